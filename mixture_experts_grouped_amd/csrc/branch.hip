// branch.hip -- the second stream of each device for the independent
// branches of a layer call (class Branch in layer.hpp).
#include "layer.hpp"

namespace moelora {

namespace {
constexpr int kMaxDevices = 64;
struct DeviceBranch {
  std::mutex mu;
  bool tried = false;  // creation attempted (once per device)
  hipStream_t side = nullptr;
  hipEvent_t ev[Branch::NEV] = {};
};
DeviceBranch g_branch[kMaxDevices];
}  // namespace

hipError_t Branch::open(hipStream_t st, bool allow) {
  main_ = side_ = st;
  ev_ = nullptr;
  if (!allow) return hipSuccess;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  hipError_t e = hipStreamIsCapturing(st, &cs);
  if (e != hipSuccess) return e;
  if (cs != hipStreamCaptureStatusNone) return hipSuccess;  // graph capture: one stream
  int dev = 0;
  if ((e = hipGetDevice(&dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipSuccess;
  DeviceBranch& b = g_branch[dev];
  std::unique_lock<std::mutex> lk(b.mu);
  if (!b.tried) {
    b.tried = true;
    bool ok = hipStreamCreateWithFlags(&b.side, hipStreamNonBlocking) == hipSuccess;
    for (int i = 0; ok && i < NEV; ++i) ok = hipEventCreateWithFlags(&b.ev[i], hipEventDisableTiming) == hipSuccess;
    if (!ok) {  // keep running on one stream
      for (int i = 0; i < NEV; ++i)
        if (b.ev[i] != nullptr) (void)hipEventDestroy(b.ev[i]);
      if (b.side != nullptr) (void)hipStreamDestroy(b.side);
      b.side = nullptr;
      (void)hipGetLastError();
    }
  }
  if (b.side == nullptr) return hipSuccess;
  lk_ = std::move(lk);
  side_ = b.side;
  ev_ = b.ev;
  // fork: the branch starts after the caller's stream so far
  if ((e = hipEventRecord(ev_[0], main_)) != hipSuccess) return e;
  return hipStreamWaitEvent(side_, ev_[0], 0);
}

hipError_t Branch::signal(hipStream_t from, int i) {
  return ev_ == nullptr ? hipSuccess : hipEventRecord(ev_[i], from);
}

hipError_t Branch::await(hipStream_t to, int i) {
  return ev_ == nullptr ? hipSuccess : hipStreamWaitEvent(to, ev_[i], 0);
}

hipError_t Branch::close() {
  if (ev_ == nullptr) return hipSuccess;
  // join: the caller's stream continues after all of the branch
  hipError_t e = hipEventRecord(ev_[0], side_);
  if (e == hipSuccess) e = hipStreamWaitEvent(main_, ev_[0], 0);
  ev_ = nullptr;
  side_ = main_;
  if (lk_.owns_lock()) lk_.unlock();
  return e;
}

}  // namespace moelora
