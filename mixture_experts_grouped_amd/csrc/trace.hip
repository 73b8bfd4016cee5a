// trace.hip -- optional per-kernel timing with HIP events recorded on the
// launch stream around every kernel of the library (off by default).
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/moelora.h"
#include "trace.hpp"

namespace moelora {

namespace {
struct Pending {
  const char* name;
  hipEvent_t a, b;
};
struct Stat {
  int64_t launches = 0;
  double ms = 0.0;
};
std::mutex g_mu;
bool g_on = false;
std::vector<hipEvent_t> g_free;
std::vector<Pending> g_pending;
hipEvent_t g_open = nullptr;
std::map<std::string, Stat> g_stats;
std::vector<std::string> g_order;

hipEvent_t get_event() {
  if (!g_free.empty()) {
    hipEvent_t e = g_free.back();
    g_free.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

bool trace_on() { return g_on; }

void trace_begin(hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_open = get_event();
  if (g_open != nullptr && hipEventRecord(g_open, st) != hipSuccess) {  // not traced
    g_free.push_back(g_open);
    g_open = nullptr;
  }
}

void trace_end(const char* name, hipStream_t st) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_open == nullptr) return;
  hipEvent_t b = get_event();
  if (b == nullptr) return;
  if (hipEventRecord(b, st) != hipSuccess) {  // drop this launch from the trace
    g_free.push_back(g_open);
    g_free.push_back(b);
    g_open = nullptr;
    return;
  }
  g_pending.push_back(Pending{name, g_open, b});
  g_open = nullptr;
}

}  // namespace moelora

using namespace moelora;

extern "C" {

void moe_lora_trace_enable(int32_t on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_on = on != 0;
}

moe_status moe_lora_trace_collect(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  for (const Pending& p : g_pending) {
    if (hipEventSynchronize(p.b) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.0f;
    if (hipEventElapsedTime(&ms, p.a, p.b) != hipSuccess) return MOE_ERR_HIP;
    std::string key(p.name);
    key = key.substr(0, key.find('<'));  // template instances count under the kernel's name
    auto it = g_stats.find(key);
    if (it == g_stats.end()) {
      g_order.push_back(key);
      it = g_stats.emplace(key, Stat{}).first;
    }
    it->second.launches += 1;
    it->second.ms += ms;
    g_free.push_back(p.a);
    g_free.push_back(p.b);
  }
  g_pending.clear();
  return MOE_OK;
}

void moe_lora_trace_reset(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_stats.clear();
  g_order.clear();
}

int32_t moe_lora_trace_count(void) {
  std::lock_guard<std::mutex> lk(g_mu);
  return (int32_t)g_order.size();
}

moe_status moe_lora_trace_entry(int32_t i, const char** name, int64_t* launches, double* total_ms) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (i < 0 || i >= (int32_t)g_order.size() || name == nullptr || launches == nullptr ||
      total_ms == nullptr)
    return MOE_ERR_INVALID;
  auto it = g_stats.find(g_order[i]);
  *name = it->first.c_str();
  *launches = it->second.launches;
  *total_ms = it->second.ms;
  return MOE_OK;
}

}  // extern "C"
