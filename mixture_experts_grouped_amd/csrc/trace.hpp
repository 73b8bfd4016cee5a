// trace.hpp -- per-kernel HIP-event tracing hooks (see trace.hip).
#pragma once
#include <hip/hip_runtime.h>

namespace moelora {
bool trace_on();
void trace_begin(hipStream_t st);
void trace_end(const char* name, hipStream_t st);
}  // namespace moelora

// Launch a kernel; with tracing on, bracket it with events on its stream and
// account it under `name` (MOE_LAUNCH: the kernel's own name).
#define MOE_LAUNCH_AS(name, kern, grid, block, lds, st, ...)         \
  do {                                                               \
    const bool moe_tr_ = ::moelora::trace_on();                      \
    if (moe_tr_) ::moelora::trace_begin(st);                         \
    hipLaunchKernelGGL(kern, grid, block, lds, st, __VA_ARGS__);     \
    if (moe_tr_) ::moelora::trace_end(name, st);                     \
  } while (0)
#define MOE_LAUNCH(kern, grid, block, lds, st, ...) \
  MOE_LAUNCH_AS(#kern, kern, grid, block, lds, st, __VA_ARGS__)
