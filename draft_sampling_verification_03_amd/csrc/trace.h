// Opt-in kernel timing: while enabled, every kernel the library launches
// carries a pair of HIP events in its own dispatch (hipExtLaunchKernel), which
// the runtime stamps when the kernel starts and when it ends, so the recorded
// time is the kernel's execution alone (no dispatch gap around it).  Disabled
// by default; the check costs one relaxed atomic load per launch.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace dspark {
bool trace_on();
// a fresh (start, stop) event pair for a launch of `name` (nullptr on failure)
void trace_events(const char *name, hipEvent_t *start, hipEvent_t *stop);
}  // namespace dspark

// DSPARK_LAUNCH(name, stream, kernel, grid, block, args...): launch `kernel`
// (parenthesize a template name that contains commas) with no dynamic LDS.
#define DSPARK_LAUNCH(name, stream, kernel, grid, block, ...)                                 \
  do {                                                                                        \
    hipEvent_t dspark_start_ = nullptr, dspark_stop_ = nullptr;                               \
    if (::dspark::trace_on()) ::dspark::trace_events(name, &dspark_start_, &dspark_stop_);    \
    hipExtLaunchKernelGGL(kernel, dim3(grid), dim3(block), 0, stream, dspark_start_,          \
                          dspark_stop_, 0, __VA_ARGS__);                                      \
  } while (0)
