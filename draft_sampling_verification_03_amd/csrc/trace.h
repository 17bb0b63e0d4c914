// Opt-in kernel timing: while enabled, every kernel the library launches is
// bracketed by two HIP events recorded on the launch stream.  Disabled by
// default; the check costs one relaxed atomic load per launch.
#pragma once
#include <hip/hip_runtime.h>

namespace dspark {
bool trace_on();
void trace_begin(const char *name, hipStream_t stream);
void trace_end(hipStream_t stream);
}  // namespace dspark

#define DSPARK_LAUNCH(name, stream, ...)                         \
  do {                                                           \
    const bool dspark_traced_ = ::dspark::trace_on();            \
    if (dspark_traced_) ::dspark::trace_begin(name, stream);     \
    __VA_ARGS__;                                                 \
    if (dspark_traced_) ::dspark::trace_end(stream);             \
  } while (0)
