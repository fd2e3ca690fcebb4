// Kernel launch helper: launches on the caller's stream, reports launch
// failures, and brackets the launch with timing events while the profiler is on.
#pragma once

#include <hip/hip_runtime.h>

namespace dspark {

bool profiler_on();
void profiler_begin(const char* name, hipStream_t stream);
void profiler_end(hipStream_t stream);

template <typename Kernel, typename... Args>
int launch_kernel(const char* name, Kernel kernel, dim3 grid, dim3 block, hipStream_t stream,
                  Args... args) {
  const bool prof = profiler_on();
  if (prof) profiler_begin(name, stream);
  hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  const hipError_t e = hipGetLastError();
  if (prof) profiler_end(stream);
  return e == hipSuccess ? 0 : -1;
}

}  // namespace dspark
