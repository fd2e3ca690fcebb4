// Kernel launch helper: launches on the caller's stream, reports launch
// failures, and while the profiler is on times the launch with the start and
// stop events of hipExtLaunchKernel, which the dispatch itself records around
// the kernel's execution (no separate event packets in the stream).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

namespace dspark {

bool profiler_on();
// Opens the timing of one launch of kernel `name`: fills the event pair (false
// when the events cannot be made; the launch then goes untimed).
bool profiler_begin(const char* name, hipEvent_t* start, hipEvent_t* stop);
// Closes it: the pair joins the pending measurements read at the next profiler_read.
void profiler_end(hipEvent_t start, hipEvent_t stop);

template <typename Kernel, typename... Args>
int launch_kernel(const char* name, Kernel kernel, dim3 grid, dim3 block, hipStream_t stream,
                  Args... args) {
  hipEvent_t start = nullptr, stop = nullptr;
  const bool prof = profiler_on() && profiler_begin(name, &start, &stop);
  if (prof) hipExtLaunchKernelGGL(kernel, grid, block, 0, stream, start, stop, 0, args...);
  else hipLaunchKernelGGL(kernel, grid, block, 0, stream, args...);
  const hipError_t e = hipGetLastError();
  if (prof) profiler_end(start, stop);
  return e == hipSuccess ? 0 : -1;
}

}  // namespace dspark
