// The per-decision uniforms as a standalone call, so that the device Philox
// can be compared word for word with an independent implementation.
#include "common.hpp"
#include "launch.hpp"

namespace dspark {

__global__ __launch_bounds__(256) void uniforms_kernel(uint64_t seed, uint64_t step, int n, uint32_t position,
                                                       uint32_t purpose, float* out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = decision_uniform(seed, step, (uint32_t)i, position, purpose);
}

int run_uniforms(uint64_t seed, uint64_t step, int n, int position, int purpose, float* out, hipStream_t stream) {
  return launch_kernel("uniforms", uniforms_kernel, dim3((n + 255) / 256), dim3(256), stream, seed, step, n,
                       (uint32_t)position, (uint32_t)purpose, out);
}

}  // namespace dspark
