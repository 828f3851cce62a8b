// Fixed-order sum of partial buffers: out[j] (+)= part[0][j] + part[1][j] + ... in
// index order, one thread per output.  No atomics, so results are bit-identical from
// run to run (the atomicAdd-free scratch-plus-reduce pattern of the foxhunt ml-alpha
// backward-scratch commit, with the partials pre-reduced in registers/LDS first).
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

__global__ __launch_bounds__(256) void k_reduce(const float* __restrict__ part, int64_t P,
                                                int64_t J, float* __restrict__ out,
                                                int accumulate) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= J) return;
  float s = 0.f;
  for (int64_t p = 0; p < P; ++p) s += part[p * J + j];
  out[j] = accumulate ? out[j] + s : s;
}

hipError_t launch_reduce(const float* part, int64_t P, int64_t J, float* out, bool accumulate,
                         hipStream_t st) {
  if (J <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_reduce, dim3((J + 255) / 256), dim3(256), 0, st, part, P, J, out,
                     accumulate ? 1 : 0);
  return hipGetLastError();
}

}  // namespace ssm
