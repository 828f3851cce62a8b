// Fixed-order sum of partial buffers, out[j] (+)= sum_p part[p][j].  No atomics: the
// order of every addition is fixed by the code, so results are bit-identical from run
// to run (the atomicAdd-free scratch-plus-reduce pattern of the foxhunt ml-alpha
// backward-scratch commit, applied after the partials were pre-reduced in registers
// and LDS).
//
// One thread per output j sums a segment of partials with kAcc independent accumulators
// (partial p goes to accumulator p mod kAcc, in increasing p; the accumulators are then
// added in index order).  Loads are issued kBatch at a time before they are added, so a
// thread waits one memory latency per kBatch partials (narrow outputs are latency-bound).  When the outputs alone fill the GPU
// (at least kWideBlocks blocks of 256) or P <= kSeg, one launch sums all P partials.
// Otherwise a first launch writes one sum per segment of kSeg partials to a temporary
// buffer and the segments are summed the same way (reduce_tmp_floats() floats of
// temporary space), so that narrow outputs still spread over many blocks.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

constexpr int kSeg = 64;
constexpr int kAcc = 4;
constexpr int kBatch = 16;  // a multiple of kAcc
constexpr int64_t kWideBlocks = 1024;

__global__ __launch_bounds__(256) void k_reduce_seg(const float* __restrict__ part, int64_t P,
                                                    int64_t J, int64_t seg,
                                                    float* __restrict__ out, int accumulate) {
  const int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (j >= J) return;
  const int64_t p0 = int64_t(blockIdx.y) * seg;
  const int64_t p1 = (p0 + seg < P) ? p0 + seg : P;
  float acc[kAcc] = {0.f, 0.f, 0.f, 0.f};
  int64_t p = p0;
  for (; p + kBatch <= p1; p += kBatch) {
    float v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) v[k] = part[(p + k) * J + j];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) acc[k % kAcc] += v[k];
  }
  if (p < p1) {  // the last, partial batch: loads clamped to the segment, extra values dropped
    float v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) v[k] = part[(p + k < p1 ? p + k : p1 - 1) * J + j];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (p + k < p1) acc[k % kAcc] += v[k];
  }
  const float s = (acc[0] + acc[1]) + (acc[2] + acc[3]);
  float* o = out + int64_t(blockIdx.y) * J;  // one row per segment (a single row if P <= kSeg)
  o[j] = accumulate ? o[j] + s : s;
}

static bool single_pass(int64_t P, int64_t J) {
  return P <= kSeg || (J + 255) / 256 >= kWideBlocks;
}

int64_t reduce_tmp_floats(int64_t P, int64_t J) {
  if (single_pass(P, J)) return 0;
  const int64_t S = (P + kSeg - 1) / kSeg;
  return S * J + reduce_tmp_floats(S, J);
}

hipError_t launch_reduce(const float* part, int64_t P, int64_t J, float* out, bool accumulate,
                         float* tmp, hipStream_t st) {
  if (J <= 0) return hipSuccess;
  const dim3 block(256);
  const int64_t gx = (J + 255) / 256;
  if (single_pass(P, J)) {
    hipLaunchKernelGGL(k_reduce_seg, dim3(gx, 1), block, 0, st, part, P, J, P, out,
                       accumulate ? 1 : 0);
    return hipGetLastError();
  }
  const int64_t S = (P + kSeg - 1) / kSeg;
  hipLaunchKernelGGL(k_reduce_seg, dim3(gx, S), block, 0, st, part, P, J, int64_t(kSeg), tmp,
                     0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_reduce(tmp, S, J, out, accumulate, tmp + S * J, st);
}

}  // namespace ssm
