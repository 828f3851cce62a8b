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
  // outputs and segments are strided over the grid (either count may exceed a grid
  // dimension); each output's sum over its segment is formed in one thread, in order
  const int64_t nseg = (P + seg - 1) / seg;
  for (int64_t sg = blockIdx.y; sg < nseg; sg += gridDim.y) {
    const int64_t p0 = sg * seg;
    const int64_t p1 = (p0 + seg < P) ? p0 + seg : P;
    float* o = out + sg * J;  // one row per segment (a single row if P <= seg)
    for (int64_t j = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; j < J;
         j += int64_t(gridDim.x) * blockDim.x) {
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
      o[j] = accumulate ? o[j] + s : s;
    }
  }
}

static bool single_pass(int64_t P, int64_t J) {
  return P <= kSeg || (J + 255) / 256 >= kWideBlocks;
}

int64_t reduce_tmp_floats(int64_t P, int64_t J) {
  if (single_pass(P, J)) return 0;
  const int64_t S = (P + kSeg - 1) / kSeg;
  return S * J + reduce_tmp_floats(S, J);
}

// Grid limits of the strided loops above (x: blocks of 256 outputs, y: segments).
constexpr int64_t kMaxReduceBlocksX = int64_t(1) << 20;
constexpr int64_t kMaxReduceBlocksY = 65535;

static dim3 reduce_grid(int64_t J, int64_t nseg) {
  const int64_t gx = (J + 255) / 256;
  return dim3(unsigned(gx < kMaxReduceBlocksX ? gx : kMaxReduceBlocksX),
              unsigned(nseg < kMaxReduceBlocksY ? nseg : kMaxReduceBlocksY));
}

hipError_t launch_reduce(const float* part, int64_t P, int64_t J, float* out, bool accumulate,
                         float* tmp, hipStream_t st) {
  if (J <= 0) return hipSuccess;
  const dim3 block(256);
  if (single_pass(P, J))
    return launch(k_reduce_seg, reduce_grid(J, 1), block, st, part, P, J, P, out,
                  accumulate ? 1 : 0);
  const int64_t S = (P + kSeg - 1) / kSeg;
  hipError_t e = launch(k_reduce_seg, reduce_grid(J, S), block, st, part, P, J, int64_t(kSeg),
                        tmp, 0);
  if (e != hipSuccess) return e;
  return launch_reduce(tmp, S, J, out, accumulate, tmp + S * J, st);
}

}  // namespace ssm
