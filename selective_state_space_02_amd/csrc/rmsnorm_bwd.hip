// Batched RMSNorm backward for gfx950, given the saved per-row rms (not its inverse),
// as the mamba-rs backward_rms_norm section defines it.  With inv = 1/rms[r] and
//   c[r] = inv^2 * (sum_i dy[r,i] scale[i] x[r,i]) / M,
// the input gradient is dx[r,i] = inv (scale[i] dy[r,i] - x[r,i] c[r]) (overwritten)
// and the scale gradient dscale[i] += sum_r dy[r,i] x[r,i] inv (accumulated).
//
// Mapping: one wavefront per row at a time (4 wavefronts per block walk disjoint
// rows); a lane owns PASSES groups of VEC consecutive columns.  Pass 1 reads the row
// and forms the dot product (wavefront DPP/shuffle sum); pass 2 re-reads it (cache
// hit), writes dx and accumulates the scale-gradient terms in registers.  At the end
// the four wavefronts' column sums are added through LDS into one partial per block;
// k_reduce sums the block partials in a fixed order.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

__device__ __forceinline__ float wave_sum(float v) {
  v = quad_sum(v);
#pragma unroll
  for (int m = 4; m < 64; m <<= 1) v += xor_lane(v, m);
  return v;
}

template <typename T, int VEC, int PASSES>
__global__ __launch_bounds__(256) void k_rms_bwd(
    int64_t R, int64_t M, int64_t rows_per_block, const T* __restrict__ dy,
    const T* __restrict__ x, const float* __restrict__ scale, const float* __restrict__ rms,
    T* __restrict__ dx, float* __restrict__ dsp) {
  __shared__ float part[4][64 * VEC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[PASSES][VEC], sc[PASSES][VEC];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t col = (int64_t(p) * 64 + lane) * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      acc[p][v] = 0.f;
      sc[p][v] = (col < M) ? scale[col + v] : 0.f;
    }
  }
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  const float invM = 1.0f / float(M);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const float inv = 1.0f / rms[r];
    const T* dyr = dy + r * M;
    const T* xr = x + r * M;
    float dot = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t col = (int64_t(p) * 64 + lane) * VEC;
      if (col < M) {
        float a[VEC], b[VEC];
        load_vec<T, VEC>(dyr + col, a);
        load_vec<T, VEC>(xr + col, b);
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot = __builtin_fmaf(a[v] * sc[p][v], b[v], dot);
      }
    }
    dot = wave_sum(dot);
    const float cr = dot * inv * inv * invM;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t col = (int64_t(p) * 64 + lane) * VEC;
      if (col < M) {
        float a[VEC], b[VEC], o[VEC];
        load_vec<T, VEC>(dyr + col, a);
        load_vec<T, VEC>(xr + col, b);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          o[v] = inv * __builtin_fmaf(sc[p][v], a[v], -b[v] * cr);
          acc[p][v] = __builtin_fmaf(a[v] * b[v], inv, acc[p][v]);
        }
        VecStore<T, VEC>::run(dx + r * M + col, o);
      }
    }
  }
  // sum the four wavefronts' column partials
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) part[wave][lane * VEC + v] = acc[p][v];
    __syncthreads();
    for (int k = tid; k < 64 * VEC; k += 256) {
      const int64_t col = int64_t(p) * 64 * VEC + k;
      if (col < M)
        dsp[int64_t(blockIdx.x) * M + col] = (part[0][k] + part[1][k]) + (part[2][k] + part[3][k]);
    }
    __syncthreads();
  }
}

template <typename T, int VEC, int PASSES>
static void rms_launch(const RmsArgs& a, const RmsPlan& p, hipStream_t st) {
  timer_mark(kKRmsBwd, false, st);
  hipLaunchKernelGGL((k_rms_bwd<T, VEC, PASSES>), dim3(p.nblk), dim3(256), 0, st, a.R, a.M,
                     p.rows_per_block, static_cast<const T*>(a.dy), static_cast<const T*>(a.x),
                     a.scale, a.rms, static_cast<T*>(a.dx), p.dsp);
  timer_mark(kKRmsBwd, true, st);
}

template <typename T, int VEC>
static hipError_t rms_v(const RmsArgs& a, const RmsPlan& p, hipStream_t st) {
  switch (p.passes) {
    case 1: rms_launch<T, VEC, 1>(a, p, st); break;
    case 2: rms_launch<T, VEC, 2>(a, p, st); break;
    case 4: rms_launch<T, VEC, 4>(a, p, st); break;
    case 8: rms_launch<T, VEC, 8>(a, p, st); break;
    case 16: rms_launch<T, VEC, 16>(a, p, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const RmsArgs& a, const RmsPlan& p, hipStream_t st) {
  hipError_t e;
  if (a.dtype == 0)
    e = (p.vec == 4) ? rms_v<float, 4>(a, p, st) : rms_v<float, 1>(a, p, st);
  else
    e = (p.vec == 8) ? rms_v<bf16_t, 8>(a, p, st) : rms_v<bf16_t, 1>(a, p, st);
  if (e != hipSuccess) return e;
  return launch_reduce(p.dsp, p.nblk, a.M, a.dscale, true, p.rtmp, st);
}

}  // namespace ssm
