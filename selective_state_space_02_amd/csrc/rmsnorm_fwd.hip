// Batched RMSNorm forward for gfx950, producing the per-row rms that the mamba-rs
// backward_rms_norm section takes as its saved statistic:
//   rms[r] = sqrt(mean_i x[r,i]^2 + eps),   y[r,i] = x[r,i] / rms[r] * scale[i].
// With a residual stream (RES), the norm's input is h = x + residual, stored (in the
// activation dtype) as residual_out, and the norm reads the stored h: the pair
// (residual_out, rms) is then exactly what the backward recomputes from.
//
// Mapping: one wavefront per row at a time (4 wavefronts per block walk disjoint rows);
// a lane owns PASSES groups of VEC consecutive columns.  The row is read once into
// registers (kept raw), its sum of squares is a wavefront DPP/shuffle sum, and y is
// written from the same registers; scale is staged in LDS.  HBM traffic: read x once,
// write y once (plus 4 bytes of rms per row).  Rows longer than sixteen groups per lane
// (k_rms_fwd_loop) are walked twice: the sum of squares, then y from a second read of
// the norm's input (with the residual stream, of the stored sum).
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

__device__ __forceinline__ float wave_sum_fwd(float v) {
  v = quad_sum(v);
#pragma unroll
  for (int m = 4; m < 64; m <<= 1) v += xor_lane(v, m);
  return v;
}

template <typename T, int VEC, int PASSES, bool RES>
__global__ __launch_bounds__(256) void k_rms_fwd(int64_t R, int64_t M, int64_t rows_per_block,
                                                 float eps, const T* __restrict__ x,
                                                 const T* __restrict__ res,
                                                 const float* __restrict__ scale,
                                                 T* __restrict__ y, float* __restrict__ rms,
                                                 T* __restrict__ res_out) {
  constexpr int CP = 64 * VEC;  // columns per pass
  __shared__ float ssc[PASSES * CP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < PASSES * CP; i += 256) ssc[i] = (i < M) ? scale[i] : 0.f;
  __syncthreads();
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  const float invM = 1.0f / float(M);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const T* xr = x + r * M;
    float v[PASSES][VEC];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int col = (p * 64 + lane) * VEC;
      if (col < M) {
        load_vec<T, VEC>(xr + col, v[p]);
        if constexpr (RES) {
          float rv[VEC];
          load_vec<T, VEC>(res + r * M + col, rv);
#pragma unroll
          for (int k = 0; k < VEC; ++k) v[p][k] = to_f32(from_f32<T>(v[p][k] + rv[k]));
          VecStore<T, VEC>::run(res_out + r * M + col, v[p]);
        }
      } else {
#pragma unroll
        for (int k = 0; k < VEC; ++k) v[p][k] = 0.f;
      }
    }
    float ss = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p)
#pragma unroll
      for (int k = 0; k < VEC; ++k) ss = __builtin_fmaf(v[p][k], v[p][k], ss);
    ss = wave_sum_fwd(ss);
    const float rr = __builtin_sqrtf(__builtin_fmaf(ss, invM, eps));
    const float inv = 1.0f / rr;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int col = (p * 64 + lane) * VEC;
      if (col < M) {
        float o[VEC];
#pragma unroll
        for (int k = 0; k < VEC; ++k) o[k] = v[p][k] * inv * ssc[col + k];
        VecStore<T, VEC>::run(y + r * M + col, o);
      }
    }
    if (lane == 0) rms[r] = rr;
  }
}

// Rows of any length: one wavefront per row, columns strided over the lanes, read twice.
template <typename T, int VEC, bool RES>
__global__ __launch_bounds__(256) void k_rms_fwd_loop(int64_t R, int64_t M,
                                                      int64_t rows_per_block, float eps,
                                                      const T* __restrict__ x,
                                                      const T* __restrict__ res,
                                                      const float* __restrict__ scale,
                                                      T* __restrict__ y, float* __restrict__ rms,
                                                      T* __restrict__ res_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  const float invM = 1.0f / float(M);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const T* xr = x + r * M;
    float ss = 0.f;
    for (int64_t col = int64_t(lane) * VEC; col < M; col += 64 * VEC) {
      float v[VEC];
      load_vec<T, VEC>(xr + col, v);
      if constexpr (RES) {
        float rv[VEC];
        load_vec<T, VEC>(res + r * M + col, rv);
#pragma unroll
        for (int k = 0; k < VEC; ++k) v[k] = to_f32(from_f32<T>(v[k] + rv[k]));
        VecStore<T, VEC>::run(res_out + r * M + col, v);
      }
#pragma unroll
      for (int k = 0; k < VEC; ++k) ss = __builtin_fmaf(v[k], v[k], ss);
    }
    ss = wave_sum_fwd(ss);
    const float rr = __builtin_sqrtf(__builtin_fmaf(ss, invM, eps));
    const float inv = 1.0f / rr;
    // the second read takes the norm's input as stored: x, or the stored sum (each lane
    // reads back the columns it wrote above)
    const T* hr = RES ? res_out + r * M : xr;
    for (int64_t col = int64_t(lane) * VEC; col < M; col += 64 * VEC) {
      float v[VEC], o[VEC];
      load_vec<T, VEC>(hr + col, v);
#pragma unroll
      for (int k = 0; k < VEC; ++k) o[k] = v[k] * inv * scale[col + k];
      VecStore<T, VEC>::run(y + r * M + col, o);
    }
    if (lane == 0) rms[r] = rr;
  }
}

template <typename T, int VEC, int PASSES>
static hipError_t rms_fwd_launch(const RmsFwdArgs& a, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  const T* res = static_cast<const T*>(a.residual);
  T* y = static_cast<T*>(a.y);
  T* ro = static_cast<T*>(a.residual_out);
  const dim3 grid(unsigned(a.nblk));
  hipError_t e;
  timer_mark(kKRmsFwd, false, st);
  if constexpr (PASSES == 0) {
    if (res)
      e = launch(k_rms_fwd_loop<T, VEC, true>, grid, dim3(256), st, a.R, a.M, a.rows_per_block,
                 a.eps, x, res, a.scale, y, a.rms, ro);
    else
      e = launch(k_rms_fwd_loop<T, VEC, false>, grid, dim3(256), st, a.R, a.M, a.rows_per_block,
                 a.eps, x, res, a.scale, y, a.rms, ro);
  } else {
    if (res)
      e = launch(k_rms_fwd<T, VEC, PASSES, true>, grid, dim3(256), st, a.R, a.M,
                 a.rows_per_block, a.eps, x, res, a.scale, y, a.rms, ro);
    else
      e = launch(k_rms_fwd<T, VEC, PASSES, false>, grid, dim3(256), st, a.R, a.M,
                 a.rows_per_block, a.eps, x, res, a.scale, y, a.rms, ro);
  }
  timer_mark(kKRmsFwd, true, st);
  return e;
}

template <typename T, int VEC>
static hipError_t rms_fwd_v(const RmsFwdArgs& a, hipStream_t st) {
  switch (a.passes) {
    case 0: return rms_fwd_launch<T, VEC, 0>(a, st);
    case 1: return rms_fwd_launch<T, VEC, 1>(a, st);
    case 2: return rms_fwd_launch<T, VEC, 2>(a, st);
    case 3: return rms_fwd_launch<T, VEC, 3>(a, st);
    case 4: return rms_fwd_launch<T, VEC, 4>(a, st);
    case 5: return rms_fwd_launch<T, VEC, 5>(a, st);
    case 6: return rms_fwd_launch<T, VEC, 6>(a, st);
    case 7: return rms_fwd_launch<T, VEC, 7>(a, st);
    case 8: return rms_fwd_launch<T, VEC, 8>(a, st);
    case 16: return rms_fwd_launch<T, VEC, 16>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_rmsnorm_fwd(const RmsFwdArgs& a, hipStream_t st) {
  if (a.dtype == 0) return (a.vec == 4) ? rms_fwd_v<float, 4>(a, st) : rms_fwd_v<float, 1>(a, st);
  return (a.vec == 8) ? rms_fwd_v<bf16_t, 8>(a, st) : rms_fwd_v<bf16_t, 1>(a, st);
}

}  // namespace ssm
