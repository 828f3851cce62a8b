// One-token decode steps for gfx950: the scan's single-step updater (the rustytorch
// commit's "single-step updater" for inference) and the causal conv1d window step.
//
// Scan step: for every (b, d, n)
//   h[b,d,n] <- exp(delta_t[b,d] A[d,n]) h[b,d,n] + delta_t[b,d] B_t[b,n] x_t[b,d]
//   y_t[b,d]  = sum_n C_t[b,n] h[b,d,n] + Dv[d] x_t[b,d]
// with the scan kernels' lane layout (four lanes per channel, NS = N/4 consecutive
// states per lane, the sum over n a quad sum) and their per-step arithmetic, so a
// sequence decoded token by token reproduces a single-chunk scan exactly.  Each
// (b, d) is computed independently in a fixed order: results do not depend on which
// other rows share the batch.
//
// Conv step: state [B][K-1][D] holds the last K-1 inputs, oldest first (channels-last,
// so a wavefront reads 64 consecutive channels); out_t = bias + sum_k W[d,k] window[k]
// over the window (state, x_t), in the conv forward kernel's order; the window then
// moves one step.
//
// Fused forms, as the sequence kernels' (same functions, same order, so decoding stays
// bit-identical to them): the scan step's time step softplus(delta_t + bias) (FZ) and
// output gate y * silu(z_t); the conv step's SiLU (ACT); and the decode token of the
// block's scan branch, conv step -> SiLU -> fused scan step in one launch.
//
// Both are HBM-bound: the scan step reads and writes h (8 bytes per state), the conv
// step reads and writes the window.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

// One scan step for the channel (b, d) of a quad (lane q holds states q*NS .. q*NS+NS-1),
// in two phases so that a caller can have every load in flight before it forms the
// step's input xv: step_load issues the step's loads (raw values, no arithmetic, no
// branch, so that no load waits for another), step_compute advances h and writes the
// output.  Shared by the scan step and the decode token.
template <typename T, int N>
struct StepOperands {
  static constexpr int NS = N / 4;
  float hv[NS], Av[NS], Bv[NS], Cv[NS];
  float bias, Dd;
  T draw, zraw;
};

template <typename T, int N, bool FZ>
__device__ __forceinline__ void step_load(StepOperands<T, N>& o, int64_t b, int64_t d,
                                          int64_t D, int q, const float* __restrict__ h,
                                          const T* __restrict__ delta_t,
                                          const float* __restrict__ A,
                                          const T* __restrict__ B_t, const T* __restrict__ C_t,
                                          const float* __restrict__ Dv,
                                          const float* __restrict__ dtb,
                                          const T* __restrict__ z_t) {
  constexpr int NS = N / 4;
  const int64_t bd = b * D + d;
  o.draw = delta_t[bd];
  if constexpr (FZ) {
    // absent operands read a valid stand-in address; the value is not used
    o.bias = (dtb ? dtb : Dv)[d];
    o.zraw = (z_t ? z_t : delta_t)[bd];
  }
  VecLoad<float, NS>::run(h + bd * N + q * NS, o.hv);
  VecLoad<float, NS>::run(A + d * N + q * NS, o.Av);
  load_vec<T, NS>(B_t + b * N + q * NS, o.Bv);
  load_vec<T, NS>(C_t + b * N + q * NS, o.Cv);
  o.Dd = Dv[d];
}

template <typename T, int N, bool FZ>
__device__ __forceinline__ void step_compute(StepOperands<T, N>& o, int64_t b, int64_t d,
                                             int64_t D, int q, float xv, float* __restrict__ h,
                                             const float* __restrict__ dtb, bool sp,
                                             const T* __restrict__ z_t, T* __restrict__ y_t) {
  constexpr int NS = N / 4;
  const int64_t bd = b * D + d;
  float dl = to_f32(o.draw);
  if constexpr (FZ) {
    dl += dtb ? o.bias : 0.f;
    if (sp) dl = softplus_f(dl);
  }
  const float u = dl * xv;
  float yp;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float a = __builtin_amdgcn_exp2f(dl * (o.Av[j] * kLog2e));
    o.hv[j] = __builtin_fmaf(a, o.hv[j], u * o.Bv[j]);
    yp = j ? __builtin_fmaf(o.Cv[j], o.hv[j], yp) : o.Cv[j] * o.hv[j];
  }
  yp = quad_sum(yp);
  VecStore<float, NS>::run(h + bd * N + q * NS, o.hv);
  // every lane forms y (the quad's lanes agree); the use below keeps the operand loads
  // where step_load put them instead of inside the single-lane store
  float yv = __builtin_fmaf(o.Dd, xv, yp);
  if constexpr (FZ) {
    const float zv = to_f32(o.zraw);
    if (z_t) yv *= zv * sigmoid_f(zv);
  }
  asm volatile("" ::"v"(yv));
  if (q == 0) y_t[bd] = from_f32<T>(yv);
}

template <typename T, int N, bool FZ>
__global__ __launch_bounds__(256) void k_scan_step(int64_t B, int64_t D, float* __restrict__ h,
                                                   const T* __restrict__ x_t,
                                                   const T* __restrict__ delta_t,
                                                   const float* __restrict__ A,
                                                   const T* __restrict__ B_t,
                                                   const T* __restrict__ C_t,
                                                   const float* __restrict__ Dv,
                                                   const float* __restrict__ dtb, bool sp,
                                                   const T* __restrict__ z_t,
                                                   T* __restrict__ y_t) {
  const int tid = threadIdx.x, q = tid & 3, cl = tid >> 2;
  const WgPos wp = wg_pos((D + 63) / 64, B);  // (channel group, batch row)
  const int64_t b = wp.b, d = wp.grp * 64 + cl;
  if (d >= D) return;  // a channel's four lanes leave together; the quad sum stays in-quad
  StepOperands<T, N> o;
  const T xr = x_t[b * D + d];
  step_load<T, N, FZ>(o, b, d, D, q, h, delta_t, A, B_t, C_t, Dv, dtb, z_t);
  step_compute<T, N, FZ>(o, b, d, D, q, to_f32(xr), h, dtb, sp, z_t, y_t);
}

// One decode token of the block's scan branch: the conv step on x_t (window [B][K-1][D]),
// its SiLU, the result rounded to T as the two-call path stores it, then the fused scan
// step on it.  The channel's four lanes share the window's loads and stores and all form
// the conv output (same operations in the conv step's order, same value).
template <typename T, int N, int K>
__global__ __launch_bounds__(256) void k_decode_step(int64_t B, int64_t D, float* __restrict__ h,
                                                     T* __restrict__ cstate,
                                                     const T* __restrict__ x_t,
                                                     const float* __restrict__ W,
                                                     const float* __restrict__ cbias,
                                                     const T* __restrict__ delta_t,
                                                     const float* __restrict__ A,
                                                     const T* __restrict__ B_t,
                                                     const T* __restrict__ C_t,
                                                     const float* __restrict__ Dv,
                                                     const float* __restrict__ dtb, bool sp,
                                                     const T* __restrict__ z_t,
                                                     T* __restrict__ out_t) {
  // The conv window of the group's 64 channels (K-1 stored rows, then x_t as tap K-1)
  // is staged through LDS: thread t moves row t/64 of channel t%64, so each row is read
  // and written as one contiguous run of 64 values.
  __shared__ float sw[K][64];
  const int tid = threadIdx.x, q = tid & 3, cl = tid >> 2;
  const WgPos wp = wg_pos((D + 63) / 64, B);  // (channel group, batch row)
  const int64_t b = wp.b, d0 = wp.grp * 64, d = d0 + cl;
  const int rc = tid & 63;
  // every load is issued before the barrier; lanes past the last channel read the last
  // channel's addresses (in bounds) and drop the values
  const int64_t dc = d < D ? d : D - 1, rcol = d0 + rc < D ? d0 + rc : D - 1;
  StepOperands<T, N> o;
  step_load<T, N, true>(o, b, dc, D, q, h, delta_t, A, B_t, C_t, Dv, dtb, z_t);
  float wk[K];
#pragma unroll
  for (int k = 0; k < K; ++k) wk[k] = W[dc * K + k];
  const float cb = cbias ? cbias[dc] : 0.f;
  T raw[(K + 3) / 4];
#pragma unroll
  for (int i = 0; i < (K + 3) / 4; ++i) {
    const int r = (tid >> 6) + 4 * i;  // uniform over the wavefront
    const T* row = x_t + b * D;  // tap K-1; the stored rows (none when K = 1) before it
    if constexpr (K > 1) {
      if (r < K - 1) row = cstate + (b * (K - 1) + r) * D;
    }
    if (r < K) raw[i] = row[rcol];
  }
#pragma unroll
  for (int i = 0; i < (K + 3) / 4; ++i) {
    const int r = (tid >> 6) + 4 * i;
    if (r < K) sw[r][rc] = to_f32(raw[i]);
  }
  __syncthreads();  // every read of the window is done before any row is rewritten
  // the window moves up one row (the values came from T, so storing them back is exact)
  if (d0 + rc < D)
    for (int r = tid >> 6; r < K - 1; r += 4)
      cstate[(b * (K - 1) + r) * D + d0 + rc] = from_f32<T>(sw[r + 1][rc]);
  if (d >= D) return;  // a channel's four lanes leave together (the quad sum stays in-quad)
  float acc = cb;
#pragma unroll
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(wk[k], sw[k][cl], acc);
  acc *= sigmoid_f(acc);
  const float xv = to_f32(from_f32<T>(acc));
  step_compute<T, N, true>(o, b, d, D, q, xv, h, dtb, sp, z_t, out_t);
}

// One token of the causal conv for VEC consecutive channels per thread (VEC = 4 when D is
// a multiple of 4, moving 8 or 16 bytes per access, else 1).  blockIdx.x picks the channel
// group; the batch rows are walked from blockIdx.y in steps of gridDim.y, which the host
// sets to about B / kConvStepRows, so the grid needs no 64-bit index division, any B fits,
// and the taps and bias of the thread's channels are read once for all its rows.
constexpr int kConvStepRows = 4;
template <typename T, int K, int ACT, int VEC>
__global__ __launch_bounds__(256) void k_conv_step(int64_t B, int64_t D, T* __restrict__ state,
                                                   const T* __restrict__ x_t,
                                                   const float* __restrict__ W,
                                                   const float* __restrict__ bias,
                                                   T* __restrict__ out_t) {
  const int64_t d0 = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) * VEC;
  if (d0 >= D) return;
  // the VEC*K taps of the thread's channels are contiguous (and 16-byte aligned for VEC =
  // 4, as W is): read them, and the biases, as 16-byte vectors
  float w[VEC][K], bv[VEC];
  if constexpr (VEC == 4) {
    float wf[4 * K];
#pragma unroll
    for (int i = 0; i < K; ++i) {
      const float4 v = reinterpret_cast<const float4*>(W + d0 * K)[i];
      wf[4 * i] = v.x; wf[4 * i + 1] = v.y; wf[4 * i + 2] = v.z; wf[4 * i + 3] = v.w;
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int k = 0; k < K; ++k) w[c][k] = wf[c * K + k];
    const float4 bb = bias ? *reinterpret_cast<const float4*>(bias + d0) : make_float4(0.f, 0.f, 0.f, 0.f);
    bv[0] = bb.x; bv[1] = bb.y; bv[2] = bb.z; bv[3] = bb.w;
  } else {
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
#pragma unroll
      for (int k = 0; k < K; ++k) w[c][k] = W[(d0 + c) * K + k];
      bv[c] = bias ? bias[d0 + c] : 0.f;
    }
  }
  for (int64_t b = blockIdx.y; b < B; b += gridDim.y) {
    float win[K][VEC];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) VecLoad<T, VEC>::run(state + (b * (K - 1) + k) * D + d0, win[k]);
    VecLoad<T, VEC>::run(x_t + b * D + d0, win[K - 1]);
    float acc[VEC];
#pragma unroll
    for (int c = 0; c < VEC; ++c) {
      acc[c] = bv[c];
#pragma unroll
      for (int k = 0; k < K; ++k) acc[c] = __builtin_fmaf(w[c][k], win[k][c], acc[c]);
      if constexpr (ACT == kActSilu) acc[c] *= sigmoid_f(acc[c]);
    }
    VecStore<T, VEC>::run(out_t + b * D + d0, acc);
    // the window moves up one row (the values came from T, so storing them back is exact)
#pragma unroll
    for (int k = 0; k < K - 1; ++k) VecStore<T, VEC>::run(state + (b * (K - 1) + k) * D + d0, win[k + 1]);
  }
}

template <typename T, int N, bool FZ>
static hipError_t scan_step_nf(const ScanStepArgs& a, hipStream_t st) {
  return launch(k_scan_step<T, N, FZ>, dim3(unsigned((a.D + 63) / 64 * a.B)), dim3(256), st,
                a.B, a.D, a.h, static_cast<const T*>(a.x_t), static_cast<const T*>(a.delta_t),
                a.A, static_cast<const T*>(a.B_t), static_cast<const T*>(a.C_t), a.Dv,
                a.dt_bias, a.dt_softplus, static_cast<const T*>(a.z_t), static_cast<T*>(a.y_t));
}

template <typename T, int N>
static hipError_t scan_step_n(const ScanStepArgs& a, hipStream_t st) {
  timer_mark(kKScanStep, false, st);
  const hipError_t e = a.fused ? scan_step_nf<T, N, true>(a, st) : scan_step_nf<T, N, false>(a, st);
  timer_mark(kKScanStep, true, st);
  return e;
}

template <typename T>
static hipError_t scan_step_t(const ScanStepArgs& a, hipStream_t st) {
  switch (a.N) {
    case 4: return scan_step_n<T, 4>(a, st);
    case 8: return scan_step_n<T, 8>(a, st);
    case 16: return scan_step_n<T, 16>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_scan_step(const ScanStepArgs& a, hipStream_t st) {
  return a.dtype == 0 ? scan_step_t<float>(a, st) : scan_step_t<bf16_t>(a, st);
}

template <typename T, int K, int ACT, int VEC>
static hipError_t conv_step_kav(const ConvStepArgs& a, hipStream_t st) {
  const int64_t groups = (a.D + VEC - 1) / VEC;
  const int64_t gy = (a.B + kConvStepRows - 1) / kConvStepRows;
  const dim3 grid(unsigned((groups + 255) / 256), unsigned(gy < 65535 ? gy : 65535));
  return launch(k_conv_step<T, K, ACT, VEC>, grid, dim3(256), st, a.B, a.D,
                static_cast<T*>(a.state), static_cast<const T*>(a.x_t), a.W, a.bias,
                static_cast<T*>(a.out_t));
}

template <typename T, int K, int ACT>
static hipError_t conv_step_ka(const ConvStepArgs& a, hipStream_t st) {
  return a.D % 4 == 0 ? conv_step_kav<T, K, ACT, 4>(a, st) : conv_step_kav<T, K, ACT, 1>(a, st);
}

template <typename T, int K>
static hipError_t conv_step_k(const ConvStepArgs& a, hipStream_t st) {
  timer_mark(kKConvStep, false, st);
  const hipError_t e = a.act == kActSilu ? conv_step_ka<T, K, kActSilu>(a, st)
                                         : conv_step_ka<T, K, kActNone>(a, st);
  timer_mark(kKConvStep, true, st);
  return e;
}

template <typename T>
static hipError_t conv_step_t(const ConvStepArgs& a, hipStream_t st) {
  switch (a.K) {
    case 1: return conv_step_k<T, 1>(a, st);
    case 2: return conv_step_k<T, 2>(a, st);
    case 3: return conv_step_k<T, 3>(a, st);
    case 4: return conv_step_k<T, 4>(a, st);
    case 5: return conv_step_k<T, 5>(a, st);
    case 6: return conv_step_k<T, 6>(a, st);
    case 7: return conv_step_k<T, 7>(a, st);
    case 8: return conv_step_k<T, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T, int N, int K>
static hipError_t decode_step_nk(const DecodeArgs& a, hipStream_t st) {
  return launch(k_decode_step<T, N, K>, dim3(unsigned((a.D + 63) / 64 * a.B)), dim3(256), st,
                a.B, a.D, a.h, static_cast<T*>(a.conv_state), static_cast<const T*>(a.x_t), a.W,
                a.conv_bias, static_cast<const T*>(a.delta_t), a.A,
                static_cast<const T*>(a.B_t), static_cast<const T*>(a.C_t), a.Dv, a.dt_bias,
                a.dt_softplus, static_cast<const T*>(a.z_t), static_cast<T*>(a.out_t));
}

template <typename T, int N>
static hipError_t decode_step_n(const DecodeArgs& a, hipStream_t st) {
  switch (a.K) {
    case 1: return decode_step_nk<T, N, 1>(a, st);
    case 2: return decode_step_nk<T, N, 2>(a, st);
    case 3: return decode_step_nk<T, N, 3>(a, st);
    case 4: return decode_step_nk<T, N, 4>(a, st);
    case 5: return decode_step_nk<T, N, 5>(a, st);
    case 6: return decode_step_nk<T, N, 6>(a, st);
    case 7: return decode_step_nk<T, N, 7>(a, st);
    case 8: return decode_step_nk<T, N, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

template <typename T>
static hipError_t decode_step_t(const DecodeArgs& a, hipStream_t st) {
  hipError_t e = hipErrorInvalidValue;
  timer_mark(kKDecodeStep, false, st);
  switch (a.N) {
    case 4: e = decode_step_n<T, 4>(a, st); break;
    case 8: e = decode_step_n<T, 8>(a, st); break;
    case 16: e = decode_step_n<T, 16>(a, st); break;
  }
  timer_mark(kKDecodeStep, true, st);
  return e;
}

hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t st) {
  return a.dtype == 0 ? decode_step_t<float>(a, st) : decode_step_t<bf16_t>(a, st);
}

hipError_t launch_conv1d_step(const ConvStepArgs& a, hipStream_t st) {
  return a.dtype == 0 ? conv_step_t<float>(a, st) : conv_step_t<bf16_t>(a, st);
}

}  // namespace ssm
