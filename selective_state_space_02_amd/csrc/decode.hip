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
// output gate y * silu(z_t); the conv step's SiLU (ACT).
//
// Both are HBM-bound: the scan step reads and writes h (8 bytes per state), the conv
// step reads and writes the window.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

template <typename T, int N, bool FZ>
__global__ __launch_bounds__(256) void k_scan_step(int64_t D, float* __restrict__ h,
                                                   const T* __restrict__ x_t,
                                                   const T* __restrict__ delta_t,
                                                   const float* __restrict__ A,
                                                   const T* __restrict__ B_t,
                                                   const T* __restrict__ C_t,
                                                   const float* __restrict__ Dv,
                                                   const float* __restrict__ dtb, bool sp,
                                                   const T* __restrict__ z_t,
                                                   T* __restrict__ y_t) {
  constexpr int NS = N / 4;
  const int tid = threadIdx.x, q = tid & 3, cl = tid >> 2;
  const int64_t b = blockIdx.y, d = int64_t(blockIdx.x) * 64 + cl;
  if (d >= D) return;  // a channel's four lanes leave together; the quad sum stays in-quad
  const int64_t bd = b * D + d;
  const float xv = to_f32(x_t[bd]);
  float dl = to_f32(delta_t[bd]);
  float zv = 0.f;  // the gate input, loaded with the other inputs (not at the store)
  if constexpr (FZ) {
    const float bias = dtb ? dtb[d] : 0.f;
    if (z_t) zv = to_f32(z_t[bd]);
    dl += bias;
    if (sp) dl = softplus_f(dl);
  }
  float hv[NS], Av[NS], Bv[NS], Cv[NS];
  VecLoad<float, NS>::run(h + bd * N + q * NS, hv);
  VecLoad<float, NS>::run(A + d * N + q * NS, Av);
  load_vec<T, NS>(B_t + b * N + q * NS, Bv);
  load_vec<T, NS>(C_t + b * N + q * NS, Cv);
  const float u = dl * xv;
  float yp;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const float a = __builtin_amdgcn_exp2f(dl * (Av[j] * kLog2e));
    hv[j] = __builtin_fmaf(a, hv[j], u * Bv[j]);
    yp = j ? __builtin_fmaf(Cv[j], hv[j], yp) : Cv[j] * hv[j];
  }
  yp = quad_sum(yp);
  VecStore<float, NS>::run(h + bd * N + q * NS, hv);
  if (q == 0) {
    float yv = __builtin_fmaf(Dv[d], xv, yp);
    if constexpr (FZ) {
      if (z_t) yv *= zv * sigmoid_f(zv);
    }
    y_t[bd] = from_f32<T>(yv);
  }
}

template <typename T, int K, int ACT>
__global__ __launch_bounds__(256) void k_conv_step(int64_t B, int64_t D, T* __restrict__ state,
                                                   const T* __restrict__ x_t,
                                                   const float* __restrict__ W,
                                                   const float* __restrict__ bias,
                                                   T* __restrict__ out_t) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= B * D) return;
  const int64_t b = i / D, d = i % D;
  float win[K];
#pragma unroll
  for (int k = 0; k < K - 1; ++k) win[k] = to_f32(state[(b * (K - 1) + k) * D + d]);
  win[K - 1] = to_f32(x_t[i]);
  float acc = bias ? bias[d] : 0.f;
#pragma unroll
  for (int k = 0; k < K; ++k) acc = __builtin_fmaf(W[d * K + k], win[k], acc);
  if constexpr (ACT == kActSilu) acc *= sigmoid_f(acc);
  out_t[i] = from_f32<T>(acc);
  // the values came from T, so storing them back in T is exact
#pragma unroll
  for (int k = 0; k < K - 1; ++k) state[(b * (K - 1) + k) * D + d] = from_f32<T>(win[k + 1]);
}

template <typename T, int N, bool FZ>
static void scan_step_nf(const ScanStepArgs& a, hipStream_t st) {
  hipLaunchKernelGGL((k_scan_step<T, N, FZ>), dim3(unsigned((a.D + 63) / 64), unsigned(a.B)),
                     dim3(256), 0, st, a.D, a.h, static_cast<const T*>(a.x_t),
                     static_cast<const T*>(a.delta_t), a.A, static_cast<const T*>(a.B_t),
                     static_cast<const T*>(a.C_t), a.Dv, a.dt_bias, a.dt_softplus,
                     static_cast<const T*>(a.z_t), static_cast<T*>(a.y_t));
}

template <typename T, int N>
static hipError_t scan_step_n(const ScanStepArgs& a, hipStream_t st) {
  timer_mark(kKScanStep, false, st);
  if (a.fused)
    scan_step_nf<T, N, true>(a, st);
  else
    scan_step_nf<T, N, false>(a, st);
  timer_mark(kKScanStep, true, st);
  return hipGetLastError();
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

template <typename T, int K, int ACT>
static void conv_step_ka(const ConvStepArgs& a, hipStream_t st) {
  const int64_t n = a.B * a.D;
  hipLaunchKernelGGL((k_conv_step<T, K, ACT>), dim3(unsigned((n + 255) / 256)), dim3(256), 0, st,
                     a.B, a.D, static_cast<T*>(a.state), static_cast<const T*>(a.x_t), a.W,
                     a.bias, static_cast<T*>(a.out_t));
}

template <typename T, int K>
static hipError_t conv_step_k(const ConvStepArgs& a, hipStream_t st) {
  timer_mark(kKConvStep, false, st);
  if (a.act == kActSilu)
    conv_step_ka<T, K, kActSilu>(a, st);
  else
    conv_step_ka<T, K, kActNone>(a, st);
  timer_mark(kKConvStep, true, st);
  return hipGetLastError();
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

hipError_t launch_conv1d_step(const ConvStepArgs& a, hipStream_t st) {
  return a.dtype == 0 ? conv_step_t<float>(a, st) : conv_step_t<bf16_t>(a, st);
}

}  // namespace ssm
