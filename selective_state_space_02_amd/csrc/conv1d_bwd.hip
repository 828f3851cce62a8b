// Depthwise causal conv1d backward for gfx950.
//
// Forward (zero left padding):  out[b,t,d] = bias[d] + sum_k W[d,k] x[b, t-K+1+k, d].
// Backward for upstream gradient g = dout (taken after the SiLU backward, as in the
// mamba-rs backward_conv1d_step section):
//   dx[b,s,d]  = sum_k g[b, s+K-1-k, d] W[d,k]          (terms with s+K-1-k < L)
//   dW[d,k]   += sum_{b,t} g[b,t,d] x[b, t-K+1+k, d]
//   db[d]     += sum_{b,t} g[b,t,d]
// The page's step function is one timestep of this (its weight and bias terms, and
// the newest-tap input term); here the whole sequence is done at once, exactly.
//
// Mapping: a thread owns VEC consecutive channels and a block of Tb timesteps.  It
// walks time forwards keeping the next K upstream values and the last K inputs in
// ring buffers (register indices fixed by unrolling over K), writes dx, and keeps
// dW/db partial sums in registers; per-(batch, time block) partials are summed in a
// fixed order by k_reduce.  HBM traffic: read g and x once, write dx once.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

template <typename T, int K, int VEC>
__global__ __launch_bounds__(256) void k_conv_bwd(
    int64_t L, int64_t D, int64_t Tb, int64_t nTb, int64_t colblocks,
    const T* __restrict__ x, const float* __restrict__ W, const T* __restrict__ g,
    T* __restrict__ dx, float* __restrict__ dWp, float* __restrict__ dbp) {
  const int64_t bid = blockIdx.x;
  const int64_t cb = bid % colblocks, rest = bid / colblocks;
  const int64_t tb = rest % nTb, b = rest / nTb;
  const int64_t d0 = (cb * 256 + threadIdx.x) * VEC;
  if (d0 >= D) return;
  const int64_t t0 = tb * Tb, t1 = (t0 + Tb < L) ? t0 + Tb : L;
  const T* xb = x + b * L * D + d0;
  const T* gb = g + b * L * D + d0;
  T* dxb = dx + b * L * D + d0;

  float w[VEC][K];
#pragma unroll
  for (int v = 0; v < VEC; ++v)
#pragma unroll
    for (int k = 0; k < K; ++k) w[v][k] = W[(d0 + v) * K + k];

  // ring buffers: slot (t - t0) mod K
  float gr[K][VEC], xr[K][VEC];
#pragma unroll
  for (int m = 0; m < K; ++m) {
    const int64_t t = t0 + m;
    if (t < L) load_vec<T, VEC>(gb + t * D, gr[m]);
    else zero(gr[m]);
  }
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int64_t t = t0 - K + 1 + k;
    if (t >= 0) load_vec<T, VEC>(xb + t * D, xr[(1 + k) % K]);
    else zero(xr[(1 + k) % K]);
  }
  float dW[VEC][K], db[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    db[v] = 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) dW[v][k] = 0.f;
  }

  for (int64_t s0 = t0; s0 < t1; s0 += K) {
#pragma unroll
    for (int r = 0; r < K; ++r) {
      const int64_t s = s0 + r;
      if (s >= t1) break;
      float o[VEC];
#pragma unroll
      for (int v = 0; v < VEC; ++v) {
        float acc = 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) acc = __builtin_fmaf(gr[(r + K - 1 - k) % K][v], w[v][k], acc);
        o[v] = acc;
        const float gv = gr[r][v];
        db[v] += gv;
#pragma unroll
        for (int k = 0; k < K; ++k) dW[v][k] = __builtin_fmaf(gv, xr[(r + 1 + k) % K][v], dW[v][k]);
      }
      VecStore<T, VEC>::run(dxb + s * D, o);
      // refill: g[s+K] into the slot of g[s]; x[s+1] into the slot of x[s+1-K]
      if (s + K < L) load_vec<T, VEC>(gb + (s + K) * D, gr[r]);
      else zero(gr[r]);
      if (s + 1 < L) load_vec<T, VEC>(xb + (s + 1) * D, xr[(r + 1) % K]);
      else zero(xr[(r + 1) % K]);
    }
  }
  const int64_t p = b * nTb + tb;
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) dWp[(p * D + d0 + v) * K + k] = dW[v][k];
    dbp[p * D + d0 + v] = db[v];
  }
}

template <typename T, int K>
static hipError_t conv_k(const ConvArgs& a, const ConvPlan& p, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  const T* g = static_cast<const T*>(a.dout);
  T* dx = static_cast<T*>(a.dx);
  const int64_t colblocks = (a.D / p.vec + 255) / 256;
  const dim3 grid(colblocks * a.B * p.nTb);
  timer_mark(kKConvBwd, false, st);
  if (p.vec == 4)
    hipLaunchKernelGGL((k_conv_bwd<T, K, 4>), grid, dim3(256), 0, st, a.L, a.D, p.Tb, p.nTb,
                       colblocks, x, a.W, g, dx, p.dWp, p.dbp);
  else
    hipLaunchKernelGGL((k_conv_bwd<T, K, 1>), grid, dim3(256), 0, st, a.L, a.D, p.Tb, p.nTb,
                       colblocks, x, a.W, g, dx, p.dWp, p.dbp);
  timer_mark(kKConvBwd, true, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t P = a.B * p.nTb;
  if ((e = launch_reduce(p.dWp, P, a.D * a.K, a.dW, true, p.rtmp, st)) != hipSuccess) return e;
  return launch_reduce(p.dbp, P, a.D, a.db, true, p.rtmp, st);
}

template <typename T>
static hipError_t conv_t(const ConvArgs& a, const ConvPlan& p, hipStream_t st) {
  switch (a.K) {
    case 1: return conv_k<T, 1>(a, p, st);
    case 2: return conv_k<T, 2>(a, p, st);
    case 3: return conv_k<T, 3>(a, p, st);
    case 4: return conv_k<T, 4>(a, p, st);
    case 5: return conv_k<T, 5>(a, p, st);
    case 6: return conv_k<T, 6>(a, p, st);
    case 7: return conv_k<T, 7>(a, p, st);
    case 8: return conv_k<T, 8>(a, p, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_bwd(const ConvArgs& a, const ConvPlan& p, hipStream_t st) {
  return a.dtype == 0 ? conv_t<float>(a, p, st) : conv_t<bf16_t>(a, p, st);
}

}  // namespace ssm
