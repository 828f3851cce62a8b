// Sigmoid-gated scan of the foxhunt ml-alpha forward-pass commit (a selective SSM scan
// over K timesteps with a sigmoid-gated state update: a_proj, b_proj, W_c and the
// zero-initialised h_s2 in, h_enriched out) for gfx950.  The page does not print the
// recurrence; the library computes this reading of it, per batch row i and state s:
//   g_k = sigmoid(a[i,k,s]),   x_k[i,s] = g_k x_{k-1}[i,s] + (1 - g_k) b[i,k,s],   x_{-1} = 0
//   h[i,j] = h0[i,j] + sum_s Wc[j,s] x_{K-1}[i,s]
// and its exact adjoint (the backward-scratch commit: d_a and d_b summed over the hidden
// channels j, d_W_c summed over the batch, d_h_s2 passed through):
//   lambda_{K-1}[i,s] = sum_j Wc[j,s] dh[i,j];  for k = K-1..0:
//   da = lambda_k (x_{k-1} - b_k) g_k (1 - g_k),  db = lambda_k (1 - g_k),
//   lambda_{k-1} = lambda_k g_k;   dWc[j,s] += sum_i dh[i,j] x_{K-1}[i,s];  dh0 = dh.
//
// Mapping: a workgroup takes rpb = max(1, 256 / S) batch rows; thread t runs the
// recurrence of (row t / S, state t % S) sequentially over K, then the workgroup forms
// its rows' hidden outputs from the final states staged in LDS.  The backward keeps the
// recomputed states x_{k-1} in the caller's workspace for its reverse loop; dWc is a
// fixed-order sum over the batch per (j, s).  No atomics.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

__global__ __launch_bounds__(256) void k_alpha_fwd(int64_t Bn, int64_t K, int64_t S, int64_t H,
                                                   int64_t rpb, const float* __restrict__ a,
                                                   const float* __restrict__ b,
                                                   const float* __restrict__ Wc,
                                                   const float* __restrict__ h0,
                                                   float* __restrict__ h) {
  __shared__ float xs[kAlphaMaxS];
  const int64_t i0 = int64_t(blockIdx.x) * rpb;
  const int tid = threadIdx.x;
  for (int64_t p = tid; p < rpb * S; p += 256) {
    const int64_t r = p / S, s = p % S, i = i0 + r;
    float x = 0.f;
    if (i < Bn) {
      const float* ap = a + i * K * S + s;
      const float* bp = b + i * K * S + s;
      for (int64_t k = 0; k < K; ++k) {
        const float g = sigmoid_f(ap[k * S]), bv = bp[k * S];
        x = __builtin_fmaf(g, x - bv, bv);  // g x + (1 - g) b
      }
    }
    xs[p] = x;
  }
  __syncthreads();
  for (int64_t q = tid; q < rpb * H; q += 256) {
    const int64_t r = q / H, j = q % H, i = i0 + r;
    if (i >= Bn) continue;
    float acc = h0 ? h0[i * H + j] : 0.f;
    for (int64_t s = 0; s < S; ++s) acc = __builtin_fmaf(Wc[j * S + s], xs[r * S + s], acc);
    h[i * H + j] = acc;
  }
}

// xh: [Bn][K][S] the states x_{k-1} (workspace); xl: [Bn][S] the final states (workspace).
__global__ __launch_bounds__(256) void k_alpha_bwd(
    int64_t Bn, int64_t K, int64_t S, int64_t H, int64_t rpb, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ Wc, const float* __restrict__ dh,
    float* __restrict__ da, float* __restrict__ db, float* __restrict__ dh0,
    float* __restrict__ xh, float* __restrict__ xl) {
  const int64_t i0 = int64_t(blockIdx.x) * rpb;
  const int tid = threadIdx.x;
  for (int64_t p = tid; p < rpb * S; p += 256) {
    const int64_t r = p / S, s = p % S, i = i0 + r;
    if (i >= Bn) continue;
    // the adjoint of the final state, through the readout: a sum over the hidden channels
    float lam = 0.f;
    for (int64_t j = 0; j < H; ++j) lam = __builtin_fmaf(Wc[j * S + s], dh[i * H + j], lam);
    // forward recompute; the state before each step is kept for the reverse loop
    float x = 0.f;
    for (int64_t k = 0; k < K; ++k) {
      const int64_t o = (i * K + k) * S + s;
      xh[o] = x;
      const float g = sigmoid_f(a[o]), bv = b[o];
      x = __builtin_fmaf(g, x - bv, bv);
    }
    xl[i * S + s] = x;
    for (int64_t k = K - 1; k >= 0; --k) {
      const int64_t o = (i * K + k) * S + s;
      const float g = sigmoid_f(a[o]), om = 1.f - g;
      da[o] = lam * (xh[o] - b[o]) * g * om;
      db[o] = lam * om;
      lam *= g;
    }
  }
  if (dh0) {
    for (int64_t q = tid; q < rpb * H; q += 256) {
      const int64_t i = i0 + q / H, j = q % H;
      if (i < Bn) dh0[i * H + j] = dh[i * H + j];
    }
  }
}

// dWc[j,s] += sum_i dh[i,j] xl[i,s], one thread per (j, s), i in order.
__global__ __launch_bounds__(256) void k_alpha_dwc(int64_t Bn, int64_t S, int64_t H,
                                                   const float* __restrict__ dh,
                                                   const float* __restrict__ xl,
                                                   float* __restrict__ dWc) {
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (idx >= H * S) return;
  const int64_t j = idx / S, s = idx % S;
  float acc = 0.f;
  for (int64_t i = 0; i < Bn; ++i) acc = __builtin_fmaf(dh[i * H + j], xl[i * S + s], acc);
  dWc[idx] += acc;
}

static int64_t alpha_rows_per_block(int64_t S) { return S >= 256 ? 1 : 256 / S; }

hipError_t launch_alpha_fwd(const AlphaArgs& a, hipStream_t st) {
  const int64_t rpb = alpha_rows_per_block(a.S);
  const int64_t nblk = (a.Bn + rpb - 1) / rpb;
  return launch(k_alpha_fwd, dim3(unsigned(nblk)), dim3(256), st, a.Bn, a.K, a.S, a.H, rpb, a.a,
                a.b, a.Wc, a.h0, a.h);
}

hipError_t launch_alpha_bwd(const AlphaArgs& a, float* xh, float* xl, hipStream_t st) {
  const int64_t rpb = alpha_rows_per_block(a.S);
  const int64_t nblk = (a.Bn + rpb - 1) / rpb;
  hipError_t e = launch(k_alpha_bwd, dim3(unsigned(nblk)), dim3(256), st, a.Bn, a.K, a.S, a.H,
                        rpb, a.a, a.b, a.Wc, a.dh, a.da, a.db, a.dh0, xh, xl);
  if (e != hipSuccess) return e;
  return launch(k_alpha_dwc, dim3(unsigned((a.H * a.S + 255) / 256)), dim3(256), st, a.Bn, a.S,
                a.H, a.dh, xl, a.dWc);
}

}  // namespace ssm
