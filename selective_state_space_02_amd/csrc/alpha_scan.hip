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
// Mapping: a workgroup of 64 threads takes rpb = max(1, 64 / S) batch rows; thread t
// runs the recurrence of (row t / S, state t % S) sequentially over K, then the workgroup
// forms its rows' hidden outputs from the final states staged in LDS.  The work per
// thread is a chain of dependent steps over a few KB, so the kernels are bound by memory
// latency: every loop issues the loads of kUnroll iterations before their arithmetic
// (the arithmetic order is the plain sequential one).  The backward keeps the recomputed
// states x_{k-1} in the caller's workspace for its reverse loop; dWc is summed over the
// batch in segments of rows (each in row order) whose partials are then added in
// segment order.  No atomics.
#include "common.hpp"
#include "launch.hpp"

namespace ssm {

constexpr int kAlphaThreads = 64;
constexpr int kUnroll = 8;

// x_{K-1} of one (row, state): a, b point at the row's step-0 value of that state.
__device__ __forceinline__ float alpha_final_state(const float* __restrict__ ap,
                                                   const float* __restrict__ bp, int64_t K,
                                                   int64_t S) {
  float x = 0.f;
  int64_t k = 0;
  for (; k + kUnroll <= K; k += kUnroll) {
    float av[kUnroll], bv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      av[u] = ap[(k + u) * S];
      bv[u] = bp[(k + u) * S];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      x = __builtin_fmaf(sigmoid_f(av[u]), x - bv[u], bv[u]);  // g x + (1 - g) b
  }
  for (; k < K; ++k) {
    const float bv = bp[k * S];
    x = __builtin_fmaf(sigmoid_f(ap[k * S]), x - bv, bv);
  }
  return x;
}

__global__ __launch_bounds__(kAlphaThreads) void k_alpha_fwd(
    int64_t Bn, int64_t K, int64_t S, int64_t H, int64_t rpb, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ Wc, const float* __restrict__ h0,
    float* __restrict__ h) {
  __shared__ float xs[kAlphaMaxS];
  const int64_t i0 = int64_t(blockIdx.x) * rpb;
  const int tid = threadIdx.x;
  for (int64_t p = tid; p < rpb * S; p += kAlphaThreads) {
    const int64_t r = p / S, s = p % S, i = i0 + r;
    xs[p] = i < Bn ? alpha_final_state(a + i * K * S + s, b + i * K * S + s, K, S) : 0.f;
  }
  __syncthreads();
  for (int64_t q = tid; q < rpb * H; q += kAlphaThreads) {
    const int64_t r = q / H, j = q % H, i = i0 + r;
    if (i >= Bn) continue;
    float acc = h0 ? h0[i * H + j] : 0.f;
    for (int64_t s = 0; s < S; ++s) acc = __builtin_fmaf(Wc[j * S + s], xs[r * S + s], acc);
    h[i * H + j] = acc;
  }
}

// xh: [Bn][K][S] the states x_{k-1} (workspace); xl: [Bn][S] the final states (workspace).
__global__ __launch_bounds__(kAlphaThreads) void k_alpha_bwd(
    int64_t Bn, int64_t K, int64_t S, int64_t H, int64_t rpb, const float* __restrict__ a,
    const float* __restrict__ b, const float* __restrict__ Wc, const float* __restrict__ dh,
    float* __restrict__ da, float* __restrict__ db, float* __restrict__ dh0,
    float* __restrict__ xh, float* __restrict__ xl) {
  const int64_t i0 = int64_t(blockIdx.x) * rpb;
  const int tid = threadIdx.x;
  for (int64_t p = tid; p < rpb * S; p += kAlphaThreads) {
    const int64_t r = p / S, s = p % S, i = i0 + r;
    if (i >= Bn) continue;
    // the adjoint of the final state, through the readout: a sum over the hidden channels
    float lam = 0.f;
    {
      const float* wp = Wc + s;
      const float* dp = dh + i * H;
      int64_t j = 0;
      for (; j + kUnroll <= H; j += kUnroll) {
        float wv[kUnroll], dv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          wv[u] = wp[(j + u) * S];
          dv[u] = dp[j + u];
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) lam = __builtin_fmaf(wv[u], dv[u], lam);
      }
      for (; j < H; ++j) lam = __builtin_fmaf(wp[j * S], dp[j], lam);
    }
    const float* ap = a + i * K * S + s;
    const float* bp = b + i * K * S + s;
    float* xp = xh + i * K * S + s;
    // forward recompute; the state before each step is kept for the reverse loop
    float x = 0.f;
    int64_t k = 0;
    for (; k + kUnroll <= K; k += kUnroll) {
      float av[kUnroll], bv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        av[u] = ap[(k + u) * S];
        bv[u] = bp[(k + u) * S];
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        xp[(k + u) * S] = x;
        x = __builtin_fmaf(sigmoid_f(av[u]), x - bv[u], bv[u]);
      }
    }
    for (; k < K; ++k) {
      xp[k * S] = x;
      const float bv = bp[k * S];
      x = __builtin_fmaf(sigmoid_f(ap[k * S]), x - bv, bv);
    }
    xl[i * S + s] = x;
    // reverse: from the last step, a tail of K % kUnroll steps first, then whole groups
    auto rstep = [&](int64_t kk, float av, float bv, float xv) {
      const float g = sigmoid_f(av), om = 1.f - g;
      da[i * K * S + kk * S + s] = lam * (xv - bv) * g * om;
      db[i * K * S + kk * S + s] = lam * om;
      lam *= g;
    };
    const int64_t kg = K - K % kUnroll;
    for (k = K - 1; k >= kg; --k) rstep(k, ap[k * S], bp[k * S], xp[k * S]);
    for (k = kg - kUnroll; k >= 0; k -= kUnroll) {
      float av[kUnroll], bv[kUnroll], xv[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        av[u] = ap[(k + u) * S];
        bv[u] = bp[(k + u) * S];
        xv[u] = xp[(k + u) * S];
      }
#pragma unroll
      for (int u = kUnroll - 1; u >= 0; --u) rstep(k + u, av[u], bv[u], xv[u]);
    }
  }
  if (dh0) {
    for (int64_t q = tid; q < rpb * H; q += kAlphaThreads) {
      const int64_t i = i0 + q / H, j = q % H;
      if (i < Bn) dh0[i * H + j] = dh[i * H + j];
    }
  }
}

// Partials of dWc: part[seg][j*S + s] = sum over the rows of segment seg (in row order) of
// dh[i,j] xl[i,s].  Workgroup (column block cb, segment seg) of a 1-D grid.
__global__ __launch_bounds__(256) void k_alpha_dwc(int64_t Bn, int64_t S, int64_t H,
                                                   int64_t rows, int64_t ncb,
                                                   const float* __restrict__ dh,
                                                   const float* __restrict__ xl,
                                                   float* __restrict__ part) {
  const int64_t cb = int64_t(blockIdx.x) % ncb, seg = int64_t(blockIdx.x) / ncb;
  const int64_t idx = cb * 256 + threadIdx.x;
  if (idx >= H * S) return;
  const int64_t j = idx / S, s = idx % S;
  const int64_t r0 = seg * rows, r1 = r0 + rows < Bn ? r0 + rows : Bn;
  float acc = 0.f;
  int64_t i = r0;
  for (; i + kUnroll <= r1; i += kUnroll) {
    float dv[kUnroll], xv[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      dv[u] = dh[(i + u) * H + j];
      xv[u] = xl[(i + u) * S + s];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc = __builtin_fmaf(dv[u], xv[u], acc);
  }
  for (; i < r1; ++i) acc = __builtin_fmaf(dh[i * H + j], xl[i * S + s], acc);
  part[seg * H * S + idx] = acc;
}

AlphaPlan alpha_plan(int64_t Bn, int64_t S, int64_t H) {
  AlphaPlan p{};
  p.rpb = S >= kAlphaThreads ? 1 : kAlphaThreads / S;
  p.nblk = (Bn + p.rpb - 1) / p.rpb;
  // dWc: about 64K partial sums in flight, segments of at least 16 rows
  const int64_t HS = H * S;
  int64_t nseg = (65536 + HS - 1) / HS;
  const int64_t most = (Bn + 15) / 16;
  if (nseg > most) nseg = most;
  if (nseg < 1) nseg = 1;
  p.rows = (Bn + nseg - 1) / nseg;
  p.nseg = (Bn + p.rows - 1) / p.rows;
  p.ncb = (HS + 255) / 256;
  return p;
}

hipError_t launch_alpha_fwd(const AlphaArgs& a, hipStream_t st) {
  const AlphaPlan p = alpha_plan(a.Bn, a.S, a.H);
  return launch(k_alpha_fwd, dim3(unsigned(p.nblk)), dim3(kAlphaThreads), st, a.Bn, a.K, a.S,
                a.H, p.rpb, a.a, a.b, a.Wc, a.h0, a.h);
}

hipError_t launch_alpha_bwd(const AlphaArgs& a, float* xh, float* xl, float* part, float* tmp,
                            hipStream_t st) {
  const AlphaPlan p = alpha_plan(a.Bn, a.S, a.H);
  hipError_t e = launch(k_alpha_bwd, dim3(unsigned(p.nblk)), dim3(kAlphaThreads), st, a.Bn,
                        a.K, a.S, a.H, p.rpb, a.a, a.b, a.Wc, a.dh, a.da, a.db, a.dh0, xh, xl);
  if (e != hipSuccess) return e;
  e = launch(k_alpha_dwc, dim3(unsigned(p.ncb * p.nseg)), dim3(256), st, a.Bn, a.S, a.H,
             p.rows, p.ncb, a.dh, xl, part);
  if (e != hipSuccess) return e;
  return launch_reduce(part, p.nseg, a.H * a.S, a.dWc, true, tmp, st);
}

}  // namespace ssm
