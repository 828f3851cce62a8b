// Depthwise causal conv1d backward for gfx950.
//
// Forward (zero left padding):  out[b,t,d] = bias[d] + sum_k W[d,k] x[b, t-K+1+k, d].
// Backward for upstream gradient g = dout of the conv output (the mamba-rs
// backward_conv1d_step section takes it after the SiLU backward); with the SiLU fused
// (act = SiLU), dout is the gradient of silu(out) and g = dout * silu'(out) is formed
// here from the recomputed pre-activation:
//   dx[b,s,d]  = sum_k g[b, s+K-1-k, d] W[d,k]          (terms with s+K-1-k < L)
//   dW[d,k]   += sum_{b,t} g[b,t,d] x[b, t-K+1+k, d]
//   db[d]     += sum_{b,t} g[b,t,d]
// The page's step function is one timestep of this (its weight and bias terms, and
// the newest-tap input term); here the whole sequence is done at once, exactly.
//
// Mapping: a lane owns VEC consecutive channels (4, 2 or 1), so every load and store
// of a wavefront is one contiguous row of 64*VEC channels; a workgroup owns those
// channels and a block of Tb timesteps, which its four wavefronts take in interleaved
// groups of R steps.  For a group a thread loads the R + K - 1 rows of g and of x the
// group touches (the K - 1 halo rows are shared with the neighbouring group, so they
// come from cache), all at once -- many rows in flight per wavefront keep HBM busy --
// then computes dx, dW and db of the group from registers.  dW/db partials are summed
// over the four wavefronts in LDS; per-(batch, time block) partials are summed in a
// fixed order by k_reduce.  HBM traffic: read g and x once, write dx once.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace ssm {

template <typename T, int K, int VEC, int ACT>
__global__ __launch_bounds__(256) void k_conv_bwd(
    int64_t L, int64_t D, int64_t Tb, int64_t nTb, int64_t cgroups,
    const T* __restrict__ x, const float* __restrict__ W, const float* __restrict__ bias,
    const T* __restrict__ g, T* __restrict__ dx, float* __restrict__ dWp,
    float* __restrict__ dbp) {
  constexpr int R = (VEC > 1) ? 8 : 16;  // steps per group
  constexpr int H = R + K - 1;           // upstream-gradient rows per group
  // input rows per group: with the SiLU backward fused, the pre-activation of every
  // gradient row is recomputed, which reaches K - 1 rows further
  constexpr int HX = (ACT == kActSilu) ? H + K - 1 : H;
  constexpr int CW = 64 * VEC;           // channels per workgroup
  using BV = BufVec<T, VEC>;
  __shared__ float red[4][K + 1][CW];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int64_t bid = blockIdx.x;
  const int64_t cg = bid % cgroups, rest = bid / cgroups;
  const int64_t tb = rest % nTb, b = rest / nTb;
  // D is a multiple of VEC: a lane's channels are all valid or all past D; lanes past
  // D read the group's last valid vector and store nothing
  const int64_t c0 = cg * CW;
  const bool act = c0 + int64_t(lane) * VEC < D;
  const uint32_t lc = act ? uint32_t(lane) * VEC : uint32_t(D - VEC - c0);
  const int64_t t0 = tb * Tb, t1 = (t0 + Tb < L) ? t0 + Tb : L;
  const T* xg = x + b * L * D + c0;
  const T* gg = g + b * L * D + c0;
  T* dxg = dx + b * L * D + c0;

  float w[VEC][K], bs[VEC], dW[VEC][K], db[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    db[v] = 0.f;
    bs[v] = bias ? bias[c0 + lc + v] : 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      w[v][k] = W[(c0 + lc + v) * K + k];
      dW[v][k] = 0.f;
    }
  }
  // each row's descriptor spans the workgroup's valid channels of that row only (built
  // from the row's 64-bit address), so no offset or size depends on D
  const uint32_t rowv = uint32_t((D - c0 < CW) ? D - c0 : CW) * uint32_t(sizeof(T));
  const uint32_t loff = lc * uint32_t(sizeof(T));
  for (int64_t ts = t0 + int64_t(wave) * R; ts < t1; ts += 4 * R) {
    // xr[i] = x[ts - K + 1 + i], gr[i] = g[ts + i]; rows outside [0, L) are zero
    typename BV::raw_t xraw[HX], graw[H];
#pragma unroll
    for (int i = 0; i < HX; ++i) {
      const int64_t tx = ts - (K - 1) + i;
      xraw[i] = (tx >= 0 && tx < L) ? BV::load(buf_rsrc(xg + tx * D, rowv), loff)
                                    : typename BV::raw_t{};
    }
#pragma unroll
    for (int i = 0; i < H; ++i)
      graw[i] = (ts + i < L) ? BV::load(buf_rsrc(gg + (ts + i) * D, rowv), loff)
                             : typename BV::raw_t{};
    // the conv output's gradient of every row the group touches; with SiLU fused, the
    // upstream value times silu'(pre), pre = bias + sum_k W x recomputed from the inputs
    float gf[H][VEC];
#pragma unroll
    for (int i = 0; i < H; ++i) {
      BV::unpack(graw[i], gf[i]);
      if constexpr (ACT == kActSilu) {
        float xw[K][VEC];
#pragma unroll
        for (int k = 0; k < K; ++k) BV::unpack(xraw[i + k], xw[k]);  // x[ts + i - K+1+k]
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float pre = bs[v];
#pragma unroll
          for (int k = 0; k < K; ++k) pre = __builtin_fmaf(w[v][k], xw[k][v], pre);
          const float sg = sigmoid_f(pre);
          gf[i][v] *= sg * __builtin_fmaf(pre, 1.f - sg, 1.f);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t t = ts + r;
      if (t < t1) {
        float xv[K][VEC], o[VEC];
#pragma unroll
        for (int k = 0; k < K; ++k) BV::unpack(xraw[r + k], xv[k]);  // x[t - K+1+k]
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float acc = 0.f;
#pragma unroll
          for (int k = 0; k < K; ++k) acc = __builtin_fmaf(gf[r + K - 1 - k][v], w[v][k], acc);
          o[v] = acc;
          const float gt = gf[r][v];  // g[t]
          db[v] += gt;
#pragma unroll
          for (int k = 0; k < K; ++k) dW[v][k] = __builtin_fmaf(gt, xv[k][v], dW[v][k]);
        }
        if (act) BV::store(BV::pack(o), buf_rsrc(dxg + t * D, rowv), loff);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[wave][k][lane * VEC + v] = dW[v][k];
    red[wave][K][lane * VEC + v] = db[v];
  }
  __syncthreads();
  if (wave == 0 && act) {
    const int64_t p = b * nTb + tb;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      const int64_t d = c0 + lc + v;
      const int j = lane * VEC + v;
#pragma unroll
      for (int k = 0; k <= K; ++k) {
        const float s = (red[0][k][j] + red[1][k][j]) + (red[2][k][j] + red[3][k][j]);
        if (k < K) dWp[(p * D + d) * K + k] = s;
        else dbp[p * D + d] = s;
      }
    }
  }
}

// lanes' channel count: 4 (2 for widths above 4, bounding registers) when D allows
template <typename T, int K, int ACT>
static hipError_t conv_ka(const ConvArgs& a, const ConvPlan& p, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  const T* g = static_cast<const T*>(a.dout);
  T* dx = static_cast<T*>(a.dx);
  constexpr int VW = (K <= 4) ? 4 : 2;
  const int vec = (a.D % 4 == 0) ? VW : 1;
  const int64_t cgroups = (a.D + 64 * vec - 1) / (64 * vec);
  const dim3 grid(unsigned(cgroups * a.B * p.nTb));
  timer_mark(kKConvBwd, false, st);
  hipError_t e;
  if (vec == VW)
    e = launch(k_conv_bwd<T, K, VW, ACT>, grid, dim3(256), st, a.L, a.D, p.Tb, p.nTb, cgroups,
               x, a.W, a.bias, g, dx, p.dWp, p.dbp);
  else
    e = launch(k_conv_bwd<T, K, 1, ACT>, grid, dim3(256), st, a.L, a.D, p.Tb, p.nTb, cgroups, x,
               a.W, a.bias, g, dx, p.dWp, p.dbp);
  timer_mark(kKConvBwd, true, st);
  if (e != hipSuccess) return e;
  const int64_t P = a.B * p.nTb;
  if ((e = launch_reduce(p.dWp, P, a.D * a.K, a.dW, true, p.rtmp, st)) != hipSuccess) return e;
  return launch_reduce(p.dbp, P, a.D, a.db, true, p.rtmp, st);
}

template <typename T, int K>
static hipError_t conv_k(const ConvArgs& a, const ConvPlan& p, hipStream_t st) {
  return a.act == kActSilu ? conv_ka<T, K, kActSilu>(a, p, st) : conv_ka<T, K, kActNone>(a, p, st);
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
