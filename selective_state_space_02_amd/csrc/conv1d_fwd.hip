// Depthwise causal conv1d forward for gfx950 (zero left padding):
//   out[b,t,d] = bias[d] + sum_k W[d,k] x[b, t-K+1+k, d]
// the forward whose per-timestep backward the mamba-rs backward_conv1d_step section
// gives (its window holds the last K inputs, tap K-1 the newest).  With act = SiLU the
// kernel stores silu(out) = out * sigmoid(out), the activation the Mamba block applies
// to the conv output before the scan.
//
// Mapping as in the backward (conv1d_bwd.hip): a lane owns VEC consecutive channels, a
// workgroup 64*VEC channels and a block of Tb steps taken by its four wavefronts in
// interleaved groups of R steps; a group's R + K - 1 input rows are loaded at once
// through one buffer descriptor (rows as scalar offsets), the K - 1 halo rows coming
// from cache.  HBM traffic: read x once, write out once.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace ssm {

template <typename T, int K, int VEC, int ACT>
__global__ __launch_bounds__(256) void k_conv_fwd(int64_t L, int64_t D, int64_t Tb, int64_t nTb,
                                                  int64_t cgroups, const T* __restrict__ x,
                                                  const float* __restrict__ W,
                                                  const float* __restrict__ bias,
                                                  T* __restrict__ out) {
  constexpr int R = (VEC > 1) ? 8 : 16;  // steps per group
  constexpr int H = R + K - 1;           // input rows per group
  constexpr int CW = 64 * VEC;           // channels per workgroup
  using BV = BufVec<T, VEC>;
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
  T* og = out + b * L * D + c0;

  float w[VEC][K], bs[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) {
    bs[v] = bias ? bias[c0 + lc + v] : 0.f;
#pragma unroll
    for (int k = 0; k < K; ++k) w[v][k] = W[(c0 + lc + v) * K + k];
  }
  // each row's descriptor spans the workgroup's valid channels of that row only (built
  // from the row's 64-bit address), so no offset or size depends on D
  const uint32_t rowv = uint32_t((D - c0 < CW) ? D - c0 : CW) * uint32_t(sizeof(T));
  const uint32_t loff = lc * uint32_t(sizeof(T));
  for (int64_t ts = t0 + int64_t(wave) * R; ts < t1; ts += 4 * R) {
    // xraw[i] = x[ts - K + 1 + i]; rows outside [0, L) are zero
    typename BV::raw_t xraw[H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
      const int64_t tx = ts - (K - 1) + i;
      xraw[i] = (tx >= 0 && tx < L) ? BV::load(buf_rsrc(xg + tx * D, rowv), loff)
                                    : typename BV::raw_t{};
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (ts + r < t1) {
        float xv[K][VEC], o[VEC];
#pragma unroll
        for (int k = 0; k < K; ++k) BV::unpack(xraw[r + k], xv[k]);  // x[t - K+1+k]
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          float acc = bs[v];
#pragma unroll
          for (int k = 0; k < K; ++k) acc = __builtin_fmaf(w[v][k], xv[k][v], acc);
          if constexpr (ACT == kActSilu) acc *= sigmoid_f(acc);
          o[v] = acc;
        }
        if (act) BV::store(BV::pack(o), buf_rsrc(og + (ts + r) * D, rowv), loff);
      }
    }
  }
}

template <typename T, int K, int ACT>
static hipError_t conv_fwd_ka(const ConvFwdArgs& a, hipStream_t st) {
  constexpr int VW = (K <= 4) ? 4 : 2;
  const int vec = (a.D % 4 == 0) ? VW : 1;
  const int64_t cgroups = (a.D + 64 * vec - 1) / (64 * vec);
  const dim3 grid(unsigned(cgroups * a.B * a.nTb));
  const T* x = static_cast<const T*>(a.x);
  T* out = static_cast<T*>(a.out);
  timer_mark(kKConvFwd, false, st);
  hipError_t e;
  if (vec == VW)
    e = launch(k_conv_fwd<T, K, VW, ACT>, grid, dim3(256), st, a.L, a.D, a.Tb, a.nTb, cgroups,
               x, a.W, a.bias, out);
  else
    e = launch(k_conv_fwd<T, K, 1, ACT>, grid, dim3(256), st, a.L, a.D, a.Tb, a.nTb, cgroups,
               x, a.W, a.bias, out);
  timer_mark(kKConvFwd, true, st);
  return e;
}

template <typename T, int K>
static hipError_t conv_fwd_k(const ConvFwdArgs& a, hipStream_t st) {
  return a.act == kActSilu ? conv_fwd_ka<T, K, kActSilu>(a, st)
                           : conv_fwd_ka<T, K, kActNone>(a, st);
}

template <typename T>
static hipError_t conv_fwd_t(const ConvFwdArgs& a, hipStream_t st) {
  switch (a.K) {
    case 1: return conv_fwd_k<T, 1>(a, st);
    case 2: return conv_fwd_k<T, 2>(a, st);
    case 3: return conv_fwd_k<T, 3>(a, st);
    case 4: return conv_fwd_k<T, 4>(a, st);
    case 5: return conv_fwd_k<T, 5>(a, st);
    case 6: return conv_fwd_k<T, 6>(a, st);
    case 7: return conv_fwd_k<T, 7>(a, st);
    case 8: return conv_fwd_k<T, 8>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t st) {
  return a.dtype == 0 ? conv_fwd_t<float>(a, st) : conv_fwd_t<bf16_t>(a, st);
}

}  // namespace ssm
