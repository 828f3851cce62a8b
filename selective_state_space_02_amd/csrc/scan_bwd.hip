// Selective-scan backward (backpropagation through time across the SSM state) for
// gfx950.
//
// With upstream gradient dy, the state adjoint obeys the reverse recurrence
//   g_t[n] = dy_t C_t[n] + a_{t+1}[n] g_{t+1}[n],      g_L = 0,
// and the gradients are
//   dx_t     = Dv dy_t + delta_t sum_n g_t[n] B_t[n]
//   ddelta_t = sum_n g_t[n] (A[n] a_t[n] h_{t-1}[n] + B_t[n] x_t)
//   dA[n]   += sum_{b,t} g_t[n] delta_t a_t[n] h_{t-1}[n]
//   dB_t[n]  = sum_d g_t[n] delta_t x_t          dC_t[n] = sum_d dy_t h_t[n]
//   dDv     += sum_{b,t} dy_t x_t                dh0[n]  = a_0[n] g_0[n]
// The forward states are recomputed from the forward's checkpoints (the forward
// recompute shared by the CPU and GPU backward in the rustytorch backward_cuda
// commit); every contribution to a cross-channel or cross-time sum is kept and
// summed in a fixed order, with no atomics (foxhunt ml-alpha backward-scratch commit:
// per-channel slots followed by a reduction, nothing dropped).
//
// Parallel form (coarse chunks as in the forward).  Running the adjoint through a
// chunk is linear: the adjoint pushed out of the chunk's first step is
//   gp_start = G + P (.) gp_end,  P[n] = prod_t a_t[n],
// with G the pushed adjoint of the chunk alone (gp_end = 0).  Launches:
//   1. k_bwd_summary: G and sum(delta) of chunks 1..nc-1 (skipped when nc == 1);
//   2. k_bwd_carry:   adjoint arriving at the end of every chunk;
//   3. k_bwd_main:    per chunk, walk the kTc-step checkpoint intervals backwards:
//                     recompute a_t and h_t of the interval from its checkpoint into
//                     registers, then run the reverse step; dx and ddelta are
//                     written, dB/dC are summed over the workgroup's 64 channels
//                     (reduce-scatter across lanes, then LDS) into per-group
//                     partials, dA/dDv into per-(batch, chunk) partials;
//   4. k_reduce (reduce.hip): fixed-order sums of the partials.
#include "common.hpp"
#include "launch.hpp"
#include "tile.hpp"

namespace ssm {

// Chunk summaries of the adjoint: G (pushed adjoint of the chunk alone) and the sum of
// delta, for chunks 1..nc-1.
// FZ: delta is the raw time step, mapped at staging (time_step_map); with z (nullable)
// dy is the gradient of the gated output y * silu(z), and the scan's upstream gradient
// dy * silu(z) is formed at staging.
template <typename T, int N, int VEC, bool FZ>
__global__ __launch_bounds__(256, 4) void k_bwd_summary(
    int64_t B, int64_t L, int64_t D, int64_t nf, int nc, int64_t g, int64_t groups,
    const T* __restrict__ delta, const float* __restrict__ A, const T* __restrict__ Cm,
    const T* __restrict__ dy, const float* __restrict__ dtb, bool sp, const T* __restrict__ z,
    float* __restrict__ GS, float* __restrict__ SD) {
  constexpr int NS = N / 4;
  __shared__ float sd[2][kTc][kTileCh], sdy[2][kTc][kTileCh], sC[2][kTc][N];
  __shared__ float sbias[FZ ? kTileCh : 1];
  const WgPos wp = wg_pos(groups, B);
  const int64_t c = wp.c + 1, b = wp.b;  // chunks 1..nc-1
  const int tid = threadIdx.x, q = tid & 3, cl = tid >> 2;
  const int64_t d0 = wp.grp * kTileCh, d = d0 + cl;
  const bool act = d < D;
  const int D32 = int(D);
  const int dvalid = (D - d0 < kTileCh) ? int(D - d0) : kTileCh;
  const T* db = delta + int64_t(b) * L * D + d0;
  const T* dyb = dy + int64_t(b) * L * D + d0;
  const T* Cb = Cm + int64_t(b) * L * N;
  float A2[NS], gp[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    A2[j] = act ? A[d * N + q * NS + j] * kLog2e : 0.f;
    gp[j] = 0.f;
  }
  // running sums of the delta this thread stages (ChTile placement): the chunk's sum of
  // delta, accumulated once per value instead of in each of a channel's lanes per step
  float dsum[VEC] = {};
  const int64_t t0 = chunk_tile(c, nf, nc, g) * kTc, te = chunk_tile(c + 1, nf, nc, g) * kTc;
  const int64_t t1 = te < L ? te : L;
  const int ntile = int((t1 - t0 + kTc - 1) / kTc);
  // tiles are walked from the last one backwards
  const ChTile<T, VEC> gt(D32, dvalid, tid);
  const uint32_t voff = VecFetch<T, N>::offset(tid);
  ChFetch<T, VEC> fd, fy, fz;
  VecFetch<T, N> fC;
  const T* zb = (FZ && z) ? z + int64_t(b) * L * D + d0 : nullptr;
  if constexpr (FZ) {
    if (tid < kTileCh) sbias[tid] = (dtb && tid < dvalid) ? dtb[d0 + tid] : 0.f;
    __syncthreads();
  }
  int pend_tv = 0;  // valid rows of the fetched tile not yet committed
  auto fetch = [&](int64_t tt, int tvalid) {
    fd.fetch(gt, db + tt * D, D32, tvalid, dvalid);
    fy.fetch(gt, dyb + tt * D, D32, tvalid, dvalid);
    fC.fetch(Cb + tt * N, tvalid, voff);
    if (zb) fz.fetch(gt, zb + tt * D, D32, tvalid, dvalid);
    pend_tv = tvalid;
  };
  auto commit = [&](int bf) {
    // (rows past L were loaded as 0, and the time-step map zeroes them)
    fd.commit_map(gt, sd[bf], [&](int k, float (&v)[VEC]) {
      if constexpr (FZ) {
        const bool ok = gt.s_in + k * ChTile<T, VEC>::RPP < pend_tv && gt.c < dvalid;
        time_step_map<VEC>(v, &sbias[gt.c], ok, sp, nullptr);
      }
#pragma unroll
      for (int i = 0; i < VEC; ++i) dsum[i] += v[i];
    });
    if constexpr (FZ) {
      if (zb)
        fy.commit_map(gt, sdy[bf], [&](int k, float (&v)[VEC]) {
          float zv[VEC];
          BufVec<T, VEC>::unpack(fz.raw[k], zv);
#pragma unroll
          for (int i = 0; i < VEC; ++i) v[i] *= zv[i] * sigmoid_f(zv[i]);
        });
      else
        fy.commit(gt, sdy[bf]);
    } else {
      fy.commit(gt, sdy[bf]);
    }
    fC.commit(sC[bf], tid);
  };
  int64_t tf = t0 + int64_t(ntile - 1) * kTc;
  fetch(tf, clamp_valid(L - tf));
  commit(0);
  __syncthreads();
  for (int it = 0; it < ntile; ++it, tf -= kTc) {
    const int buf = it & 1;
    const bool more = it + 1 < ntile;
    if (more) fetch(tf - kTc, kTc);  // every tile but the last one is full
    // the LDS operands of step s-1 are read during step s
    float ndl = sd[buf][kTc - 1][cl], ndy = sdy[buf][kTc - 1][cl], nC[NS];
    tile_read_vec<N, NS>(sC[buf], kTc - 1, q, nC);
#pragma unroll
    for (int s = kTc - 1; s >= 0; --s) {
      const float dl = ndl, dyv = ndy;
      float Cv[NS];
#pragma unroll
      for (int j = 0; j < NS; ++j) Cv[j] = nC[j];
      if (s > 0) {
        ndl = sd[buf][s - 1][cl];
        ndy = sdy[buf][s - 1][cl];
        tile_read_vec<N, NS>(sC[buf], s - 1, q, nC);
      }
#pragma unroll
      for (int j = 0; j < NS; ++j) {
        const float g = __builtin_fmaf(dyv, Cv[j], gp[j]);
        gp[j] = __builtin_amdgcn_exp2f(dl * A2[j]) * g;
      }
      step_fence_arr(gp);
      step_fence_arr(nC);
      step_fence(ndl, ndy);
    }
    if (more) commit(buf ^ 1);
    __syncthreads();
  }
  if (act) {
    const int64_t o = (b * nc + c) * D + d;
#pragma unroll
    for (int j = 0; j < NS; ++j) GS[o * N + q * NS + j] = gp[j];
  }
  // the tile buffers are free after the loop's last barrier
  const float sdl = chan_rows_sum(gt, dsum, &sd[0][0][0], tid);
  if (tid < dvalid) SD[(b * nc + c) * D + d0 + tid] = sdl;
}

template <int N>
__global__ __launch_bounds__(256) void k_bwd_carry(
    int64_t B, int64_t D, int nc, const float* __restrict__ A, const float* __restrict__ GS,
    const float* __restrict__ SD, const float* __restrict__ dh_last, float* __restrict__ gin) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= B * D * N) return;
  const int64_t n = idx % N, bd = idx / N, d = bd % D, b = bd / D;
  const float A2 = A[d * N + n] * kLog2e;
  // what arrives at the end of the last chunk: the final state's own gradient, if given
  float gp = dh_last ? dh_last[idx] : 0.f;
  // sequential over chunks (last to first); a batch of kCarryAhead chunk summaries is
  // loaded before it is composed
  for (int c0 = nc - 1; c0 >= 0; c0 -= kCarryAhead) {
    float sdv[kCarryAhead], gv[kCarryAhead];
#pragma unroll
    for (int i = 0; i < kCarryAhead; ++i) {
      // (index clamped into [0, nc): before the start the value is loaded but not used;
      // chunk 0's summary slot is never written nor used)
      const int c = c0 - i >= 0 ? c0 - i : 0;
      const int64_t o = (b * nc + c) * D + d;
      sdv[i] = SD[o];
      gv[i] = GS[o * N + n];
    }
#pragma unroll
    for (int i = 0; i < kCarryAhead; ++i) {
      const int c = c0 - i;
      if (c >= 0) {
        const int64_t o = (b * nc + c) * D + d;
        gin[o * N + n] = gp;
        if (c > 0) {
          const float P = __builtin_amdgcn_exp2f(A2 * sdv[i]);
          gp = __builtin_fmaf(P, gp, gv[i]);
        }
      }
    }
  }
}

// Regeneration of dense states for the sparse-checkpoint backward: workgroup (channel
// group, batch row, run) runs the segments k = k0 + run*nrun .. (at most nrun of them,
// below k1), each the steps [k*ck_every, min((k+1)*ck_every, L)) from the state the
// forward saved before its first step (cks: [B][nck_s][D][N]), and stores the state
// before every CK-th step (CK = ckpt_base(N), the dense interval the main pass
// recomputes from) into ckd, whose batch rows hold nckd states from state index f0 on.
// The recurrence is the forward's (the tile's x staged as u = delta * x); rows past L
// are zero, the identity step.
template <typename T, int N, int VEC>
__global__ __launch_bounds__(256, 4) void k_ckpt_regen(
    int64_t B, int64_t L, int64_t D, int64_t groups, int64_t ck_every, int64_t k0,
    int64_t k1, int nrun, const T* __restrict__ x, const T* __restrict__ delta,
    const float* __restrict__ A, const T* __restrict__ Bm, const float* __restrict__ cks,
    int64_t nck_s, float* __restrict__ ckd, int64_t nckd, int64_t f0) {
  constexpr int NS = N / 4;
  constexpr int CK = int(ckpt_base(N));
  __shared__ float sx[2][kTc][kTileCh], sd[2][kTc][kTileCh], sB[2][kTc][N];
  const WgPos wp = wg_pos(groups, B);
  const int64_t kr = k0 + wp.c * nrun, kre = kr + nrun < k1 ? kr + nrun : k1, b = wp.b;
  const int tid = threadIdx.x, q = tid & 3, cl = tid >> 2;
  const int64_t d0 = wp.grp * kTileCh, d = d0 + cl;
  const bool act = d < D;
  const int D32 = int(D);
  const int dvalid = (D - d0 < kTileCh) ? int(D - d0) : kTileCh;
  const T* xb = x + b * L * D + d0;
  const T* db = delta + b * L * D + d0;
  const T* Bb = Bm + b * L * N;
  float A2[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) A2[j] = act ? A[d * N + q * NS + j] * kLog2e : 0.f;
  const uint32_t ckoff = act ? uint32_t(cl * N + q * NS) * 4u : kOffNone;
  const uint32_t ckbytes = uint32_t(dvalid * N) * 4u;
  float h[NS];
  float* ckg = ckd + (b * nckd * D + d0) * N;
  const float* ckr = cks + (b * nck_s * D + d0) * N;
  const int64_t t0 = kr * ck_every, te = kre * ck_every, t1 = te < L ? te : L;
  const int ntile = int((t1 - t0 + kTc - 1) / kTc);
  const int seg_tiles = int(ck_every / kTc);
  const ChTile<T, VEC> gt(D32, dvalid, tid);
  const uint32_t voff = VecFetch<T, N>::offset(tid);
  ChFetch<T, VEC> fx, fd;
  VecFetch<T, N> fB;
  auto fetch = [&](int64_t tt) {
    const int tv = clamp_valid(L - tt);
    fx.fetch(gt, xb + tt * D, D32, tv, dvalid);
    fd.fetch(gt, db + tt * D, D32, tv, dvalid);
    fB.fetch(Bb + tt * N, tv, voff);
  };
  auto commit = [&](int bf) {
    fd.commit(gt, sd[bf]);
    fx.commit_map(gt, sx[bf], [&](int kk, float (&v)[VEC]) {
      const float* dv = &sd[bf][gt.s_in + kk * ChTile<T, VEC>::RPP][gt.c];
#pragma unroll
      for (int i = 0; i < VEC; ++i) v[i] *= dv[i];
    });
    fB.commit(sB[bf], tid);
  };
  fetch(t0);
  commit(0);
  __syncthreads();
  for (int it = 0; it < ntile; ++it) {
    const int buf = it & 1;
    const int64_t tf = t0 + int64_t(it) * kTc;
    if (it + 1 < ntile) fetch(tf + kTc);
    // each segment starts from the state the forward saved before it
    if (it % seg_tiles == 0)
      buf_load_states<NS>(buf_rsrc(ckr + (kr + it / seg_tiles) * D * N, ckbytes), ckoff, h);
#pragma unroll
    for (int part = 0; part < kTc / CK; ++part) {
      const int64_t ts = tf + part * CK;
      if (ts < L) buf_store_states<NS>(h, buf_rsrc(ckg + (ts / CK - f0) * D * N, ckbytes), ckoff);
#pragma unroll 4
      for (int s = part * CK; s < (part + 1) * CK; ++s) {
        const float dl = sd[buf][s][cl], u = sx[buf][s][cl];
        float Bv[NS];
        tile_read_vec<N, NS>(sB[buf], s, q, Bv);
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float a = __builtin_amdgcn_exp2f(dl * A2[j]);
          h[j] = __builtin_fmaf(a, h[j], u * Bv[j]);
        }
      }
    }
    if (it + 1 < ntile) commit(buf ^ 1);
    __syncthreads();
  }
}

// Main backward pass: one chunk of one batch row for 64 channels.  Tiles of kTc steps
// are walked from the last one backwards.  A tile holds SPLIT checkpoint intervals
// (SPLIT = ckpt_per_tile(N)); from the last interval to the first, the states of the
// interval are recomputed from its checkpoint into a register stash, then the reverse
// step runs over the stashed steps.  dx and ddelta
// of a step overwrite the step's x and delta in LDS (a channel's slots are read and
// written only by the channel's four lanes, reads first) and are stored after the tile
// with coalesced writes; the dB/dC partials of each lane go to LDS and are summed there.
// Two barriers per tile: after the compute (outputs complete) and after the next
// tile's inputs are committed.
//
// FZ: the Mamba-block neighbours.  delta is the raw time step, mapped at staging
// (time_step_map), whose derivative there (sigmoid, or 1) is kept in LDS for the tile's
// ddelta store: the stored ddelta is the raw input's gradient, and its per-channel sum
// over the chunk goes to dbp (time-step bias partials, [B*nc][D]).  With z (nullable),
// dy is the gradient of the gated output y * silu(z); at staging it becomes the scan's
// upstream gradient dy * silu(z), and dz = dy * ysave * silu'(z) is stored (ysave: y
// before the gate, saved by the forward).  The gate's inputs are loaded after the
// previous tile's compute, so their registers are not held across it.
template <typename T, int N, int VEC, int SPLIT, int WAVES, bool FZ>
__global__ __launch_bounds__(256, WAVES) void k_bwd_main(
    int64_t B, int64_t L, int64_t D, int64_t nf, int nc, int64_t g, int64_t groups, int c_off,
    int64_t nck, int64_t f0, const T* __restrict__ x, const T* __restrict__ delta, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ Dv,
    const T* __restrict__ dy, const float* __restrict__ ckpt, const float* __restrict__ gin,
    const float* __restrict__ dtb, bool sp, const T* __restrict__ z,
    const T* __restrict__ ysave, T* __restrict__ dx, T* __restrict__ ddelta,
    T* __restrict__ dz, float* __restrict__ dBp, float* __restrict__ dCp,
    float* __restrict__ dAp, float* __restrict__ dDp, float* __restrict__ dbp,
    float* __restrict__ dh0) {
  constexpr int NS = N / 4;       // states per lane
  constexpr int V = 2 * NS;       // per-lane values summed over channels: dB, dC
  constexpr int NP = 16 / V;      // partials per value left in LDS by chan_reduce_scatter
  constexpr int SL = kTc / SPLIT; // stashed steps = checkpoint interval
  static_assert(SPLIT == ckpt_per_tile(N), "stash split must match the checkpoints");
  // Four states per lane take the permuted state order (perm_quarter / perm_xor), whose
  // channel reduce-scatter costs one DPP add per pair.  B and C rows then take the
  // two-copy layout of VecFetch::commit_perm, interleaved per step in sBC (B's row, then
  // C's), so that the reverse step reads both with two LDS instructions.  The fused
  // variant keeps the plain order: its LDS would no longer admit three workgroups per CU
  // with the second copies.
  constexpr bool PERM = NS == 4 && !FZ;
  __shared__ float sx[2][kTc][kTileCh], sd[2][kTc][kTileCh], sdy[2][kTc][kTileCh];
  __shared__ float sB[2][kTc][PERM ? 1 : N], sC[2][kTc][PERM ? 1 : N];
  __shared__ float sBC[PERM ? 2 : 1][kTc][PERM ? 4 * N : 1];
  __shared__ float red[4][kTc][64];  // [wavefront][step][lane]
  // FZ: time-step bias, the time-step map's derivative for the current tile, and each
  // thread's running ddelta sums of its VEC channels
  __shared__ float sbias[FZ ? kTileCh : 1], ssg[FZ ? kTc : 1][kTileCh];
  __shared__ float sdb[FZ ? kTileThreads * VEC : 1];

  const WgPos wp = wg_pos(groups, B);
  const int64_t c = wp.c + c_off, b = wp.b, grp = wp.grp;  // this launch's chunks from c_off
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, q = tid & 3, cl = tid >> 2;
  const int64_t d0 = grp * kTileCh, d = d0 + cl;
  const bool act = d < D;
  const int D32 = int(D);
  const int dvalid = (D - d0 < kTileCh) ? int(D - d0) : kTileCh;
  // register j of the lane holds state Qs*NS + (j ^ ms)
  const int Qs = PERM ? perm_quarter(lane) : q, ms = PERM ? perm_xor(lane) : 0;
  const uint32_t pa = uint32_t(16 * (ms & 1) + 4 * Qs + 2 * (ms >> 1)) * 4u;  // PERM reads
  const T* xb = x + int64_t(b) * L * D + d0;
  const T* db = delta + int64_t(b) * L * D + d0;
  const T* dyb = dy + int64_t(b) * L * D + d0;
  const T* Bb = Bm + int64_t(b) * L * N;
  const T* Cb = Cm + int64_t(b) * L * N;
  T* dxb = dx + int64_t(b) * L * D + d0;
  T* ddb = ddelta + int64_t(b) * L * D + d0;
  // checkpoint f (the state before step f*SL) of this group: ckpt + ((b*nck + f - f0)*D +
  // d0)*N, lane at (cl*N + Qs*NS); the buffer holds the states from index f0 on
  const float* ckg = ckpt + (int64_t(b) * nck * D + d0) * N;
  const uint32_t ckoff = act ? uint32_t(cl * N + Qs * NS) * 4u : kOffNone;
  const uint32_t ckbytes = uint32_t(dvalid * N) * 4u;
  float* pB = dBp + (int64_t(grp) * B + b) * L * N;
  float* pC = dCp + (int64_t(grp) * B + b) * L * N;

  float A2[NS], gp[NS], dA_acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    A2[j] = act ? A[d * N + Qs * NS + (j ^ ms)] * kLog2e : 0.f;
    gp[j] = (act && gin) ? gin[((b * nc + c) * D + d) * N + Qs * NS + (j ^ ms)] : 0.f;
    dA_acc[j] = 0.f;
  }
  const float Dd = act ? Dv[d] : 0.f;
  float dD_acc = 0.f;

  const int64_t t0 = chunk_tile(c, nf, nc, g) * kTc, te = chunk_tile(c + 1, nf, nc, g) * kTc;
  const int64_t t1 = te < L ? te : L;
  const int ntile = int((t1 - t0 + kTc - 1) / kTc);

  const ChTile<T, VEC> gt(D32, dvalid, tid);
  using G = ChTile<T, VEC>;
  const uint32_t voff = VecFetch<T, N>::offset(tid);
  ChFetch<T, VEC> fx, fd, fy;
  VecFetch<T, N> fB, fC;
  const T* zb = (FZ && z) ? z + int64_t(b) * L * D + d0 : nullptr;
  const T* ysb = (FZ && z) ? ysave + int64_t(b) * L * D + d0 : nullptr;
  T* dzb = (FZ && z) ? dz + int64_t(b) * L * D + d0 : nullptr;
  if constexpr (FZ) {
    if (tid < kTileCh) sbias[tid] = (dtb && tid < dvalid) ? dtb[d0 + tid] : 0.f;
#pragma unroll
    for (int i = 0; i < VEC; ++i) sdb[tid * VEC + i] = 0.f;
    __syncthreads();
  }
  float hcur[SPLIT][NS], hnxt[SPLIT][NS];  // checkpoints of the current and the next tile
  int pend_tv = 0;                         // valid rows of the fetched, uncommitted tile
  int64_t pend_tt = 0;                     // and its first step
  auto fetch = [&](int64_t tt, int tvalid, float (&hk)[SPLIT][NS]) {
    fx.fetch(gt, xb + tt * D, D32, tvalid, dvalid);
    fd.fetch(gt, db + tt * D, D32, tvalid, dvalid);
    fy.fetch(gt, dyb + tt * D, D32, tvalid, dvalid);
    fB.fetch(Bb + tt * N, tvalid, voff);
    fC.fetch(Cb + tt * N, tvalid, voff);
    pend_tv = tvalid;
    pend_tt = tt;
    // Every load is issued unconditionally, straight into the registers the loop carries:
    // an interval wholly past L, or the empty fetch past the chunk's first tile
    // (tvalid 0), reads zeros through an empty descriptor.  (A load under a branch ends
    // in a register copy at the join, whose wait would also cover the loads just issued.)
#pragma unroll
    for (int hf = 0; hf < SPLIT; ++hf) {
      const bool has = tvalid > 0 && (hf == 0 || tt + hf * SL < L);
      const auto rs = buf_rsrc(ckg + (has ? tt / SL + hf - f0 : 0) * D * N, has ? ckbytes : 0u);
      if constexpr (PERM) buf_load_states_perm(rs, ckoff, ms, hk[hf]);
      else buf_load_states<NS>(rs, ckoff, hk[hf]);
    }
  };
  // the gate's inputs of the pending tile (FZ with z), loaded just before its commit
  ChFetch<T, VEC> fz, fys;
  auto fetch_gate = [&]() {
    if (zb) {
      fz.fetch(gt, zb + pend_tt * D, D32, pend_tv, dvalid);
      fys.fetch(gt, ysb + pend_tt * D, D32, pend_tv, dvalid);
    }
  };
  auto commit = [&](int bf) {
    fx.commit(gt, sx[bf]);
    if constexpr (FZ) {
      // (LDS addresses from opaque copies: rebuilt per tile, not held across the compute)
      fd.commit_map(gt, sd[bf], [&](int k, float (&v)[VEC]) {
        const int row = opaque(gt.s_in) + k * G::RPP, cc = opaque(gt.c);
        time_step_map<VEC>(v, &sbias[cc], row < pend_tv && cc < dvalid, sp, &ssg[row][cc]);
      });
      if (zb) {
        fy.commit_map(gt, sdy[bf], [&](int k, float (&v)[VEC]) {
          float zv[VEC], yv[VEC], dzv[VEC];
          BufVec<T, VEC>::unpack(fz.raw[k], zv);
          BufVec<T, VEC>::unpack(fys.raw[k], yv);
#pragma unroll
          for (int i = 0; i < VEC; ++i) {
            const float sg = sigmoid_f(zv[i]);
            dzv[i] = v[i] * yv[i] * sg * __builtin_fmaf(zv[i], 1.f - sg, 1.f);
            v[i] *= zv[i] * sg;
          }
          tile_store_regs(gt, dzb + pend_tt * D, k, dzv, D32, pend_tv, dvalid);
        });
      } else {
        fy.commit(gt, sdy[bf]);
      }
    } else {
      fd.commit(gt, sd[bf]);
      fy.commit(gt, sdy[bf]);
    }
    if constexpr (PERM) {
      // (addresses rebuilt per tile from an opaque copy, not held across the compute)
      const int ot = opaque(tid);
      fB.commit_perm(&sBC[bf][0][0], 4 * N, ot);
      fC.commit_perm(&sBC[bf][0][2 * N], 4 * N, ot);
    } else {
      fB.commit(sB[bf], tid);
      fC.commit(sC[bf], tid);
    }
  };
  // the lane's NS values of B, or of B and C, at step s of tile buffer bf
  auto read_B = [&](int bf, int s, float (&o)[NS]) {
    if constexpr (PERM) tile_read_perm(&sBC[bf][s][0], pa, o);
    else tile_read_vec<N, NS>(sB[bf], s, q, o);
  };
  auto read_BC = [&](int bf, int s, float (&ob)[NS], float (&oc)[NS]) {
    if constexpr (PERM) {
      tile_read_perm2(&sBC[bf][s][0], pa, ob, oc);
    } else {
      tile_read_vec<N, NS>(sB[bf], s, q, ob);
      tile_read_vec<N, NS>(sC[bf], s, q, oc);
    }
  };

  int64_t tf = t0 + int64_t(ntile - 1) * kTc;  // first step of the current tile
  fetch(tf, clamp_valid(L - tf), hcur);
  if constexpr (FZ) fetch_gate();
  commit(0);
  // every tile but the last one is full; past the first tile an empty fetch (at a valid
  // address) keeps the loads unconditional
  fetch(ntile > 1 ? tf - kTc : tf, ntile > 1 ? kTc : 0, hnxt);
  __syncthreads();

  float pv[V];  // channel-sum values of the step above the current one
  for (int it = 0; it < ntile; ++it, tf -= kTc) {
    const int buf = it & 1;
#pragma unroll
    for (int half = SPLIT - 1; half >= 0; --half) {
      const int s0 = half * SL;
      // Recompute the interval's steps s0 .. s0+SL-1 from its checkpoint into the stash.
      // The LDS operands of step s+1 are read during step s.
      // each step's state is written straight into its stash slot (and fenced there),
      // so the stash costs no register copies
      float as[SL][NS], hs[SL][NS];
      float ndl = sd[buf][s0][cl], nxv = sx[buf][s0][cl], nB[NS];
      read_B(buf, s0, nB);
#pragma unroll
      for (int i = 0; i < SL; ++i) {
        const int s = s0 + i;
        const float dl = ndl, u = dl * nxv;
        float Bv[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) Bv[j] = nB[j];
        if (i + 1 < SL) {
          ndl = sd[buf][s + 1][cl];
          nxv = sx[buf][s + 1][cl];
          read_B(buf, s + 1, nB);
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float a = __builtin_amdgcn_exp2f(dl * A2[j]);
          hs[i][j] = __builtin_fmaf(a, i ? hs[i - 1][j] : hcur[half][j], u * Bv[j]);
          as[i][j] = a;
        }
        step_fence_arr(hs[i]);
        step_fence_arr(nB);
        step_fence(ndl, nxv);
      }
      // Reverse step over the stash; the channel sums of step s+1 are formed during
      // step s, and the LDS operands of step s-1 are read during step s.
      float rdl, rxv, rdy, rB[NS], rC[NS];
      {
        const int s = s0 + SL - 1;
        rdl = sd[buf][s][cl];
        rxv = sx[buf][s][cl];
        rdy = sdy[buf][s][cl];
        read_BC(buf, s, rB, rC);
      }
#pragma unroll
      for (int i = SL - 1; i >= 0; --i) {
        const int s = s0 + i;
        const float dl = rdl, xv = rxv, dyv = rdy;
        float Bv[NS], Cv[NS];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          Bv[j] = rB[j];
          Cv[j] = rC[j];
        }
        if (i > 0) {
          rdl = sd[buf][s - 1][cl];
          rxv = sx[buf][s - 1][cl];
          rdy = sdy[buf][s - 1][cl];
          read_BC(buf, s - 1, rB, rC);
        }
        const float u = dl * xv;
        float sBg, sAq;
        float vals[V];
#pragma unroll
        for (int j = 0; j < NS; ++j) {
          const float g = __builtin_fmaf(dyv, Cv[j], gp[j]);
          const float qq = __builtin_fmaf(-u, Bv[j], hs[i][j]);  // a_t h_{t-1}
          const float gq = g * qq;
          dA_acc[j] = __builtin_fmaf(gq, dl, dA_acc[j]);
          sAq = j ? __builtin_fmaf(gq, A2[j], sAq) : gq * A2[j];
          sBg = j ? __builtin_fmaf(g, Bv[j], sBg) : g * Bv[j];
          // channel-sum values: dB then dC of each state (PERM), or all dB then all dC
          vals[PERM ? 2 * j : j] = g * u;
          vals[PERM ? 2 * j + 1 : NS + j] = dyv * hs[i][j];
          gp[j] = as[i][j] * g;
        }
        // identical in the channel's four lanes, which all write the same values
        sBg = quad_sum(sBg);
        sAq = quad_sum(sAq);
        sx[buf][s][cl] = __builtin_fmaf(Dd, dyv, dl * sBg);   // dx
        sd[buf][s][cl] = __builtin_fmaf(kLn2, sAq, xv * sBg);  // ddelta
        dD_acc = __builtin_fmaf(dyv, xv, dD_acc);
        if (s < kTc - 1) {
          if constexpr (PERM) chan_reduce_scatter_perm(pv);
          else chan_reduce_scatter<V>(pv, lane);
          red[wave][s + 1][lane] = pv[0];
        }
#pragma unroll
        for (int k = 0; k < V; ++k) pv[k] = vals[k];
        step_fence_arr(gp);
        step_fence_arr(dA_acc);
        step_fence_arr(rB);
        step_fence_arr(rC);
        step_fence(dD_acc, rdl, rxv, rdy);
      }
    }
    if constexpr (PERM) chan_reduce_scatter_perm(pv);
    else chan_reduce_scatter<V>(pv, lane);
    red[wave][0][lane] = pv[0];
    // The plain variant commits the next tile's inputs to the other buffer (free since
    // the previous tile's second barrier) right after the wavefront's own compute, where
    // it overlaps the workgroup's slower wavefronts, not between the barriers, where the
    // whole workgroup waits.  The fused variant loads its gate inputs after the barrier
    // (registers), so it commits after the stores.
    if constexpr (!FZ) {
      if (it + 1 < ntile) commit(buf ^ 1);
    }
    __syncthreads();
    if constexpr (FZ) {
      if (it + 1 < ntile) fetch_gate();  // the next tile's, consumed by its commit below
    }

    // this tile's dx and ddelta, and the channel sums -> this group's dB/dC partials
    const int smax = (t1 - tf < kTc) ? int(t1 - tf) : kTc;
    tile_store_ch(gt, dxb + tf * D, sx[buf], D32, smax, dvalid);
    if constexpr (FZ) {
      tile_store_ch_map(gt, ddb + tf * D, sd[buf], D32, smax, dvalid,
                        [&](int k, float (&v)[VEC]) {
                          const int row = opaque(gt.s_in) + k * G::RPP, cc = opaque(gt.c);
                          const int ti = opaque(tid) * VEC;
#pragma unroll
                          for (int i = 0; i < VEC; ++i) {
                            v[i] *= ssg[row][cc + i];
                            if (row < smax) sdb[ti + i] += v[i];
                          }
                        });
    } else {
      tile_store_ch(gt, ddb + tf * D, sd[buf], D32, smax, dvalid);
    }
    for (int k = tid; k < kTc * 2 * N; k += 256) {
      const int s = k / (2 * N), r = k % (2 * N);
      if (s < smax) {
        // value index and state quarter of output r (dB_n for r < N, dC_n above)
        const int n = r % N, vi = (r / N) * NS + n % NS, qr = n / NS;
        float sum = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          float part;
          if constexpr (PERM) {
            part = red[w][s][perm_partial_lane(r / N, n, 0)] +
                   red[w][s][perm_partial_lane(r / N, n, 1)];
          } else {
            part = red[w][s][chan_partial_lane<V>(vi, 0, qr)];
#pragma unroll
            for (int pi = 1; pi < NP; ++pi) part += red[w][s][chan_partial_lane<V>(vi, pi, qr)];
          }
          sum = w ? sum + part : part;
        }
        const int64_t o = (tf + s) * N;
        if (r < N) pB[o + r] = sum;
        else pC[o + r - N] = sum;
      }
    }
    if (it + 1 < ntile) {
      if constexpr (FZ) commit(buf ^ 1);
#pragma unroll
      for (int hf = 0; hf < SPLIT; ++hf) {
#pragma unroll
        for (int j = 0; j < NS; ++j) reg_move(hcur[hf][j], hnxt[hf][j]);
      }
      step_fence();
      fetch(it + 2 < ntile ? tf - 2 * kTc : tf, it + 2 < ntile ? kTc : 0, hnxt);
    }
    __syncthreads();
  }

  if constexpr (FZ) {
    // time-step bias partial of each channel: the sum over the threads that share its
    // channels (rows of the ChTile placement), in row order
    if (dbp && tid < kTileCh && tid < dvalid) {
      const int tc = tid / VEC, ci = tid % VEC;  // thread column and channel within it
      float sum = 0.f;
      for (int r = 0; r < G::RPP; ++r) sum += sdb[(r * G::TPR + tc) * VEC + ci];
      dbp[(b * nc + c) * D + d0 + tid] = sum;
    }
  }
  if (act) {
    const int64_t o = (b * nc + c) * D + d;
#pragma unroll
    for (int j = 0; j < NS; ++j) dAp[o * N + Qs * NS + (j ^ ms)] = dA_acc[j];
    if (q == 0) dDp[o] = dD_acc;
    if (dh0 && c == 0) {
#pragma unroll
      for (int j = 0; j < NS; ++j) dh0[(int64_t(b) * D + d) * N + Qs * NS + (j ^ ms)] = gp[j];
    }
  }
}

// Steps a regeneration workgroup covers at least (runs of short checkpoint intervals).
constexpr int64_t kRegenSteps = 128;

// Waves per SIMD of k_bwd_main.  Its LDS (41-45 KB) admits three workgroups per CU; at
// N = 16 a full-tile stash does not fit the register budget of three waves per SIMD, a
// half-tile one does, hence the mid-tile checkpoints at N = 16 (ckpt_per_tile).
template <int N>
struct BwdMainCfg {
  static constexpr int kSplit = ckpt_per_tile(N);
  static constexpr int kWaves = 3;
};

// ---------------------------------------------------------------------------------
// host launcher
// ---------------------------------------------------------------------------------
template <typename T, int N, int VEC, bool FZ>
static hipError_t bwd_impl(const ScanArgs& a, const BwdPlan& p, hipStream_t st) {
  const T* x = static_cast<const T*>(a.x);
  const T* delta = static_cast<const T*>(a.delta);
  const T* Bm = static_cast<const T*>(a.Bm);
  const T* Cm = static_cast<const T*>(a.Cm);
  const T* dy = static_cast<const T*>(a.dy);
  const dim3 block(256);
  // the adjoint arriving at each chunk's end, [B][nc][D][N]: with one chunk that is the
  // final state's gradient alone, whose [B][D][N] layout is the same array
  const float* gin = a.dh_last;
  hipError_t e;
  if (p.nc > 1) {
    timer_mark(kKBwdSummary, false, st);
    e = launch(k_bwd_summary<T, N, VEC, FZ>, dim3(unsigned(p.ng * a.B * (p.nc - 1))), block, st,
               a.B, a.L, a.D, p.nf, p.nc, p.g, p.ng, delta, a.A, Cm, dy, a.dt_bias,
               a.dt_softplus, static_cast<const T*>(a.z), p.GS, p.SD);
    timer_mark(kKBwdSummary, true, st);
    if (e != hipSuccess) return e;
    const int64_t tot = a.B * a.D * N;
    timer_mark(kKBwdCarry, false, st);
    e = launch(k_bwd_carry<N>, dim3(unsigned((tot + 255) / 256)), block, st, a.B, a.D, p.nc,
               a.A, p.GS, p.SD, a.dh_last, p.gin);
    timer_mark(kKBwdCarry, true, st);
    if (e != hipSuccess) return e;
    gin = p.gin;
  }
  using Cfg = BwdMainCfg<N>;
  // the main pass over chunks [c0, c1) with the dense states in ck (batch rows of nck
  // states from index f0 on)
  auto main_pass = [&](int c0, int c1, const float* ck, int64_t nck, int64_t f0) {
    timer_mark(kKBwdMain, false, st);
    const hipError_t r = launch(
        k_bwd_main<T, N, VEC, Cfg::kSplit, Cfg::kWaves, FZ>, dim3(unsigned(p.ng * a.B * (c1 - c0))),
        block, st, a.B, a.L, a.D, p.nf, p.nc, p.g, p.ng, c0, nck, f0, x, delta, a.A, Bm, Cm, a.Dv,
        dy, ck, gin, a.dt_bias, a.dt_softplus, static_cast<const T*>(a.z),
        static_cast<const T*>(a.ysave), static_cast<T*>(a.dx), static_cast<T*>(a.ddelta),
        static_cast<T*>(a.dz), p.dBp, p.dCp, p.dAp, p.dDp, a.ddt_bias ? p.dbp : nullptr, a.dh0);
    timer_mark(kKBwdMain, true, st);
    return r;
  };
  if (p.slab_chunks == 0) {
    if ((e = main_pass(0, p.nc, p.ckpt, p.nck, 0)) != hipSuccess) return e;
  } else {
    // sparse checkpoints: slab by slab, regenerate the dense states, then the main pass
    // (the timing hook sees each kernel's last launch)
    constexpr int64_t CK = ckpt_base(N);
    for (int c0 = 0; c0 < p.nc; c0 += p.slab_chunks) {
      const int c1 = c0 + p.slab_chunks < p.nc ? c0 + p.slab_chunks : p.nc;
      const int64_t ts = chunk_tile(c0, p.nf, p.nc, p.g) * kTc;
      const int64_t te0 = chunk_tile(c1, p.nf, p.nc, p.g) * kTc, te = te0 < a.L ? te0 : a.L;
      const int64_t k0 = ts / p.ck_every, nseg = (te - ts + p.ck_every - 1) / p.ck_every;
      // a workgroup regenerates runs of consecutive intervals, about kRegenSteps steps,
      // longer where the grid would pass one launch's limit (every interval restarts from
      // its saved state, so the run length does not change the states)
      int64_t nrun = p.ck_every >= kRegenSteps ? 1 : kRegenSteps / p.ck_every;
      const int64_t cap = kMaxGridX / (p.ng * a.B);
      if ((nseg + nrun - 1) / nrun > cap) nrun = (nseg + cap - 1) / cap;
      const int64_t nruns = (nseg + nrun - 1) / nrun;
      timer_mark(kKCkptRegen, false, st);
      e = launch(k_ckpt_regen<T, N, VEC>, dim3(unsigned(p.ng * a.B * nruns)), block, st, a.B,
                 a.L, a.D, p.ng, p.ck_every, k0, k0 + nseg, int(nrun), x, delta, a.A, Bm, p.ckpt,
                 p.nck, p.ckd, p.nckd, ts / CK);
      timer_mark(kKCkptRegen, true, st);
      if (e != hipSuccess) return e;
      if ((e = main_pass(c0, c1, p.ckd, p.nckd, ts / CK)) != hipSuccess) return e;
    }
  }
  const int64_t BLN = a.B * a.L * N;
  if ((e = launch_reduce(p.dBp, p.ng, BLN, a.dB, false, p.rtmp, st)) != hipSuccess) return e;
  if ((e = launch_reduce(p.dCp, p.ng, BLN, a.dC, false, p.rtmp, st)) != hipSuccess) return e;
  if ((e = launch_reduce(p.dAp, a.B * p.nc, a.D * N, a.dA, true, p.rtmp, st)) != hipSuccess)
    return e;
  if (FZ && a.ddt_bias &&
      (e = launch_reduce(p.dbp, a.B * p.nc, a.D, a.ddt_bias, true, p.rtmp, st)) != hipSuccess)
    return e;
  return launch_reduce(p.dDp, a.B * p.nc, a.D, a.dD, true, p.rtmp, st);
}

template <typename T, int N>
static hipError_t bwd_vec(const ScanArgs& a, const BwdPlan& p, hipStream_t st) {
  if (a.fused) return a.vec4 ? bwd_impl<T, N, 4, true>(a, p, st) : bwd_impl<T, N, 1, true>(a, p, st);
  return a.vec4 ? bwd_impl<T, N, 4, false>(a, p, st) : bwd_impl<T, N, 1, false>(a, p, st);
}

hipError_t launch_scan_bwd(const ScanArgs& a, const BwdPlan& p, hipStream_t st) {
  if (a.dtype == 0) {
    switch (a.N) {
      case 4: return bwd_vec<float, 4>(a, p, st);
      case 8: return bwd_vec<float, 8>(a, p, st);
      case 16: return bwd_vec<float, 16>(a, p, st);
    }
  } else {
    switch (a.N) {
      case 4: return bwd_vec<bf16_t, 4>(a, p, st);
      case 8: return bwd_vec<bf16_t, 8>(a, p, st);
      case 16: return bwd_vec<bf16_t, 16>(a, p, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace ssm
