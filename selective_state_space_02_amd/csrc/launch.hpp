// Internal interface between the C ABI (api.cpp) and the kernel translation units.
// Arguments arrive here already validated; plans carry workspace pointers carved
// out of the caller's workspace.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <tuple>
#include <utility>

namespace ssm {

// Kernel launch that returns the status of this launch alone: the arguments are
// converted to the kernel's parameter types and passed to hipLaunchKernel, whose return
// value is that launch's own status.  An error that an earlier runtime call left pending
// on the calling thread (the caller's, or another library's) is neither returned nor
// cleared, so it stays for its owner to read.
template <typename... P, size_t... I>
hipError_t launch_tuple(const void* fn, dim3 grid, dim3 block, hipStream_t st,
                        std::tuple<P...>& args, std::index_sequence<I...>) {
  void* argv[sizeof...(P) + 1] = {static_cast<void*>(&std::get<I>(args))..., nullptr};
  return hipLaunchKernel(fn, grid, block, argv, 0, st);
}
template <typename... P, typename... A>
hipError_t launch(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t st, A&&... args) {
  static_assert(sizeof...(P) == sizeof...(A), "kernel argument count");
  std::tuple<P...> vals(std::forward<A>(args)...);
  return launch_tuple(reinterpret_cast<const void*>(kernel), grid, block, st, vals,
                      std::index_sequence_for<P...>{});
}
// Largest grid dimension x a launch may use (hipLaunchKernel's limit for gridDim.x).
constexpr int64_t kMaxGridX = 0x7fffffff;

// Tile length of the scan kernels (steps staged through LDS at a time).
constexpr int kTc = 16;

// Checkpoints per tile: the backward recomputes states from the state before every
// (kTc / ckpt_per_tile)-th step (the dense interval, ckpt_base).  At N = 16 the backward
// stashes half a tile at a time (its register budget), so it needs the state at mid-tile
// too.  The forward saves the states at the dense interval by default, or every
// ck_every steps (a multiple of kTc); the backward then regenerates the dense states of
// one slab of chunks at a time (k_ckpt_regen) before its main pass over that slab.
constexpr int ckpt_per_tile(int64_t N) { return N == 16 ? 2 : 1; }
constexpr int64_t ckpt_base(int64_t N) { return kTc / ckpt_per_tile(N); }

// Chunk summaries the carry kernels load ahead of their sequential composition.
constexpr int kCarryAhead = 16;

struct ScanArgs {
  int dtype;  // 0 f32, 1 bf16
  int64_t B, L, D, N;
  bool vec4;  // D % 4 == 0: per-channel tiles move 4 channels per thread
  const void* x;
  const void* delta;
  const float* A;
  const void* Bm;
  const void* Cm;
  const float* Dv;
  const float* h0;  // nullable [B][D][N]
  void* y;          // fwd output
  float* h_last;    // nullable
  // backward
  const void* dy;
  void* dx;
  void* ddelta;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dh0;  // nullable
  const float* dh_last;  // nullable [B][D][N]: gradient arriving at h_{L-1} (zero if null)
  // The scan's Mamba-block neighbours (fused entry points only).  The delta input is
  // then the raw time step: delta_eff = dt_softplus ? softplus(delta + dt_bias[d])
  // : delta + dt_bias[d]; with z the output is y * silu(z).
  bool fused;            // selects the kernel variants that apply them
  const float* dt_bias;  // nullable [D] (zero)
  bool dt_softplus;
  const void* z;         // nullable [B,L,D]
  void* ysave;           // forward: nullable, y before the gate; backward: that input
  void* dz;              // backward, with z
  float* ddt_bias;       // backward, nullable, accumulated
};

// Coarse chunking of the sequence (shared rule for forward and backward).
struct Chunking {
  int nc;       // number of coarse chunks
  int64_t nf;   // number of tiles, ceil(L / kTc)
};

// Chunk c of nc covers the tiles [chunk_tile(c), chunk_tile(c + 1)) of the nf tiles of
// the sequence: an even split of units of g tiles (chunk lengths differing by at most
// one unit; the last unit may be short), so every chunk boundary is a multiple of g
// tiles.  Only the last chunk can hold the sequence's partial tile, so chunks 0..nc-2
// are full.  nc must not exceed the unit count.  floor(c * nu / nc) is formed as
// c * q + floor(c * r / nc) with nu = q * nc + r, exact without the c * nu product, which
// could pass 2^63 for sequences near the size limit cut into very many chunks.
__host__ __device__ __forceinline__ int64_t chunk_tile(int64_t c, int64_t nf, int64_t nc,
                                                      int64_t g) {
  const int64_t nu = (nf + g - 1) / g;
  const int64_t q = nu / nc, r = nu % nc;
  const int64_t t = g * (c * q + c * r / nc);
  return t < nf ? t : nf;
}

// Most slabs a sparse-checkpoint backward may split its chunks into (it keeps the chunk
// count, and every grid the backward launches, far from the 32-bit and grid limits).
constexpr int64_t kMaxSlabs = 65536;

// Position of a scan workgroup in its 1-D grid: the channel group varies fastest, then
// the batch row, then the chunk (the order of the former 3-D grid), so the grid is not
// bounded by the 65535 limit of a grid's y and z dimensions.  All three factors are
// below 2^31 (the grid's x limit), so 32-bit division suffices.
struct WgPos {
  int64_t grp, b, c;
};
__device__ __forceinline__ WgPos wg_pos(int64_t groups, int64_t B) {
  const uint32_t wg = blockIdx.x, g = uint32_t(groups), nb = uint32_t(B);
  const uint32_t r = wg / g;
  return {int64_t(wg - r * g), int64_t(r % nb), int64_t(r / nb)};
}

struct FwdPlan {
  int nc;
  int64_t nf;
  int64_t ck_every;  // steps between saved states: ckpt_base(N) or a multiple of kTc
  int64_t nck;       // number of saved states, ceil(L / ck_every)
  float* S;     // [B][nc][D][N]   (nc > 1)
  float* SD;    // [B][nc][D]      (nc > 1)
  float* hin;   // [B][nc][D][N]   (nc > 1)
  float* ckpt;  // [B][nck][D][N]  nullable
};

struct BwdPlan {
  int nc;
  int64_t nf, ng;
  int64_t g;          // chunk granularity in tiles (sparse checkpoints: every / kTc)
  int64_t nck;        // number of checkpoints
  const float* ckpt;  // [B][nck][D][N]
  // sparse checkpoints (ck_every > ckpt_base(N)): the dense states of one slab of
  // slab_chunks chunks at a time are regenerated into ckd ([B][nckd][D][N], the slab's
  // states from its first step on) before the main pass over the slab
  int64_t ck_every;
  int slab_chunks;    // 0: dense checkpoints given, one main pass over every chunk
  float* ckd;
  int64_t nckd;
  float* GS;          // [B][nc][D][N]  (nc > 1)
  float* SD;          // [B][nc][D]     (nc > 1)
  float* gin;         // [B][nc][D][N]  (nc > 1)
  float* dBp;         // [ng][B][L][N]
  float* dCp;         // [ng][B][L][N]
  float* dAp;         // [B*nc][D][N]
  float* dDp;         // [B*nc][D]
  float* dbp;         // [B*nc][D]  time-step bias partials (fused backward)
  float* rtmp;        // reduction scratch
};

struct ConvArgs {
  int dtype;
  int64_t B, L, D, K;
  int act;             // kActNone or kActSilu (dout is then the gradient of silu(conv))
  const void* x;
  const float* W;
  const float* bias;   // nullable; read only with act = kActSilu
  const void* dout;
  void* dx;
  float* dW;
  float* db;
};

struct ConvPlan {
  int64_t Tb, nTb;  // time block (a multiple of 64 steps) and the number of blocks
  float* dWp;  // [B*nTb][D][K]
  float* dbp;  // [B*nTb][D]
  float* rtmp; // reduction scratch
};

struct RmsArgs {
  int dtype;
  int64_t R, M;
  const void* dy;
  const void* x;
  const float* scale;
  const float* rms;
  void* dx;
  float* dscale;
};

struct RmsPlan {
  int64_t vec;
  int64_t passes;  // column groups per lane held at once; 0: the looped path (any M)
  int64_t rows_per_block, nblk;
  float* dsp;   // [nblk][M]
  float* crow;  // [R] per-row coefficients (looped path only)
  float* rtmp;  // reduction scratch
};

// Kernel identifiers of the timing hook (values are part of the C ABI, see
// ssm_set_kernel_timer in ssm_scan.h).
enum KernelId {
  kKFwdSummary = 1,
  kKFwdCarry = 2,
  kKFwdOutput = 3,
  kKBwdSummary = 4,
  kKBwdCarry = 5,
  kKBwdMain = 6,
  kKConvBwd = 7,
  kKRmsBwd = 8,
  kKConvFwd = 9,
  kKRmsFwd = 10,
  kKScanStep = 11,
  kKConvStep = 12,
  kKDecodeStep = 13,
  kKCkptRegen = 14,
  kKNumIds = 15
};

// Records the caller's event for kernel `id` on stream st (stop = false: before the
// launch, true: after it), if the calling thread armed one; otherwise does nothing.
void timer_mark(int id, bool stop, hipStream_t st);

hipError_t launch_scan_fwd(const ScanArgs& a, const FwdPlan& p, hipStream_t st);
hipError_t launch_scan_bwd(const ScanArgs& a, const BwdPlan& p, hipStream_t st);
hipError_t launch_conv1d_bwd(const ConvArgs& a, const ConvPlan& p, hipStream_t st);

struct ConvFwdArgs {
  int dtype;
  int64_t B, L, D, K;
  int64_t Tb, nTb;  // time blocks, as ConvPlan
  int act;          // kActNone or kActSilu (out = silu(conv))
  const void* x;
  const float* W;
  const float* bias;  // nullable
  void* out;
};
hipError_t launch_conv1d_fwd(const ConvFwdArgs& a, hipStream_t st);

struct RmsFwdArgs {
  int dtype;
  int64_t R, M;
  int64_t vec, passes, rows_per_block, nblk;  // as RmsPlan
  float eps;
  const void* x;
  const void* residual;  // nullable: added to x first
  const float* scale;
  void* y;
  float* rms;
  void* residual_out;    // with residual: x + residual, the norm's input
};
hipError_t launch_rmsnorm_fwd(const RmsFwdArgs& a, hipStream_t st);

struct ScanStepArgs {
  int dtype;
  int64_t B, D, N;
  float* h;  // [B][D][N], in place
  const void* x_t;
  const void* delta_t;
  const float* A;
  const void* B_t;
  const void* C_t;
  const float* Dv;
  void* y_t;
  // the fused step (time-step bias and softplus, output gate), as ScanArgs
  bool fused;
  const float* dt_bias;  // nullable
  bool dt_softplus;
  const void* z_t;       // nullable [B][D]
};
hipError_t launch_scan_step(const ScanStepArgs& a, hipStream_t st);

struct ConvStepArgs {
  int dtype;
  int64_t B, D, K;
  void* state;  // [B][K-1][D], in place (unused when K == 1)
  const void* x_t;
  const float* W;
  const float* bias;  // nullable
  int act;            // kActNone or kActSilu (out_t = silu(conv))
  void* out_t;
};
hipError_t launch_conv1d_step(const ConvStepArgs& a, hipStream_t st);

struct DecodeArgs {
  int dtype;
  int64_t B, D, N, K;
  float* h;          // [B][D][N], in place
  void* conv_state;  // [B][K-1][D], in place (unused when K == 1)
  const void* x_t;   // the conv's input [B][D]
  const float* W;
  const float* conv_bias;  // nullable
  const void* delta_t;
  const float* A;
  const void* B_t;
  const void* C_t;
  const float* Dv;
  const float* dt_bias;  // nullable
  bool dt_softplus;
  const void* z_t;       // nullable
  void* out_t;
};
hipError_t launch_decode_step(const DecodeArgs& a, hipStream_t st);
hipError_t launch_rmsnorm_bwd(const RmsArgs& a, const RmsPlan& p, hipStream_t st);

// The sigmoid-gated scan (alpha_scan.hip): a, b, da, db [Bn][K][S]; Wc, dWc [H][S];
// h0, h, dh, dh0 [Bn][H]; f32.
constexpr int64_t kAlphaMaxS = 1024;
struct AlphaArgs {
  int64_t Bn, K, S, H;
  const float* a;
  const float* b;
  const float* Wc;
  const float* h0;  // nullable (zero)
  float* h;
  const float* dh;
  float* da;
  float* db;
  float* dWc;  // accumulated
  float* dh0;  // nullable
};
// Launch plan of the sigmoid-gated scan: rpb batch rows per workgroup (nblk workgroups);
// dWc summed over nseg segments of `rows` batch rows, ncb column blocks of 256 (j, s).
struct AlphaPlan {
  int64_t rpb, nblk, rows, nseg, ncb;
};
AlphaPlan alpha_plan(int64_t Bn, int64_t S, int64_t H);
hipError_t launch_alpha_fwd(const AlphaArgs& a, hipStream_t st);
// Workspace: xh Bn*K*S floats, xl Bn*S, part nseg*H*S, tmp reduce_tmp_floats(nseg, H*S).
hipError_t launch_alpha_bwd(const AlphaArgs& a, float* xh, float* xl, float* part, float* tmp,
                            hipStream_t st);
// The static scratch of rmsnorm_bwd_noalloc: its size, and the device address of the
// current device's copy (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);
// out[j] (+)= sum_{p < P} part[p*J + j] in a fixed order; tmp holds
// reduce_tmp_floats(P, J) floats (may be null when that is 0).
hipError_t launch_reduce(const float* part, int64_t P, int64_t J, float* out, bool accumulate,
                         float* tmp, hipStream_t st);
int64_t reduce_tmp_floats(int64_t P, int64_t J);

}  // namespace ssm
