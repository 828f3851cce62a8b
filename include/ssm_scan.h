/*
 * ssm_scan.h -- C ABI of libssmscan.so, the MI355X (gfx950) selective-scan hot path.
 *
 * Operations on already-projected tensors:
 *   ssm_scan_fwd       selective-SSM scan, forward
 *   ssm_scan_bwd       its backward (backpropagation through time across the state)
 *   ssm_scan_fused_fwd / ssm_scan_fused_bwd
 *                      the scan with its Mamba-block neighbours fused in: time-step
 *                      bias and softplus, output gate y * silu(z)
 *   conv1d_causal_bwd  depthwise causal conv1d backward (optionally through a SiLU)
 *   rmsnorm_bwd        batched RMSNorm backward
 *   conv1d_causal_fwd  depthwise causal conv1d forward (optionally followed by SiLU)
 *   rmsnorm_fwd        batched RMSNorm forward (also returns the saved rms), optionally
 *                      after adding the residual stream
 *   ssm_scan_step      one-token decode step of the scan (state updated in place)
 *   conv1d_causal_step one-token decode step of the conv (window updated in place)
 *   ssm_scan_fused_step one-token decode step of the fused scan
 *   ssm_decode_step    one decode token of the block's scan branch (conv step, SiLU,
 *                      fused scan step) in one launch
 *   ssm_scan_fwd_every / ssm_scan_bwd_every
 *                      the scan with sparse checkpoints (states regenerated per slab);
 *                      the backward also takes the gradient arriving at the final state
 *   ssm_scan_chunks    the coarse chunk counts the scan plans (host query)
 *   ssm_alpha_scan_fwd / ssm_alpha_scan_bwd
 *                      the sigmoid-gated scan of the ml-alpha kernel (one reading)
 *   rmsnorm_bwd_noalloc  rmsnorm_bwd without a workspace (static scratch)
 *
 * Common conventions
 * ------------------
 * - Pointers.  Every tensor pointer is a DEVICE pointer to a dense, row-major,
 *   contiguous buffer; no strides or offsets cross this ABI (a strided view read as
 *   dense silently gives wrong numbers -- the failure the rustytorch backward_cuda
 *   commit reports for its matmul path).  Every tensor pointer must be 16-byte
 *   aligned.  The caller owns every buffer; the library never allocates or frees
 *   device memory.
 * - dtype.  ssm_dtype_t selects the storage type of the activations (x, delta, B, C,
 *   y, dy, dx, ddelta, conv x/dout/dx, norm x/dy/dx): f32 or bf16.  Parameters and
 *   their gradients (A, D, W, scale, rms, dA, dD, dW, db, dscale), states (h0,
 *   h_last, dh0, checkpoints) and dB/dC are always f32.  Arithmetic is f32 with f32
 *   state; bf16 outputs are rounded to nearest even.
 * - Streams.  `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Calls only enqueue work: they return before the GPU finishes and never
 *   synchronize.  Buffers must stay alive until the stream work completes.  Calls
 *   are re-entrant; the library keeps no state except a per-thread error message
 *   and the per-thread timing hook below.
 * - Workspace.  Scratch (partial sums, chunk carries) lives in a caller buffer `ws`
 *   of at least the size the matching *_workspace_bytes() query returns for the
 *   same arguments; ws may be NULL when that size is 0.  Its content on entry is
 *   ignored.  Two calls that run concurrently need separate workspaces.
 * - Accumulation.  Parameter gradients (dA, dD, dW, db, dscale) are ADDED to the
 *   caller's buffer (as the mamba-rs backward_ops.rs functions accumulate their
 *   weight and scale gradients); every other output is overwritten.
 * - Determinism.  No atomics: every sum runs in a fixed order, so repeated calls
 *   with the same inputs give bit-identical outputs.
 * - Errors.  Arguments are validated on the host before any HIP call; a rejected
 *   call enqueues nothing and leaves every output untouched.  The return value is
 *   SSM_OK or a negative SSM_ERR_* code; ssm_last_error() then describes the
 *   problem.  Nothing aborts and no exception crosses the ABI.  SSM_ERR_HIP
 *   reports only this call's launches, each taken from its own launch status: a HIP
 *   error still pending on the calling thread from earlier runtime calls (the
 *   caller's, or another library's) is neither reported as this call's failure nor
 *   cleared; it stays pending for its owner.
 * - Sizes.  Batch, sequence, channel and row counts are int64.  A size is refused
 *   (SSM_ERR_UNSUPPORTED) only where one launch's grid (2^31 - 1 workgroups) could not
 *   cover it, as stated per operation; element counts must stay below 2^46.
 */
#ifndef SSM_SCAN_H
#define SSM_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SSM_F32 = 0, SSM_BF16 = 1 } ssm_dtype_t;

/* Activation applied to the conv output: none, or SiLU, silu(p) = p * sigmoid(p) (the
 * activation the Mamba block puts between its conv and the scan; the mamba-rs
 * backward_conv1d_step section takes its gradient after the SiLU backward). */
typedef enum { SSM_ACT_NONE = 0, SSM_ACT_SILU = 1 } ssm_act_t;

enum {
    SSM_OK = 0,
    SSM_ERR_ARG = -1,          /* null required pointer, size <= 0, size overflow */
    SSM_ERR_UNSUPPORTED = -2,  /* N not in {4,8,16}, K not in [1,8], dtype, act, M too large */
    SSM_ERR_WORKSPACE = -3,    /* ws_bytes smaller than the query's answer */
    SSM_ERR_ALIGN = -4,        /* a tensor pointer is not 16-byte aligned */
    SSM_ERR_HIP = -5           /* the HIP runtime rejected a launch */
};

/* Message for the last non-OK return on the calling thread ("" if none). */
const char *ssm_last_error(void);

/* Library version string. */
const char *ssm_version(void);

/* Timing hook (measurement only; for benchmarks and profilers).  Arms, for the calling
 * thread, a pair of caller-owned hipEvent_t (passed as void*) around one kernel: every
 * later launch of that kernel by this thread records `start` on the call's stream just
 * before the launch and `stop` just after it (the pair is re-recorded at each launch,
 * so read it before the next call).  start = stop = NULL disarms.  The kernels:
 *   1 scan-forward chunk summary    2 scan-forward carry    3 scan-forward output
 *   4 scan-backward chunk summary   5 scan-backward carry   6 scan-backward main
 *   7 conv1d backward               8 RMSNorm backward
 *   9 conv1d forward               10 RMSNorm forward
 *  11 scan decode step             12 conv1d decode step
 *  13 decode token (conv step + SiLU + fused scan step)
 *  14 scan-backward regeneration of dense states from sparse checkpoints
 * (Kernels launched several times in one call -- the sparse-checkpoint backward's main
 * pass and regeneration, once per slab -- leave the pair on their last launch.)
 * Returns SSM_ERR_ARG for an unknown id or a half-set pair.  Has no effect on results. */
int ssm_set_kernel_timer(int kernel, void *start, void *stop);

/* ---------------------------------------------------------------------------------
 * Selective scan (Mamba S6).  The pages name this scan and its reverse pass -- the
 * rustytorch commit "feat(mamba): GPU-accelerated backward pass (backward_cuda)"
 * (sequential scan, its BPTT reverse pass, the shared forward recompute) and the
 * mamba-rs 0.5.1 crate summary (training by backpropagation through the SSM
 * state) -- without printing it.  Per batch row b, channel d, state n:
 *     a_t[n] = exp(delta[b,t,d] * A[d,n])
 *     h_t[n] = a_t[n] * h_{t-1}[n] + delta[b,t,d] * Bm[b,t,n] * x[b,t,d]
 *     y[b,t,d] = sum_n Cm[b,t,n] * h_t[n] + Dv[d] * x[b,t,d]
 * with h_{-1} = h0[b,d,:] or 0 (the zero-initialised state of the foxhunt ml-alpha
 * forward-pass commit).  delta is used as given (already softplus'd); A is used as
 * given (not A_log).
 *
 * Shapes: x, delta, y, dy, dx, ddelta [B,L,D]; Bm, Cm [B,L,N] (shared by all
 * channels); A, dA [D,N]; Dv, dD [D]; h0, h_last, dh0 [B,D,N]; dB, dC [B,L,N] f32.
 * Supported: N in {4, 8, 16}; 1 <= D <= 2^24 (a 16-step tile of one 64-channel
 * group is addressed with 32-bit buffer offsets); any L >= 1 (tails handled, no
 * multiple required; D a multiple of 4 takes the vectorised path); any B with
 * B * ceil(D/64) and ceil(B * D * N / 256) below 2^31 (the 1-D grids).
 *
 * Checkpoints.  The forward can save the state before every 8th step (N = 16) or
 * every 16th step (N = 4, 8) into `ckpt`
 * (ssm_scan_ckpt_bytes() bytes; layout private to this library version) for the
 * backward to recompute states from.  The backward given ckpt == NULL recomputes
 * the forward itself into its workspace.
 * ------------------------------------------------------------------------------- */
size_t ssm_scan_ckpt_bytes(int64_t B, int64_t L, int64_t D, int64_t N);
/* Plan query (host only, no GPU work): the number of coarse chunks the forward and the
 * backward split the sequence into for these sizes (chunks of whole 16-step tiles,
 * lengths differing by at most one tile).  Either pointer may be NULL.  Returns SSM_OK,
 * or SSM_ERR_ARG for non-positive sizes. */
int ssm_scan_chunks(int64_t B, int64_t L, int64_t D, int64_t N, int *fwd_chunks,
                    int *bwd_chunks);
size_t ssm_scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                    ssm_dtype_t dtype);
/* with_ckpt = 1 if the backward will be given the forward's checkpoints */
size_t ssm_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                    ssm_dtype_t dtype, int with_ckpt);

/* Forward.  Required: x, delta, A, Bm, Cm, Dv, y.  Optional (NULL to skip): h0
 * (initial state; zero if NULL), ckpt (out: checkpoints), h_last (out: state after
 * the last step). */
int ssm_scan_fwd(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                 int64_t N, const void *x, const void *delta, const float *A,
                 const void *Bm, const void *Cm, const float *Dv, const float *h0,
                 void *y, float *ckpt, float *h_last, void *ws, size_t ws_bytes);

/* Backward for upstream gradient dy [B,L,D].  Required: x, delta, A, Bm, Cm, Dv, dy,
 * dx, ddelta, dA, dB, dC, dD.  Optional: h0 (the forward's initial state; used only
 * when ckpt is NULL), ckpt (the forward's checkpoints for these same inputs and h0),
 * dh0 (out: gradient of the initial state, overwritten).
 * dx, ddelta, dB, dC, dh0 are overwritten; dA, dD are accumulated. */
int ssm_scan_bwd(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                 int64_t N, const void *x, const void *delta, const float *A,
                 const void *Bm, const void *Cm, const float *Dv, const float *h0,
                 const void *dy, const float *ckpt, void *dx, void *ddelta, float *dA,
                 float *dB, float *dC, float *dD, float *dh0, void *ws, size_t ws_bytes);

/* Checkpoint interval as a memory/compute trade (the forward cache the foxhunt ml-alpha
 * backward-scratch commit keeps, against the forward recompute of the rustytorch
 * backward_cuda commit).  ck_every = 0 is the default interval above (8 steps at N = 16,
 * 16 below), which ssm_scan_fwd/ssm_scan_bwd use; any other value must be a positive
 * multiple of 16 steps: the forward then saves the state before every ck_every-th step
 * only (ssm_scan_ckpt_bytes_every() bytes, 1/m of the default for ck_every = m x the
 * default), and the backward splits its coarse chunks (whole intervals) into `slabs`
 * slabs, regenerating the default-interval states of one slab at a time from the saved
 * ones into its workspace before its main pass over that slab: one more forward pass over
 * the sequence, and a workspace holding one slab's states (about 1/slabs of the default
 * checkpoints).  The same ck_every must be given to the forward and the backward;
 * with ckpt == NULL the backward runs the forward at that interval into its workspace.
 * Results are the default path's to within summation order (the chunks differ).
 * Returns 0 (the byte queries) or SSM_ERR_ARG for another ck_every, or slabs outside
 * [1, 65536].
 *
 * The backward also takes dh_last (nullable [B,D,N] f32): the gradient arriving at the
 * final state h_{L-1} from outside the sequence, added to that state's adjoint (NULL:
 * zero).  With it a sequence cut into consecutive pieces runs piece by piece: the forward
 * of piece k + 1 starts from the h_last of piece k (h0), and the backward of piece k
 * takes as dh_last the dh0 of piece k + 1; dA and dD then accumulate over the pieces. */
size_t ssm_scan_ckpt_bytes_every(int64_t B, int64_t L, int64_t D, int64_t N,
                                 int64_t ck_every);
size_t ssm_scan_bwd_workspace_bytes_every(int64_t B, int64_t L, int64_t D, int64_t N,
                                          ssm_dtype_t dtype, int with_ckpt, int64_t ck_every,
                                          int64_t slabs);
int ssm_scan_fwd_every(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void *x, const void *delta, const float *A,
                       const void *Bm, const void *Cm, const float *Dv, const float *h0,
                       void *y, float *ckpt, float *h_last, int64_t ck_every, void *ws,
                       size_t ws_bytes);
int ssm_scan_bwd_every(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void *x, const void *delta, const float *A,
                       const void *Bm, const void *Cm, const float *Dv, const float *h0,
                       const void *dy, const float *ckpt, void *dx, void *ddelta, float *dA,
                       float *dB, float *dC, float *dD, float *dh0, const float *dh_last,
                       int64_t ck_every, int64_t slabs, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * The scan between its neighbours in the Mamba block, fused into the scan's kernels.
 * The pages name the time-step projection's gradient (dt_proj, rustytorch backward_cuda
 * commit) and the SiLU that precedes the scan's input (mamba-rs backward_conv1d_step
 * section); the time step's activation and the output gate are not written out there and
 * are taken as in Mamba: the time step is the projection's output plus a per-channel bias
 * through a softplus, and the scan output is gated by SiLU of a second branch z.
 *     pre[b,t,d]   = delta[b,t,d] + delta_bias[d]        (delta_bias NULL: zero)
 *     dt[b,t,d]    = delta_softplus ? softplus(pre) : pre,  softplus(p) = log(1 + e^p)
 *     y            = the scan of ssm_scan_fwd with time step dt
 *     out[b,t,d]   = z ? y[b,t,d] * silu(z[b,t,d]) : y[b,t,d],  silu(p) = p * sigmoid(p)
 * Forward: y_save (optional, only with z) receives y before the gate, which the backward
 * with z needs; ckpt and h_last as in ssm_scan_fwd (the state runs on dt).
 * Backward, for upstream gradient dout of out (chain rule through the three steps):
 *     dz      = dout * y_save * silu'(z)                    (with z; dz overwritten)
 *     dy      = z ? dout * silu(z) : dout, the scan's upstream gradient
 *     ddelta  = d(dt) * (delta_softplus ? sigmoid(pre) : 1), the gradient of delta
 *     ddelta_bias[d] += sum_{b,t} ddelta[b,t,d]            (optional, accumulated)
 * and dx, dA, dB, dC, dD, dh0 as ssm_scan_bwd gives them for dt and dy.  With z, y_save
 * and dz are required; without z they must be NULL.  delta_softplus is 0 or 1.
 * Shapes and dtypes as the plain scan; z, y_save, out, dz [B,L,D] (dtype); delta_bias,
 * ddelta_bias [D] f32.  Workspace: ssm_scan_fwd_workspace_bytes /
 * ssm_scan_bwd_workspace_bytes with the same arguments.  Numerics: softplus and sigmoid
 * in f32 from the hardware exp2 and log2 (a few ulp); rows past L are zero steps.
 * ------------------------------------------------------------------------------- */
int ssm_scan_fused_fwd(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void *x, const void *delta, const float *A,
                       const void *Bm, const void *Cm, const float *Dv, const float *h0,
                       const float *delta_bias, int delta_softplus, const void *z, void *out,
                       void *y_save, float *ckpt, float *h_last, void *ws, size_t ws_bytes);
int ssm_scan_fused_bwd(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void *x, const void *delta, const float *A,
                       const void *Bm, const void *Cm, const float *Dv, const float *h0,
                       const float *delta_bias, int delta_softplus, const void *z,
                       const void *y_save, const void *dout, const float *ckpt, void *dx,
                       void *ddelta, float *dA, float *dB, float *dC, float *dD, float *dh0,
                       void *dz, float *ddelta_bias, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * Depthwise causal conv1d backward.  The mamba-rs 0.5.1 backward_ops.rs section
 * backward_conv1d_step gives one timestep of it for a shift-register conv (bias grad
 * = upstream value; weight grad = upstream value times the saved window; input grad
 * through the newest tap).  Here the whole sequence at once, for the forward
 *     out[b,t,d] = bias[d] + sum_{k<K} W[d,k] * x[b, t-K+1+k, d]   (x = 0 for t < 0):
 *     dx[b,s,d] = sum_k dout[b, s+K-1-k, d] * W[d,k]     (terms with s+K-1-k < L)
 *     dW[d,k]  += sum_{b,t} dout[b,t,d] * x[b, t-K+1+k, d]
 *     db[d]    += sum_{b,t} dout[b,t,d]
 With act = SSM_ACT_NONE, dout is the gradient of the conv output itself and bias is
 * not read.  With act = SSM_ACT_SILU, dout is the gradient of u = silu(out), and the
 * SiLU backward is fused: the kernel recomputes out (which is why bias is an input) and
 * uses g = dout * sigmoid(out) * (1 + out * (1 - sigmoid(out))) in place of dout above.
 * Shapes: x, dout, dx [B,L,D] (dtype); W, dW [D,K] f32 (tap K-1 = newest input);
 * bias, db [D] f32; bias may be NULL (zero).  Supported: K in [1, 8].
 * ------------------------------------------------------------------------------- */
size_t conv1d_causal_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t K,
                                         ssm_dtype_t dtype);
int conv1d_causal_bwd(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                      int64_t K, const void *x, const float *W, const float *bias,
                      ssm_act_t act, const void *dout, void *dx, float *dW, float *db,
                      void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * Batched RMSNorm backward given the saved per-row rms (not its inverse), as the
 * mamba-rs 0.5.1 backward_ops.rs section backward_rms_norm states it, for the
 * forward y[r,i] = x[r,i] / rms[r] * scale[i], rms[r] = sqrt(mean_i x[r,i]^2 + eps):
 *     inv = 1/rms[r],  c = inv^2 * (sum_i dy[r,i] scale[i] x[r,i]) / M
 *     dx[r,i]    = inv * (scale[i] dy[r,i] - x[r,i] * c)      (overwritten)
 *     dscale[i] += sum_r dy[r,i] * x[r,i] * inv              (accumulated)
 * Shapes: dy, x, dx [R,M] (dtype); scale, dscale [M] f32; rms [R] f32.
 * Supported: any R and M (R * M < 2^46).  Rows of up to 16 column groups per lane
 * (M <= 8192 bf16 with M a multiple of 8, M <= 4096 f32 with M a multiple of 4,
 * otherwise M <= 1024) are read once or twice by one kernel; longer rows take two
 * kernels (per-row coefficients, then column slabs of 8 groups per lane) that read
 * the row twice; the slab grid must stay below 2^31 workgroups (M below about 2^31).
 * ------------------------------------------------------------------------------- */
size_t rmsnorm_bwd_workspace_bytes(int64_t R, int64_t M, ssm_dtype_t dtype);
int rmsnorm_bwd(void *stream, ssm_dtype_t dtype, int64_t R, int64_t M, const void *dy,
                const void *x, const float *scale, const float *rms, void *dx,
                float *dscale, void *ws, size_t ws_bytes);

/* ---------------------------------------------------------------------------------
 * Sigmoid-gated scan: the foxhunt ml-alpha forward-pass commit's "selective SSM scan
 * over K timesteps with sigmoid-gated state update" (a_proj, b_proj, W_c and the
 * zero-initialised h_s2 in, h_enriched out).  The page does not print the recurrence;
 * this library computes the reading below (its results are not pinned to the pages),
 * per batch row i and state s:
 *     g_k = sigmoid(a[i,k,s]),   x_k[i,s] = g_k x_{k-1}[i,s] + (1 - g_k) b[i,k,s]
 *     h[i,j] = h0[i,j] + sum_s Wc[j,s] x_{K-1}[i,s]          (x_{-1} = 0)
 * and its exact adjoint for dh = dL/dh, with the gradient structure the backward-scratch
 * commit states (d_a and d_b summed over the hidden channels, d_W_c over the batch, d_h_s2
 * passed through):
 *     da[i,k,s], db[i,k,s] (overwritten);  dWc[j,s] += sum_i dh[i,j] x_{K-1}[i,s];
 *     dh0 = dh (overwritten; NULL to skip)
 * Shapes (f32, row-major): a, b, da, db [Bn,K,S]; Wc, dWc [H,S]; h0, h, dh, dh0 [Bn,H].
 * Supported: 1 <= S <= 1024 (states staged in LDS), any Bn, K, H whose grids fit one
 * launch (ceil(Bn / max(1, 64/S)) and ceil(H*S/256) workgroups below 2^31).  The
 * backward's workspace (ssm_alpha_scan_bwd_workspace_bytes) holds the recomputed states
 * and the dWc partial sums of batch segments (added in segment order: deterministic).
 * ------------------------------------------------------------------------------- */
size_t ssm_alpha_scan_bwd_workspace_bytes(int64_t Bn, int64_t K, int64_t S, int64_t H);
int ssm_alpha_scan_fwd(void *stream, int64_t Bn, int64_t K, int64_t S, int64_t H,
                       const float *a, const float *b, const float *Wc, const float *h0,
                       float *h);
int ssm_alpha_scan_bwd(void *stream, int64_t Bn, int64_t K, int64_t S, int64_t H,
                       const float *a, const float *b, const float *Wc, const float *dh,
                       float *da, float *db, float *dWc, float *dh0, void *ws,
                       size_t ws_bytes);

/* rmsnorm_bwd for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops, harnesses that forbid hipMalloc.  Same operation, arguments
 * and results as rmsnorm_bwd (bit for bit), without a workspace: its scratch (block
 * partials of dscale, reduction temporaries, per-row coefficients) lives in a static
 * device array of 16 MiB, one per GPU, held until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree).  It uses the current device's array: `stream`
 * must belong to the current device.  Calls on one GPU share its array, so calls whose
 * work overlaps on one GPU (other threads, other streams) race; serialize them.
 * Returns SSM_ERR_UNSUPPORTED when the plan's scratch exceeds 16 MiB (about
 * 512 x M + R floats: M up to about 8000 for long batches), SSM_ERR_HIP if the array's
 * address cannot be taken; otherwise as rmsnorm_bwd. */
int rmsnorm_bwd_noalloc(void *stream, ssm_dtype_t dtype, int64_t R, int64_t M,
                        const void *dy, const void *x, const float *scale, const float *rms,
                        void *dx, float *dscale);

/* ---------------------------------------------------------------------------------
 * Depthwise causal conv1d forward, the forward of conv1d_causal_bwd above (the window
 * of the mamba-rs backward_conv1d_step section holds the last K inputs, tap K-1 the
 * newest; the sequence starts from a zero window):
 *     out[b,t,d] = bias[d] + sum_{k<K} W[d,k] * x[b, t-K+1+k, d]   (x = 0 for t < 0)
 * With act = SSM_ACT_SILU the stored value is silu(out[b,t,d]) instead.
 * Shapes: x, out [B,L,D] (dtype); W [D,K] f32; bias [D] f32 or NULL (zero).  No
 * workspace.  Supported: K in [1, 8].
 * ------------------------------------------------------------------------------- */
int conv1d_causal_fwd(void *stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                      int64_t K, const void *x, const float *W, const float *bias,
                      ssm_act_t act, void *out);

/* ---------------------------------------------------------------------------------
 * Batched RMSNorm forward, the forward of rmsnorm_bwd above; it also writes the
 * per-row rms that the backward takes as its saved statistic (the mamba-rs
 * backward_rms_norm section saves rms, not its inverse):
 *     rms[r] = sqrt(mean_i x[r,i]^2 + eps),   y[r,i] = x[r,i] / rms[r] * scale[i]
 * With the residual stream (residual and residual_out both given, or both NULL), the
 * block's add comes first: h = x + residual is computed in f32, rounded to the dtype and
 * written to residual_out (the stream passed on), and the norm above is applied to that
 * stored h, so that rmsnorm_bwd with x = residual_out and this rms is exact.
 * Shapes: x, residual, residual_out, y [R,M] (dtype); scale [M] f32; rms [R] f32 (out).
 * eps finite, >= 0.  No workspace.  Supported M: as rmsnorm_bwd.
 * ------------------------------------------------------------------------------- */
int rmsnorm_fwd(void *stream, ssm_dtype_t dtype, int64_t R, int64_t M, const void *x,
                const void *residual, const float *scale, float eps, void *y, float *rms,
                void *residual_out);

/* ---------------------------------------------------------------------------------
 * One-token decode step of the selective scan: the single-step updater the rustytorch
 * backward_cuda commit describes for inference.  For every batch row b, channel d,
 * state n:
 *     h[b,d,n] <- exp(delta_t[b,d] * A[d,n]) * h[b,d,n] + delta_t[b,d] * B_t[b,n] * x_t[b,d]
 *     y_t[b,d]  = sum_n C_t[b,n] * h[b,d,n] + Dv[d] * x_t[b,d]
 * i.e. one timestep of ssm_scan_fwd; a sequence decoded token by token from h = h0 gives
 * the scan's outputs.  Each (b, d) is computed independently, in a fixed order, so the
 * results do not depend on which other rows share the batch.
 * Shapes: h [B,D,N] f32 (in/out, updated in place); x_t, delta_t, y_t [B,D] (dtype);
 * B_t, C_t [B,N] (dtype); A [D,N] f32; Dv [D] f32.  No workspace.  Supported sizes as
 * ssm_scan_fwd.
 * ------------------------------------------------------------------------------- */
int ssm_scan_step(void *stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t N, float *h,
                  const void *x_t, const void *delta_t, const float *A, const void *B_t,
                  const void *C_t, const float *Dv, void *y_t);

/* ---------------------------------------------------------------------------------
 * One-token decode step of the depthwise causal conv1d.  state [B,K-1,D] (dtype) holds
 * the last K-1 inputs, oldest first (all zero at the start of a sequence):
 *     out_t[b,d] = bias[d] + sum_{k<K-1} W[d,k] * state[b,k,d] + W[d,K-1] * x_t[b,d]
 * then the window moves one step in place (the oldest input drops out, x_t becomes the
 * newest).  A sequence stepped token by token gives conv1d_causal_fwd's outputs (with
 * the same act: SSM_ACT_SILU stores silu of the sum).
 * Shapes: x_t, out_t [B,D] (dtype); W [D,K] f32; bias [D] f32 or NULL (zero); state may
 * be NULL when K = 1.  No workspace.  Supported: K in [1, 8], B*D <= 2^38.
 * ------------------------------------------------------------------------------- */
int conv1d_causal_step(void *stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t K,
                       void *state, const void *x_t, const float *W, const float *bias,
                       ssm_act_t act, void *out_t);

/* ---------------------------------------------------------------------------------
 * One token of ssm_scan_fused_fwd: the time step dt = softplus(delta_t + delta_bias)
 * (delta_softplus = 1) or delta_t + delta_bias (0; delta_bias NULL = zero), one step of
 * ssm_scan_step with it, and out_t = y_t * silu(z_t) when z_t is given (else y_t).  A
 * sequence decoded token by token from h = h0 gives ssm_scan_fused_fwd's out and final
 * state.  Shapes as ssm_scan_step; delta_bias [D] f32; z_t [B,D] (dtype).  No workspace.
 * ------------------------------------------------------------------------------- */
int ssm_scan_fused_step(void *stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t N,
                        float *h, const void *x_t, const void *delta_t, const float *A,
                        const void *B_t, const void *C_t, const float *Dv,
                        const float *delta_bias, int delta_softplus, const void *z_t,
                        void *out_t);

/* ---------------------------------------------------------------------------------
 * One decode token of the Mamba block's scan branch in one launch: the conv step on x_t
 * (conv1d_causal_step with act = SSM_ACT_SILU; its output rounded to the dtype, as that
 * call stores it), then ssm_scan_fused_step on that input.  Same results, bit for bit, as
 * those two calls in sequence; conv_state and h are updated in place.
 * Shapes: h [B,D,N] f32; conv_state [B,K-1,D] (dtype; may be NULL when K = 1); x_t,
 * delta_t, z_t, out_t [B,D] (dtype); W [D,K] f32; conv_bias, delta_bias [D] f32 or NULL;
 * A [D,N] f32; B_t, C_t [B,N] (dtype); Dv [D] f32.  No workspace.  Supported: as
 * ssm_scan_step, K in [1, 8].
 * ------------------------------------------------------------------------------- */
int ssm_decode_step(void *stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t N,
                    int64_t K, float *h, void *conv_state, const void *x_t, const float *W,
                    const float *conv_bias, const void *delta_t, const float *A,
                    const void *B_t, const void *C_t, const float *Dv, const float *delta_bias,
                    int delta_softplus, const void *z_t, void *out_t);

#ifdef __cplusplus
}
#endif

#endif /* SSM_SCAN_H */
