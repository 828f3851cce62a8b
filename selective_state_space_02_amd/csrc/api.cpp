// C ABI of libssmscan.so: host-side validation, workspace sizing and carving, and the
// launch sequence of each operation.  All validation happens before the first HIP
// call, so every rejection path runs (and is tested) without a GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <initializer_list>
#include <string>
#include <utility>

#include "../../include/ssm_scan.h"
#include "launch.hpp"

namespace {

thread_local std::string g_err;

// Timing hook: per-thread caller events recorded around one kernel's launch.
struct TimerSlot {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local TimerSlot g_timer[ssm::kKNumIds];

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return SSM_OK;
}

constexpr int64_t kMaxElems = int64_t(1) << 46;  // guards int64 index arithmetic
constexpr size_t kAlign = 256;                    // workspace sub-buffer alignment

size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Carves consecutive 256-byte-aligned regions out of a workspace.
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base(static_cast<char*>(b)) {}
  float* take(size_t nfloats) {
    float* p = base ? reinterpret_cast<float*>(base + off) : nullptr;
    off += round_up(nfloats * sizeof(float));
    return p;
  }
};

// ---------------------------------------------------------------------------------
// scan plans
// ---------------------------------------------------------------------------------
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// MI355X: 256 compute units.  Workgroups a scan launch aims for: every pass kernel
// (summary and main) is latency- and issue-bound per SIMD, and a single wave per SIMD
// issues at about a third of the rate of several, so a grid many times larger than the
// resident set keeps every SIMD loaded to the end (measured on the 2 x 16384 x 5120
// layer: chunk counts from 3 to 32 take the backward from 3.06 to 2.56 ms and the
// forward from 1.64 to 1.13 ms, flat beyond).
constexpr int64_t kCUs = 256;
constexpr int64_t kFwdTargetWG = kCUs * 32;
constexpr int64_t kBwdTargetWG = kCUs * 20;
// Every chunk costs a fixed prologue and epilogue in each pass (addressing, the first
// tiles' loads, the carried state, its dA/dD partials), so chunks shorter than about 16
// tiles pay for themselves only where the grid would otherwise be too small.  Measured on
// 8 x 2048 x 1536 (f32): 64 + 32 chunks (2 and 4 tiles) 0.620 ms, 8 + 8 chunks 0.558 ms;
// on 4 x 8192 x 2560 (bf16) 57 + 32 chunks 1.563 ms, 32 + 32 1.548 ms; on 2 x 16384 x
// 5120 the plan is unchanged.
constexpr int64_t kLongChunkTiles = 16;
constexpr int64_t kMinChunkWG = kCUs * 4;

// Coarse chunking of the sequence: whole units of g tiles per chunk (g = 1, or the tiles
// of one sparse-checkpoint interval), the longest chunks whose count reaches the target
// grid (nu / want units each), but at least two tiles per chunk: below that the summary
// pass costs as much as it saves.  Chunks are then lengthened towards kLongChunkTiles
// tiles as far as the grid keeps kMinChunkWG workgroups.  The chunks split the units
// evenly (ssm::chunk_tile).
ssm::Chunking choose_chunks(int64_t B, int64_t L, int64_t D, int64_t target, int64_t g = 1) {
  ssm::Chunking c;
  c.nf = cdiv(L, ssm::kTc);
  const int64_t nu = cdiv(c.nf, g);   // units
  const int64_t W = B * cdiv(D, 64);  // workgroups per chunk
  const int64_t want = cdiv(target, W);
  int64_t units = want > 1 ? nu / want : nu;  // units per chunk
  const int64_t umin = g >= 2 ? 1 : (nu < 2 ? nu : 2);
  if (units < umin) units = umin;
  const int64_t ulong = cdiv(kLongChunkTiles, g);
  if (units < ulong) {
    // the longest units up to ulong whose chunk count still gives kMinChunkWG workgroups
    const int64_t nc_min = cdiv(kMinChunkWG, W);
    int64_t u = nc_min <= 1 ? nu : nu / nc_min;
    if (u > ulong) u = ulong;
    if (u > units) units = u;
  }
  c.nc = int(cdiv(nu, units));
  return c;
}

// The checkpoint interval a call uses: every = 0 selects the dense interval
// (ssm::ckpt_base: 8 steps at N = 16, 16 below).
int64_t ck_interval(int64_t N, int64_t every) { return every == 0 ? ssm::ckpt_base(N) : every; }

// checkpoints: the state before every `every`-th step
int64_t ckpt_count(int64_t L, int64_t every) { return cdiv(L, every); }

// Largest reduction scratch (floats) over the (partials, outputs) pairs one call reduces.
int64_t max_tmp(std::initializer_list<std::pair<int64_t, int64_t>> pj) {
  int64_t m = 0;
  for (const auto& q : pj) {
    const int64_t t = ssm::reduce_tmp_floats(q.first, q.second);
    if (t > m) m = t;
  }
  return m;
}

size_t fwd_ws(int64_t B, int64_t L, int64_t D, int64_t N, int64_t every, ssm::FwdPlan* plan,
              void* ws) {
  const ssm::Chunking c = choose_chunks(B, L, D, kFwdTargetWG);
  Carver cv(ws);
  ssm::FwdPlan p{};
  p.nc = c.nc;
  p.nf = c.nf;
  p.ck_every = ck_interval(N, every);
  p.nck = ckpt_count(L, p.ck_every);
  if (c.nc > 1) {
    p.S = cv.take(size_t(B) * c.nc * D * N);
    p.SD = cv.take(size_t(B) * c.nc * D);
    p.hin = cv.take(size_t(B) * c.nc * D * N);
  }
  if (plan) *plan = p;
  return cv.off;
}

size_t ckpt_floats(int64_t B, int64_t L, int64_t D, int64_t N, int64_t every) {
  return size_t(B) * size_t(ckpt_count(L, ck_interval(N, every))) * size_t(D) * size_t(N);
}

// Backward plan.  With sparse checkpoints (every above the dense interval) the chunks are
// whole checkpoint intervals (g = every / kTc tiles), and the main pass runs over slabs
// of slab_chunks chunks, each after regenerating its dense states into ckd.  The chunk
// target then also gives each slab's main launch about two rounds of resident
// workgroups (three per CU): measured on the 2 x 16384 x 5120 layer, the backward's time
// is flat in the chunk count (32 to 256 chunks within 2%) but drops when a slab's launch
// would not fill the GPU (4 chunks of 160 workgroups per slab: +0.35 ms), while the
// per-chunk buffers (carries, dA partials) grow with the count.
size_t bwd_ws(int64_t B, int64_t L, int64_t D, int64_t N, bool with_ckpt, int64_t every,
              int64_t slabs, ssm::BwdPlan* plan, float** ckpt_out, ssm::FwdPlan* fplan,
              void* ws) {
  const int64_t ev = ck_interval(N, every);
  const bool sparse = ev != ssm::ckpt_base(N);
  const int64_t g = sparse ? ev / ssm::kTc : 1;
  const int64_t slab_target = slabs * kCUs * 6;
  const int64_t target = sparse && slab_target > kBwdTargetWG ? slab_target : kBwdTargetWG;
  const ssm::Chunking c = choose_chunks(B, L, D, target, g);
  Carver cv(ws);
  ssm::BwdPlan p{};
  p.nc = c.nc;
  p.nf = c.nf;
  p.g = g;
  p.ck_every = ev;
  p.nck = ckpt_count(L, ev);
  p.ng = cdiv(D, 64);
  if (c.nc > 1) {
    p.GS = cv.take(size_t(B) * c.nc * D * N);
    p.SD = cv.take(size_t(B) * c.nc * D);
    p.gin = cv.take(size_t(B) * c.nc * D * N);
  }
  p.dBp = cv.take(size_t(p.ng) * B * L * N);
  p.dCp = cv.take(size_t(p.ng) * B * L * N);
  p.dAp = cv.take(size_t(B) * c.nc * D * N);
  p.dDp = cv.take(size_t(B) * c.nc * D);
  p.dbp = cv.take(size_t(B) * c.nc * D);
  {
    // scratch for every reduction the backward runs (dB/dC, dA, dD and the time-step
    // bias share it in turn); the need is not monotone in the output count
    const int64_t t = max_tmp({{p.ng, B * L * N}, {B * c.nc, D * N}, {B * c.nc, D}});
    p.rtmp = cv.take(size_t(t));
  }
  if (sparse) {
    p.slab_chunks = int(cdiv(c.nc, slabs));
    int64_t mx = 0;  // dense states of the longest slab
    for (int64_t c0 = 0; c0 < c.nc; c0 += p.slab_chunks) {
      const int64_t c1 = c0 + p.slab_chunks < c.nc ? c0 + p.slab_chunks : c.nc;
      const int64_t ts = ssm::chunk_tile(c0, c.nf, c.nc, g) * ssm::kTc;
      int64_t te = ssm::chunk_tile(c1, c.nf, c.nc, g) * ssm::kTc;
      if (te > L) te = L;
      const int64_t n = cdiv(te - ts, ssm::ckpt_base(N));
      if (n > mx) mx = n;
    }
    p.nckd = mx;
    p.ckd = cv.take(size_t(B) * size_t(mx) * size_t(D) * size_t(N));
  }
  if (!with_ckpt) {
    float* ck = cv.take(ckpt_floats(B, L, D, N, every));
    if (ckpt_out) *ckpt_out = ck;
    // the forward's own workspace follows
    char* fbase = ws ? static_cast<char*>(ws) + cv.off : nullptr;
    cv.off += fwd_ws(B, L, D, N, every, fplan, fbase);
  }
  if (plan) *plan = p;
  return cv.off;
}

// every: 0 (the dense interval), the dense interval itself, or a positive multiple of
// kTc; slabs >= 1
int check_ckpt_every(int64_t N, int64_t every, int64_t slabs) {
  if (every < 0 || (every != 0 && every != ssm::ckpt_base(N) && every % ssm::kTc != 0))
    return fail(SSM_ERR_ARG,
                "checkpoint interval %lld must be 0, %lld or a positive multiple of %d steps",
                (long long)every, (long long)ssm::ckpt_base(N), ssm::kTc);
  if (slabs < 1 || slabs > ssm::kMaxSlabs)
    return fail(SSM_ERR_ARG, "slabs must be in [1, %lld] (got %lld)", (long long)ssm::kMaxSlabs,
                (long long)slabs);
  return SSM_OK;
}

int check_scan_dims(ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D, int64_t N) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (B=%lld L=%lld D=%lld N=%lld)",
                (long long)B, (long long)L, (long long)D, (long long)N);
  if (dtype != SSM_F32 && dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "dtype %d not supported (SSM_F32 or SSM_BF16)", int(dtype));
  if (N != 4 && N != 8 && N != 16)
    return fail(SSM_ERR_UNSUPPORTED, "state size N=%lld not supported (4, 8 or 16)", (long long)N);
  // a 16-step tile of one channel group spans < 2^31 bytes (32-bit buffer offsets)
  if (D > (int64_t(1) << 24))
    return fail(SSM_ERR_UNSUPPORTED, "channels D=%lld exceed 2^24", (long long)D);
  if (B > kMaxElems / L || B * L > kMaxElems / D || B * L * D > kMaxElems / N)
    return fail(SSM_ERR_ARG, "tensor sizes overflow");
  // one workgroup per (64-channel group, batch row) of a chunk, on a 1-D grid; the carry
  // kernels take one thread per (batch row, channel, state)
  if (B * cdiv(D, 64) > ssm::kMaxGridX || cdiv(B * D * N, 256) > ssm::kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "B*D=%lld channels exceed one launch's grid",
                (long long)(B * D));
  return SSM_OK;
}

struct Ptr {
  const void* p;
  const char* name;
};

constexpr const char* kAlignHint =
    " (a view at an offset into a larger buffer keeps the offset: pass a copy)";

int check_ptrs(std::initializer_list<Ptr> required, std::initializer_list<Ptr> optional) {
  for (const Ptr& q : required)
    if (!q.p) return fail(SSM_ERR_ARG, "required pointer '%s' is NULL", q.name);
  for (const Ptr& q : required)
    if (!aligned16(q.p))
      return fail(SSM_ERR_ALIGN, "pointer '%s' is not 16-byte aligned%s", q.name, kAlignHint);
  for (const Ptr& q : optional)
    if (q.p && !aligned16(q.p))
      return fail(SSM_ERR_ALIGN, "pointer '%s' is not 16-byte aligned%s", q.name, kAlignHint);
  return SSM_OK;
}

int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(SSM_ERR_WORKSPACE, "workspace too small: %zu bytes given, %zu needed", ws_bytes,
                need);
  if (need > 0 && !ws) return fail(SSM_ERR_WORKSPACE, "workspace pointer is NULL");
  if (ws && !aligned16(ws)) return fail(SSM_ERR_ALIGN, "workspace is not 16-byte aligned");
  return SSM_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

// conv plan
void conv_plan(int64_t B, int64_t L, int64_t D, int64_t K, ssm::ConvPlan* p) {
  // about 4096 workgroups; a workgroup spans 64 lanes of 4 channels (2 above width 4;
  // 1 when D is not a multiple of 4); time blocks are multiples of 64 steps (four
  // wavefronts x groups of 8 or 16 steps)
  const int64_t vec = (D % 4 != 0) ? 1 : (K <= 4 ? 4 : 2);
  const int64_t cgroups = cdiv(D, 64 * vec);
  int64_t nTb = cdiv(4096, cgroups * B);  // (cgroups * B <= kMaxGridX, check_conv_dims)
  const int64_t maxTb = cdiv(L, 64);
  if (nTb > maxTb) nTb = maxTb;
  if (nTb < 1) nTb = 1;
  p->Tb = cdiv(cdiv(L, nTb), 64) * 64;
  p->nTb = cdiv(L, p->Tb);
}

size_t conv_ws(int64_t B, int64_t L, int64_t D, int64_t K, ssm_dtype_t dt, ssm::ConvPlan* plan,
               void* ws) {
  ssm::ConvPlan p{};
  conv_plan(B, L, D, K, &p);
  Carver cv(ws);
  p.dWp = cv.take(size_t(B) * p.nTb * D * K);
  p.dbp = cv.take(size_t(B) * p.nTb * D);
  p.rtmp = cv.take(size_t(max_tmp({{B * p.nTb, D * K}, {B * p.nTb, D}})));
  if (plan) *plan = p;
  return cv.off;
}

// rms plan (every R and M: rows of more than 16 column groups per lane take the looped
// path, passes = 0)
void rms_plan(int64_t R, int64_t M, ssm_dtype_t dt, ssm::RmsPlan* p) {
  const int64_t full = (dt == SSM_BF16) ? 8 : 4;
  p->vec = (M % full == 0) ? full : 1;
  const int64_t per_pass = 64 * p->vec;
  const int64_t need = cdiv(M, per_pass);
  // rows of up to 8 passes stay in registers, up to 16 are read twice
  p->passes = need <= 8 ? need : (need <= 16 ? 16 : 0);
  // about 512 blocks of 4 wavefronts (each block leaves one dscale partial row; 2048
  // blocks measured no faster and cost a 4x larger reduce), at least 4 rows per block
  int64_t rpb = cdiv(R, 512);
  if (rpb < 4) rpb = 4;
  p->rows_per_block = rpb;
  p->nblk = cdiv(R, rpb);
}

size_t rms_ws(int64_t R, int64_t M, ssm_dtype_t dt, ssm::RmsPlan* plan, void* ws) {
  ssm::RmsPlan p{};
  rms_plan(R, M, dt, &p);
  Carver cv(ws);
  p.dsp = cv.take(size_t(p.nblk) * M);
  if (p.passes == 0) p.crow = cv.take(size_t(R));
  p.rtmp = cv.take(size_t(ssm::reduce_tmp_floats(p.nblk, M)));
  if (plan) *plan = p;
  return cv.off;
}

}  // namespace

void ssm::timer_mark(int id, bool stop, hipStream_t st) {
  if (id <= 0 || id >= kKNumIds) return;
  hipEvent_t e = stop ? g_timer[id].stop : g_timer[id].start;
  if (e) (void)hipEventRecord(e, st);
}

extern "C" {

int ssm_set_kernel_timer(int kernel, void* start, void* stop) {
  if (kernel <= 0 || kernel >= ssm::kKNumIds)
    return fail(SSM_ERR_ARG, "unknown kernel id %d", kernel);
  if ((start == nullptr) != (stop == nullptr))
    return fail(SSM_ERR_ARG, "start and stop events must both be set or both be NULL");
  g_timer[kernel].start = static_cast<hipEvent_t>(start);
  g_timer[kernel].stop = static_cast<hipEvent_t>(stop);
  return ok();
}


const char* ssm_last_error(void) { return g_err.c_str(); }

const char* ssm_version(void) { return "ssmscan-gfx950 0.1.0"; }

size_t ssm_scan_ckpt_bytes_every(int64_t B, int64_t L, int64_t D, int64_t N, int64_t every) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 0;
  if (every < 0 || (every != 0 && every != ssm::ckpt_base(N) && every % ssm::kTc != 0)) return 0;
  return ckpt_floats(B, L, D, N, every) * sizeof(float);
}

size_t ssm_scan_ckpt_bytes(int64_t B, int64_t L, int64_t D, int64_t N) {
  return ssm_scan_ckpt_bytes_every(B, L, D, N, 0);
}

int ssm_scan_chunks(int64_t B, int64_t L, int64_t D, int64_t N, int* fwd_chunks,
                    int* bwd_chunks) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (B=%lld L=%lld D=%lld N=%lld)",
                (long long)B, (long long)L, (long long)D, (long long)N);
  if (fwd_chunks) *fwd_chunks = choose_chunks(B, L, D, kFwdTargetWG).nc;
  if (bwd_chunks) *bwd_chunks = choose_chunks(B, L, D, kBwdTargetWG).nc;
  return ok();
}

size_t ssm_scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype_t) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 0;
  return fwd_ws(B, L, D, N, 0, nullptr, nullptr);
}

size_t ssm_scan_bwd_workspace_bytes_every(int64_t B, int64_t L, int64_t D, int64_t N,
                                          ssm_dtype_t, int with_ckpt, int64_t every,
                                          int64_t slabs) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 0;
  if (every < 0 || (every != 0 && every != ssm::ckpt_base(N) && every % ssm::kTc != 0) ||
      slabs < 1 || slabs > ssm::kMaxSlabs)
    return 0;
  return bwd_ws(B, L, D, N, with_ckpt != 0, every, slabs, nullptr, nullptr, nullptr, nullptr);
}

size_t ssm_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N,
                                    ssm_dtype_t dtype, int with_ckpt) {
  return ssm_scan_bwd_workspace_bytes_every(B, L, D, N, dtype, with_ckpt, 0, 1);
}

int ssm_scan_fwd_every(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void* x, const void* delta, const float* A,
                       const void* Bm, const void* Cm, const float* Dv, const float* h0,
                       void* y, float* ckpt, float* h_last, int64_t ck_every, void* ws,
                       size_t ws_bytes) {
  int rc = check_scan_dims(dtype, B, L, D, N);
  if (rc) return rc;
  if ((rc = check_ckpt_every(N, ck_every, 1))) return rc;
  rc = check_ptrs({{x, "x"}, {delta, "delta"}, {A, "A"}, {Bm, "Bm"}, {Cm, "Cm"}, {Dv, "Dv"}, {y, "y"}},
                  {{h0, "h0"}, {ckpt, "ckpt"}, {h_last, "h_last"}});
  if (rc) return rc;
  ssm::FwdPlan p{};
  const size_t need = fwd_ws(B, L, D, N, ck_every, &p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  fwd_ws(B, L, D, N, ck_every, &p, ws);
  p.ckpt = ckpt;
  ssm::ScanArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dv = Dv; a.h0 = h0;
  a.y = y; a.h_last = h_last;
  a.vec4 = D % 4 == 0;
  return hip_status(ssm::launch_scan_fwd(a, p, static_cast<hipStream_t>(stream)), "ssm_scan_fwd");
}

int ssm_scan_fwd(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D, int64_t N,
                 const void* x, const void* delta, const float* A, const void* Bm,
                 const void* Cm, const float* Dv, const float* h0, void* y, float* ckpt,
                 float* h_last, void* ws, size_t ws_bytes) {
  return ssm_scan_fwd_every(stream, dtype, B, L, D, N, x, delta, A, Bm, Cm, Dv, h0, y, ckpt,
                            h_last, 0, ws, ws_bytes);
}

int ssm_scan_bwd_every(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void* x, const void* delta, const float* A,
                       const void* Bm, const void* Cm, const float* Dv, const float* h0,
                       const void* dy, const float* ckpt, void* dx, void* ddelta, float* dA,
                       float* dB, float* dC, float* dD, float* dh0, const float* dh_last,
                       int64_t ck_every, int64_t slabs, void* ws, size_t ws_bytes) {
  int rc = check_scan_dims(dtype, B, L, D, N);
  if (rc) return rc;
  if ((rc = check_ckpt_every(N, ck_every, slabs))) return rc;
  rc = check_ptrs({{x, "x"}, {delta, "delta"}, {A, "A"}, {Bm, "Bm"}, {Cm, "Cm"}, {Dv, "Dv"},
                   {dy, "dy"}, {dx, "dx"}, {ddelta, "ddelta"}, {dA, "dA"}, {dB, "dB"},
                   {dC, "dC"}, {dD, "dD"}},
                  {{h0, "h0"}, {ckpt, "ckpt"}, {dh0, "dh0"}, {dh_last, "dh_last"}});
  if (rc) return rc;
  const bool with_ckpt = ckpt != nullptr;
  ssm::BwdPlan p{};
  ssm::FwdPlan fp{};
  float* own_ckpt = nullptr;
  const size_t need = bwd_ws(B, L, D, N, with_ckpt, ck_every, slabs, &p, &own_ckpt, &fp, nullptr);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  bwd_ws(B, L, D, N, with_ckpt, ck_every, slabs, &p, &own_ckpt, &fp, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  ssm::ScanArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dv = Dv; a.h0 = h0;
  a.dy = dy; a.dx = dx; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD;
  a.dh0 = dh0;
  a.dh_last = dh_last;
  a.vec4 = D % 4 == 0;
  if (with_ckpt) {
    p.ckpt = ckpt;
  } else {
    // recompute the forward's checkpoints (at the same interval; y is not needed)
    fp.ckpt = own_ckpt;
    ssm::ScanArgs f = a;
    f.y = nullptr;
    f.h_last = nullptr;
    hipError_t e = ssm::launch_scan_fwd(f, fp, st);
    if (e != hipSuccess) return hip_status(e, "ssm_scan_bwd (forward recompute)");
    p.ckpt = own_ckpt;
  }
  return hip_status(ssm::launch_scan_bwd(a, p, st), "ssm_scan_bwd");
}

int ssm_scan_bwd(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D, int64_t N,
                 const void* x, const void* delta, const float* A, const void* Bm,
                 const void* Cm, const float* Dv, const float* h0, const void* dy,
                 const float* ckpt, void* dx, void* ddelta, float* dA, float* dB, float* dC,
                 float* dD, float* dh0, void* ws, size_t ws_bytes) {
  return ssm_scan_bwd_every(stream, dtype, B, L, D, N, x, delta, A, Bm, Cm, Dv, h0, dy, ckpt,
                            dx, ddelta, dA, dB, dC, dD, dh0, nullptr, 0, 1, ws, ws_bytes);
}

int ssm_scan_fused_fwd(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void* x, const void* delta, const float* A,
                       const void* Bm, const void* Cm, const float* Dv, const float* h0,
                       const float* delta_bias, int delta_softplus, const void* z, void* out,
                       void* y_save, float* ckpt, float* h_last, void* ws, size_t ws_bytes) {
  int rc = check_scan_dims(dtype, B, L, D, N);
  if (rc) return rc;
  rc = check_ptrs({{x, "x"}, {delta, "delta"}, {A, "A"}, {Bm, "Bm"}, {Cm, "Cm"}, {Dv, "Dv"},
                   {out, "out"}},
                  {{h0, "h0"}, {delta_bias, "delta_bias"}, {z, "z"}, {y_save, "y_save"},
                   {ckpt, "ckpt"}, {h_last, "h_last"}});
  if (rc) return rc;
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_ARG, "delta_softplus must be 0 or 1 (got %d)", delta_softplus);
  if (y_save && !z) return fail(SSM_ERR_ARG, "y_save is only written with the gate input z");
  ssm::FwdPlan p{};
  const size_t need = fwd_ws(B, L, D, N, 0, &p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  fwd_ws(B, L, D, N, 0, &p, ws);
  p.ckpt = ckpt;
  ssm::ScanArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dv = Dv; a.h0 = h0;
  a.y = out; a.h_last = h_last;
  a.vec4 = D % 4 == 0;
  a.fused = true;
  a.dt_bias = delta_bias; a.dt_softplus = delta_softplus != 0;
  a.z = z; a.ysave = y_save;
  return hip_status(ssm::launch_scan_fwd(a, p, static_cast<hipStream_t>(stream)),
                    "ssm_scan_fused_fwd");
}

int ssm_scan_fused_bwd(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                       int64_t N, const void* x, const void* delta, const float* A,
                       const void* Bm, const void* Cm, const float* Dv, const float* h0,
                       const float* delta_bias, int delta_softplus, const void* z,
                       const void* y_save, const void* dout, const float* ckpt, void* dx,
                       void* ddelta, float* dA, float* dB, float* dC, float* dD, float* dh0,
                       void* dz, float* ddelta_bias, void* ws, size_t ws_bytes) {
  int rc = check_scan_dims(dtype, B, L, D, N);
  if (rc) return rc;
  rc = check_ptrs({{x, "x"}, {delta, "delta"}, {A, "A"}, {Bm, "Bm"}, {Cm, "Cm"}, {Dv, "Dv"},
                   {dout, "dout"}, {dx, "dx"}, {ddelta, "ddelta"}, {dA, "dA"}, {dB, "dB"},
                   {dC, "dC"}, {dD, "dD"}},
                  {{h0, "h0"}, {delta_bias, "delta_bias"}, {z, "z"}, {y_save, "y_save"},
                   {ckpt, "ckpt"}, {dh0, "dh0"}, {dz, "dz"}, {ddelta_bias, "ddelta_bias"}});
  if (rc) return rc;
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_ARG, "delta_softplus must be 0 or 1 (got %d)", delta_softplus);
  if (z && (!y_save || !dz))
    return fail(SSM_ERR_ARG, "with the gate input z, y_save and dz are required");
  if (!z && (y_save || dz))
    return fail(SSM_ERR_ARG, "y_save and dz are only used with the gate input z");
  const bool with_ckpt = ckpt != nullptr;
  ssm::BwdPlan p{};
  ssm::FwdPlan fp{};
  float* own_ckpt = nullptr;
  const size_t need = bwd_ws(B, L, D, N, with_ckpt, 0, 1, &p, &own_ckpt, &fp, nullptr);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  bwd_ws(B, L, D, N, with_ckpt, 0, 1, &p, &own_ckpt, &fp, ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  ssm::ScanArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.L = L; a.D = D; a.N = N;
  a.x = x; a.delta = delta; a.A = A; a.Bm = Bm; a.Cm = Cm; a.Dv = Dv; a.h0 = h0;
  a.dy = dout; a.dx = dx; a.ddelta = ddelta; a.dA = dA; a.dB = dB; a.dC = dC; a.dD = dD;
  a.dh0 = dh0;
  a.vec4 = D % 4 == 0;
  a.fused = true;
  a.dt_bias = delta_bias; a.dt_softplus = delta_softplus != 0;
  a.z = z; a.ysave = const_cast<void*>(y_save); a.dz = dz; a.ddt_bias = ddelta_bias;
  if (with_ckpt) {
    p.ckpt = ckpt;
  } else {
    // recompute the forward's checkpoints with the same time step (no output, no gate)
    fp.ckpt = own_ckpt;
    ssm::ScanArgs f = a;
    f.y = nullptr;
    f.h_last = nullptr;
    f.z = nullptr;
    f.ysave = nullptr;
      hipError_t e = ssm::launch_scan_fwd(f, fp, st);
    if (e != hipSuccess) return hip_status(e, "ssm_scan_fused_bwd (forward recompute)");
    p.ckpt = own_ckpt;
  }
  return hip_status(ssm::launch_scan_bwd(a, p, st), "ssm_scan_fused_bwd");
}

static int check_conv_dims(ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D, int64_t K,
                           ssm_act_t act) {
  if (B <= 0 || L <= 0 || D <= 0 || K <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (B=%lld L=%lld D=%lld K=%lld)",
                (long long)B, (long long)L, (long long)D, (long long)K);
  if (dtype != SSM_F32 && dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (act != SSM_ACT_NONE && act != SSM_ACT_SILU)
    return fail(SSM_ERR_UNSUPPORTED, "activation %d not supported (0 none, 1 SiLU)", int(act));
  if (K > 8) return fail(SSM_ERR_UNSUPPORTED, "conv width K=%lld not supported (1..8)", (long long)K);
  if (B > kMaxElems / L || B * L > kMaxElems / D) return fail(SSM_ERR_ARG, "tensor sizes overflow");
  // one workgroup per (channel group, batch row, time block) on a 1-D grid, at least one
  // time block; a channel group spans 64 lanes of 1 to 4 channels
  if (B * cdiv(D, 64) > ssm::kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "B*D=%lld channels exceed one launch's grid",
                (long long)(B * D));
  return SSM_OK;
}

size_t conv1d_causal_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t K,
                                         ssm_dtype_t dtype) {
  if (B <= 0 || L <= 0 || D <= 0 || K <= 0) return 0;
  return conv_ws(B, L, D, K, dtype, nullptr, nullptr);
}

int conv1d_causal_bwd(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                      int64_t K, const void* x, const float* W, const float* bias,
                      ssm_act_t act, const void* dout, void* dx, float* dW, float* db,
                      void* ws, size_t ws_bytes) {
  int rc = check_conv_dims(dtype, B, L, D, K, act);
  if (rc) return rc;
  rc = check_ptrs({{x, "x"}, {W, "W"}, {dout, "dout"}, {dx, "dx"}, {dW, "dW"}, {db, "db"}},
                  {{bias, "bias"}});
  if (rc) return rc;
  ssm::ConvPlan p{};
  const size_t need = conv_ws(B, L, D, K, dtype, &p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  conv_ws(B, L, D, K, dtype, &p, ws);
  ssm::ConvArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.L = L; a.D = D; a.K = K;
  a.act = int(act);
  a.x = x; a.W = W; a.bias = act == SSM_ACT_SILU ? bias : nullptr;
  a.dout = dout; a.dx = dx; a.dW = dW; a.db = db;
  return hip_status(ssm::launch_conv1d_bwd(a, p, static_cast<hipStream_t>(stream)),
                    "conv1d_causal_bwd");
}

int conv1d_causal_fwd(void* stream, ssm_dtype_t dtype, int64_t B, int64_t L, int64_t D,
                      int64_t K, const void* x, const float* W, const float* bias,
                      ssm_act_t act, void* out) {
  int rc = check_conv_dims(dtype, B, L, D, K, act);
  if (rc) return rc;
  rc = check_ptrs({{x, "x"}, {W, "W"}, {out, "out"}}, {{bias, "bias"}});
  if (rc) return rc;
  ssm::ConvPlan p{};
  conv_plan(B, L, D, K, &p);
  ssm::ConvFwdArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.L = L; a.D = D; a.K = K;
  a.Tb = p.Tb; a.nTb = p.nTb;
  a.act = int(act);
  a.x = x; a.W = W; a.bias = bias; a.out = out;
  return hip_status(ssm::launch_conv1d_fwd(a, static_cast<hipStream_t>(stream)),
                    "conv1d_causal_fwd");
}

int rmsnorm_fwd(void* stream, ssm_dtype_t dtype, int64_t R, int64_t M, const void* x,
                const void* residual, const float* scale, float eps, void* y, float* rms,
                void* residual_out) {
  if (R <= 0 || M <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (R=%lld M=%lld)", (long long)R, (long long)M);
  if (!(eps >= 0.f) || eps > 3.0e38f)
    return fail(SSM_ERR_ARG, "eps must be finite and >= 0 (got %g)", double(eps));
  if (dtype != SSM_F32 && dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (R > kMaxElems / M) return fail(SSM_ERR_ARG, "tensor sizes overflow");
  ssm::RmsPlan p{};
  rms_plan(R, M, dtype, &p);
  // the looped backward runs one workgroup per (row block, column slab of 8 x 64 x vec
  // columns) on a 1-D grid (at most 512 row blocks)
  if (p.passes == 0 && p.nblk * cdiv(M, 8 * 64 * p.vec) > ssm::kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "row length M=%lld exceeds one launch's grid", (long long)M);
  int rc = check_ptrs({{x, "x"}, {scale, "scale"}, {y, "y"}, {rms, "rms"}},
                      {{residual, "residual"}, {residual_out, "residual_out"}});
  if (rc) return rc;
  if ((residual == nullptr) != (residual_out == nullptr))
    return fail(SSM_ERR_ARG, "residual and residual_out must both be given or both be NULL");
  ssm::RmsFwdArgs a{};
  a.dtype = int(dtype);
  a.R = R; a.M = M;
  // no per-block partials in the forward: small blocks (two rows per wavefront) give
  // every SIMD several wavefronts' rows in flight
  int64_t rpb = 8;
  while (cdiv(R, rpb) > INT32_MAX) rpb *= 2;
  a.vec = p.vec; a.passes = p.passes; a.rows_per_block = rpb; a.nblk = cdiv(R, rpb);
  a.eps = eps;
  a.x = x; a.residual = residual; a.scale = scale; a.y = y; a.rms = rms;
  a.residual_out = residual_out;
  return hip_status(ssm::launch_rmsnorm_fwd(a, static_cast<hipStream_t>(stream)), "rmsnorm_fwd");
}

int ssm_scan_step(void* stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t N, float* h,
                  const void* x_t, const void* delta_t, const float* A, const void* B_t,
                  const void* C_t, const float* Dv, void* y_t) {
  int rc = check_scan_dims(dtype, B, 1, D, N);
  if (rc) return rc;
  rc = check_ptrs({{h, "h"}, {x_t, "x_t"}, {delta_t, "delta_t"}, {A, "A"}, {B_t, "B_t"},
                   {C_t, "C_t"}, {Dv, "Dv"}, {y_t, "y_t"}}, {});
  if (rc) return rc;
  ssm::ScanStepArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.D = D; a.N = N;
  a.h = h; a.x_t = x_t; a.delta_t = delta_t; a.A = A; a.B_t = B_t; a.C_t = C_t; a.Dv = Dv;
  a.y_t = y_t;
  return hip_status(ssm::launch_scan_step(a, static_cast<hipStream_t>(stream)), "ssm_scan_step");
}

int ssm_scan_fused_step(void* stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t N,
                        float* h, const void* x_t, const void* delta_t, const float* A,
                        const void* B_t, const void* C_t, const float* Dv,
                        const float* delta_bias, int delta_softplus, const void* z_t,
                        void* out_t) {
  int rc = check_scan_dims(dtype, B, 1, D, N);
  if (rc) return rc;
  rc = check_ptrs({{h, "h"}, {x_t, "x_t"}, {delta_t, "delta_t"}, {A, "A"}, {B_t, "B_t"},
                   {C_t, "C_t"}, {Dv, "Dv"}, {out_t, "out_t"}},
                  {{delta_bias, "delta_bias"}, {z_t, "z_t"}});
  if (rc) return rc;
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_ARG, "delta_softplus must be 0 or 1 (got %d)", delta_softplus);
  ssm::ScanStepArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.D = D; a.N = N;
  a.h = h; a.x_t = x_t; a.delta_t = delta_t; a.A = A; a.B_t = B_t; a.C_t = C_t; a.Dv = Dv;
  a.y_t = out_t;
  a.fused = true;
  a.dt_bias = delta_bias; a.dt_softplus = delta_softplus != 0; a.z_t = z_t;
  return hip_status(ssm::launch_scan_step(a, static_cast<hipStream_t>(stream)),
                    "ssm_scan_fused_step");
}

int ssm_decode_step(void* stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t N,
                    int64_t K, float* h, void* conv_state, const void* x_t, const float* W,
                    const float* conv_bias, const void* delta_t, const float* A,
                    const void* B_t, const void* C_t, const float* Dv, const float* delta_bias,
                    int delta_softplus, const void* z_t, void* out_t) {
  int rc = check_scan_dims(dtype, B, 1, D, N);
  if (rc) return rc;
  if (K <= 0) return fail(SSM_ERR_ARG, "conv width must be positive (K=%lld)", (long long)K);
  if (K > 8) return fail(SSM_ERR_UNSUPPORTED, "conv width K=%lld not supported (1..8)", (long long)K);
  rc = K > 1 ? check_ptrs({{h, "h"}, {conv_state, "conv_state"}, {x_t, "x_t"}, {W, "W"},
                           {delta_t, "delta_t"}, {A, "A"}, {B_t, "B_t"}, {C_t, "C_t"},
                           {Dv, "Dv"}, {out_t, "out_t"}},
                          {{conv_bias, "conv_bias"}, {delta_bias, "delta_bias"}, {z_t, "z_t"}})
             : check_ptrs({{h, "h"}, {x_t, "x_t"}, {W, "W"}, {delta_t, "delta_t"}, {A, "A"},
                           {B_t, "B_t"}, {C_t, "C_t"}, {Dv, "Dv"}, {out_t, "out_t"}},
                          {{conv_state, "conv_state"}, {conv_bias, "conv_bias"},
                           {delta_bias, "delta_bias"}, {z_t, "z_t"}});
  if (rc) return rc;
  if (delta_softplus != 0 && delta_softplus != 1)
    return fail(SSM_ERR_ARG, "delta_softplus must be 0 or 1 (got %d)", delta_softplus);
  ssm::DecodeArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.D = D; a.N = N; a.K = K;
  a.h = h; a.conv_state = conv_state; a.x_t = x_t; a.W = W; a.conv_bias = conv_bias;
  a.delta_t = delta_t; a.A = A; a.B_t = B_t; a.C_t = C_t; a.Dv = Dv;
  a.dt_bias = delta_bias; a.dt_softplus = delta_softplus != 0; a.z_t = z_t; a.out_t = out_t;
  return hip_status(ssm::launch_decode_step(a, static_cast<hipStream_t>(stream)),
                    "ssm_decode_step");
}

int conv1d_causal_step(void* stream, ssm_dtype_t dtype, int64_t B, int64_t D, int64_t K,
                       void* state, const void* x_t, const float* W, const float* bias,
                       ssm_act_t act, void* out_t) {
  if (B <= 0 || D <= 0 || K <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (B=%lld D=%lld K=%lld)", (long long)B,
                (long long)D, (long long)K);
  if (dtype != SSM_F32 && dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (act != SSM_ACT_NONE && act != SSM_ACT_SILU)
    return fail(SSM_ERR_UNSUPPORTED, "activation %d not supported (0 none, 1 SiLU)", int(act));
  if (K > 8) return fail(SSM_ERR_UNSUPPORTED, "conv width K=%lld not supported (1..8)", (long long)K);
  // element counts well inside int64 (the grid walks batch rows, so B itself is not bounded)
  if (B > kMaxElems / D || B * D > (int64_t(1) << 38))
    return fail(SSM_ERR_ARG, "tensor sizes overflow");
  int rc = K > 1 ? check_ptrs({{state, "state"}, {x_t, "x_t"}, {W, "W"}, {out_t, "out_t"}},
                              {{bias, "bias"}})
                 : check_ptrs({{x_t, "x_t"}, {W, "W"}, {out_t, "out_t"}},
                              {{state, "state"}, {bias, "bias"}});
  if (rc) return rc;
  ssm::ConvStepArgs a{};
  a.dtype = int(dtype);
  a.B = B; a.D = D; a.K = K;
  a.act = int(act);
  a.state = state; a.x_t = x_t; a.W = W; a.bias = bias; a.out_t = out_t;
  return hip_status(ssm::launch_conv1d_step(a, static_cast<hipStream_t>(stream)),
                    "conv1d_causal_step");
}

size_t rmsnorm_bwd_workspace_bytes(int64_t R, int64_t M, ssm_dtype_t dtype) {
  if (R <= 0 || M <= 0) return 0;
  return rms_ws(R, M, dtype, nullptr, nullptr);
}

int rmsnorm_bwd(void* stream, ssm_dtype_t dtype, int64_t R, int64_t M, const void* dy,
                const void* x, const float* scale, const float* rms, void* dx, float* dscale,
                void* ws, size_t ws_bytes) {
  if (R <= 0 || M <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (R=%lld M=%lld)", (long long)R, (long long)M);
  if (dtype != SSM_F32 && dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (R > kMaxElems / M) return fail(SSM_ERR_ARG, "tensor sizes overflow");
  ssm::RmsPlan p{};
  rms_plan(R, M, dtype, &p);
  // the looped backward runs one workgroup per (row block, column slab of 8 x 64 x vec
  // columns) on a 1-D grid (at most 512 row blocks)
  if (p.passes == 0 && p.nblk * cdiv(M, 8 * 64 * p.vec) > ssm::kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "row length M=%lld exceeds one launch's grid", (long long)M);
  int rc = check_ptrs({{dy, "dy"}, {x, "x"}, {scale, "scale"}, {rms, "rms"}, {dx, "dx"},
                       {dscale, "dscale"}}, {});
  if (rc) return rc;
  const size_t need = rms_ws(R, M, dtype, &p, nullptr);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  rms_ws(R, M, dtype, &p, ws);
  ssm::RmsArgs a{};
  a.dtype = int(dtype);
  a.R = R; a.M = M;
  a.dy = dy; a.x = x; a.scale = scale; a.rms = rms; a.dx = dx; a.dscale = dscale;
  return hip_status(ssm::launch_rmsnorm_bwd(a, p, static_cast<hipStream_t>(stream)), "rmsnorm_bwd");
}

static int check_alpha_dims(int64_t Bn, int64_t K, int64_t S, int64_t H) {
  if (Bn <= 0 || K <= 0 || S <= 0 || H <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (Bn=%lld K=%lld S=%lld H=%lld)",
                (long long)Bn, (long long)K, (long long)S, (long long)H);
  if (S > ssm::kAlphaMaxS)
    return fail(SSM_ERR_UNSUPPORTED, "state size S=%lld exceeds %lld", (long long)S,
                (long long)ssm::kAlphaMaxS);
  if (Bn > kMaxElems / K || Bn * K > kMaxElems / S || Bn > kMaxElems / H || H * S > kMaxElems)
    return fail(SSM_ERR_ARG, "tensor sizes overflow");
  const ssm::AlphaPlan p = ssm::alpha_plan(Bn, S, H);
  if (p.nblk > ssm::kMaxGridX || p.ncb * p.nseg > ssm::kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "sizes exceed one launch's grid (Bn=%lld H*S=%lld)",
                (long long)Bn, (long long)(H * S));
  return SSM_OK;
}

size_t ssm_alpha_scan_bwd_workspace_bytes(int64_t Bn, int64_t K, int64_t S, int64_t H) {
  if (Bn <= 0 || K <= 0 || S <= 0 || H <= 0) return 0;
  const ssm::AlphaPlan p = ssm::alpha_plan(Bn, S, H);
  Carver cv(nullptr);
  cv.take(size_t(Bn) * size_t(K) * size_t(S));
  cv.take(size_t(Bn) * size_t(S));
  cv.take(size_t(p.nseg) * size_t(H) * size_t(S));
  cv.take(size_t(ssm::reduce_tmp_floats(p.nseg, H * S)));
  return cv.off;
}

int ssm_alpha_scan_fwd(void* stream, int64_t Bn, int64_t K, int64_t S, int64_t H,
                       const float* a, const float* b, const float* Wc, const float* h0,
                       float* h) {
  int rc = check_alpha_dims(Bn, K, S, H);
  if (rc) return rc;
  rc = check_ptrs({{a, "a"}, {b, "b"}, {Wc, "Wc"}, {h, "h"}}, {{h0, "h0"}});
  if (rc) return rc;
  ssm::AlphaArgs x{};
  x.Bn = Bn; x.K = K; x.S = S; x.H = H;
  x.a = a; x.b = b; x.Wc = Wc; x.h0 = h0; x.h = h;
  return hip_status(ssm::launch_alpha_fwd(x, static_cast<hipStream_t>(stream)),
                    "ssm_alpha_scan_fwd");
}

int ssm_alpha_scan_bwd(void* stream, int64_t Bn, int64_t K, int64_t S, int64_t H,
                       const float* a, const float* b, const float* Wc, const float* dh,
                       float* da, float* db, float* dWc, float* dh0, void* ws, size_t ws_bytes) {
  int rc = check_alpha_dims(Bn, K, S, H);
  if (rc) return rc;
  rc = check_ptrs({{a, "a"}, {b, "b"}, {Wc, "Wc"}, {dh, "dh"}, {da, "da"}, {db, "db"},
                   {dWc, "dWc"}},
                  {{dh0, "dh0"}});
  if (rc) return rc;
  const size_t need = ssm_alpha_scan_bwd_workspace_bytes(Bn, K, S, H);
  if ((rc = check_ws(ws, ws_bytes, need))) return rc;
  Carver cv(ws);
  const ssm::AlphaPlan p = ssm::alpha_plan(Bn, S, H);
  float* xh = cv.take(size_t(Bn) * size_t(K) * size_t(S));
  float* xl = cv.take(size_t(Bn) * size_t(S));
  float* part = cv.take(size_t(p.nseg) * size_t(H) * size_t(S));
  float* tmp = cv.take(size_t(ssm::reduce_tmp_floats(p.nseg, H * S)));
  ssm::AlphaArgs x{};
  x.Bn = Bn; x.K = K; x.S = S; x.H = H;
  x.a = a; x.b = b; x.Wc = Wc; x.dh = dh; x.da = da; x.db = db; x.dWc = dWc; x.dh0 = dh0;
  return hip_status(ssm::launch_alpha_bwd(x, xh, xl, part, tmp, static_cast<hipStream_t>(stream)),
                    "ssm_alpha_scan_bwd");
}

int rmsnorm_bwd_noalloc(void* stream, ssm_dtype_t dtype, int64_t R, int64_t M, const void* dy,
                        const void* x, const float* scale, const float* rms, void* dx,
                        float* dscale) {
  if (R <= 0 || M <= 0)
    return fail(SSM_ERR_ARG, "sizes must be positive (R=%lld M=%lld)", (long long)R, (long long)M);
  if (dtype != SSM_F32 && dtype != SSM_BF16)
    return fail(SSM_ERR_UNSUPPORTED, "dtype %d not supported", int(dtype));
  if (R > kMaxElems / M) return fail(SSM_ERR_ARG, "tensor sizes overflow");
  ssm::RmsPlan p{};
  rms_plan(R, M, dtype, &p);
  if (p.passes == 0 && p.nblk * cdiv(M, 8 * 64 * p.vec) > ssm::kMaxGridX)
    return fail(SSM_ERR_UNSUPPORTED, "row length M=%lld exceeds one launch's grid", (long long)M);
  int rc = check_ptrs({{dy, "dy"}, {x, "x"}, {scale, "scale"}, {rms, "rms"}, {dx, "dx"},
                       {dscale, "dscale"}}, {});
  if (rc) return rc;
  // the same plan as rmsnorm_bwd, carved out of the static scratch instead of a workspace
  const size_t need = rms_ws(R, M, dtype, &p, nullptr);
  if (need > ssm::kNoAllocScratchBytes)
    return fail(SSM_ERR_UNSUPPORTED,
                "rmsnorm_bwd_noalloc: R=%lld M=%lld needs %zu bytes of scratch, above the static "
                "buffer's %zu (use rmsnorm_bwd with a workspace)",
                (long long)R, (long long)M, need, ssm::kNoAllocScratchBytes);
  void* ws = nullptr;
  hipError_t e = ssm::noalloc_scratch(&ws);
  if (e != hipSuccess) return hip_status(e, "rmsnorm_bwd_noalloc (scratch address)");
  rms_ws(R, M, dtype, &p, ws);
  ssm::RmsArgs a{};
  a.dtype = int(dtype);
  a.R = R; a.M = M;
  a.dy = dy; a.x = x; a.scale = scale; a.rms = rms; a.dx = dx; a.dscale = dscale;
  return hip_status(ssm::launch_rmsnorm_bwd(a, p, static_cast<hipStream_t>(stream)),
                    "rmsnorm_bwd_noalloc");
}

}  // extern "C"
