// Staging of scan inputs and outputs through LDS, one tile at a time, with buffer
// (descriptor-based) memory instructions.
//
// A tile is kTc consecutive steps of one batch row for the workgroup's 64 channels.
// Every element of a per-channel tensor ([B,L,D]: x, delta, dy; outputs y, dx, ddelta)
// and of a per-step vector ([B,L,N]: B, C) moves once, coalesced: a thread owns VEC
// consecutive channels of one step (VEC = 4 when D is a multiple of 4, else 1), so a
// wavefront covers whole rows of 64 channels.  Loads are issued into registers while
// the previous tile is being computed and written to one of two LDS buffers only after
// that compute ("commit"), so their latency overlaps the compute.
//
// Bounds are handled by the buffer hardware: a descriptor spans only the valid part of
// the tile (loads beyond it return 0, stores beyond it are dropped), and a thread whose
// channels lie past D carries an offset beyond every descriptor.  A zero step is an
// exact identity of the recurrence (a = exp(0) = 1, no input, no output), so the
// compute loops carry no tail branches.  The per-thread offset does not depend on the
// tile; only the descriptors (scalar registers) are rebuilt per tile.
#pragma once
#include "common.hpp"

namespace ssm {

constexpr int kTileThreads = 256;
constexpr int kTileCh = 64;  // channels per workgroup

// Descriptor over [base, base + bytes): gfx9-family raw buffer (stride 0), with the
// default data format word of that family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
constexpr uint32_t kOffNone = 0x80000000u;  // beyond every descriptor built here

// VEC elements of T moved by one buffer instruction (at vector offset off plus scalar
// offset soff).
template <typename T, int VEC>
struct BufVec;
template <>
struct BufVec<float, 4> {
  using raw_t = __attribute__((ext_vector_type(4))) unsigned;
  __device__ static raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  }
  __device__ static void store(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, soff, 0);
  }
  __device__ static void unpack(raw_t v, float (&o)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
  }
  __device__ static raw_t pack(const float (&f)[4]) {
    raw_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(f[i]);
    return v;
  }
};
template <>
struct BufVec<bf16_t, 4> {
  using raw_t = __attribute__((ext_vector_type(2))) unsigned;
  __device__ static raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
  }
  __device__ static void store(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, soff, 0);
  }
  __device__ static void unpack(raw_t v, float (&o)[4]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      o[2 * i] = __uint_as_float(v[i] << 16);
      o[2 * i + 1] = __uint_as_float(v[i] & 0xFFFF0000u);
    }
  }
  __device__ static raw_t pack(const float (&f)[4]) {
    raw_t v;
#pragma unroll
    for (int i = 0; i < 2; ++i) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
  }
};
template <>
struct BufVec<float, 1> {
  using raw_t = unsigned;
  __device__ static raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
  }
  __device__ static void store(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, soff, 0);
  }
  __device__ static void unpack(raw_t v, float (&o)[1]) { o[0] = __uint_as_float(v); }
  __device__ static raw_t pack(const float (&f)[1]) { return __float_as_uint(f[0]); }
};
template <>
struct BufVec<bf16_t, 1> {
  using raw_t = unsigned short;
  __device__ static raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, soff, 0);
  }
  __device__ static void store(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b16(v, r, off, soff, 0);
  }
  __device__ static void unpack(raw_t v, float (&o)[1]) {
    o[0] = __uint_as_float(uint32_t(v) << 16);
  }
  __device__ static raw_t pack(const float (&f)[1]) { return from_f32<bf16_t>(f[0]); }
};

template <>
struct BufVec<float, 2> {
  using raw_t = __attribute__((ext_vector_type(2))) unsigned;
  __device__ static raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, off, soff, 0);
  }
  __device__ static void store(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b64(v, r, off, soff, 0);
  }
  __device__ static void unpack(raw_t v, float (&o)[2]) {
    o[0] = __uint_as_float(v[0]);
    o[1] = __uint_as_float(v[1]);
  }
  __device__ static raw_t pack(const float (&f)[2]) {
    raw_t v;
    v[0] = __float_as_uint(f[0]);
    v[1] = __float_as_uint(f[1]);
    return v;
  }
};
template <>
struct BufVec<bf16_t, 2> {
  using raw_t = unsigned;
  __device__ static raw_t load(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, soff, 0);
  }
  __device__ static void store(raw_t v, __amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
    __builtin_amdgcn_raw_buffer_store_b32(v, r, off, soff, 0);
  }
  __device__ static void unpack(raw_t v, float (&o)[2]) {
    o[0] = __uint_as_float(v << 16);
    o[1] = __uint_as_float(v & 0xFFFF0000u);
  }
  __device__ static raw_t pack(const float (&f)[2]) { return pack_bf16x2(f[0], f[1]); }
};

// Placement of a thread in a per-channel tile: TPR threads per step row, RPP rows per
// pass of the 256 threads, kPer passes per tile.  Pass k covers rows s_in + k*RPP.
template <typename T, int VEC>
struct ChTile {
  static constexpr int TPR = kTileCh / VEC;
  static constexpr int RPP = kTileThreads / TPR;
  static constexpr int kPer = kTc / RPP;
  int s_in, c;   // row (in pass 0) and first channel of this thread
  uint32_t off;  // byte offset of (s_in, c) from the tile start, or kOffNone
  __device__ __forceinline__ ChTile(int D32, int dvalid, int tid) {
    s_in = tid / TPR;
    c = (tid % TPR) * VEC;
    off = c < dvalid ? uint32_t(s_in * D32 + c) * uint32_t(sizeof(T)) : kOffNone;
  }
  // Descriptor of pass k of the tile at `tile` (= base + tf*D + d0) with tvalid valid
  // rows and dvalid valid channels: rows k*RPP .. tvalid-1, the last one up to dvalid.
  __device__ __forceinline__ static __amdgpu_buffer_rsrc_t rsrc(const T* tile, int D32,
                                                                int tvalid, int dvalid, int k) {
    const int tv = tvalid - k * RPP;
    const uint32_t bytes = tv > 0 ? uint32_t((tv - 1) * D32 + dvalid) * uint32_t(sizeof(T)) : 0u;
    return buf_rsrc(tile + int64_t(k) * RPP * D32, bytes);
  }
};

// One per-channel input tensor's share of a tile.
template <typename T, int VEC>
struct ChFetch {
  using G = ChTile<T, VEC>;
  using BV = BufVec<T, VEC>;
  typename BV::raw_t raw[G::kPer];
  __device__ __forceinline__ void fetch(const G& g, const T* tile, int D32, int tvalid,
                                        int dvalid) {
#pragma unroll
    for (int k = 0; k < G::kPer; ++k)
      raw[k] = BV::load(G::rsrc(tile, D32, tvalid, dvalid, k), g.off);
  }
  __device__ __forceinline__ void commit(const G& g, float (*sm)[kTileCh]) const {
    commit_map(g, sm, [](int, float (&)[VEC]) {});
  }
  // As commit, with f(k, v) applied to pass k's values (rows g.s_in + k*RPP) first.
  template <class F>
  __device__ __forceinline__ void commit_map(const G& g, float (*sm)[kTileCh], F&& f) const {
#pragma unroll
    for (int k = 0; k < G::kPer; ++k) {
      float v[VEC];
      BV::unpack(raw[k], v);
      f(k, v);
      float* dst = &sm[g.s_in + k * G::RPP][g.c];
      if constexpr (VEC == 4) {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        dst[0] = v[0];
      }
    }
  }
};

// Per-channel total of values the threads have accumulated in ChTile placement: each
// thread holds running sums `part` of its VEC channels over its rows (s_in + k*RPP, every
// tile), and the RPP threads that share a channel column are added in row order through
// `scratch` (kTileThreads*VEC floats of LDS, free on entry).  Thread tid < kTileCh gets
// the total of channel tid.  Contains a barrier: every thread of the block must call it.
template <typename T, int VEC>
__device__ __forceinline__ float chan_rows_sum(const ChTile<T, VEC>& g, const float (&part)[VEC],
                                               float* scratch, int tid) {
  using G = ChTile<T, VEC>;
#pragma unroll
  for (int i = 0; i < VEC; ++i) scratch[tid * VEC + i] = part[i];
  __syncthreads();
  float t = 0.f;
  if (tid < kTileCh) {
    const int tc = tid / VEC, ci = tid % VEC;  // thread column and channel within it
    for (int r = 0; r < G::RPP; ++r) t += scratch[(r * G::TPR + tc) * VEC + ci];
  }
  return t;
}

// Writes an LDS tile of per-channel outputs to a [.,L,D] tensor; tile = base + tf*D + d0;
// rows >= tvalid and channels >= dvalid are not written.
// tile_store_ch_map applies f(k, v) to pass k's values (rows g.s_in + k*RPP) before the
// store.
template <typename T, int VEC, class F>
__device__ __forceinline__ void tile_store_ch_map(const ChTile<T, VEC>& g, T* tile,
                                                  const float (*sm)[kTileCh], int D32,
                                                  int tvalid, int dvalid, F&& f) {
  using G = ChTile<T, VEC>;
  using BV = BufVec<T, VEC>;
#pragma unroll
  for (int k = 0; k < G::kPer; ++k) {
    const float* src = &sm[g.s_in + k * G::RPP][g.c];
    float v[VEC];
    if constexpr (VEC == 4) {
      const float4 q = *reinterpret_cast<const float4*>(src);
      v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    } else {
      v[0] = src[0];
    }
    f(k, v);
    BV::store(BV::pack(v), G::rsrc(tile, D32, tvalid, dvalid, k), g.off);
  }
}
template <typename T, int VEC>
__device__ __forceinline__ void tile_store_ch(const ChTile<T, VEC>& g, T* tile,
                                              const float (*sm)[kTileCh], int D32, int tvalid,
                                              int dvalid) {
  tile_store_ch_map(g, tile, sm, D32, tvalid, dvalid, [](int, float (&)[VEC]) {});
}

// Pass k of a per-channel output tile straight from registers (the ChTile placement).
template <typename T, int VEC>
__device__ __forceinline__ void tile_store_regs(const ChTile<T, VEC>& g, T* tile, int k,
                                                const float (&v)[VEC], int D32, int tvalid,
                                                int dvalid) {
  using BV = BufVec<T, VEC>;
  BV::store(BV::pack(v), ChTile<T, VEC>::rsrc(tile, D32, tvalid, dvalid, k), g.off);
}

// The fused scan's time step from its raw input, in place: raw + bias[c] through a
// softplus when sp (the Mamba time step), zero where !ok (rows past the sequence and
// channels past D: the identity step).  sg, when given, receives the derivative of that
// map at the point, sigmoid(raw + bias) or 1.
template <int VEC>
__device__ __forceinline__ void time_step_map(float (&v)[VEC], const float* bias, bool ok,
                                              bool sp, float* sg) {
#pragma unroll
  for (int i = 0; i < VEC; ++i) {
    const float p = v[i] + bias[i];
    float s = p, d = 1.f;
    if (sp) s = sg ? softplus_sigmoid(p, d) : softplus_f(p);
    if (sg) sg[i] = d;
    v[i] = ok ? s : 0.f;
  }
}

// One per-step vector's share of a tile ([kTc][N] contiguous): thread tid < kTc*N owns
// element tid (step tid/N, state tid%N).
template <typename T, int N>
struct VecFetch {
  using BV = BufVec<T, 1>;
  typename BV::raw_t raw;
  __device__ __forceinline__ static uint32_t offset(int tid) {
    return tid < kTc * N ? uint32_t(tid) * uint32_t(sizeof(T)) : kOffNone;
  }
  // tile = base + tf*N
  __device__ __forceinline__ void fetch(const T* tile, int tvalid, uint32_t off) {
    raw = BV::load(buf_rsrc(tile, uint32_t(tvalid * N) * uint32_t(sizeof(T))), off);
  }
  __device__ __forceinline__ void commit(float (*sm)[N], int tid) const {
    float v[1];
    BV::unpack(raw, v);
    if (tid < kTc * N) sm[tid / N][tid % N] = v[0];
  }
  // Row layout of the permuted state order (N = 16): 2N floats, the step's vector (copy
  // 0: state n at n) and the same vector with adjacent states swapped (copy 1: state n at
  // N + (n ^ 1)); rows of consecutive steps start `stride` floats apart.
  __device__ __forceinline__ void commit_perm(float* tile, int stride, int tid) const {
    static_assert(N == 16, "the permuted state order is defined for four states per lane");
    float v[1];
    BV::unpack(raw, v);
    if (tid < kTc * N) {
      const int s = tid / N, n = tid % N;
      float* r = tile + s * stride;
      r[n] = v[0];
      r[N + (n ^ 1)] = v[0];
    }
  }
};

// The NS state values of state group q (states q*NS .. q*NS+NS-1) at step s of an LDS
// vector tile.
template <int N, int NS>
__device__ __forceinline__ void tile_read_vec(const float (*sm)[N], int s, int q, float (&o)[NS]) {
  if constexpr (NS == 4) {
    const float4 v = *reinterpret_cast<const float4*>(&sm[s][q * 4]);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else if constexpr (NS == 2) {
    const float2 v = *reinterpret_cast<const float2*>(&sm[s][q * 2]);
    o[0] = v.x; o[1] = v.y;
  } else {
    o[0] = sm[s][q];
  }
}

// A lane's four values of one step row of the permuted layout (VecFetch::commit_perm),
// in the order of perm_quarter / perm_xor: register r gets state 4*Q + (r ^ m).  `a0` is
// the lane's byte offset ((m & 1)*16 + 4*Q + 2*(m >> 1))*4: registers 0, 1 come from there
// (copy m & 1 swaps the pair when m is odd) and 2, 3 from the quarter's other pair
// (a0 ^ 8).  Each 8-byte read stays inside the row's 32 floats, one per LDS bank.
__device__ __forceinline__ void tile_read_perm(const float* row, uint32_t a0, float (&o)[4]) {
  const char* r = reinterpret_cast<const char*>(row);
  const float2 lo = *reinterpret_cast<const float2*>(r + a0);
  const float2 hi = *reinterpret_cast<const float2*>(r + (a0 ^ 8u));
  o[0] = lo.x; o[1] = lo.y; o[2] = hi.x; o[3] = hi.y;
}
// The same for two rows 128 bytes apart (B's and C's rows of one step): the matching
// reads of the two rows pair into one two-address LDS instruction each.
__device__ __forceinline__ void tile_read_perm2(const float* row, uint32_t a0, float (&b)[4],
                                                float (&c)[4]) {
  const char* r = reinterpret_cast<const char*>(row);
  const float2 b01 = *reinterpret_cast<const float2*>(r + a0);
  const float2 c01 = *reinterpret_cast<const float2*>(r + a0 + 128);
  const float2 b23 = *reinterpret_cast<const float2*>(r + (a0 ^ 8u));
  const float2 c23 = *reinterpret_cast<const float2*>(r + (a0 ^ 8u) + 128);
  b[0] = b01.x; b[1] = b01.y; b[2] = b23.x; b[3] = b23.y;
  c[0] = c01.x; c[1] = c01.y; c[2] = c23.x; c[3] = c23.y;
}

// NS consecutive f32 state values of one lane through a descriptor (loads past it
// return 0, stores past it are dropped).
template <int NS>
__device__ __forceinline__ void buf_load_states(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                float (&o)[NS]) {
  if constexpr (NS == 4) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __uint_as_float(v[j]);
  } else if constexpr (NS == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    o[0] = __uint_as_float(v[0]);
    o[1] = __uint_as_float(v[1]);
  } else {
    o[0] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
  }
}
// Four f32 state values of one lane in the permuted order: register r gets the value at
// byte offset off + 4*(r ^ m) (off = the lane's 16-byte state quarter, or kOffNone).
__device__ __forceinline__ void buf_load_states_perm(__amdgpu_buffer_rsrc_t r, uint32_t off,
                                                     int m, float (&o)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j)
    o[j] = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(r, off + uint32_t((j ^ m) * 4), 0, 0));
}
template <int NS>
__device__ __forceinline__ void buf_store_states(const float (&v)[NS], __amdgpu_buffer_rsrc_t r,
                                                 uint32_t off) {
  if constexpr (NS == 4) {
    __attribute__((ext_vector_type(4))) unsigned u;
#pragma unroll
    for (int j = 0; j < 4; ++j) u[j] = __float_as_uint(v[j]);
    __builtin_amdgcn_raw_buffer_store_b128(u, r, off, 0, 0);
  } else if constexpr (NS == 2) {
    __attribute__((ext_vector_type(2))) unsigned u;
    u[0] = __float_as_uint(v[0]);
    u[1] = __float_as_uint(v[1]);
    __builtin_amdgcn_raw_buffer_store_b64(u, r, off, 0, 0);
  } else {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v[0]), r, off, 0, 0);
  }
}

__device__ __forceinline__ int clamp_valid(int64_t v) {
  return v < 0 ? 0 : (v > kTc ? kTc : int(v));
}

}  // namespace ssm
