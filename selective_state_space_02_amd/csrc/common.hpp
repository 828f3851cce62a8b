// Device helpers shared by the gfx950 kernels: storage-type loads and stores, DPP
// quad sums and the butterfly reduction across the channels of a wavefront.
//
// Lane layout used by every scan kernel ("quad = channel"): a wavefront holds 16
// channels; lane l works on channel l/4 and on the NS = N/4 consecutive states
// starting at n = (l%4)*NS.  Sums over the state index are quad sums (two DPP adds);
// sums over channels are butterflies over lane bits 2..5.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

typedef uint16_t bf16_t;  // raw bf16 bits

// ---------------------------------------------------------------------------------
// storage-type conversion
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) {
  // round to nearest even (v_cvt_pk_bf16_f32 on gfx950)
  return __builtin_bit_cast(bf16_t, (__bf16)v);
}

// sigmoid(p) = 1 / (1 + exp(-p)) from the hardware exp2 and reciprocal (about one ulp
// each); saturates to 0 and 1 in the tails.
__device__ __forceinline__ float sigmoid_f(float p) {
  return __builtin_amdgcn_rcpf(1.f + __builtin_amdgcn_exp2f(-p * kLog2e));
}
// Activation after the conv: 0 none, 1 SiLU (p * sigmoid(p)).
constexpr int kActNone = 0, kActSilu = 1;

// log1p(t) for t in [0, 1] from one logarithm: with u = fl(1 + t), the rounding error
// c = t - (u - 1) is exact (both differences are exact for u in [1, 2]) and at most 2^-24;
// log1p(t) = log(u) + log(1 + c/u), and log(1 + c/u) = c to within 2^-24 t.  log(u)
// alone would lose the low bits of t that the rounding of u drops.
__device__ __forceinline__ float log1p_unit(float t) {
  const float u = 1.f + t;
  return __builtin_fmaf(__builtin_amdgcn_logf(u), kLn2, t - (u - 1.f));
}
// softplus(v) = log(1 + exp(v)) = max(v, 0) + log1p(exp(-|v|)).
__device__ __forceinline__ float softplus_f(float v) {
  return __builtin_fmaxf(v, 0.f) + log1p_unit(__builtin_amdgcn_exp2f(-__builtin_fabsf(v) * kLog2e));
}
// softplus(v) and its derivative sigmoid(v) from one exponential: with t = exp(-|v|),
// sigmoid(v) = 1 / (1 + t) for v >= 0 and t / (1 + t) below.
__device__ __forceinline__ float softplus_sigmoid(float v, float& sg) {
  const float t = __builtin_amdgcn_exp2f(-__builtin_fabsf(v) * kLog2e);
  const float r = __builtin_amdgcn_rcpf(1.f + t);
  sg = v >= 0.f ? r : t * r;
  return __builtin_fmaxf(v, 0.f) + log1p_unit(t);
}

// Two floats as packed bf16 (lo in bits 0-15), rounded to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 r = __builtin_convertvector(f2{lo, hi}, b2);
  return __builtin_bit_cast(uint32_t, r);
}

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float v) { p[i] = from_f32<T>(v); }

// NS consecutive values starting at p (p aligned to NS*sizeof(T)).
template <typename T, int NS> struct VecLoad;

template <> struct VecLoad<float, 4> {
  static __device__ __forceinline__ void run(const float* p, float (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(p);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct VecLoad<float, 2> {
  static __device__ __forceinline__ void run(const float* p, float (&o)[2]) {
    const float2 v = *reinterpret_cast<const float2*>(p);
    o[0] = v.x; o[1] = v.y;
  }
};
template <> struct VecLoad<float, 1> {
  static __device__ __forceinline__ void run(const float* p, float (&o)[1]) { o[0] = p[0]; }
};
template <> struct VecLoad<bf16_t, 4> {
  static __device__ __forceinline__ void run(const bf16_t* p, float (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(v.x << 16); o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16); o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};
template <> struct VecLoad<bf16_t, 2> {
  static __device__ __forceinline__ void run(const bf16_t* p, float (&o)[2]) {
    const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
    o[0] = __uint_as_float(v << 16); o[1] = __uint_as_float(v & 0xffff0000u);
  }
};
template <> struct VecLoad<bf16_t, 1> {
  static __device__ __forceinline__ void run(const bf16_t* p, float (&o)[1]) { o[0] = to_f32(p[0]); }
};

template <> struct VecLoad<bf16_t, 8> {
  static __device__ __forceinline__ void run(const bf16_t* p, float (&o)[8]) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = __uint_as_float(w[k] << 16);
      o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};

// VEC consecutive values stored at p (p aligned to VEC*sizeof(T)).
template <typename T, int VEC> struct VecStore;
template <> struct VecStore<float, 4> {
  static __device__ __forceinline__ void run(float* p, const float (&v)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};
template <> struct VecStore<float, 2> {
  static __device__ __forceinline__ void run(float* p, const float (&v)[2]) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  }
};
template <> struct VecStore<float, 1> {
  static __device__ __forceinline__ void run(float* p, const float (&v)[1]) { p[0] = v[0]; }
};
template <> struct VecStore<bf16_t, 8> {
  static __device__ __forceinline__ void run(bf16_t* p, const float (&v)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = uint32_t(from_f32<bf16_t>(v[2 * k])) | (uint32_t(from_f32<bf16_t>(v[2 * k + 1])) << 16);
    *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
  }
};
template <> struct VecStore<bf16_t, 4> {
  static __device__ __forceinline__ void run(bf16_t* p, const float (&v)[4]) {
    uint2 o;
    o.x = uint32_t(from_f32<bf16_t>(v[0])) | (uint32_t(from_f32<bf16_t>(v[1])) << 16);
    o.y = uint32_t(from_f32<bf16_t>(v[2])) | (uint32_t(from_f32<bf16_t>(v[3])) << 16);
    *reinterpret_cast<uint2*>(p) = o;
  }
};
template <> struct VecStore<bf16_t, 1> {
  static __device__ __forceinline__ void run(bf16_t* p, const float (&v)[1]) {
    p[0] = from_f32<bf16_t>(v[0]);
  }
};

template <typename T, int NS>
__device__ __forceinline__ void load_vec(const T* p, float (&o)[NS]) { VecLoad<T, NS>::run(p, o); }

template <int NS>
__device__ __forceinline__ void zero(float (&o)[NS]) {
#pragma unroll
  for (int j = 0; j < NS; ++j) o[j] = 0.f;
}

// ---------------------------------------------------------------------------------
// cross-lane sums
// ---------------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over the 4 lanes of a quad; every lane of the quad gets the total.
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(v);  // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);  // quad_perm [2,3,0,1]
  return v;
}

__device__ __forceinline__ float xor_lane(float v, int mask) {
  return __shfl_xor(v, mask, 64);
}

// DPP move within rows of 16 lanes, writing only the banks (groups of 4 lanes) set in
// BANK; other lanes return `old`.  row_ror:n (CTRL 0x120 + n) reads lane (i - n) mod 16.
// Ordering fence for unrolled step loops: each value is treated as redefined here and
// no memory access moves across.  Work of later steps that depends on these values
// (or on loads issued after the fence) cannot be hoisted above it, so the compiler
// does not interleave whole steps (which would keep the operands of many steps live
// at once); independent work inside a step is still scheduled freely.
__device__ __forceinline__ void step_fence() { asm volatile("" ::: "memory"); }
template <typename T0, typename... Ts>
__device__ __forceinline__ void step_fence(T0& v, Ts&... rest) {
  asm volatile("" : "+v"(v));
  step_fence(rest...);
}
// A copy of v the compiler cannot see through: values derived from it are computed
// where they are used rather than hoisted out of a loop and held in registers.
template <typename T>
__device__ __forceinline__ T opaque(T v) {
  asm volatile("" : "+v"(v));
  return v;
}
// An explicit register move into a register other than src's.  Where a loop hands a
// loop-carried value over (the next tile's checkpoint becoming the current one) right
// before src's register is reloaded, this keeps the reload landing in src's own
// register: a plain assignment may leave the loads in temporaries that are copied back
// at the loop edge, and that copy waits for every load in flight.
__device__ __forceinline__ void reg_move(float& dst, float src) {
  asm volatile("v_mov_b32 %0, %1" : "=&v"(dst) : "v"(src));
}
template <int K>
__device__ __forceinline__ void step_fence_arr(float (&v)[K]) {
#pragma unroll
  for (int k = 0; k < K; ++k) asm volatile("" : "+v"(v[k]));
}

// gfx950 lane swap between rows 0/1 and 2/3 of a wavefront (lane distance 16): after
// swap16(a, b), lanes with bit 4 clear hold (a, a of lane+16) and the others
// (b of lane-16, b).
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Reduce-scatter of V (2, 4 or 8) values per lane over the 16 lanes that share
// (lane & 3), i.e. over the 16 channels of a wavefront: the halving steps of a
// butterfly over lane bits 3, 2 (V >= 4) and 4 (V == 8), cheapest first.  At each step
// a lane keeps half of its values (the lower half if its bit is 0) and adds the
// partner's copy of that half.  Bits 3 and 2 lie inside a row of 16 lanes, where two
// masked DPP adds per pair do it (dpp_halve); bit 4 takes a lane swap, which moves a
// whole pair at once.  On return v[0] of a lane holds the
// value index whose bits, most significant first, are the lane's bits 3, 2, 4 (as many
// as log2 V), summed over the channels that agree with the lane in the remaining
// channel bits: the 16/V partial sums of (k, q) sit in lanes chan_partial_lane<V>(k, p,
// q), p < 16/V, and are added by the caller.
// One halving step of the reduce-scatter inside a row of 16 lanes, for the value pair
// (a, b): lanes whose bit (3 or 2) is clear get a + a of the partner, the others
// b + b of the partner.  DPP's bank mask (bank = lanes 4i .. 4i+3 of a row) writes each
// half of the lanes with its own add, so no select is needed; the partner is read in the
// add (row_ror:8 is lane^8; for bit 2, row_shl:4 reads lane+4 in banks 0 and 2 and
// row_shr:4 lane-4 in banks 1 and 3).  The compiler emits DPP only with full masks,
// hence the asm; s_nop 1 covers the wait states a DPP read needs after a VALU write.
template <int BIT>
__device__ __forceinline__ float dpp_halve(float a, float b) {
  float r;
  if constexpr (BIT == 3)
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
        "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xc"
        : "=&v"(r) : "v"(a), "v"(b));
  else
    asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_shl:4 row_mask:0xf bank_mask:0x5\n\t"
        "v_add_f32_dpp %0, %2, %2 row_shr:4 row_mask:0xf bank_mask:0xa"
        : "=&v"(r) : "v"(a), "v"(b));
  return r;
}

template <int V>
__device__ __forceinline__ void chan_reduce_scatter(float (&v)[V], int) {
  static_assert(V == 2 || V == 4 || V == 8, "V must be 2, 4 or 8");
#pragma unroll
  for (int k = 0; k < V / 2; ++k) v[k] = dpp_halve<3>(v[k], v[k + V / 2]);  // bit 3
  if constexpr (V >= 4) {
#pragma unroll
    for (int k = 0; k < V / 4; ++k) v[k] = dpp_halve<2>(v[k], v[k + V / 4]);  // bit 2
  }
  if constexpr (V >= 8) {  // bit 4 (distance 16)
    float a = v[0], b = v[1];
    swap16(a, b);
    v[0] = a + b;
  }
}

// Permuted state order for four states per lane (N = 16), which lets every in-row
// halving of the channel reduce-scatter below take one full-mask DPP add per pair.
// Within a row of 16 lanes DPP pairs lanes by XOR only for the masks 8 (row_ror:8) and
// 7 (row_half_mirror); a halving step with one add per pair also needs the partner to
// hold, in the registers the lane keeps, the states the partner sends.  So lane l
// (quad lane q = l & 3, lane bits b2, b3) holds the state quarter Q = q ^ (3*b2), and in
// register r the state 4*Q + (r ^ m) with m = 2*b3 + b2: the partner across bit 3 (l ^ 8)
// has the same Q and m ^ 2, the partner across bits 0..2 (l ^ 7) the same Q and m ^ 1.
// A channel's four lanes still hold all 16 states (q -> q ^ 3*b2 is a permutation).
__host__ __device__ __forceinline__ constexpr int perm_quarter(int lane) {
  return (lane & 3) ^ (3 * ((lane >> 2) & 1));
}
__host__ __device__ __forceinline__ constexpr int perm_xor(int lane) {
  return ((lane >> 2) & 1) | (((lane >> 3) & 1) << 1);
}

// Reduce-scatter over the 16 channels of a wavefront of the 8 values (index 2r + t:
// register r's state, t = 0 for dB and 1 for dC) of the permuted order: halving across
// lane bit 3 (row_ror:8, keeps r < 2), across lane bits 0..2 (row_half_mirror, keeps
// r = 0), then across bit 4 (lane swap: bit 4 clear keeps t = 0).  On return v[0] of lane
// l holds value t = bit 4 of l for state 4*perm_quarter(l) + perm_xor(l), summed over the
// channels that agree with l's in channel bit 3 (lane bit 5): two partials per output, at
// perm_partial_lane(t, n, 0 and 1).
__device__ __forceinline__ void chan_reduce_scatter_perm(float (&v)[8]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) v[k] += dpp<0x128>(v[k + 4]);  // row_ror:8 = lane ^ 8
#pragma unroll
  for (int k = 0; k < 2; ++k) v[k] += dpp<0x141>(v[k + 2]);  // row_half_mirror = lane ^ 7
  float a = v[0], b = v[1];
  swap16(a, b);
  v[0] = a + b;
}

// Lane holding partial p (0 or 1) of output (t, n) after chan_reduce_scatter_perm.
__host__ __device__ __forceinline__ constexpr int perm_partial_lane(int t, int n, int p) {
  const int m = n & 3, b2 = m & 1, b3 = m >> 1, q = (n >> 2) ^ (3 * b2);
  return q | (b2 << 2) | (b3 << 3) | (t << 4) | (p << 5);
}

// Lane that holds partial p (p < 16/V) of value index k for state quarter q after
// chan_reduce_scatter<V>: k's bits (most significant first) at lane bits 3, 2, 4, p's
// bits (least significant first) at the channel bits left over.
template <int V>
__host__ __device__ __forceinline__ constexpr int chan_partial_lane(int k, int p, int q) {
  constexpr int S = V == 8 ? 3 : (V == 4 ? 2 : 1);
  constexpr int sb[3] = {3, 2, 4};
  int l = q;
  for (int s = 0; s < S; ++s) l |= ((k >> (S - 1 - s)) & 1) << sb[s];
  int j = 0;
  for (int bit = 2; bit <= 5; ++bit) {
    bool used = false;
    for (int s = 0; s < S; ++s) used = used || sb[s] == bit;
    if (!used) {
      l |= ((p >> j) & 1) << bit;
      ++j;
    }
  }
  return l;
}

}  // namespace ssm
