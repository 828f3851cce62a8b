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
template <int CTRL, int BANK>
__device__ __forceinline__ float dpp_masked(float old, float src) {
  return __int_as_float(
      __builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(src), CTRL, 0xF, BANK, false));
}

// gfx950 lane swaps: after swap32(a, b), lanes 0-31 hold (a, a of lane+32) and lanes
// 32-63 hold (b of lane-32, b); swap16 does the same between rows 0/1 and 2/3.
__device__ __forceinline__ void swap32(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Sum V (2, 4 or 8) values per lane over the 16 lanes that share (lane & 3), i.e. over
// the 16 channels of a wavefront.  Butterfly reduce-scatter over lane bits 5, 4, 3: at
// each halving step a lane keeps half of its values (the lower half if its bit is 0)
// and adds the partner's copy of that half -- a lane swap does the exchange for bits
// 5 and 4, bank-masked DPP rotations for bit 3.  Lane bits left over once one value
// remains are summed pairwise.  On return lane l holds in v[0] the total of value
// index chan_reduce_index<V>(l); every lane holds a total (duplicated over the
// leftover bits; chan_reduce_writer<V>(l) picks one lane per value).
template <int V>
__device__ __forceinline__ void chan_reduce(float (&v)[V], int lane) {
  static_assert(V == 2 || V == 4 || V == 8, "V must be 2, 4 or 8");
  // bit 5 (lane distance 32)
#pragma unroll
  for (int k = 0; k < V / 2; ++k) {
    float a = v[k], b = v[k + V / 2];
    swap32(a, b);
    v[k] = a + b;
  }
  // bit 4 (distance 16)
  if constexpr (V >= 4) {
#pragma unroll
    for (int k = 0; k < V / 4; ++k) {
      float a = v[k], b = v[k + V / 4];
      swap16(a, b);
      v[k] = a + b;
    }
  } else {
    float a = v[0], b = v[0];
    swap16(a, b);
    v[0] = a + b;
  }
  // bit 3 (distance 8, inside a row: row_ror:8 pairs lane i with i^8)
  if constexpr (V >= 8) {
    const float lo = v[0], hi = v[1];
    const float t = dpp_masked<0x128, 0xC>(0.f, hi);  // lanes 8-15: hi of lane i-8
    const float r = dpp_masked<0x128, 0x3>(t, lo);    // lanes 0-7: lo of lane i+8
    v[0] = ((lane & 8) ? hi : lo) + r;
  } else {
    v[0] += dpp_masked<0x128, 0xF>(0.f, v[0]);
  }
  // bit 2 (distance 4): banks 0,2 read lane i+4 (row_ror:12), banks 1,3 lane i-4 (row_ror:4)
  {
    const float t = dpp_masked<0x124, 0xA>(0.f, v[0]);
    v[0] += dpp_masked<0x12C, 0x5>(t, v[0]);
  }
}

template <int V>
__device__ __forceinline__ int chan_reduce_index(int lane) {
  int idx = 0, bit = 5;
#pragma unroll
  for (int half = V / 2; half >= 1; half /= 2, --bit)
    if ((lane >> bit) & 1) idx += half;
  return idx;
}

template <int V>
__device__ __forceinline__ bool chan_reduce_writer(int lane) {
  constexpr int H = (V >= 8) ? 3 : (V >= 4) ? 2 : (V >= 2) ? 1 : 0;  // log2(V)
  constexpr int R = 4 - H;                                           // leftover bits
  return ((lane >> 2) & ((1 << R) - 1)) == 0;
}

}  // namespace ssm
