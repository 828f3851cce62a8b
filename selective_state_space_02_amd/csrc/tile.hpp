// Staging of scan inputs through LDS, one tile at a time.
//
// A tile is kTc consecutive steps of one batch row for the workgroup's 64 channels.
// Every element of a per-channel tensor ([B,L,D]: x, delta, dy) and of a per-step
// vector ([B,L,N]: B, C) is fetched once with a coalesced load -- a wavefront reads 64
// consecutive channels of one step -- and held in a register, raw, while the previous
// tile is being computed; it is converted to f32 and written to one of two LDS buffers
// only after that compute ("commit"), so the load latency overlaps the compute.
//
// Loads are unconditional: an element outside the tensor (step >= L or channel >= D)
// is read from the tile's first element instead (always inside) and replaced by zero
// at commit.  A zero step is an exact identity of the recurrence (a = exp(0) = 1, no
// input, no output), so the compute loops carry no tail branches.
#pragma once
#include "common.hpp"

namespace ssm {

constexpr int kTileThreads = 256;
constexpr int kTileCh = 64;                                 // channels per workgroup
constexpr int kChPerThread = kTc * kTileCh / kTileThreads;  // 4

// One per-channel tensor's share of a tile: element e = tid + 256 k sits at step e/64,
// channel e%64 of the tile.
template <typename T>
struct ChFetch {
  T raw[kChPerThread];
  // tile = base + tf*D + d0 (the tile's first element); tvalid = L - tf; dvalid = D - d0.
  __device__ __forceinline__ void fetch(const T* __restrict__ tile, int D32, int tvalid,
                                        int dvalid, int tid) {
#pragma unroll
    for (int k = 0; k < kChPerThread; ++k) {
      const int e = tid + kTileThreads * k, s = e >> 6, c = e & 63;
      const bool ok = s < tvalid && c < dvalid;
      raw[k] = tile[ok ? s * D32 + c : 0];
    }
  }
  __device__ __forceinline__ void commit(float (*sm)[kTileCh], int tvalid, int dvalid,
                                         int tid) const {
#pragma unroll
    for (int k = 0; k < kChPerThread; ++k) {
      const int e = tid + kTileThreads * k, s = e >> 6, c = e & 63;
      const bool ok = s < tvalid && c < dvalid;
      sm[s][c] = ok ? to_f32(raw[k]) : 0.f;
    }
  }
};

// One per-step vector's share of a tile: thread tid < kTc*N owns element tid (step
// tid/N, state tid%N).
template <typename T, int N>
struct VecFetch {
  T raw;
  __device__ __forceinline__ void fetch(const T* __restrict__ tile /* base + tf*N */,
                                        int tvalid, int tid) {
    const bool ok = tid < kTc * N && tid / N < tvalid;
    raw = tile[ok ? tid : 0];
  }
  __device__ __forceinline__ void commit(float (*sm)[N], int tvalid, int tid) const {
    if (tid < kTc * N) sm[tid / N][tid % N] = (tid / N < tvalid) ? to_f32(raw) : 0.f;
  }
};

// Writes an LDS tile of per-channel outputs back to a [.,L,D] tensor with the same
// coalesced mapping as the fetch (a wavefront stores 64 consecutive channels of one
// step); tile = base + tf*D + d0; only steps < tvalid and channels < dvalid are written.
template <typename T>
__device__ __forceinline__ void tile_store_ch(T* __restrict__ tile, const float (*sm)[kTileCh],
                                              int D32, int tvalid, int dvalid, int tid) {
#pragma unroll
  for (int k = 0; k < kChPerThread; ++k) {
    const int e = tid + kTileThreads * k, s = e >> 6, c = e & 63;
    if (s < tvalid && c < dvalid) tile[s * D32 + c] = from_f32<T>(sm[s][c]);
  }
}

// The NS state values of lane quarter q at step s of an LDS vector tile.
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

__device__ __forceinline__ int clamp_valid(int64_t v) {
  return v < 0 ? 0 : (v > kTc ? kTc : int(v));
}

}  // namespace ssm
