// Batched RMSNorm backward for gfx950, given the saved per-row rms (not its inverse),
// as the mamba-rs backward_rms_norm section defines it.  With inv = 1/rms[r] and
//   c[r] = inv^2 * (sum_i dy[r,i] scale[i] x[r,i]) / M,
// the input gradient is dx[r,i] = inv (scale[i] dy[r,i] - x[r,i] c[r]) (overwritten)
// and the scale gradient dscale[i] += sum_r dy[r,i] x[r,i] inv (accumulated).
//
// Mapping: one wavefront per row at a time (4 wavefronts per block walk disjoint
// rows); a lane owns PASSES groups of VEC consecutive columns.  Rows of at most eight
// groups per lane (k_rms_bwd_res) are read once into registers: the dot product is
// formed (wavefront DPP/shuffle sum), then dx is written from the same registers and
// the scale-gradient terms accumulate in registers; scale is staged in LDS.  Rows of up
// to sixteen groups per lane (k_rms_bwd) are read twice, the second time for dx.  At the
// end the four wavefronts' column sums are added through LDS into one partial per block;
// k_reduce sums the block partials in a fixed order.
//
// Rows of any other length (the looped path) take two kernels: k_rms_bwd_rowc forms each
// row's coefficient c[r] (one read of the row), then k_rms_bwd_slab covers the row in
// column slabs of kSlabPasses groups per lane, one slab per workgroup column, writing dx
// and each block's scale-gradient partials of its slab (a second read of the row).
#include <atomic>

#include "common.hpp"
#include "launch.hpp"

namespace ssm {

__device__ __forceinline__ float wave_sum(float v) {
  v = quad_sum(v);
#pragma unroll
  for (int m = 4; m < 64; m <<= 1) v += xor_lane(v, m);
  return v;
}

// VEC consecutive row values kept raw (as stored) in registers.
template <typename T, int VEC>
struct RowVec;
template <>
struct RowVec<bf16_t, 8> {
  using raw_t = uint4;
  __device__ static raw_t load(const bf16_t* p) { return *reinterpret_cast<const uint4*>(p); }
  __device__ static void fence(raw_t& v) { step_fence(v.x, v.y, v.z, v.w); }
  __device__ static void unpack(raw_t v, float (&o)[8]) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      o[2 * k] = __uint_as_float(w[k] << 16);
      o[2 * k + 1] = __uint_as_float(w[k] & 0xffff0000u);
    }
  }
};
template <>
struct RowVec<float, 4> {
  using raw_t = float4;
  __device__ static raw_t load(const float* p) { return *reinterpret_cast<const float4*>(p); }
  __device__ static void fence(raw_t& v) { step_fence(v.x, v.y, v.z, v.w); }
  __device__ static void unpack(raw_t v, float (&o)[4]) {
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <>
struct RowVec<bf16_t, 1> {
  using raw_t = uint32_t;
  __device__ static raw_t load(const bf16_t* p) { return p[0]; }
  __device__ static void fence(raw_t& v) { step_fence(v); }
  __device__ static void unpack(raw_t v, float (&o)[1]) { o[0] = __uint_as_float(v << 16); }
};
template <>
struct RowVec<float, 1> {
  using raw_t = float;
  __device__ static raw_t load(const float* p) { return p[0]; }
  __device__ static void fence(raw_t& v) { step_fence(v); }
  __device__ static void unpack(raw_t v, float (&o)[1]) { o[0] = v; }
};

template <typename T, int VEC, int PASSES>
__global__ __launch_bounds__(256) void k_rms_bwd_res(
    int64_t R, int64_t M, int64_t rows_per_block, const T* __restrict__ dy,
    const T* __restrict__ x, const float* __restrict__ scale, const float* __restrict__ rms,
    T* __restrict__ dx, float* __restrict__ dsp) {
  using RV = RowVec<T, VEC>;
  constexpr int CP = 64 * VEC;  // columns per pass
  __shared__ float ssc[PASSES * CP];
  __shared__ float part[4][CP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  for (int i = tid; i < PASSES * CP; i += 256) ssc[i] = (i < M) ? scale[i] : 0.f;
  float acc[PASSES][VEC];
#pragma unroll
  for (int p = 0; p < PASSES; ++p)
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[p][v] = 0.f;
  __syncthreads();
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  const float invM = 1.0f / float(M);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const T* dyr = dy + r * M;
    const T* xr = x + r * M;
    typename RV::raw_t rd[PASSES], rx[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int col = (p * 64 + lane) * VEC;
      if (col < M) {
        rd[p] = RV::load(dyr + col);
        rx[p] = RV::load(xr + col);
      } else {
        rd[p] = {};
        rx[p] = {};
      }
    }
    const float inv = 1.0f / rms[r];
    float dot = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int col = (p * 64 + lane) * VEC;
      float a[VEC], b[VEC];
      RV::unpack(rd[p], a);
      RV::unpack(rx[p], b);
#pragma unroll
      for (int v = 0; v < VEC; ++v) dot = __builtin_fmaf(a[v] * ssc[col + v], b[v], dot);
    }
    // the output pass unpacks the raw row again rather than keeping it unpacked
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      RV::fence(rd[p]);
      RV::fence(rx[p]);
    }
    dot = wave_sum(dot);
    const float cr = dot * inv * inv * invM;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int col = (p * 64 + lane) * VEC;
      if (col < M) {
        float a[VEC], b[VEC], o[VEC];
        RV::unpack(rd[p], a);
        RV::unpack(rx[p], b);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          o[v] = inv * __builtin_fmaf(ssc[col + v], a[v], -b[v] * cr);
          acc[p][v] = __builtin_fmaf(a[v] * b[v], inv, acc[p][v]);
        }
        VecStore<T, VEC>::run(dx + r * M + col, o);
      }
    }
  }
  // sum the four wavefronts' column partials
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) part[wave][lane * VEC + v] = acc[p][v];
    __syncthreads();
    for (int k = tid; k < CP; k += 256) {
      const int64_t col = int64_t(p) * CP + k;
      if (col < M)
        dsp[int64_t(blockIdx.x) * M + col] = (part[0][k] + part[1][k]) + (part[2][k] + part[3][k]);
    }
    __syncthreads();
  }
}

template <typename T, int VEC, int PASSES>
__global__ __launch_bounds__(256) void k_rms_bwd(
    int64_t R, int64_t M, int64_t rows_per_block, const T* __restrict__ dy,
    const T* __restrict__ x, const float* __restrict__ scale, const float* __restrict__ rms,
    T* __restrict__ dx, float* __restrict__ dsp) {
  __shared__ float part[4][64 * VEC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[PASSES][VEC], sc[PASSES][VEC];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int64_t col = (int64_t(p) * 64 + lane) * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      acc[p][v] = 0.f;
      sc[p][v] = (col < M) ? scale[col + v] : 0.f;
    }
  }
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  const float invM = 1.0f / float(M);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const float inv = 1.0f / rms[r];
    const T* dyr = dy + r * M;
    const T* xr = x + r * M;
    float dot = 0.f;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t col = (int64_t(p) * 64 + lane) * VEC;
      if (col < M) {
        float a[VEC], b[VEC];
        load_vec<T, VEC>(dyr + col, a);
        load_vec<T, VEC>(xr + col, b);
#pragma unroll
        for (int v = 0; v < VEC; ++v) dot = __builtin_fmaf(a[v] * sc[p][v], b[v], dot);
      }
    }
    dot = wave_sum(dot);
    const float cr = dot * inv * inv * invM;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int64_t col = (int64_t(p) * 64 + lane) * VEC;
      if (col < M) {
        float a[VEC], b[VEC], o[VEC];
        load_vec<T, VEC>(dyr + col, a);
        load_vec<T, VEC>(xr + col, b);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          o[v] = inv * __builtin_fmaf(sc[p][v], a[v], -b[v] * cr);
          acc[p][v] = __builtin_fmaf(a[v] * b[v], inv, acc[p][v]);
        }
        VecStore<T, VEC>::run(dx + r * M + col, o);
      }
    }
  }
  // sum the four wavefronts' column partials
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) part[wave][lane * VEC + v] = acc[p][v];
    __syncthreads();
    for (int k = tid; k < 64 * VEC; k += 256) {
      const int64_t col = int64_t(p) * 64 * VEC + k;
      if (col < M)
        dsp[int64_t(blockIdx.x) * M + col] = (part[0][k] + part[1][k]) + (part[2][k] + part[3][k]);
    }
    __syncthreads();
  }
}

// Looped path, first kernel: c[r] = inv^2 * (sum_i dy scale x) / M for every row, one
// wavefront per row (four rows per workgroup at a time), columns strided over the lanes.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void k_rms_bwd_rowc(
    int64_t R, int64_t M, int64_t rows_per_block, const T* __restrict__ dy,
    const T* __restrict__ x, const float* __restrict__ scale, const float* __restrict__ rms,
    float* __restrict__ cr) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t r0 = int64_t(blockIdx.x) * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  const float invM = 1.0f / float(M);
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const T* dyr = dy + r * M;
    const T* xr = x + r * M;
    float dot = 0.f;
    for (int64_t col = int64_t(lane) * VEC; col < M; col += 64 * VEC) {
      float a[VEC], b[VEC];
      load_vec<T, VEC>(dyr + col, a);
      load_vec<T, VEC>(xr + col, b);
#pragma unroll
      for (int v = 0; v < VEC; ++v) dot = __builtin_fmaf(a[v] * scale[col + v], b[v], dot);
    }
    dot = wave_sum(dot);
    const float inv = 1.0f / rms[r];
    if (lane == 0) cr[r] = dot * inv * inv * invM;
  }
}

// Groups of VEC columns per lane in one column slab of the looped path.
constexpr int kSlabPasses = 8;

// Looped path, second kernel: workgroup (row block, column slab) writes dx of its slab
// for its rows and the block's scale-gradient partial of the slab's columns.
template <typename T, int VEC>
__global__ __launch_bounds__(256) void k_rms_bwd_slab(
    int64_t R, int64_t M, int64_t rows_per_block, int64_t nblk, const T* __restrict__ dy,
    const T* __restrict__ x, const float* __restrict__ scale, const float* __restrict__ rms,
    const float* __restrict__ cr, T* __restrict__ dx, float* __restrict__ dsp) {
  constexpr int CP = 64 * VEC;  // columns per pass
  __shared__ float part[4][CP];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t blk = int64_t(blockIdx.x) % nblk, slab = int64_t(blockIdx.x) / nblk;
  const int64_t cs = slab * kSlabPasses * CP;  // first column of the slab
  float acc[kSlabPasses][VEC], sc[kSlabPasses][VEC];
#pragma unroll
  for (int p = 0; p < kSlabPasses; ++p) {
    const int64_t col = cs + (int64_t(p) * 64 + lane) * VEC;
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
      acc[p][v] = 0.f;
      sc[p][v] = (col < M) ? scale[col + v] : 0.f;
    }
  }
  const int64_t r0 = blk * rows_per_block;
  const int64_t r1 = (r0 + rows_per_block < R) ? r0 + rows_per_block : R;
  for (int64_t r = r0 + wave; r < r1; r += 4) {
    const float inv = 1.0f / rms[r], c = cr[r];
    const T* dyr = dy + r * M;
    const T* xr = x + r * M;
#pragma unroll
    for (int p = 0; p < kSlabPasses; ++p) {
      const int64_t col = cs + (int64_t(p) * 64 + lane) * VEC;
      if (col < M) {
        float a[VEC], b[VEC], o[VEC];
        load_vec<T, VEC>(dyr + col, a);
        load_vec<T, VEC>(xr + col, b);
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
          o[v] = inv * __builtin_fmaf(sc[p][v], a[v], -b[v] * c);
          acc[p][v] = __builtin_fmaf(a[v] * b[v], inv, acc[p][v]);
        }
        VecStore<T, VEC>::run(dx + r * M + col, o);
      }
    }
  }
  // sum the four wavefronts' column partials
#pragma unroll
  for (int p = 0; p < kSlabPasses; ++p) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) part[wave][lane * VEC + v] = acc[p][v];
    __syncthreads();
    for (int k = tid; k < CP; k += 256) {
      const int64_t col = cs + int64_t(p) * CP + k;
      if (col < M)
        dsp[blk * M + col] = (part[0][k] + part[1][k]) + (part[2][k] + part[3][k]);
    }
    __syncthreads();
  }
}

template <typename T, int VEC, int PASSES>
static hipError_t rms_launch(const RmsArgs& a, const RmsPlan& p, hipStream_t st) {
  const T* dy = static_cast<const T*>(a.dy);
  const T* x = static_cast<const T*>(a.x);
  T* dx = static_cast<T*>(a.dx);
  hipError_t e;
  timer_mark(kKRmsBwd, false, st);
  if constexpr (PASSES == 0) {  // the looped path
    e = launch(k_rms_bwd_rowc<T, VEC>, dim3(unsigned(p.nblk)), dim3(256), st, a.R, a.M,
               p.rows_per_block, dy, x, a.scale, a.rms, p.crow);
    const int64_t nslab = (a.M + kSlabPasses * 64 * VEC - 1) / (kSlabPasses * 64 * VEC);
    if (e == hipSuccess)
      e = launch(k_rms_bwd_slab<T, VEC>, dim3(unsigned(p.nblk * nslab)), dim3(256), st, a.R,
                 a.M, p.rows_per_block, p.nblk, dy, x, a.scale, a.rms, p.crow, dx, p.dsp);
  } else if constexpr (PASSES <= 8) {
    e = launch(k_rms_bwd_res<T, VEC, PASSES>, dim3(unsigned(p.nblk)), dim3(256), st, a.R, a.M,
               p.rows_per_block, dy, x, a.scale, a.rms, dx, p.dsp);
  } else {
    e = launch(k_rms_bwd<T, VEC, PASSES>, dim3(unsigned(p.nblk)), dim3(256), st, a.R, a.M,
               p.rows_per_block, dy, x, a.scale, a.rms, dx, p.dsp);
  }
  timer_mark(kKRmsBwd, true, st);
  return e;
}

// passes: exact count up to 8 (row resident in registers), 16 (read twice), or 0 (the
// looped path, any row length)
template <typename T, int VEC>
static hipError_t rms_v(const RmsArgs& a, const RmsPlan& p, hipStream_t st) {
  switch (p.passes) {
    case 0: return rms_launch<T, VEC, 0>(a, p, st);
    case 1: return rms_launch<T, VEC, 1>(a, p, st);
    case 2: return rms_launch<T, VEC, 2>(a, p, st);
    case 3: return rms_launch<T, VEC, 3>(a, p, st);
    case 4: return rms_launch<T, VEC, 4>(a, p, st);
    case 5: return rms_launch<T, VEC, 5>(a, p, st);
    case 6: return rms_launch<T, VEC, 6>(a, p, st);
    case 7: return rms_launch<T, VEC, 7>(a, p, st);
    case 8: return rms_launch<T, VEC, 8>(a, p, st);
    case 16: return rms_launch<T, VEC, 16>(a, p, st);
  }
  return hipErrorInvalidValue;
}

// Scratch of rmsnorm_bwd_noalloc, for callers that cannot allocate (code under HIP graph
// capture, serving loops, harnesses that forbid hipMalloc): a static device array of
// kNoAllocScratchBytes, one copy per GPU for the life of the process.  Host code never
// uses the array's name as an address: the device address of each GPU's copy is taken
// once per device with hipGetSymbolAddress (with that device current) and kept in
// g_scratch_ptr; that pointer is what reaches the kernels.  Calls on one GPU share its
// copy, so calls that overlap on one GPU race.  Nothing in it needs clearing: every
// partial the kernels read was written by the same call.
static __device__ __align__(256) float scratch[kNoAllocScratchBytes / sizeof(float)];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* q = g_scratch_ptr[dev].load();
  if (!q) {
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev].store(q);
  }
  *ptr = q;
  return hipSuccess;
}

hipError_t launch_rmsnorm_bwd(const RmsArgs& a, const RmsPlan& p, hipStream_t st) {
  hipError_t e;
  if (a.dtype == 0)
    e = (p.vec == 4) ? rms_v<float, 4>(a, p, st) : rms_v<float, 1>(a, p, st);
  else
    e = (p.vec == 8) ? rms_v<bf16_t, 8>(a, p, st) : rms_v<bf16_t, 1>(a, p, st);
  if (e != hipSuccess) return e;
  return launch_reduce(p.dsp, p.nblk, a.M, a.dscale, true, p.rtmp, st);
}

}  // namespace ssm
