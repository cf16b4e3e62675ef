// Device-side helpers shared by the Twilight kernels for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "twl_launch.h"

namespace twl {

constexpr int kWave = 64;

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// ---- device-side guards on caller data ----------------------------------------------

// Number of valid tokens of sequence b: seq_lens clamped to [0, max_pages * 16].
__device__ __forceinline__ int seq_len_clamped(const int32_t* seq_lens, int b, int max_pages) {
  int n = seq_lens[b];
  n = n < 0 ? 0 : n;
  const int cap = max_pages * kPage;
  return n > cap ? cap : n;
}

__device__ __forceinline__ bool phys_ok(int phys, int num_phys) {
  return phys >= 0 && phys < num_phys;
}

// ---- wave reductions (64 lanes) -------------------------------------------------------

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t w = __shfl_xor(v, o);
    v = w > v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const uint32_t w = __shfl_xor(v, o);
    v = w < v ? w : v;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t w = __shfl_up(v, o);
    if (l >= o) v += w;
  }
  return v;
}

__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  const int l = lane_id();
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint64_t w = __shfl_up(v, o);
    if (l >= o) v += w;
  }
  return v;
}

// ---- block-wide primitives (blockDim.x == NT, a multiple of 64) -----------------------

// Exclusive prefix sum of one value per thread, in thread order. `lds` holds NT/64 + 1
// words. Returns the exclusive prefix; *total receives the block total.
template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* lds,
                                                        uint32_t* total) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave;
  const uint32_t incl = wave_incl_scan_u32(v);
  if (lane_id() == kWave - 1) lds[w] = incl;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t run = 0;
    for (int i = 0; i < NW; ++i) {
      const uint32_t t = lds[i];
      lds[i] = run;
      run += t;
    }
    lds[NW] = run;
  }
  __syncthreads();
  const uint32_t res = lds[w] + incl - v;
  *total = lds[NW];
  __syncthreads();
  return res;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* lds) {
  constexpr int NW = NT / kWave;
  v = wave_max(v);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = fmaxf(r, lds[i]);
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* lds) {
  constexpr int NW = NT / kWave;
  v = wave_sum(v);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += lds[i];
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
  constexpr int NW = NT / kWave;
  v = wave_max_u32(v);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = lds[i] > r ? lds[i] : r;
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* lds) {
  constexpr int NW = NT / kWave;
  v = wave_min_u32(v);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  uint32_t r = lds[0];
#pragma unroll
  for (int i = 1; i < NW; ++i) r = lds[i] < r ? lds[i] : r;
  __syncthreads();
  return r;
}

template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* lds) {
  constexpr int NW = NT / kWave;
  v = wave_sum_u64(v);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) r += lds[i];
  __syncthreads();
  return r;
}

// ---- number formats -------------------------------------------------------------------

__device__ __forceinline__ float h2f(uint16_t bits) {
  return static_cast<float>(__builtin_bit_cast(f16, bits));
}

// fp16 bit pattern nearest (ties to even) to a finite v in [0, 65520): one rounding of the
// fp64 value, done by exact power-of-two scaling and rint.
__device__ __forceinline__ uint16_t f64_to_f16_bits_nonneg(double v) {
  if (v < 0x1p-14) {
    const double m = rint(v * 0x1p24);  // subnormal step 2^-24; 1024 is the smallest normal
    return static_cast<uint16_t>(m);
  }
  int e;
  const double f = frexp(v, &e);       // v = f * 2^e, f in [0.5, 1)
  double m = rint(ldexp(f, 11));        // [1024, 2048]
  int E = e - 1;
  if (m == 2048.0) {
    m = 1024.0;
    ++E;
  }
  return static_cast<uint16_t>(((E + 15) << 10) | (static_cast<int>(m) - 1024));
}

// Order-preserving map of a double onto uint64 (larger double -> larger key).
__device__ __forceinline__ uint64_t f64_order_key(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

}  // namespace twl
