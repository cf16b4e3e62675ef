// Device-side helpers shared by the Twilight kernels for gfx950 (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "twl_launch.h"

namespace twl {

constexpr int kWave = 64;

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
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

// Makes a loaded value count as used at this point: its load is issued (and waited for)
// here, so the compiler cannot sink it past a later branch.
__device__ __forceinline__ void keep_loaded(int v) { asm volatile("" ::"v"(v)); }

// A load of a value that is the same for the whole wave, issued on the vector path: its
// address depends on an opaque zero held in a VGPR. Vector loads return in order, so waiting
// for a later load (a kernel argument, say) does not also wait for this one, as it would for
// a scalar load, and it can be issued alongside the wave's first vector loads. The caller
// makes the value scalar (readfirstlane) where it is needed.
__device__ __forceinline__ int vgpr_zero() {
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return z;
}
__device__ __forceinline__ int load_uniform_vec(const int32_t* p) { return p[vgpr_zero()]; }

__device__ __forceinline__ bool phys_ok(int phys, int num_phys) {
  return phys >= 0 && phys < num_phys;
}

// ---- cross-lane moves ------------------------------------------------------------------
// DPP controls (GFX9 encoding).
constexpr int kQuadXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kRowShr1 = 0x111;
constexpr int kRowShr2 = 0x112;
constexpr int kRowShr4 = 0x114;
constexpr int kRowShr8 = 0x118;
constexpr int kRowRor8 = 0x128;
constexpr int kRowMirror = 0x140;
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowBcast15 = 0x142;
constexpr int kRowBcast31 = 0x143;

// DPP move; lanes without a source (or outside row_mask) read 0.
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(
      __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, RM, 0xF, true));
}
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL, RM>(__builtin_bit_cast(uint32_t, v)));
}
// Lane n (0..15, a constant after unrolling) of each 16-lane row, broadcast to its row
// (DPP row_newbcast).
__device__ __forceinline__ float row_bcast_f32(float v, int n) {
  switch (n) {
    case 0: return dpp_f32<0x150>(v);
    case 1: return dpp_f32<0x151>(v);
    case 2: return dpp_f32<0x152>(v);
    case 3: return dpp_f32<0x153>(v);
    case 4: return dpp_f32<0x154>(v);
    case 5: return dpp_f32<0x155>(v);
    case 6: return dpp_f32<0x156>(v);
    case 7: return dpp_f32<0x157>(v);
    case 8: return dpp_f32<0x158>(v);
    case 9: return dpp_f32<0x159>(v);
    case 10: return dpp_f32<0x15A>(v);
    case 11: return dpp_f32<0x15B>(v);
    case 12: return dpp_f32<0x15C>(v);
    case 13: return dpp_f32<0x15D>(v);
    case 14: return dpp_f32<0x15E>(v);
    default: return dpp_f32<0x15F>(v);
  }
}
template <int CTRL, int RM = 0xF>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, RM>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp_u32<CTRL, RM>(static_cast<uint32_t>(v >> 32));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}

template <typename T>
__device__ __forceinline__ T readlane(T v, int lane) {
  if constexpr (sizeof(T) == 8) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(u), lane);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(u >> 32), lane);
    return __builtin_bit_cast(T, (static_cast<uint64_t>(hi) << 32) | lo);
  } else {
    return __builtin_bit_cast(
        T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
  }
}

template <int CTRL, typename T>
__device__ __forceinline__ T dpp_any(T v) {
  if constexpr (sizeof(T) == 8) {
    return __builtin_bit_cast(T, dpp_u64<CTRL>(__builtin_bit_cast(uint64_t, v)));
  } else {
    return __builtin_bit_cast(T, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
  }
}

struct OpSum {
  template <typename T> __device__ T operator()(T a, T b) const { return a + b; }
};
struct OpMax {
  template <typename T> __device__ T operator()(T a, T b) const { return a > b ? a : b; }
  __device__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OpMin {
  template <typename T> __device__ T operator()(T a, T b) const { return a < b ? a : b; }
};

// Reduction over the whole wave, result uniform: DPP inside each 16-lane row (every lane of
// a row ends with the row result, each step combining a commutative pair), then the four
// rows combined through readlane in a fixed order. Every lane must be active.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
  v = op(v, dpp_any<kQuadXor1>(v));
  v = op(v, dpp_any<kQuadXor2>(v));
  v = op(v, dpp_any<kRowHalfMirror>(v));
  v = op(v, dpp_any<kRowMirror>(v));
  return op(op(readlane(v, 0), readlane(v, 16)), op(readlane(v, 32), readlane(v, 48)));
}

__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax()); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpSum()); }

// Sum over aligned groups of W lanes (W in {2, 4, 8, 16}) with DPP; every lane of a group
// ends with the bit-identical total.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group width");
  v += dpp_f32<kQuadXor1>(v);
  if constexpr (W >= 4) v += dpp_f32<kQuadXor2>(v);
  if constexpr (W >= 8) v += dpp_f32<kRowHalfMirror>(v);
  if constexpr (W >= 16) v += dpp_f32<kRowMirror>(v);
  return v;
}

// Reduction with `op` over aligned groups of W lanes (W in {2, 4, 8, 16}); every lane of a
// group ends with the group's result.
template <int W, typename Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
  static_assert(W == 2 || W == 4 || W == 8 || W == 16, "group width");
  v = op(v, dpp_f32<kQuadXor1>(v));
  if constexpr (W >= 4) v = op(v, dpp_f32<kQuadXor2>(v));
  if constexpr (W >= 8) v = op(v, dpp_f32<kRowHalfMirror>(v));
  if constexpr (W >= 16) v = op(v, dpp_f32<kRowMirror>(v));
  return v;
}

// Combine the lanes that hold the same position within their W-lane group, over all
// 64 / W groups of the wave (W in {8, 16}); every lane ends with the combined value. Uses
// a DPP rotate inside rows and the gfx950 permlane swaps across rows.
template <int W, typename Op>
__device__ __forceinline__ float across_groups(float v, Op op) {
  static_assert(W == 8 || W == 16, "group width");
  if constexpr (W == 8) v = op(v, dpp_f32<kRowRor8>(v));
  {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, v),
                                                    __builtin_bit_cast(int, v), false, false);
    v = op(__builtin_bit_cast(float, static_cast<int>(r[0])),
           __builtin_bit_cast(float, static_cast<int>(r[1])));
  }
  {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, v),
                                                    __builtin_bit_cast(int, v), false, false);
    v = op(__builtin_bit_cast(float, static_cast<int>(r[0])),
           __builtin_bit_cast(float, static_cast<int>(r[1])));
  }
  return v;
}

// Sum over the wave's four 16-lane rows, scattered: on return, row r (lanes 16r..16r+15)
// holds in y[i] the four-row sum of x[r * N / 4 + i], lane by lane. Each permlane swap
// carries two different values, so a value costs half a swap and half an add per step,
// where an all-reduce costs a full swap, two copies and an add.
template <int N>
__device__ __forceinline__ void sum_rows_scatter(const float (&x)[N], float (&y)[N / 4]) {
  static_assert(N % 4 == 0, "value count");
  float h[N / 2];
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    // lanes 0-31 end with x[k] summed over rows {r, r ^ 2}, lanes 32-63 with x[k + N/2]
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(int, x[k]),
                                                    __builtin_bit_cast(int, x[k + N / 2]),
                                                    false, false);
    h[k] = __builtin_bit_cast(float, static_cast<int>(r[0])) +
           __builtin_bit_cast(float, static_cast<int>(r[1]));
  }
#pragma unroll
  for (int k = 0; k < N / 4; ++k) {
    // even rows end with h[k] summed over rows {r, r ^ 1}, odd rows with h[k + N/4]
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(int, h[k]),
                                                    __builtin_bit_cast(int, h[k + N / 4]),
                                                    false, false);
    y[k] = __builtin_bit_cast(float, static_cast<int>(r[0])) +
           __builtin_bit_cast(float, static_cast<int>(r[1]));
  }
}

// 2^x on the transcendental unit alone: exact for -inf (0) and within an ulp of exp2f for
// x >= -126; below that it returns 0 where exp2f returns a denormal.
__device__ __forceinline__ float exp2_unit(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the 64 lanes: row-local Hillis-Steele shifts, then the row
// totals carried across rows with row_bcast.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T x) {
  x += dpp_any<kRowShr1>(x);
  x += dpp_any<kRowShr2>(x);
  x += dpp_any<kRowShr4>(x);
  x += dpp_any<kRowShr8>(x);
  if constexpr (sizeof(T) == 8) {
    x += __builtin_bit_cast(T, dpp_u64<kRowBcast15, 0xA>(__builtin_bit_cast(uint64_t, x)));
    x += __builtin_bit_cast(T, dpp_u64<kRowBcast31, 0xC>(__builtin_bit_cast(uint64_t, x)));
  } else {
    x += __builtin_bit_cast(T, dpp_u32<kRowBcast15, 0xA>(__builtin_bit_cast(uint32_t, x)));
    x += __builtin_bit_cast(T, dpp_u32<kRowBcast31, 0xC>(__builtin_bit_cast(uint32_t, x)));
  }
  return x;
}

// ---- block-wide primitives (blockDim.x == NT, a multiple of 64, at most 1024) ----------
// Each takes an LDS scratch of NT/64 elements and ends with a barrier, so the scratch may
// be reused by the next call.

template <int NT, typename T, typename Op>
__device__ __forceinline__ T block_reduce(T v, T* lds, Op op, T identity) {
  constexpr int NW = NT / kWave;
  v = wave_reduce(v, op);
  if (lane_id() == 0) lds[threadIdx.x / kWave] = v;
  __syncthreads();
  T x = lane_id() < NW ? lds[lane_id()] : identity;
  x = wave_reduce(x, op);
  __syncthreads();
  return x;
}

template <int NT>
__device__ __forceinline__ float block_max(float v, float* lds) {
  return block_reduce<NT>(v, lds, OpMax(), -INFINITY);
}
template <int NT>
__device__ __forceinline__ float block_sum(float v, float* lds) {
  return block_reduce<NT>(v, lds, OpSum(), 0.f);
}
template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, uint32_t* lds) {
  return block_reduce<NT>(v, lds, OpMax(), 0u);
}
template <int NT>
__device__ __forceinline__ uint32_t block_min_u32(uint32_t v, uint32_t* lds) {
  return block_reduce<NT>(v, lds, OpMin(), 0xffffffffu);
}
template <int NT>
__device__ __forceinline__ uint64_t block_sum_u64(uint64_t v, uint64_t* lds) {
  return block_reduce<NT>(v, lds, OpSum(), uint64_t(0));
}
template <int NT>
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t* lds) {
  return block_reduce<NT>(v, lds, OpMax(), uint64_t(0));
}
template <int NT>
__device__ __forceinline__ uint64_t block_min_u64(uint64_t v, uint64_t* lds) {
  return block_reduce<NT>(v, lds, OpMin(), ~uint64_t(0));
}

// Minimum and maximum of one value per thread in a single exchange.
template <int NT, typename T>
__device__ __forceinline__ void block_minmax(T vmin, T vmax, T* lds_min, T* lds_max, T id_min,
                                             T id_max, T* out_min, T* out_max) {
  constexpr int NW = NT / kWave;
  vmin = wave_reduce(vmin, OpMin());
  vmax = wave_reduce(vmax, OpMax());
  if (lane_id() == 0) {
    lds_min[threadIdx.x / kWave] = vmin;
    lds_max[threadIdx.x / kWave] = vmax;
  }
  __syncthreads();
  T a = lane_id() < NW ? lds_min[lane_id()] : id_min;
  T b = lane_id() < NW ? lds_max[lane_id()] : id_max;
  *out_min = wave_reduce(a, OpMin());
  *out_max = wave_reduce(b, OpMax());
  __syncthreads();
}

// Exclusive prefix sum of one value per thread, in thread order; *total gets the sum.
template <int NT, typename T>
__device__ __forceinline__ T block_excl_scan(T v, T* lds, T* total) {
  constexpr int NW = NT / kWave;
  const int w = threadIdx.x / kWave;
  const T incl = wave_incl_scan(v);
  if (lane_id() == kWave - 1) lds[w] = incl;
  __syncthreads();
  T x = lane_id() < NW ? lds[lane_id()] : T(0);
  x = wave_incl_scan(x);
  const T before = w > 0 ? readlane(x, w - 1) : T(0);
  *total = readlane(x, NW - 1);
  __syncthreads();
  return before + incl - v;
}

template <int NT>
__device__ __forceinline__ uint32_t block_excl_scan_u32(uint32_t v, uint32_t* lds,
                                                        uint32_t* total) {
  return block_excl_scan<NT, uint32_t>(v, lds, total);
}

// Boundary bucket of a descending selection over NT * BPT buckets kept in LDS, bucket b at
// bins[b] (`bins` aligned to BPT elements). Thread t owns the contiguous buckets
// [t*BPT, (t+1)*BPT) and reads them in one vector load, so the wave's reads are one
// contiguous, conflict-free stretch. Returns the bucket b* with
// weight(buckets > b*) < rem <= weight(buckets >= b*); *above = weight(buckets > b*),
// *in = weight(b*). `lds` holds NT/64 elements, `pick` 3. Requires
// 0 < rem <= total weight. When frac > 0, rem is replaced by
// max(1, ceil(frac * total weight)) and *rem_used receives it, so a first pass needs no
// separate reduction for the total. It ends without a barrier: every thread has read `lds`
// before the second barrier and reads `pick` after it, so the caller must pass a block
// barrier before it writes `pick` or `lds` again (the radix selections here always do, in
// the passes between two picks).
template <int NT, int BPT, typename T>
__device__ __forceinline__ uint32_t block_pick_bucket_lds(const T* bins, T rem, T* lds, T* pick,
                                                          T* above, T* in, float frac = 0.f,
                                                          T* rem_used = nullptr) {
  constexpr int NW = NT / kWave;
  const int t = threadIdx.x;
  const int w = t / kWave;
  typedef T TV __attribute__((ext_vector_type(BPT)));
  const TV bvv = *reinterpret_cast<const TV*>(bins + t * BPT);
  T bv[BPT];
  T mine = T(0);
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    bv[i] = bvv[i];
    mine += bv[i];
  }
  const T incl = wave_incl_scan(mine);
  if (lane_id() == kWave - 1) lds[w] = incl;
  __syncthreads();
  T x = lane_id() < NW ? lds[lane_id()] : T(0);
  x = wave_incl_scan(x);
  const T before = w > 0 ? readlane(x, w - 1) : T(0);
  const T total = readlane(x, NW - 1);
  if (frac > 0.f) {
    rem = static_cast<T>(ceil(static_cast<double>(frac) * static_cast<double>(total)));
    rem = rem < T(1) ? T(1) : rem;
    if (rem_used) *rem_used = rem;
  }
  T abv = total - (before + incl);  // weight of the buckets above this thread's range
#pragma unroll
  for (int i = BPT - 1; i >= 0; --i) {
    if (abv < rem && rem <= abv + bv[i]) {
      pick[0] = static_cast<T>(t * BPT + i);
      pick[1] = abv;
      pick[2] = bv[i];
    }
    abv += bv[i];
  }
  __syncthreads();
  const uint32_t b = static_cast<uint32_t>(pick[0]);
  *above = pick[1];
  *in = pick[2];
  return b;
}

// ---- softmax normalisation from split partials ----------------------------------------

// Global (max, sum of exp2) of a row of log2-unit logits from its chunks' (max, sum of
// exp2) pairs, one wave: lane i merges chunks i, i + 64, ... online, then the lanes are
// combined on the common maximum. Every lane returns the same pair. Chunks with max -inf
// (no valid slot) are skipped. The estimate's normalising pass and the top-p that
// normalises for itself both use this, so they agree bit for bit.
__device__ __forceinline__ float2 merge_max_sum_wave(const float2* pr, int n_chunks) {
  float m = -INFINITY, l = 0.f;
  for (int i = lane_id(); i < n_chunks; i += kWave) {
    const float2 p = pr[i];
    if (p.x > -INFINITY) {
      const float mn = fmaxf(m, p.x);
      l = (m > -INFINITY ? l * exp2_unit(m - mn) : 0.f) + p.y * exp2_unit(p.x - mn);
      m = mn;
    }
  }
  const float M = wave_max(m);
  const float L = wave_sum(m > -INFINITY ? l * exp2_unit(m - M) : 0.f);
  return make_float2(M, L);
}

// 1 / (sum of exp2) of a row, 0 for an empty row.
__device__ __forceinline__ float softmax_inv_sum(float L) { return L > 0.f ? 1.f / L : 0.f; }

// Normalised weight of a log2-unit logit v given the row's max and 1 / (sum of exp2); 0 for
// a slot that is not a candidate (v = -inf) or an empty row (M = -inf, taken as 0 so that no
// -inf - -inf arises). The exponential runs on the transcendental unit alone: weights below
// 2^-126 / sum come out 0 instead of subnormal.
__device__ __forceinline__ float softmax_weight(float v, float M, float inv_l) {
  // one rounded product, never contracted into the caller's next add, so that every kernel
  // that forms this weight gets the same bits whether it stores it or sums it at once
#pragma clang fp contract(off)
  const float mref = M == -INFINITY ? 0.f : M;
  return exp2_unit(v - mref) * inv_l;
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
