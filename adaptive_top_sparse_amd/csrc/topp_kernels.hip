// Top-p (nucleus) pruning of the candidates and compaction of the kept tokens (Twilight
// pages, atlas.scime.ai summary: "Approach" for top-p thresholding of the estimated weights
// with binary-search top-p kernels, "Limitations" for the group-wise budget under GQA).
//
// The search for tau runs on chip, one 1024-thread block per (sequence, KV head):
//  * W_j = mean over the group's heads of the weights (fp32, fixed head order).
//  * Masses are exact integers: M_j = floor(W_j * 2^(40 - e)), e the binary exponent of the
//    unit's largest W, so every sum is independent of order and the result is
//    deterministic. The truncation costs less than 2^-40 of max W per slot.
//  * tau is the largest fp32 value with sum_{W_j >= tau} M_j >= ceil(p * sum_j M_j). The
//    search narrows the range of fp32 bit patterns (monotone for W >= 0) with 2048-bucket
//    mass histograms, instead of halving it once per pass: a 31-bit range closes in at
//    most three passes, each one read of the registers.
//  * Kept = {W_j >= tau, W_j > 0}, compacted with a block scan in slot order, which is
//    ascending token order because candidate pages are ascending.
#include "twl_device.h"
#include "twl_launch.h"

TWL_PHASE_STORAGE(topp)

namespace twl {
namespace {

constexpr int kToppThreads = 1024;
constexpr int kBins = 2048;

// floor(W * 2^(40 - e)) for a non-negative fp32 W given by its bits, e the binary exponent
// of the unit's largest W: integer shifts of the 24-bit significand (W < 2^(e+1), so the
// result is below 2^41). Subnormal W (a tiny share of any sum) counts as 0.
__device__ __forceinline__ uint64_t fixed_mass(uint32_t key, int e) {
  const int ew = static_cast<int>(key >> 23) - 127;
  if (ew < -126) return 0;
  const uint64_t sig = (key & 0x7fffffu) | 0x800000u;
  const int sh = ew - e + 17;  // W * 2^(40-e) = sig * 2^(ew - 23 + 40 - e)
  if (sh >= 0) return sig << sh;
  return sh <= -24 ? 0 : (sig >> (-sh));
}

// Each thread owns SPT consecutive slots. Up to 16 stay in registers for the whole search;
// larger rows are processed as 16-slot tiles, with W staged once in the workspace (each
// thread re-reads only what it wrote). A slot is a candidate when its page rank is below the
// unit's candidate count and its token is inside the sequence; slots of unmapped pages
// carry weight 0 from the estimate and are never kept (W > 0 is required).
template <int SPT>
__global__ __launch_bounds__(kToppThreads) void topp_kernel(
    const float* __restrict__ weights, const int32_t* __restrict__ cand_pages,
    const int32_t* __restrict__ cand_count, int cand_stride_pages,
    const int32_t* __restrict__ seq_lens, int Hkv, int G, int max_pages, float p,
    int32_t* __restrict__ kept, int32_t* __restrict__ kept_count, float* __restrict__ tau_out,
    float* __restrict__ stage) {
  constexpr int TILE = SPT < 16 ? SPT : 16;
  constexpr int NT = SPT / TILE;
  constexpr int PG = (TILE + kPage - 1) / kPage;  // candidate pages a tile touches
  __shared__ unsigned long long mass[kBins];
  __shared__ uint32_t scan_u32[kToppThreads / kWave + 1], scan_u32b[kToppThreads / kWave];
  __shared__ uint64_t red64[kToppThreads / kWave];
  __shared__ uint64_t pick[3];
  TWL_PHASE(0);
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const long unit = static_cast<long>(b) * Hkv + g;
  const int Hq = Hkv * G;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int n_slots = cand_stride_pages * kPage;
  const int32_t* cand_row = cand_pages ? cand_pages + unit * cand_stride_pages : nullptr;
  int cnt = 0;
  if (cand_pages != nullptr) {
    cnt = cand_count ? cand_count[unit] : (n + kPage - 1) / kPage;
    cnt = cnt < cand_stride_pages ? cnt : cand_stride_pages;
  }
  const int first = threadIdx.x * SPT;
  float* my_stage = NT > 1 ? stage + unit * n_slots + first : nullptr;
  const float inv_g = 1.0f / static_cast<float>(G);  // exact: G is a power of two

  // logical token of the tile's slot i, or -1 (tile-local page ids preloaded in pg[])
  auto token_of = [&](int f0, const int (&pg)[PG], int i) -> int {
    const int slot = f0 + i;
    if (slot >= n_slots) return -1;
    int t;
    if (cand_row == nullptr) {
      t = slot;
    } else {
      const int pid = pg[(i + (f0 % kPage)) / kPage];
      if (slot / kPage >= cnt || pid < 0) return -1;
      t = pid * kPage + slot % kPage;
    }
    return t < n ? t : -1;
  };
  auto load_pages = [&](int f0, int (&pg)[PG]) {
#pragma unroll
    for (int j = 0; j < PG; ++j) {
      const int r = f0 / kPage + j;
      pg[j] = (cand_row != nullptr && r < cnt) ? cand_row[r] : -1;
    }
  };

  // pass 0: W_j = mean of the group's weights on candidate slots (0 elsewhere)
  float W[TILE];
  uint32_t kmax = 0, kmin = 0xffffffffu;
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
    const int f0 = first + t * TILE;
    int pg[PG];
    load_pages(f0, pg);
#pragma unroll
    for (int i = 0; i < TILE; ++i) W[i] = 0.f;
    if (f0 < n_slots) {
      for (int h = 0; h < G; ++h) {
        const float* row = weights + (static_cast<long>(b) * Hq + g * G + h) * n_slots + f0;
        if constexpr (TILE % 4 == 0) {
          // n_slots % 16 == 0, so a tile that starts inside the row ends inside it
#pragma unroll
          for (int i = 0; i < TILE; i += 4) {
            const f32x4 v = *reinterpret_cast<const f32x4*>(row + i);
            W[i] += v[0];
            W[i + 1] += v[1];
            W[i + 2] += v[2];
            W[i + 3] += v[3];
          }
        } else {
#pragma unroll
          for (int i = 0; i < TILE; ++i)
            if (f0 + i < n_slots) W[i] += row[i];
        }
      }
    }
#pragma unroll
    for (int i = 0; i < TILE; ++i) {
      W[i] = token_of(f0, pg, i) >= 0 ? fmaxf(W[i] * inv_g, 0.f) : 0.f;
      const uint32_t k = __float_as_uint(W[i]);
      if (k > 0) {
        kmax = k > kmax ? k : kmax;
        kmin = k < kmin ? k : kmin;
      }
    }
    if (NT > 1 && f0 < n_slots) {
#pragma unroll
      for (int i = 0; i < TILE; i += 4)
        *reinterpret_cast<f32x4*>(my_stage + t * TILE + i) =
            f32x4{W[i], W[i + 1], W[i + 2], W[i + 3]};
    }
  }
  TWL_PHASE(1);
  block_minmax<kToppThreads, uint32_t>(kmin, kmax, scan_u32, scan_u32b, 0xffffffffu, 0u, &kmin,
                                       &kmax);
  TWL_PHASE(2);

  // reload tile t of this thread's W (no-op when everything fits one tile)
  auto load_tile = [&](int t) {
    if constexpr (NT > 1) {
      if (first + t * TILE < n_slots) {
#pragma unroll
        for (int i = 0; i < TILE; i += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(my_stage + t * TILE + i);
          W[i] = v[0];
          W[i + 1] = v[1];
          W[i + 2] = v[2];
          W[i + 3] = v[3];
        }
      } else {
#pragma unroll
        for (int i = 0; i < TILE; ++i) W[i] = 0.f;
      }
    }
  };

  float tau = 0.f;
  if (kmax != 0 && p >= 1.0f) {
    tau = __uint_as_float(kmin);
  } else if (kmax != 0) {
    // fixed-point masses relative to the largest weight's binade
    const int e = static_cast<int>((kmax >> 23) & 0xff) - 127;
    TWL_PHASE(3);
    // the first pass covers every positive W, so its scan yields the total mass and the
    // target ceil(p * total)
    uint64_t rem = 0;
    uint32_t lo = kmin, hi = kmax;
    int pass_no = 0;
    for (;;) {
      const uint32_t range = hi - lo;
      const int bits = range == 0 ? 0 : 32 - __clz(range);
      const int shift = bits > 11 ? bits - 11 : 0;
      mass[threadIdx.x] = 0ull;
      mass[threadIdx.x + kToppThreads] = 0ull;
      __syncthreads();
#pragma unroll 1
      for (int t = 0; t < NT; ++t) {
        load_tile(t);
#pragma unroll
        for (int i = 0; i < TILE; ++i) {
          const uint32_t k = __float_as_uint(W[i]);
          if (k >= lo && k <= hi) {
            const uint64_t m = fixed_mass(k, e);
            if (m != 0) atomicAdd(&mass[(k - lo) >> shift], m);
          }
        }
      }
      __syncthreads();
      uint64_t above, inb;
      const uint32_t bucket = block_pick_bucket<kToppThreads, uint64_t>(
          mass[2 * threadIdx.x], mass[2 * threadIdx.x + 1], rem, red64, pick, &above, &inb,
          pass_no == 0 ? p : 0.f, &rem);
      rem -= above;
      const uint32_t nlo = lo + (bucket << shift);
      const uint32_t span = (1u << shift) - 1u;
      const uint32_t nhi = (hi - nlo) < span ? hi : nlo + span;
      lo = nlo;
      hi = nhi;
      TWL_PHASE(4 + (pass_no < 4 ? pass_no : 4));
      ++pass_no;
      if (shift == 0) break;
    }
    tau = __uint_as_float(lo);
  }

  TWL_PHASE(9);
  // compaction in slot order
  uint32_t nk = 0;
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
    load_tile(t);
#pragma unroll
    for (int i = 0; i < TILE; ++i) nk += (W[i] > 0.f && W[i] >= tau) ? 1u : 0u;
  }
  uint32_t total;
  uint32_t pos = block_excl_scan_u32<kToppThreads>(nk, scan_u32, &total);
  TWL_PHASE(10);
  int32_t* out = kept + unit * n_slots;
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
    const int f0 = first + t * TILE;
    int pg[PG];
    load_pages(f0, pg);
    load_tile(t);
#pragma unroll
    for (int i = 0; i < TILE; ++i) {
      if (W[i] > 0.f && W[i] >= tau) out[pos++] = token_of(f0, pg, i);
    }
  }
  if (threadIdx.x == 0) {
    kept_count[unit] = static_cast<int32_t>(total);
    if (tau_out) tau_out[unit] = tau;
  }
  TWL_PHASE(11);
}

template <int SPT>
void topp_launch(const Layout& L, const float* weights, const int32_t* cand_pages,
                 const int32_t* cand_count, int stride, float p, int32_t* kept,
                 int32_t* kept_count, float* tau, float* stage, hipStream_t s) {
  topp_kernel<SPT><<<dim3(L.Hkv, L.B), kToppThreads, 0, s>>>(
      weights, cand_pages, cand_count, stride, L.seq_lens, L.Hkv, L.G(), L.max_pages, p, kept,
      kept_count, tau, stage);
}

}  // namespace

size_t topp_workspace_bytes(const Layout& L, int cand_stride_pages) {
  const long n_slots = static_cast<long>(cand_stride_pages) * kPage;
  if (n_slots <= 16L * kToppThreads) return 0;
  return align_up(static_cast<size_t>(L.B) * L.Hkv * n_slots * sizeof(float), 256);
}

hipError_t launch_topp(const Layout& L, const float* weights, const int32_t* cand_pages,
                       const int32_t* cand_count, int cand_stride_pages, float p,
                       int32_t* kept, int32_t* kept_count, float* tau, void* ws,
                       hipStream_t s) {
  const int n_slots = cand_stride_pages * kPage;
  const int spt = (n_slots + kToppThreads - 1) / kToppThreads;
  float* st = static_cast<float*>(stage_scratch(ws, L));
  if (spt <= 1) topp_launch<1>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  else if (spt <= 2) topp_launch<2>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  else if (spt <= 4) topp_launch<4>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  else if (spt <= 8) topp_launch<8>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  else if (spt <= 16) topp_launch<16>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  else if (spt <= 32) topp_launch<32>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  else topp_launch<64>(L, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau, st, s);
  return hipGetLastError();
}

}  // namespace twl
