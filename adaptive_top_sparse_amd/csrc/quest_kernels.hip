// Quest page selection, the page-level top-k stage that Twilight prunes further (Twilight
// pages, atlas.scime.ai summary: "Approach" names Quest as a base selector, "Surprising
// findings" its per-page max-pooled key layout).
//
// score(page) = sum_h sum_c max(q_hc * lo_c, q_hc * hi_c) over the KV head's G query heads.
// Regrouped per channel: score = sum_c (lo_c * A_c + hi_c * B_c) with
// A_c = sum of the group's negative q_hc and B_c = sum of the non-negative ones, which is
// the same real number. Every fp16 x fp16 product is a multiple of 2^-48 and the regrouped
// terms are partial sums of those products, so as long as the page's terms stay within
// 2^53 of their finest step (always true for finite fp16 data of ordinary range) each fp64
// FMA and add is exact, whatever the order. Exact scores make ties real ties; they are
// broken by the lower page index.
#include "twl_device.h"
#include "twl_launch.h"

TWL_PHASE_STORAGE(quest)
TWL_SPAN_STORAGE(quest)

namespace twl {
namespace {

#ifndef TWL_SCORE_THREADS
#define TWL_SCORE_THREADS 256
#endif
#ifndef TWL_SCORE_ROUNDS
#define TWL_SCORE_ROUNDS 4
#endif
constexpr int kScoreThreads = TWL_SCORE_THREADS;
constexpr int kScoreRounds = TWL_SCORE_ROUNDS;

// Lanes per page = D/8 (each lane owns 8 channels = 16 B of lo and 16 B of hi). A block
// covers kScoreThreads/LPP consecutive logical pages per round, kScoreRounds rounds, read
// as one contiguous stretch of the KV head's bounds; all rounds' loads are issued before
// any arithmetic, so each lane has 2 * rounds loads in flight.
template <int D>
constexpr int score_pages_per_block() {
  return kScoreThreads / (D / 8) * kScoreRounds;
}

template <int D>
__global__ __launch_bounds__(kScoreThreads) void quest_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ minmax,
    const int32_t* __restrict__ seq_lens, int Hq, int Hkv, int max_pages,
    double* __restrict__ scores) {
  constexpr int LPP = D / 8;
  constexpr int PPI = kScoreThreads / LPP;  // pages per round
  constexpr int ROUNDS = kScoreRounds;
  constexpr int PPB = PPI * ROUNDS;
  TWL_PHASE(0);
  TWL_SPAN_BEGIN();
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int G = Hq / Hkv;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int P = (n + kPage - 1) / kPage;
  const int p0 = blockIdx.x * PPB;
  if (p0 >= P) return;
  const int sub = threadIdx.x % LPP;
  const int c0 = sub * 8;
  // this KV head's bounds, in logical page order
  const uint16_t* unit_mm = minmax + (static_cast<long>(b) * Hkv + g) * max_pages * 2 * D;
  u32x4 lo[ROUNDS], hi[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = p0 + r * PPI + threadIdx.x / LPP;
    if (p < P) {
      const uint16_t* blk = unit_mm + static_cast<long>(p) * 2 * D + c0;
      lo[r] = *reinterpret_cast<const u32x4*>(blk);
      hi[r] = *reinterpret_cast<const u32x4*>(blk + D);
    } else {
      lo[r] = u32x4{0u, 0u, 0u, 0u};
      hi[r] = u32x4{0u, 0u, 0u, 0u};
    }
  }
  double A[8], Bc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    A[c] = 0.0;
    Bc[c] = 0.0;
  }
  for (int h = 0; h < G; ++h) {
    const u32x4 qv =
        *reinterpret_cast<const u32x4*>(q + (static_cast<long>(b) * Hq + g * G + h) * D + c0);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const uint16_t bits = static_cast<uint16_t>((qv[c / 2] >> (16 * (c % 2))) & 0xffffu);
      const double x = static_cast<double>(h2f(bits));
      if (x < 0.0) A[c] += x; else Bc[c] += x;
    }
  }
  TWL_PHASE(1);
  double* out = scores + (static_cast<long>(b) * Hkv + g) * max_pages;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    double acc = 0.0;
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int sh = 16 * (c % 2);
      const double l = static_cast<double>(h2f(static_cast<uint16_t>((lo[r][c / 2] >> sh) & 0xffffu)));
      const double u = static_cast<double>(h2f(static_cast<uint16_t>((hi[r][c / 2] >> sh) & 0xffffu)));
      acc = fma(l, A[c], acc);
      acc = fma(u, Bc[c], acc);
    }
#pragma unroll
    for (int o = LPP / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    const int p = p0 + r * PPI + threadIdx.x / LPP;
    if (sub == 0 && p < P) out[p] = acc;
  }
  TWL_PHASE(2);
  TWL_SPAN_END();
}

// One 1024-thread block per (sequence, KV head); thread t owns pages [t*KPT, t*KPT+KPT).
// Radix select over order-preserving 64-bit keys of the exact scores: the bits the keys
// all share are skipped (block min/max), then 11-bit digits are examined from the top,
// stopping as soon as the boundary bucket is taken whole or holds at most 64 pages (one
// wave then ranks those by score, then page index, and the last one taken becomes a
// (score, page) threshold); more than 64 exact ties go to the lower page indices by a
// block scan. A block scan then compacts the chosen pages in page order.
template <int KPT>
__global__ __launch_bounds__(1024) void quest_select_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv,
    int max_pages, int budget, int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_count) {
  constexpr int NT = 1024;
  constexpr int kBins = 2 * NT;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_lds[NT / kWave + 1];
  __shared__ uint64_t red64[NT / kWave], red64b[NT / kWave];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t n_short;
  __shared__ uint64_t short_key[kWave + 1];
  __shared__ int short_page[kWave + 1];
  TWL_PHASE(4);
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int P = (n + kPage - 1) / kPage;
  const int m = min(budget, P);
  const long unit = static_cast<long>(b) * Hkv + g;
  int32_t* out = sel_pages + unit * budget;
  if (threadIdx.x == 0) sel_count[unit] = m;
  if (m == P) {
    for (int i = threadIdx.x; i < P; i += NT) out[i] = i;
    return;
  }
  const double* sc = scores + unit * max_pages;
  const int first = threadIdx.x * KPT;
  uint64_t key[KPT];
  uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = first + i;
    key[i] = p < P ? f64_order_key(sc[p]) : 0ull;
    if (p < P) {
      kmin = key[i] < kmin ? key[i] : kmin;
      kmax = key[i] > kmax ? key[i] : kmax;
    }
  }
  TWL_PHASE(5);
  block_minmax<NT, uint64_t>(kmin, kmax, red64, red64b, ~0ull, 0ull, &kmin, &kmax);
  TWL_PHASE(6);

  // bits above `top` are common to every key
  uint64_t prefix = 0, mask = 0;
  uint32_t rem = static_cast<uint32_t>(m);
  // how the boundary is decided: kTies = the first `rem` keys equal to the final prefix in
  // page order; kAllIn = every key equal to the prefix; kPair = (key, page) >= (t_key, t_page)
  // in the selection order (key descending, then page ascending)
  enum { kTies, kAllIn, kPair } mode = kTies;
  uint64_t t_key = 0;
  int t_page = 0;
  if (kmin == kmax) {
    // every score ties: the first m pages
    mode = kPair;
    t_key = kmax;
    t_page = m - 1;
  } else {
    int top = 63 - __clzll(kmin ^ kmax);
    mask = top == 63 ? 0ull : ~((2ull << top) - 1ull);
    prefix = kmax & mask;
    if (threadIdx.x == 0) n_short = 0u;
    int npass = 0;
    for (;;) {
      const int lo_bit = top >= 10 ? top - 10 : 0;
      const int nbits = top - lo_bit + 1;
      const uint64_t dmask = (1ull << nbits) - 1ull;
      hist[threadIdx.x] = 0;
      hist[threadIdx.x + NT] = 0;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (first + i < P && (key[i] & mask) == prefix)
          atomicAdd(&hist[(key[i] >> lo_bit) & dmask], 1u);
      }
      __syncthreads();
      uint32_t above, cnt;
      const uint32_t digit = block_pick_bucket<NT, uint32_t>(
          hist[2 * threadIdx.x], hist[2 * threadIdx.x + 1], rem, scan_lds, pick, &above, &cnt);
      rem -= above;
      prefix |= static_cast<uint64_t>(digit) << lo_bit;
      mask |= dmask << lo_bit;
      TWL_PHASE(7 + (npass < 4 ? npass : 4));
      ++npass;
      if (cnt == rem) {
        mode = kAllIn;
        break;
      }
      if (cnt <= static_cast<uint32_t>(kWave)) {
        // short boundary bucket: one wave ranks its pages in the selection order and the
        // rem-th becomes the threshold pair
#pragma unroll
        for (int i = 0; i < KPT; ++i) {
          if (first + i < P && (key[i] & mask) == prefix) {
            const uint32_t idx = atomicAdd(&n_short, 1u);
            if (idx < static_cast<uint32_t>(kWave)) {  // always: idx < cnt <= 64
              short_key[idx] = key[i];
              short_page[idx] = first + i;
            }
          }
        }
        TWL_PHASE(14);
        __syncthreads();
        TWL_PHASE(15);
        if (threadIdx.x < kWave) {
          // lane l holds page l of the bucket; the loop broadcasts each with readlane
          const int l = threadIdx.x;
          const int n_in = __builtin_amdgcn_readfirstlane(static_cast<int>(cnt));
          const bool live = l < n_in;
          const uint64_t mk = live ? short_key[l] : 0ull;
          const int mp = live ? short_page[l] : 0;
          uint32_t rank = 0;
          for (int j = 0; j < n_in; ++j) {
            const uint64_t kj = readlane(mk, j);
            const int pj = readlane(mp, j);
            rank += (kj > mk || (kj == mk && pj < mp)) ? 1u : 0u;
          }
          if (live && rank == rem - 1) {
            short_key[kWave] = mk;
            short_page[kWave] = mp;
          }
        }
        TWL_PHASE(16);
        __syncthreads();
        TWL_PHASE(17);
        mode = kPair;
        t_key = short_key[kWave];
        t_page = short_page[kWave];
        break;
      }
      if (lo_bit == 0) break;
      top = lo_bit - 1;
    }
  }

  // pages strictly above the boundary prefix are in; of the pages equal to it, the first
  // `rem` in page order are in (all of them unless exact ties remain)
  uint32_t tot;
  uint32_t eq_before = 0;
  if (mode == kTies) {
    uint32_t n_eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      n_eq += (first + i < P && (key[i] & mask) == prefix) ? 1u : 0u;
    eq_before = block_excl_scan_u32<NT>(n_eq, scan_lds, &tot);
  }
  bool chosen[KPT];
  uint32_t n_sel = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    bool c = false;
    if (first + i < P) {
      if (mode == kPair) {
        c = key[i] > t_key || (key[i] == t_key && first + i <= t_page);
      } else {
        const uint64_t km = key[i] & mask;
        if (km > prefix) {
          c = true;
        } else if (km == prefix) {
          c = mode == kAllIn || eq_before < rem;
          ++eq_before;
        }
      }
    }
    chosen[i] = c;
    n_sel += c ? 1u : 0u;
  }
  uint32_t pos = block_excl_scan_u32<NT>(n_sel, scan_lds, &tot);
  TWL_PHASE(12);
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (chosen[i]) out[pos++] = first + i;
  TWL_PHASE(13);
}

template <int KPT>
void select_launch(const Layout& L, int budget, int32_t* sel_pages, int32_t* sel_count,
                   const double* scores, hipStream_t s) {
  quest_select_kernel<KPT><<<dim3(L.Hkv, L.B), 1024, 0, s>>>(scores, L.seq_lens, L.Hkv,
                                                             L.max_pages, budget, sel_pages,
                                                             sel_count);
}

}  // namespace

size_t quest_workspace_bytes(const Layout& L) {
  return align_up(static_cast<size_t>(L.B) * L.Hkv * L.max_pages * sizeof(double), 256);
}

hipError_t launch_quest_select(const Layout& L, const void* q, const void* minmax, int budget,
                               int32_t* sel_pages, int32_t* sel_count, void* ws, hipStream_t s) {
  double* scores = static_cast<double*>(stage_scratch(ws, L));
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* mm = static_cast<const uint16_t*>(minmax);
  if (L.d == 128) {
    constexpr int ppb = score_pages_per_block<128>();
    const dim3 grid((L.max_pages + ppb - 1) / ppb, L.Hkv, L.B);
    quest_score_kernel<128><<<grid, kScoreThreads, 0, s>>>(qq, mm, L.seq_lens, L.Hq, L.Hkv,
                                                           L.max_pages, scores);
  } else {
    constexpr int ppb = score_pages_per_block<64>();
    const dim3 grid((L.max_pages + ppb - 1) / ppb, L.Hkv, L.B);
    quest_score_kernel<64><<<grid, kScoreThreads, 0, s>>>(qq, mm, L.seq_lens, L.Hq, L.Hkv,
                                                          L.max_pages, scores);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int kpt_needed = (L.max_pages + 1023) / 1024;
  if (kpt_needed <= 1) select_launch<1>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt_needed <= 2) select_launch<2>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt_needed <= 4) select_launch<4>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt_needed <= 8) select_launch<8>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt_needed <= 16) select_launch<16>(L, budget, sel_pages, sel_count, scores, s);
  else select_launch<32>(L, budget, sel_pages, sel_count, scores, s);
  return hipGetLastError();
}

}  // namespace twl
