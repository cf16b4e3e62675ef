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
#include <type_traits>

#include "twl_device.h"
#include "twl_launch.h"

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
typedef double f64x2 __attribute__((ext_vector_type(2)));

// Row stride of the score workspace: max_pages rounded up to a multiple of 64.
__host__ __device__ inline long score_row_stride(int max_pages) {
  return (static_cast<long>(max_pages) + 63) / 64 * 64;
}

template <int D>
constexpr int score_pages_per_block() {
  return kScoreThreads / (D / 8) * kScoreRounds;
}

// Sum of one value per round over the LPP lanes of a page, for 4 rounds at once: two
// exchanges halve the values per lane (each lane keeping the rounds its bits select), then
// a butterfly finishes. The partners differ by lane-index masks (LPP-1, LPP/2-1, then 2, 1
// for LPP = 16, or 7, 2, 1 for LPP = 8) that span the page's lanes, so every lane ends with
// the total of round round_of_lane(); fp64 adds of exact partial sums are exact in any
// order.
template <int LPP>
__device__ __forceinline__ double reduce_rounds4(const double (&v)[4]) {
  constexpr int kA = LPP == 16 ? kRowMirror : kRowHalfMirror;   // flips bit log2(LPP) - 1
  constexpr int kB = LPP == 16 ? kRowHalfMirror : kQuadXor2;    // flips bit log2(LPP) - 2
  const int lane = lane_id();
  const bool ba = (lane & (LPP / 2)) != 0;
  const bool bb = (lane & (LPP / 4)) != 0;
  double h[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const double keep = ba ? v[2 * i + 1] : v[2 * i];
    const double send = ba ? v[2 * i] : v[2 * i + 1];
    h[i] = keep + dpp_any<kA>(send);
  }
  const double keep = bb ? h[1] : h[0];
  const double send = bb ? h[0] : h[1];
  double x = keep + dpp_any<kB>(send);
  if constexpr (LPP == 16) x += dpp_any<kQuadXor2>(x);
  x += dpp_any<kQuadXor1>(x);
  return x;
}

// Round whose total reduce_rounds4 leaves in this lane, and whether the lane writes it.
template <int LPP>
__device__ __forceinline__ int round_of_lane() {
  const int lane = lane_id();
  return ((lane & (LPP / 2)) != 0 ? 1 : 0) + ((lane & (LPP / 4)) != 0 ? 2 : 0);
}
template <int LPP>
__device__ __forceinline__ bool writes_round() {
  return (lane_id() & (LPP / 4 - 1)) == 0;
}

template <int D, int G>
__global__ __launch_bounds__(kScoreThreads) void quest_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ minmax,
    const int32_t* __restrict__ seq_lens, int Hkv, int max_pages,
    double* __restrict__ scores) {
  constexpr int LPP = D / 8;
  constexpr int PPI = kScoreThreads / LPP;  // pages per round
  constexpr int ROUNDS = kScoreRounds;
  constexpr int PPB = PPI * ROUNDS;
  static_assert(ROUNDS == 4, "the round reduction handles four rounds");
  const int b = blockIdx.z;
  const int bx = blockIdx.x, by = blockIdx.y;
  const int g = by;
  const int Hq = Hkv * G;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int P = (n + kPage - 1) / kPage;
  const int p0 = bx * PPB;
  if (p0 >= P) return;
  const int sub = threadIdx.x % LPP;
  const int c0 = sub * 8;
  // this KV head's bounds, in logical page order; pages past the sequence load page p0
  // (so that no load sits behind a branch) and are not written
  const uint16_t* unit_mm = minmax + (static_cast<long>(b) * Hkv + g) * max_pages * 2 * D;
  // The bounds are read once per step: non-temporal loads (measured 8.4 -> 7.7 us at the
  // 128k GQA layer and 122 -> 116 us at the B = 32 ragged batch).
  u32x4 lo[ROUNDS], hi[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int p = p0 + r * PPI + threadIdx.x / LPP;
    const uint16_t* blk = unit_mm + static_cast<long>(p < P ? p : p0) * 2 * D + c0;
    lo[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk));
    hi[r] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(blk + D));
  }
  // A_c / B_c: sums of the group's negative / non-negative q_hc, formed once per block
  // (while the bounds are in flight) and read back per lane. Sums of at most 8 fp16 values
  // are exact in fp64.
  __shared__ double sA[D], sB[D];
  if (threadIdx.x < D) {
    const uint16_t* qh = q + (static_cast<long>(b) * Hq + g * G) * D + threadIdx.x;
    double a = 0.0, bsum = 0.0;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const double x = static_cast<double>(h2f(qh[h * D]));
      a += fmin(x, 0.0);
      bsum += fmax(x, 0.0);
    }
    sA[threadIdx.x] = a;
    sB[threadIdx.x] = bsum;
  }
  __syncthreads();
  double A[8], Bc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    A[c] = sA[c0 + c];
    Bc[c] = sB[c0 + c];
  }
  double part[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    double acc_lo = 0.0, acc_hi = 0.0;  // two chains per round
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int sh = 16 * (c % 2);
      const double l = static_cast<double>(h2f(static_cast<uint16_t>((lo[r][c / 2] >> sh) & 0xffffu)));
      const double u = static_cast<double>(h2f(static_cast<uint16_t>((hi[r][c / 2] >> sh) & 0xffffu)));
      acc_lo = fma(l, A[c], acc_lo);
      acc_hi = fma(u, Bc[c], acc_hi);
    }
    part[r] = acc_lo + acc_hi;
  }
  const double total = reduce_rounds4<LPP>(part);
  const int p = p0 + round_of_lane<LPP>() * PPI + threadIdx.x / LPP;
  if (writes_round<LPP>() && p < P)
    scores[(static_cast<long>(b) * Hkv + g) * score_row_stride(max_pages) + p] = total;
}

// One 1024-thread block per (sequence, KV head); thread t owns pages [t*KPT, t*KPT+KPT).
// Radix select over order-preserving 64-bit keys of the exact scores: the bits the keys
// all share are skipped (block min/max), then 11-bit digits are examined from the top,
// stopping as soon as the boundary bucket is taken whole or holds at most 64 pages (one
// wave then ranks those by score, then page index, and the last one taken becomes a
// (score, page) threshold); more than 64 exact ties go to the lower page indices by a
// block scan. A block scan then compacts the chosen pages in page order.
template <int NT, int KPT>
__global__ __launch_bounds__(NT) void quest_select_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv,
    int max_pages, int budget, int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_count) {
  constexpr int kBins = 2048;
  constexpr int BPT = kBins / NT;
  constexpr int NW = NT / kWave;
  // digit histogram, digit d at hist[d]; after a pass has picked its digit
  // it doubles as scratch for the short-bucket finish
  __shared__ __attribute__((aligned(16))) uint32_t hist[kBins];
  __shared__ uint32_t scan_lds[NT / kWave + 1];
  __shared__ uint64_t red64[NT / kWave], red64b[NT / kWave];
  __shared__ uint32_t pick[3];
  __shared__ uint32_t n_short;
  __shared__ uint64_t short_key[kWave + 1];
  __shared__ int short_page[kWave + 1];
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const long unit = static_cast<long>(b) * Hkv + g;
  const double* sc = scores + unit * score_row_stride(max_pages);
  const int first = threadIdx.x * KPT;
  // The scores are requested before the sequence length is known (bounded by the row, whose
  // stride is even and at least max_pages), and the length comes on the vector path, so the
  // two round trips overlap; pages past the sequence are masked below.
  const int n_lane = load_uniform_vec(seq_lens + b);
  constexpr int VW = KPT < 2 ? 1 : 2;  // pairs of scores in 16-byte loads
  double sv[KPT];
#pragma unroll
  for (int i = 0; i < KPT; i += VW) {
    const int pl = first + i < max_pages ? first + i : 0;
    if constexpr (VW == 2) {
      const f64x2 v = *reinterpret_cast<const f64x2*>(sc + pl);
      sv[i] = v[0];
      sv[i + 1] = v[1];
    } else {
      sv[i] = sc[pl];
    }
  }
  const int nv = __builtin_amdgcn_readfirstlane(n_lane);
  const int n = nv < 0 ? 0 : (nv > max_pages * kPage ? max_pages * kPage : nv);
  const int P = (n + kPage - 1) / kPage;
  const int m = min(budget, P);
  int32_t* out = sel_pages + unit * budget;
  if (threadIdx.x == 0) sel_count[unit] = m;
  if (m == P) {
    for (int i = threadIdx.x; i < P; i += NT) out[i] = i;
    return;
  }
  // the first pass's histogram is cleared now; the barrier of the min/max reduction below
  // orders these stores before its atomics
#pragma unroll
  for (int i = 0; i < BPT; ++i) hist[i * NT + threadIdx.x] = 0;
  // pages past the sequence get key 0, below every score's key, so they never raise kmax
  // (selects rather than branches: the loop stays straight-line code)
  uint64_t key[KPT];
  uint64_t kmin = ~0ull, kmax = 0ull;
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const bool ok = first + i < P;
    const uint64_t k = f64_order_key(sv[i]);
    key[i] = ok ? k : 0ull;
    const uint64_t kl = ok ? k : ~0ull;
    kmin = kl < kmin ? kl : kmin;
    kmax = key[i] > kmax ? key[i] : kmax;
  }
  block_minmax<NT, uint64_t>(kmin, kmax, red64, red64b, ~0ull, 0ull, &kmin, &kmax);

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
      if (npass > 0) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) hist[i * NT + threadIdx.x] = 0;
        __syncthreads();
      }
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        if (first + i < P && (key[i] & mask) == prefix)
          atomicAdd(&hist[static_cast<uint32_t>((key[i] >> lo_bit) & dmask)], 1u);
      }
      __syncthreads();
      uint32_t above, cnt;
      const uint32_t digit = block_pick_bucket_lds<NT, BPT, uint32_t>(hist, rem, scan_lds, pick,
                                                                      &above, &cnt);
      rem -= above;
      prefix |= static_cast<uint64_t>(digit) << lo_bit;
      mask |= dmask << lo_bit;
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
        __syncthreads();
        {
          // page i = lane; wave w counts the bucket's pages in its share that come before
          // page i in the selection order, then wave 0 totals the shares
          constexpr int JPW = kWave / NW;
          uint32_t* part = hist;  // free until the next pass clears it
          const int l = lane_id();
          const int wv = threadIdx.x / kWave;
          const int n_in = static_cast<int>(cnt);
          const bool live = l < n_in;
          const uint64_t mk = live ? short_key[l] : 0ull;
          const int mp = live ? short_page[l] : 0;
          uint32_t r_part = 0;
#pragma unroll
          for (int q = 0; q < JPW; ++q) {
            const int j = wv * JPW + q;
            const int jj = j < kWave ? j : 0;
            const uint64_t kj = short_key[jj];
            const int pj = short_page[jj];
            r_part += (j < n_in && (kj > mk || (kj == mk && pj < mp))) ? 1u : 0u;
          }
          part[wv * kWave + l] = r_part;
          __syncthreads();
          if (wv == 0) {
            uint32_t rank = 0;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) rank += part[w2 * kWave + l];
            if (live && rank == rem - 1) {
              short_key[kWave] = mk;
              short_page[kWave] = mp;
            }
          }
        }
        __syncthreads();
        mode = kPair;
        t_key = short_key[kWave];
        t_page = short_page[kWave];
        break;
      }
      if (lo_bit == 0) break;
      top = lo_bit - 1;
    }
  }

  // Pages strictly above the boundary prefix are in; of the pages equal to it, the first
  // `rem` in page order are in (all of them unless exact ties remain). When all of them
  // are in, that is key >= prefix (the bits below the mask are free), one pair test.
  if (mode == kAllIn) {
    mode = kPair;
    t_key = prefix;
    t_page = P;
  }
  uint32_t tot;
  bool chosen[KPT];
  uint32_t n_sel = 0;
  if (mode == kPair) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int pg = first + i;
      chosen[i] = (pg < P) & ((key[i] > t_key) | ((key[i] == t_key) & (pg <= t_page)));
      n_sel += chosen[i] ? 1u : 0u;
    }
  } else {
    uint32_t n_eq = 0;
#pragma unroll
    for (int i = 0; i < KPT; ++i)
      n_eq += (first + i < P && (key[i] & mask) == prefix) ? 1u : 0u;
    uint32_t eq_before = block_excl_scan_u32<NT>(n_eq, scan_lds, &tot);
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      bool c = false;
      if (first + i < P) {
        const uint64_t km = key[i] & mask;
        if (km > prefix) {
          c = true;
        } else if (km == prefix) {
          c = eq_before < rem;
          ++eq_before;
        }
      }
      chosen[i] = c;
      n_sel += c ? 1u : 0u;
    }
  }
  uint32_t pos = block_excl_scan_u32<NT>(n_sel, scan_lds, &tot);
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (chosen[i]) out[pos++] = first + i;
}

template <int NT, int KPT>
void select_launch(const Layout& L, int budget, int32_t* sel_pages, int32_t* sel_count,
                   const double* scores, hipStream_t s) {
  quest_select_kernel<NT, KPT><<<dim3(L.Hkv, L.B), NT, 0, s>>>(scores, L.seq_lens, L.Hkv,
                                                               L.max_pages, budget, sel_pages,
                                                               sel_count);
}

}  // namespace

size_t quest_workspace_bytes(const Layout& L) {
  return align_up(static_cast<size_t>(L.B) * L.Hkv * score_row_stride(L.max_pages) * sizeof(double),
                  256);
}

long quest_score_stride(int max_pages) { return score_row_stride(max_pages); }

hipError_t launch_quest_scores(const Layout& L, const void* q, const void* minmax, double* scores,
                               hipStream_t s) {
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* mm = static_cast<const uint16_t*>(minmax);
  auto score = [&](auto d_tag, auto g_tag) {
    constexpr int D = decltype(d_tag)::value;
    constexpr int G = decltype(g_tag)::value;
    constexpr int ppb = score_pages_per_block<D>();
    const dim3 grid((L.max_pages + ppb - 1) / ppb, L.Hkv, L.B);
    quest_score_kernel<D, G><<<grid, kScoreThreads, 0, s>>>(qq, mm, L.seq_lens, L.Hkv,
                                                            L.max_pages, scores);
  };
  auto score_d = [&](auto d_tag) {
    switch (L.G()) {
      case 1: score(d_tag, std::integral_constant<int, 1>()); break;
      case 2: score(d_tag, std::integral_constant<int, 2>()); break;
      case 4: score(d_tag, std::integral_constant<int, 4>()); break;
      default: score(d_tag, std::integral_constant<int, 8>()); break;
    }
  };
  if (L.d == 128) score_d(std::integral_constant<int, 128>());
  else score_d(std::integral_constant<int, 64>());
  return hipGetLastError();
}

hipError_t launch_quest_top(const Layout& L, const double* scores, int budget,
                            int32_t* sel_pages, int32_t* sel_count, hipStream_t s) {
  // up to 2048 pages per sequence: 512-thread blocks, four to a CU, so a large batch of
  // units selects in one round (13.5 -> 10.4 us on the B = 32 ragged MHA step)
  if (L.max_pages <= 2048) {
    const int k5 = (L.max_pages + 511) / 512;
    if (k5 <= 1) select_launch<512, 1>(L, budget, sel_pages, sel_count, scores, s);
    else if (k5 <= 2) select_launch<512, 2>(L, budget, sel_pages, sel_count, scores, s);
    else select_launch<512, 4>(L, budget, sel_pages, sel_count, scores, s);
    return hipGetLastError();
  }
  const int kpt = (L.max_pages + 1023) / 1024;
  if (kpt <= 1) select_launch<1024, 1>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt <= 2) select_launch<1024, 2>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt <= 4) select_launch<1024, 4>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt <= 8) select_launch<1024, 8>(L, budget, sel_pages, sel_count, scores, s);
  else if (kpt <= 16) select_launch<1024, 16>(L, budget, sel_pages, sel_count, scores, s);
  else select_launch<1024, 32>(L, budget, sel_pages, sel_count, scores, s);
  return hipGetLastError();
}

hipError_t launch_quest_select(const Layout& L, const void* q, const void* minmax, int budget,
                               int32_t* sel_pages, int32_t* sel_count, void* ws, hipStream_t s) {
  double* scores = static_cast<double*>(stage_scratch(ws, L));
  const hipError_t e = launch_quest_scores(L, q, minmax, scores, s);
  if (e != hipSuccess) return e;
  return launch_quest_top(L, scores, budget, sel_pages, sel_count, s);
}

}  // namespace twl
