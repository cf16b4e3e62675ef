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

namespace twl {
namespace {

constexpr int kScorePagesPerBlock = 64;

// Lanes per page = D/8 (each lane owns 8 channels = 16 B of lo and 16 B of hi).
template <int D>
__global__ __launch_bounds__(256) void quest_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ minmax,
    const int32_t* __restrict__ page_table, const int32_t* __restrict__ seq_lens, int Hq,
    int Hkv, int max_pages, int num_phys, double* __restrict__ scores) {
  constexpr int LPP = D / 8;
  constexpr int PPI = 256 / LPP;  // pages per block iteration
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int G = Hq / Hkv;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int P = (n + kPage - 1) / kPage;
  const int p0 = blockIdx.x * kScorePagesPerBlock;
  if (p0 >= P) return;
  const int sub = threadIdx.x % LPP;
  const int c0 = sub * 8;

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

  double* out = scores + (static_cast<long>(b) * Hkv + g) * max_pages;
  const int p_end = min(P, p0 + kScorePagesPerBlock);
  // the LPP lanes of a page group share p and trip count, so the shuffles stay in-group
  for (int p = p0 + threadIdx.x / LPP; p < p_end; p += PPI) {
    double acc = 0.0;
    const int phys = page_table[static_cast<long>(b) * max_pages + p];
    if (phys_ok(phys, num_phys)) {
      const uint16_t* blk = minmax + (static_cast<long>(phys) * Hkv + g) * 2 * D + c0;
      const u32x4 lo = *reinterpret_cast<const u32x4*>(blk);
      const u32x4 hi = *reinterpret_cast<const u32x4*>(blk + D);
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const int sh = 16 * (c % 2);
        const double l = static_cast<double>(h2f(static_cast<uint16_t>((lo[c / 2] >> sh) & 0xffffu)));
        const double u = static_cast<double>(h2f(static_cast<uint16_t>((hi[c / 2] >> sh) & 0xffffu)));
        acc = fma(l, A[c], acc);
        acc = fma(u, Bc[c], acc);
      }
    }
#pragma unroll
    for (int o = LPP / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (sub == 0) out[p] = acc;
  }
}

// One 1024-thread block per (sequence, KV head). Thread t owns pages [t*KPT, t*KPT+KPT).
// Radix select over order-preserving 64-bit keys of the exact scores, 8 bits per pass from
// the top, stopping as soon as the boundary digit's bucket is taken whole; remaining exact
// ties are resolved by page index. Then a block scan compacts the chosen pages in order.
template <int KPT>
__global__ __launch_bounds__(1024) void quest_select_kernel(
    const double* __restrict__ scores, const int32_t* __restrict__ seq_lens, int Hkv,
    int max_pages, int budget, int32_t* __restrict__ sel_pages, int32_t* __restrict__ sel_count) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_lds[1024 / kWave + 1];
  __shared__ uint32_t pick[3];
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int P = (n + kPage - 1) / kPage;
  const int m = min(budget, P);
  const long unit = static_cast<long>(b) * Hkv + g;
  int32_t* out = sel_pages + unit * budget;
  if (threadIdx.x == 0) sel_count[unit] = m;
  if (m == P) {
    for (int i = threadIdx.x; i < P; i += blockDim.x) out[i] = i;
    return;
  }
  const double* sc = scores + unit * max_pages;
  const int first = threadIdx.x * KPT;
  uint64_t key[KPT];
#pragma unroll
  for (int i = 0; i < KPT; ++i) {
    const int p = first + i;
    key[i] = p < P ? f64_order_key(sc[p]) : 0ull;
  }

  uint64_t prefix = 0, mask = 0;
  uint32_t rem = static_cast<uint32_t>(m);
  for (int shift = 56; shift >= 0; shift -= 8) {
    if (threadIdx.x < 256) hist[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      if (first + i < P && (key[i] & mask) == prefix)
        atomicAdd(&hist[(key[i] >> shift) & 0xff], 1u);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // lane l holds digits 4l..4l+3; count of keys with a larger digit than each
      const int l = threadIdx.x;
      uint32_t c[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = hist[4 * l + j];
      const uint32_t mine = c[0] + c[1] + c[2] + c[3];
      // suffix sum over lanes > l
      uint32_t incl = mine;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t w = __shfl_down(incl, o);
        if (l + o < 64) incl += w;
      }
      uint32_t above = incl - mine;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < rem && rem <= above + c[j]) {
          pick[0] = static_cast<uint32_t>(4 * l + j);
          pick[1] = above;
          pick[2] = c[j];
        }
        above += c[j];
      }
    }
    __syncthreads();
    const uint32_t digit = pick[0], above = pick[1], cnt = pick[2];
    __syncthreads();
    rem -= above;
    prefix |= static_cast<uint64_t>(digit) << shift;
    mask |= 0xffull << shift;
    if (cnt == rem) break;
  }

  // pages strictly above the boundary prefix are in; of the pages equal to it, the first
  // `rem` in page order are in
  uint32_t n_eq = 0;
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    n_eq += (first + i < P && (key[i] & mask) == prefix) ? 1u : 0u;
  uint32_t tot;
  uint32_t eq_before = block_excl_scan_u32<1024>(n_eq, scan_lds, &tot);
  bool chosen[KPT];
  uint32_t n_sel = 0;
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
  uint32_t pos = block_excl_scan_u32<1024>(n_sel, scan_lds, &tot);
#pragma unroll
  for (int i = 0; i < KPT; ++i)
    if (chosen[i]) out[pos++] = first + i;
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
  double* scores = static_cast<double*>(ws);
  const dim3 grid((L.max_pages + kScorePagesPerBlock - 1) / kScorePagesPerBlock, L.Hkv, L.B);
  const auto* qq = static_cast<const uint16_t*>(q);
  const auto* mm = static_cast<const uint16_t*>(minmax);
  if (L.d == 128) {
    quest_score_kernel<128><<<grid, 256, 0, s>>>(qq, mm, L.page_table, L.seq_lens, L.Hq, L.Hkv,
                                                 L.max_pages, L.num_phys, scores);
  } else {
    quest_score_kernel<64><<<grid, 256, 0, s>>>(qq, mm, L.page_table, L.seq_lens, L.Hq, L.Hkv,
                                                L.max_pages, L.num_phys, scores);
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
