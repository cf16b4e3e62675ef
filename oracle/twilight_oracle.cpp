// Twilight hierarchical top-p sparse decode: the CPU oracle.
//
// TEST INFRASTRUCTURE ONLY. This file is the plain, slow, obviously correct reference that
// the HIP path is checked against. Only the test suite, the smoke check and the CPU
// baseline leg of the benchmark may load it. It shares no code, header, table or helper
// with the GPU library, and the product path never calls it.
//
// Everything is computed per (sequence, KV head) unit on plain logical arrays, in fp64,
// with exact integer arithmetic wherever a decision (a code, a page choice) must be
// bit-exact. fp16 values travel as their IEEE binary16 bit patterns (uint16_t).
//
// Sources (the Twilight pages):
//  * atlas.scime.ai summary, "Approach": a base sparse-attention method pre-selects
//    tokens, then top-p (nucleus) thresholding of their estimated attention weights
//    prunes them; the estimate uses a 4-bit quantized key cache.
//  * atlas.scime.ai summary, "Surprising findings": Quest's per-page max pooling makes
//    plain top-p unworkable there, so top-p runs as a second, token-level stage after the
//    page-level top-k ("hierarchical").
//  * atlas.scime.ai summary, "Limitations": under GQA the budget is per KV-head group.
//  * The quantizer (per token, group of 32 channels, scale = (max-min)/15, zero = min,
//    round to nearest) and the Quest page bound (per-page channelwise min/max) are the
//    workload definitions that accompany the pages; every point the pages leave open is a
//    reading listed in the design notes and repeated at the function that takes it.
//
// Parity pins: every function below is checked by the CPU tests against something other
// than itself (brute force, closed forms, invariants, an independent numpy formulation).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <numeric>
#include <vector>

namespace {

// ---- binary16 <-> exact values ------------------------------------------------------

// Exact value of a finite binary16 number.
double h2d(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  double v;
  if (e == 0) {
    v = std::ldexp(static_cast<double>(m), -24);
  } else {
    v = std::ldexp(static_cast<double>(1024 + m), e - 25);
  }
  return sign ? -v : v;
}

// Exact value of a finite binary16 number as an integer count of 2^-24.
int64_t h2units(uint16_t h) {
  const int sign = (h >> 15) & 1;
  const int e = (h >> 10) & 0x1f;
  const int m = h & 0x3ff;
  int64_t u;
  if (e == 0) {
    u = m;
  } else {
    u = static_cast<int64_t>(1024 + m) << (e - 1);
  }
  return sign ? -u : u;
}

bool h_is_finite(uint16_t h) { return ((h >> 10) & 0x1f) != 0x1f; }

// The binary16 value nearest to num/den for num >= 0, den > 0, ties to the even
// significand (round-to-nearest-even). Exact: with num a multiple of 2^-24 below 2^18
// and den <= 15, both num and den*h are exactly representable doubles, and so are
// their differences. Searches the non-negative finite bit patterns, which are ordered
// like their values.
uint16_t nearest_h_of_ratio(double num, int den) {
  // largest pattern h with den*h <= num
  int lo = 0, hi = 0x7bff;  // 0x7bff = 65504, the largest finite
  if (den * h2d(0x7bff) <= num) return 0x7bff;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (den * h2d(static_cast<uint16_t>(mid)) <= num) lo = mid; else hi = mid - 1;
  }
  const uint16_t a = static_cast<uint16_t>(lo);
  const uint16_t b = static_cast<uint16_t>(lo + 1);
  const double da = num - den * h2d(a);
  const double db = den * h2d(b) - num;
  if (da < db) return a;
  if (db < da) return b;
  return (a & 1) ? b : a;  // tie: even significand
}

// ---- exact 128-bit helpers ------------------------------------------------------------

using i128 = __int128;

double i128_to_double(i128 x) { return static_cast<double>(x); }

int trailing_zeros_u128(unsigned __int128 x) {
  int n = 0;
  while (x != 0 && (x & 1) == 0) { x >>= 1; ++n; }
  return n;
}

}  // namespace

extern "C" {

// Oracle ABI version, bumped when a function's contract changes.
int orc_version() { return 2; }

// ---- c1: key quantizer (4-bit, and the 2-bit variant the pages ablate) ------------------
// Per token and per group of 32 consecutive channels, with L = 2^bits - 1 levels above
// zero: zero = min, scale = the binary16 value nearest (ties to even) to (max - min)/L,
// code_c = the c in 0..L whose dequantized value zero + c*scale is nearest to x_c (ties to
// the even code), and every code is 0 when scale is 0. Nearest-code is the same as
// clamp(round((x-zero)/scale), 0, L) with half-to-even rounding, written as a brute-force
// search over the L + 1 codes. The 2-bit form (atlas.scime.ai ablation table: 4-bit is
// preferred over 2-bit for the estimate's stability) keeps the same group of 32 channels.
// k: [n_tokens, d] binary16; codes: [n_tokens, d] one code per byte;
// scale, zero: [n_tokens, d/32] binary16. Returns 0, or -1 on bad input.
int orc_quantize_keys_bits(const uint16_t* k, int64_t n_tokens, int d, int bits,
                           uint8_t* codes, uint16_t* scale, uint16_t* zero) {
  if (d <= 0 || d % 32 != 0 || n_tokens < 0 || (bits != 2 && bits != 4)) return -1;
  const int levels = (1 << bits) - 1;
  const int ng = d / 32;
  for (int64_t t = 0; t < n_tokens; ++t) {
    for (int g = 0; g < ng; ++g) {
      const uint16_t* x = k + t * d + g * 32;
      double mn = h2d(x[0]), mx = h2d(x[0]);
      uint16_t mn_bits = x[0];
      for (int c = 0; c < 32; ++c) {
        if (!h_is_finite(x[c])) return -1;
        const double v = h2d(x[c]);
        if (v < mn) { mn = v; mn_bits = x[c]; }
        if (v > mx) mx = v;
      }
      // -0.0 and +0.0 are both the minimum value 0; store the bit pattern that occurred.
      const uint16_t s_bits = nearest_h_of_ratio(mx - mn, levels);
      const double s = h2d(s_bits);
      scale[t * ng + g] = s_bits;
      zero[t * ng + g] = mn_bits;
      for (int c = 0; c < 32; ++c) {
        uint8_t best = 0;
        if (s > 0.0) {
          const double xv = h2d(x[c]);
          double best_err = -1.0;
          for (int code = 0; code <= levels; ++code) {
            const double err = std::fabs((xv - mn) - code * s);  // exact
            if (best_err < 0.0 || err < best_err ||
                (err == best_err && (code % 2 == 0) && (best % 2 == 1))) {
              best_err = err;
              best = static_cast<uint8_t>(code);
            }
          }
        }
        codes[t * d + g * 32 + c] = best;
      }
    }
  }
  return 0;
}

// The 4-bit quantizer of the estimate (atlas.scime.ai "Approach": a 4-bit key cache).
int orc_quantize_keys(const uint16_t* k, int64_t n_tokens, int d, uint8_t* codes,
                      uint16_t* scale, uint16_t* zero) {
  return orc_quantize_keys_bits(k, n_tokens, d, 4, codes, scale, zero);
}

// ---- c2: Quest per-page channelwise key bounds ----------------------------------------
// For each page of page_size tokens, lo_c / hi_c are the minimum / maximum of channel c
// over the page's valid tokens (a partial last page uses only the tokens that exist).
// k: [n_tokens, d]; lo, hi: [ceil(n/page_size), d] binary16.
int orc_page_bounds(const uint16_t* k, int64_t n_tokens, int d, int page_size,
                    uint16_t* lo, uint16_t* hi) {
  if (d <= 0 || page_size <= 0 || n_tokens < 0) return -1;
  const int64_t P = (n_tokens + page_size - 1) / page_size;
  for (int64_t p = 0; p < P; ++p) {
    const int64_t t0 = p * page_size;
    const int64_t t1 = std::min<int64_t>(n_tokens, t0 + page_size);
    for (int c = 0; c < d; ++c) {
      uint16_t bl = k[t0 * d + c], bh = k[t0 * d + c];
      for (int64_t t = t0; t < t1; ++t) {
        const uint16_t x = k[t * d + c];
        if (h2d(x) < h2d(bl)) bl = x;
        if (h2d(x) > h2d(bh)) bh = x;
      }
      lo[p * d + c] = bl;
      hi[p * d + c] = bh;
    }
  }
  return 0;
}

// ---- c3: Quest page selection ---------------------------------------------------------
// score(page) = sum over the group's G query heads h and channels c of
// max(q_hc * lo_c, q_hc * hi_c): for each head, the largest value q_h . k can take over
// the page's bounding box, summed over the heads that share the KV head. Computed exactly
// as an integer count of 2^-48. Pages are ranked by (score descending, page index
// ascending); the first min(budget, P) are kept and written in ascending page order.
// q: [G, d]; lo, hi: [P, d]; sel: [min(budget, P)]; scores_out: [P] (nearest double of
// the exact score) or NULL. *n_order_sensitive counts pages whose score an fp64 sum could
// round in some order: the terms are multiples of 2^g and the sum of their magnitudes is
// at least 2^(g+53). Returns the number of pages kept, or -1.
int orc_quest_select(const uint16_t* q, int G, int d, const uint16_t* lo, const uint16_t* hi,
                     int64_t P, int budget, int32_t* sel, double* scores_out,
                     int64_t* n_order_sensitive) {
  if (G <= 0 || d <= 0 || P < 0 || budget <= 0) return -1;
  std::vector<i128> score(static_cast<size_t>(P));
  int64_t sensitive = 0;
  for (int64_t p = 0; p < P; ++p) {
    i128 s = 0;
    unsigned __int128 abs_sum = 0;
    int finest = 1 << 30;
    for (int h = 0; h < G; ++h) {
      for (int c = 0; c < d; ++c) {
        const i128 qv = h2units(q[h * d + c]);
        const i128 a = qv * h2units(lo[p * d + c]);
        const i128 b = qv * h2units(hi[p * d + c]);
        const i128 term = a > b ? a : b;
        s += term;
        const unsigned __int128 mag = term < 0 ? static_cast<unsigned __int128>(-term)
                                               : static_cast<unsigned __int128>(term);
        abs_sum += mag;
        if (mag != 0) finest = std::min(finest, trailing_zeros_u128(mag));
      }
    }
    score[p] = s;
    if (abs_sum != 0 && (abs_sum >> finest) >= (static_cast<unsigned __int128>(1) << 53))
      ++sensitive;
    if (scores_out) scores_out[p] = std::ldexp(i128_to_double(s), -48);
  }
  std::vector<int64_t> order(static_cast<size_t>(P));
  std::iota(order.begin(), order.end(), 0);
  std::sort(order.begin(), order.end(), [&](int64_t a, int64_t b) {
    if (score[a] != score[b]) return score[a] > score[b];
    return a < b;
  });
  const int64_t m = std::min<int64_t>(budget, P);
  std::vector<int64_t> kept(order.begin(), order.begin() + m);
  std::sort(kept.begin(), kept.end());
  for (int64_t i = 0; i < m; ++i) sel[i] = static_cast<int32_t>(kept[i]);
  if (n_order_sensitive) *n_order_sensitive = sensitive;
  return static_cast<int>(m);
}

// ---- c4: estimated attention weights from the int4 key cache --------------------------
// Candidate slot j = (rank r of the page in cand_pages) * page_size + offset; its token
// is cand_pages[r]*page_size + offset (or j itself when cand_pages is NULL: every token
// is a candidate). A slot is valid when r < n_cand_pages and the token < n_tokens.
// For each head h: s_hj = sm_scale * sum_c q_hc * (zero + code_c * scale) over the token's
// dequantized key; w_h = softmax of s_h over the valid slots; invalid slots get 0.
// Reading: the softmax temperature is the attention scale sm_scale, and the softmax
// normalizes over the candidates only.
// q: [G, d]; codes: [n_tokens, d]; scale, zero: [n_tokens, d/32]; w: [G, n_slots].
int orc_estimate_weights(const uint16_t* q, int G, int d, const uint8_t* codes,
                         const uint16_t* scale, const uint16_t* zero, int64_t n_tokens,
                         const int32_t* cand_pages, int64_t n_cand_pages, int page_size,
                         float sm_scale, double* w, int64_t n_slots) {
  if (G <= 0 || d <= 0 || d % 32 != 0 || page_size <= 0 || n_slots < 0) return -1;
  const int ng = d / 32;
  std::vector<int64_t> token(static_cast<size_t>(n_slots), -1);
  for (int64_t j = 0; j < n_slots; ++j) {
    int64_t t = -1;
    if (cand_pages == nullptr) {
      t = j;
    } else {
      const int64_t r = j / page_size;
      if (r < n_cand_pages) t = static_cast<int64_t>(cand_pages[r]) * page_size + j % page_size;
    }
    if (t >= 0 && t < n_tokens) token[j] = t;
  }
  for (int h = 0; h < G; ++h) {
    std::vector<double> s(static_cast<size_t>(n_slots), 0.0);
    double mx = -INFINITY;
    for (int64_t j = 0; j < n_slots; ++j) {
      const int64_t t = token[j];
      if (t < 0) continue;
      double acc = 0.0;
      for (int c = 0; c < d; ++c) {
        const double kq = h2d(zero[t * ng + c / 32]) +
                          codes[t * d + c] * h2d(scale[t * ng + c / 32]);
        acc += h2d(q[h * d + c]) * kq;
      }
      s[j] = static_cast<double>(sm_scale) * acc;
      mx = std::max(mx, s[j]);
    }
    double sum = 0.0;
    for (int64_t j = 0; j < n_slots; ++j)
      if (token[j] >= 0) sum += std::exp(s[j] - mx);
    for (int64_t j = 0; j < n_slots; ++j)
      w[h * n_slots + j] = token[j] >= 0 ? std::exp(s[j] - mx) / sum : 0.0;
  }
  return 0;
}

// ---- c5 + c6: top-p threshold (minimal nucleus) and compaction ------------------------
// W_j = (1/G) * sum_h w_hj (the group's budget is shared: one kept set per KV head).
// Valid slots are sorted by (W descending, slot ascending) and accumulated in that order
// until the running mass reaches p * sum_j W_j; that prefix is the smallest set with at
// least that mass. For p >= 1 every valid slot is kept, whatever its W: top-p at p = 1
// prunes nothing (the estimate's softmax weights are all positive in exact arithmetic, so
// this is also the nucleus of the full mass; an underflowed weight does not drop its
// token). tau is the smallest kept W. The kept slots are mapped to logical token ids as in orc_estimate_weights and
// written in ascending order (compaction).
// w: [G, n_slots]; valid: [n_slots] 0/1; kept: [n_slots]. Returns the kept count or -1.
int64_t orc_topp_select(const double* w, const uint8_t* valid, int G, int64_t n_slots,
                        float p, const int32_t* cand_pages, int64_t n_cand_pages,
                        int page_size, int32_t* kept, double* tau) {
  if (G <= 0 || n_slots < 0 || !(p > 0.0f) || page_size <= 0) return -1;
  std::vector<double> W(static_cast<size_t>(n_slots), 0.0);
  std::vector<int64_t> idx;
  double total = 0.0;
  for (int64_t j = 0; j < n_slots; ++j) {
    if (!valid[j]) continue;
    double acc = 0.0;
    for (int h = 0; h < G; ++h) acc += w[h * n_slots + j];
    W[j] = acc / G;
    idx.push_back(j);
    total += W[j];
  }
  std::sort(idx.begin(), idx.end(), [&](int64_t a, int64_t b) {
    if (W[a] != W[b]) return W[a] > W[b];
    return a < b;
  });
  std::vector<int64_t> chosen;
  if (p >= 1.0f) {
    chosen = idx;
  } else {
    const double target = static_cast<double>(p) * total;
    double run = 0.0;
    for (int64_t j : idx) {
      if (run >= target) break;
      chosen.push_back(j);
      run += W[j];
    }
  }
  double t = 0.0;
  if (!chosen.empty()) t = W[chosen.back()];
  if (tau) *tau = t;
  std::vector<int64_t> toks;
  for (int64_t j : chosen) {
    if (cand_pages == nullptr) {
      toks.push_back(j);
    } else {
      toks.push_back(static_cast<int64_t>(cand_pages[j / page_size]) * page_size +
                     j % page_size);
    }
  }
  std::sort(toks.begin(), toks.end());
  for (size_t i = 0; i < toks.size(); ++i) kept[i] = static_cast<int32_t>(toks[i]);
  (void)n_cand_pages;
  return static_cast<int64_t>(toks.size());
}

// ---- c7: attention over the kept tokens -----------------------------------------------
// For each head h: o_h = sum_{j in kept} e^{s_j - m} v_j / sum_{j in kept} e^{s_j - m},
// with s_j = sm_scale * q_h . k_j on the fp16 keys (not the int4 estimate) and m the
// largest s_j; an empty kept set gives o_h = 0.
// q: [G, d]; k, v: [n_tokens, d]; kept: [n_kept] token ids; out: [G, d].
int orc_sparse_attention(const uint16_t* q, int G, int d, const uint16_t* k,
                         const uint16_t* v, int64_t n_tokens, const int32_t* kept,
                         int64_t n_kept, float sm_scale, double* out) {
  if (G <= 0 || d <= 0 || n_kept < 0) return -1;
  for (int64_t i = 0; i < n_kept; ++i)
    if (kept[i] < 0 || kept[i] >= n_tokens) return -1;
  for (int h = 0; h < G; ++h) {
    double* o = out + static_cast<int64_t>(h) * d;
    for (int c = 0; c < d; ++c) o[c] = 0.0;
    if (n_kept == 0) continue;
    std::vector<double> s(static_cast<size_t>(n_kept));
    double mx = -INFINITY;
    for (int64_t i = 0; i < n_kept; ++i) {
      const int64_t t = kept[i];
      double acc = 0.0;
      for (int c = 0; c < d; ++c) acc += h2d(q[h * d + c]) * h2d(k[t * d + c]);
      s[i] = static_cast<double>(sm_scale) * acc;
      mx = std::max(mx, s[i]);
    }
    double denom = 0.0;
    for (int64_t i = 0; i < n_kept; ++i) {
      const double e = std::exp(s[i] - mx);
      denom += e;
      const int64_t t = kept[i];
      for (int c = 0; c < d; ++c) o[c] += e * h2d(v[t * d + c]);
    }
    for (int c = 0; c < d; ++c) o[c] /= denom;
  }
  return 0;
}

// Exact binary16 value of a bit pattern (lets tests check the decoder itself).
double orc_half_to_double(uint16_t h) { return h2d(h); }

// Nearest binary16 (ties to even) of num/den (lets tests check the encoder itself).
uint16_t orc_nearest_half_of_ratio(double num, int den) { return nearest_h_of_ratio(num, den); }

}  // extern "C"
