// Top-p (nucleus) pruning of the candidates and compaction of the kept tokens (Twilight
// pages, atlas.scime.ai summary: "Approach" for top-p thresholding of the estimated weights
// with binary-search top-p kernels, "Limitations" for the group-wise budget under GQA).
//
// The search for tau runs on chip, one block per (sequence, KV head) (1024 threads; 512 for
// units of up to 4096 slots):
//  * W_j = mean over the group's heads of the weights (fp32, fixed head order).
//  * Masses are exact integers: M_j = floor(W_j * 2^(40 - e)), e the binary exponent of the
//    unit's largest W, so every sum is independent of order and the result is
//    deterministic. The truncation costs less than 2^-40 of max W per slot.
//  * tau is the largest fp32 value with sum_{W_j >= tau} M_j >= ceil(p * sum_j M_j). The
//    search narrows the range of fp32 bit patterns (monotone for W >= 0) with 2048-bucket
//    mass histograms, instead of halving it once per pass: a 31-bit range closes in at
//    most three passes. The range starts at the smallest key of nonzero mass (lighter
//    weights add nothing and cannot hold tau), so a pass tests each key with one unsigned
//    comparison and adds its mass with one LDS atomic. As soon as the boundary bucket
//    holds at most 64 weights, they are gathered and one wave finishes the search.
//  * W is read from memory once and stays resident for every pass: up to 32 values per
//    lane in VGPRs, the rest (units above 32768 slots) in LDS.
//  * Kept = {W_j >= tau} (tau > 0), compacted in slot order (per-wave scans, then one
//    exchange of wave totals), which is ascending token order because candidate pages are
//    ascending. p = 1 keeps every valid slot, whatever its W.
// When the group is large relative to the unit (G * slots-per-thread above 32, what one
// block's registers take), a wide pass first forms W over many work-groups into the
// workspace, so that the per-unit block does not stream G rows of weights through one CU.
#include <type_traits>

#include "twl_device.h"
#include "twl_launch.h"

namespace twl {
namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kBins = 2048;
constexpr int kMeanThreads = 256;
constexpr int kMeanSlots = kMeanThreads * 16;  // slots per work-group of the group-mean pass

// Per block size: W vectors per lane held in VGPRs (the rest live in LDS) and the largest
// G * slots-per-thread read straight from the weights (a 1024-thread block has 128 VGPRs
// per lane, a 512-thread block, with units of at most 4096 slots, needs no more).
template <int NT>
struct ToppShape {
  static constexpr int kWaves = NT / kWave;
  static constexpr int kRegVecs = 8;
  static constexpr int kDirectLoads = 32;
  static constexpr int kRegBatch = 4;  // vectors whose loads go out together
  static constexpr int kBpt = kBins / NT;              // histogram buckets per thread
};

// floor(W * 2^(40 - e)) for a non-negative fp32 W given by its bits, e the binary exponent
// of the unit's largest W (W < 2^(e+1), so the result is below 2^41). Subnormal W (a tiny
// share of any sum) counts as 0. x = W * 2^(40-e) is exact in fp32 (a power-of-two
// scaling); its integer part above 2^32 converts exactly, and x minus that part is again
// exact in fp32 (it keeps at most x's 24 significant bits), so two truncating conversions
// give floor(x) with no 64-bit shifts.
__device__ __forceinline__ uint64_t fixed_mass_normal(uint32_t key, int e) {
  const float x = ldexpf(__uint_as_float(key), 40 - e);
  const uint32_t hi = static_cast<uint32_t>(x * 0x1p-32f);
  const uint32_t lo = static_cast<uint32_t>(fmaf(-static_cast<float>(hi), 0x1p32f, x));
  return (static_cast<uint64_t>(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t fixed_mass(uint32_t key, int e) {
  return (key >> 23) == 0 ? 0ull : fixed_mass_normal(key, e);
}

template <int VW>
__device__ __forceinline__ void load_vec(const float* p, float (&x)[VW]) {
  if constexpr (VW == 4) {
    const f32x4 t = *reinterpret_cast<const f32x4*>(p);
    x[0] = t[0];
    x[1] = t[1];
    x[2] = t[2];
    x[3] = t[3];
  } else if constexpr (VW == 2) {
    const f32x2 t = *reinterpret_cast<const f32x2*>(p);
    x[0] = t[0];
    x[1] = t[1];
  } else {
    x[0] = *p;
  }
}

// Page id behind slot s0, loaded unconditionally so that loads can be issued before any is
// used (and before the candidate count is known): entry 0 stands in when the slot's page
// rank is past the row's `bound` entries. Ranks past the candidate count read entries that
// page_token rejects.
__device__ __forceinline__ int page_id_of(const int32_t* cand_row, int bound, int s0) {
  if (cand_row == nullptr) return 0;
  const int r = s0 / kPage;
  return cand_row[r < bound ? r : 0];
}

// Logical token of slot s0 (s0 a multiple of 4 or less, so its vector stays in one page)
// given its page id from page_id_of, or -1 when the slot's page is not a candidate. Tokens
// past seq_len are filtered by the caller.
__device__ __forceinline__ int page_token(const int32_t* cand_row, int cnt, int max_pages,
                                          int s0, int pid) {
  if (cand_row == nullptr) return s0;
  if (s0 / kPage >= cnt || pid < 0 || pid >= max_pages) return -1;
  return pid * kPage + s0 % kPage;
}

// Marks a vector whose first token is not known yet (tokens are >= -1).
constexpr int kNoToken = -2;

// Candidate pages in the row of unit `unit` (0 without a page list).
__device__ __forceinline__ int candidate_pages(const int32_t* cand_pages,
                                               const int32_t* cand_count, long unit,
                                               int cand_stride_pages, int n) {
  if (cand_pages == nullptr) return 0;
  int cnt = cand_count ? cand_count[unit] : (n + kPage - 1) / kPage;
  return cnt < cand_stride_pages ? cnt : cand_stride_pages;
}

// Group mean of the weights on candidate slots (0 elsewhere), for units whose block would
// otherwise read G rows alone. Work-group (chunk, g, b) covers kMeanSlots slots; each
// thread four vectors of four, contiguous across the work-group.
template <int G>
__global__ __launch_bounds__(kMeanThreads) void topp_mean_kernel(
    const float* __restrict__ weights, const int32_t* __restrict__ cand_pages,
    const int32_t* __restrict__ cand_count, int cand_stride_pages,
    const int32_t* __restrict__ seq_lens, int Hkv, int max_pages, float* __restrict__ stage,
    const float2* __restrict__ norm, int norm_chunks) {
  __shared__ float s_norm[2][G];
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const long unit = static_cast<long>(b) * Hkv + g;
  // with norm given, weights hold logits: each head's max and 1 / (sum of exp2) first, by
  // the same wave merge as the estimate's normalising pass
  float nM[G], nL[G];
  if (norm != nullptr) {
    for (int h = threadIdx.x / kWave; h < G; h += kMeanThreads / kWave) {
      const float2 ml = merge_max_sum_wave(norm + (unit * G + h) * norm_chunks, norm_chunks);
      if (lane_id() == 0) {
        s_norm[0][h] = ml.x;
        s_norm[1][h] = softmax_inv_sum(ml.y);  // once per head, not per thread
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      nM[h] = s_norm[0][h];
      nL[h] = s_norm[1][h];
    }
  }
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int n_slots = cand_stride_pages * kPage;
  const int32_t* cand_row = cand_pages ? cand_pages + unit * cand_stride_pages : nullptr;
  const int cnt = candidate_pages(cand_pages, cand_count, unit, cand_stride_pages, n);
  const float* row0 = weights + unit * G * n_slots;
  const float inv_g = 1.0f / static_cast<float>(G);  // exact: G is a power of two
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int s0 = blockIdx.x * kMeanSlots + v * (kMeanThreads * 4) + threadIdx.x * 4;
    const bool in_row = s0 < n_slots;
    const int sl = in_row ? s0 : 0;  // loads stay unconditional (and in bounds)
    float x[G][4];
#pragma unroll
    for (int h = 0; h < G; ++h) load_vec<4>(row0 + static_cast<long>(h) * n_slots + sl, x[h]);
    if (norm != nullptr) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) x[h][j] = softmax_weight(x[h][j], nM[h], nL[h]);
    }
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += x[h][j];
    const int t0 = page_token(cand_row, cnt, max_pages, sl, page_id_of(cand_row, cnt, sl));
    f32x4 w;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (t0 >= 0 && t0 + j < n) ? fmaxf(acc[j] * inv_g, 0.f) : 0.f;
    if (in_row) *reinterpret_cast<f32x4*>(stage + unit * n_slots + s0) = w;
  }
}

// Slot layout of a unit inside its block: wave w owns SPT*64 consecutive slots from
// w*SPT*64; its vector v covers 64*VW consecutive slots, lane l holding VW of them from
// v*64*VW + l*VW. Loads are contiguous across the wave, and slot order is
// (wave, vector, lane, element), which the compaction keeps.
template <int NT, int SPT>
struct SlotMap {
  static constexpr int VW = SPT < 4 ? SPT : 4;
  static constexpr int NV = SPT / VW;
  static constexpr int NR = NV < ToppShape<NT>::kRegVecs ? NV : ToppShape<NT>::kRegVecs;
  static constexpr int NL = NV - NR;  // vectors in LDS (VW == 4)
};

// `src` holds G rows of n_slots values per unit: the estimate's weights, or (G == 1) the
// group means formed by topp_mean_kernel, which are already 0 off the candidates. With
// `norm` given, src holds the estimate's logits instead and norm its per-chunk (max, sum of
// exp) pairs, norm_chunks per query head; the kernel then normalises each head's logits
// itself, with the same arithmetic as the estimate's normalising pass, so the weights it
// sees are bit-identical and that pass (a launch and a round trip of the weights) is saved.
template <int NT, int G, int SPT>
__global__ __launch_bounds__(NT) void topp_kernel(
    const float* __restrict__ src, const int32_t* __restrict__ cand_pages,
    const int32_t* __restrict__ cand_count, int cand_stride_pages,
    const int32_t* __restrict__ seq_lens, int units, int cand_div, int max_pages, float p,
    int32_t* __restrict__ kept, int32_t* __restrict__ kept_count,
    float* __restrict__ tau_out, const float2* __restrict__ norm, int norm_chunks) {
  using M = SlotMap<NT, SPT>;
  using S = ToppShape<NT>;
  constexpr int VW = M::VW, NR = M::NR, NL = M::NL;
  constexpr int NW = S::kWaves, BPT = S::kBpt;
  static_assert(NL == 0 || VW == 4, "LDS-resident vectors are four wide");
  // the mass histogram, bucket b at mass[b]; after a pass has picked its bucket it doubles
  // as scratch for the short-bucket finish
  __shared__ __attribute__((aligned(16))) uint64_t mass[kBins];
  __shared__ f32x4 w_lds[NL > 0 ? NL * NT : 1];
  __shared__ uint32_t red_a[NW], red_b[NW], wave_tot[NW];
  __shared__ uint64_t red64[NW];
  __shared__ uint64_t pick[3];
  __shared__ uint32_t n_short[2], short_keys[kWave + 1];
  __shared__ float s_norm[2][G];
  const int b = blockIdx.y;
  const int g = blockIdx.x;
  const long unit = static_cast<long>(b) * units + g;
  // a head-wise unit (one query head) reads its KV head's candidates: cand_div = G
  const long cunit = unit / cand_div;
  const int n_slots = cand_stride_pages * kPage;
  const int32_t* cand_row = cand_pages ? cand_pages + cunit * cand_stride_pages : nullptr;
  // the sequence length and candidate count come on the vector path and are made scalar
  // where the first batch is formed, so that neither holds up the weight loads (the page-id
  // loads are bounded by the row's stride, not by the count)
  const int n_lane = load_uniform_vec(seq_lens + b);
  const int cnt_lane = load_uniform_vec(cand_count != nullptr ? cand_count + cunit : seq_lens + b);
  int n = 0, cnt = 0;
  auto resolve_counts = [&]() {
    const int nv = __builtin_amdgcn_readfirstlane(n_lane);
    n = nv < 0 ? 0 : (nv > max_pages * kPage ? max_pages * kPage : nv);
    const int cv = __builtin_amdgcn_readfirstlane(cnt_lane);
    const int c = cand_count != nullptr ? cv : (n + kPage - 1) / kPage;
    cnt = cand_pages == nullptr ? 0 : (c < cand_stride_pages ? c : cand_stride_pages);
  };
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int wbase = wv * SPT * kWave;
  const float* row0 = src + unit * G * n_slots;
  const float inv_g = 1.0f / static_cast<float>(G);  // exact: G is a power of two
  // the first pass's histogram is cleared now; the barrier of the min/max reduction that
  // ends pass 0 orders these stores before its atomics
#pragma unroll
  for (int i = 0; i < BPT; ++i) mass[i * NT + threadIdx.x] = 0ull;
  if (threadIdx.x == 0) n_short[0] = 0u;

  // pass 0: W = mean of the group's weights on candidate slots (0 elsewhere). A batch of
  // vectors first issues all its loads (weights and page ids), then forms W; n_slots is a
  // multiple of 16, so a vector that starts inside the row ends inside it, and vectors past
  // the row load slot 0 instead, so that no load sits behind a branch.
  float W[NR][VW];
  // token of each register vector's first slot (-1: not a candidate), kept while it costs
  // few registers; wider shapes look the tokens up again when compacting
  constexpr bool kKeepT0 = SPT <= 16;
  int T0[NR];
  uint32_t kmax = 0, kmin = 0xffffffffu;
  // each head's max and 1 / (sum of exp2) when normalising here: wave h merges head h's
  // chunks
  float nM[G], nL[G];
  auto norm_stats = [&]() {
    for (int h = wv; h < G; h += NW) {
      const float2 ml = merge_max_sum_wave(norm + (unit * G + h) * norm_chunks, norm_chunks);
      if (lane == 0) {
        s_norm[0][h] = ml.x;
        s_norm[1][h] = softmax_inv_sum(ml.y);  // once per head, not per thread
      }
    }
    __syncthreads();
#pragma unroll
    for (int h = 0; h < G; ++h) {
      nM[h] = s_norm[0][h];
      nL[h] = s_norm[1][h];
    }
  };
  // a batch of NB vectors: all loads (weights and page ids) first, then W
  auto load_batch = [&](int v0, auto& x, auto& pid) {
    constexpr int NB = sizeof(pid) / sizeof(pid[0]);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s0 = wbase + (v0 + i) * kWave * VW + lane * VW;
      const int sl = s0 < n_slots ? s0 : 0;
#pragma unroll
      for (int h = 0; h < G; ++h)
        load_vec<VW>(row0 + static_cast<long>(h) * n_slots + sl, x[i][h]);
      pid[i] = page_id_of(cand_row, cand_stride_pages, sl);
    }
  };
  auto finish_batch = [&](int v0, auto& x, auto& pid, float (*dst)[VW], int* t0_out) {
    constexpr int NB = sizeof(pid) / sizeof(pid[0]);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s0 = wbase + (v0 + i) * kWave * VW + lane * VW;
      const int t0 = s0 < n_slots ? page_token(cand_row, cnt, max_pages, s0, pid[i]) : -1;
      if (t0_out != nullptr) t0_out[i] = t0;
      if (norm != nullptr) {
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int j = 0; j < VW; ++j) x[i][h][j] = softmax_weight(x[i][h][j], nM[h], nL[h]);
      }
#pragma unroll
      for (int j = 0; j < VW; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < G; ++h) acc += x[i][h][j];
        // a slot off the candidates holds -1 (never kept); a candidate holds its mean
        // weight, +0 when that is not positive (so p = 1 can keep it all the same)
        const float mw = acc * inv_g;
        const float w = (t0 >= 0 && t0 + j < n) ? (mw > 0.f ? mw : 0.f) : -1.0f;
        dst[i][j] = w;
        const uint32_t k = __float_as_uint(w);
        if (w > 0.f) {
          kmax = k > kmax ? k : kmax;
          kmin = k < kmin ? k : kmin;
        }
      }
    }
  };
  if constexpr (NL > 0) {
    if (norm != nullptr) norm_stats();
    constexpr int kBatch = 4;
    static_assert(NL % kBatch == 0, "LDS vectors come in batches of four");
#pragma unroll 1
    for (int v = 0; v < NL; v += kBatch) {
      float x[kBatch][G][VW];
      int pid[kBatch];
      float w[kBatch][VW];
      load_batch(NR + v, x, pid);
      if (v == 0) resolve_counts();
      finish_batch(NR + v, x, pid, w, nullptr);
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        w_lds[(v + i) * NT + threadIdx.x] =
            f32x4{w[i][0], w[i][1 % VW], w[i][2 % VW], w[i][3 % VW]};
    }
  }
  // register vectors in batches, which bounds the loads held in flight; when normalising
  // here with no LDS vectors, the first batch's loads go out before the heads' statistics
  // are merged, so the two latencies overlap
  constexpr int kRegBatch = NR < S::kRegBatch ? NR : S::kRegBatch;
#pragma unroll
  for (int v = 0; v < NR; v += kRegBatch) {
    float x[kRegBatch][G][VW];
    int pid[kRegBatch];
    load_batch(v, x, pid);
    if (NL == 0 && v == 0 && norm != nullptr) norm_stats();
    if (NL == 0 && v == 0) resolve_counts();
    finish_batch(v, x, pid, W + v, kKeepT0 ? T0 + v : nullptr);
  }
  block_minmax<NT, uint32_t>(kmin, kmax, red_a, red_b, 0xffffffffu, 0u, &kmin, &kmax);

  // f(v, w) for every vector v of this lane's resident W, in vector order
  auto for_each_w = [&](auto&& f) {
#pragma unroll
    for (int v = 0; v < NR; ++v) f(v, W[v]);
    if constexpr (NL > 0) {
#pragma unroll 2
      for (int v = 0; v < NL; ++v) {
        const f32x4 t = w_lds[v * NT + threadIdx.x];
        float w[VW];
#pragma unroll
        for (int j = 0; j < VW; ++j) w[j] = t[j];
        f(NR + v, w);
      }
    }
  };

  // p = 1 keeps every candidate, whatever its weight (an fp32 weight may underflow to 0);
  // otherwise the kept set is {W >= tau} with tau > 0
  const bool keep_all = p >= 1.0f;
  float tau = 0.f;
  if (keep_all) {
    tau = kmax != 0 ? __uint_as_float(kmin) : 0.f;
  } else if (kmax != 0) {
    // fixed-point masses relative to the largest weight's binade
    const int e = static_cast<int>((kmax >> 23) & 0xff) - 127;
    // the first pass covers every W of nonzero mass, so its scan yields the total mass and
    // the target ceil(p * total). Keys below kz (W < 2^(e - 40), subnormals included) have
    // mass 0 at this resolution: they add nothing and cannot hold tau (the target is at
    // least 1), so the search range starts at kz and every key inside it has mass >= 1.
    const uint32_t kz = e + 87 > 0 ? static_cast<uint32_t>(e + 87) << 23 : 0x00800000u;
    uint64_t rem = 0;
    uint32_t lo = kmin > kz ? kmin : kz, hi = kmax;
    int pass_no = 0;
    for (;;) {
      const uint32_t range = hi - lo;
      const int bits = range == 0 ? 0 : 32 - __clz(range);
      const int shift = bits > 11 ? bits - 11 : 0;
      if (pass_no > 0) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) mass[i * NT + threadIdx.x] = 0ull;
        if (threadIdx.x == 0) n_short[pass_no & 1] = 0u;
        __syncthreads();
      }
      for_each_w([&](int, const float(&w)[VW]) {
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          // k in [lo, hi] as one unsigned comparison of its offset
          const uint32_t k = __float_as_uint(w[j]);
          const uint32_t d = k - lo;
          if (d <= range) {
            atomicAdd(&mass[d >> shift], fixed_mass_normal(k, e));
          }
        }
        // keep the scheduler from forming every vector's 64-bit masses ahead of the
        // atomics (which would need two VGPRs per slot)
        __builtin_amdgcn_sched_barrier(0);
      });
      __syncthreads();
      uint64_t above, inb;
      const uint32_t bucket = block_pick_bucket_lds<NT, BPT, uint64_t>(
          mass, rem, red64, pick, &above, &inb, pass_no == 0 ? p : 0.f, &rem);
      rem -= above;
      const uint32_t nlo = lo + (bucket << shift);
      const uint32_t span = (1u << shift) - 1u;
      const uint32_t nhi = (hi - nlo) < span ? hi : nlo + span;
      lo = nlo;
      hi = nhi;
      if (shift == 0) break;
      {
        // No key of the bucket has a mass above fixed_mass(hi), so it holds at least
        // inb / fixed_mass(hi) keys; when that bound exceeds 64 the collection below would
        // come back too long, so the next pass starts at once. (fp64: inb < 2^57 rounds by
        // at most one part in 2^53, and 64.5 * mh is exact, so the test implies > 64 keys.)
        const uint64_t mh = fixed_mass(hi, e);
        if (mh != 0 && static_cast<double>(inb) > 64.5 * static_cast<double>(mh)) {
          ++pass_no;
          continue;
        }
      }
      // Short boundary bucket: collect its keys and let one wave finish the search.
      // tau is then the largest key whose mass together with every larger key of the
      // bucket reaches rem (0 < rem <= the bucket's mass, so one exists).
      const int par = pass_no & 1;
      const uint32_t brange = hi - lo;
      for_each_w([&](int, const float(&w)[VW]) {
#pragma unroll
        for (int j = 0; j < VW; ++j) {
          const uint32_t k = __float_as_uint(w[j]);
          if (k - lo <= brange) {
            const uint32_t idx = atomicAdd(&n_short[par], 1u);
            if (idx < kWave) short_keys[idx] = k;
          }
        }
      });
      __syncthreads();
      const uint32_t n_in = __builtin_amdgcn_readfirstlane(n_short[par]);
      ++pass_no;
      if (n_in > kWave) continue;
      {
        // element i = lane; wave w adds the masses of its share of the bucket's keys that
        // are >= key i, then wave 0 totals the shares
        constexpr int JPW = kWave / NW;
        uint64_t* part = mass;  // free until the next pass clears it
        const bool live = lane < static_cast<int>(n_in);
        const uint32_t my_key = live ? short_keys[lane] : 0u;
        uint64_t s_part = 0;
#pragma unroll
        for (int q = 0; q < JPW; ++q) {
          const int j = wv * JPW + q;
          const uint32_t kj = short_keys[j < kWave ? j : 0];
          s_part += (j < static_cast<int>(n_in) && kj >= my_key) ? fixed_mass(kj, e) : 0ull;
        }
        part[wv * kWave + lane] = s_part;
        __syncthreads();
        if (wv == 0) {
          uint64_t s_ge = 0;  // mass of the bucket's keys >= my_key
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) s_ge += part[w2 * kWave + lane];
          const uint32_t cand = (live && s_ge >= rem) ? my_key : 0u;
          const uint32_t best = wave_reduce(cand, OpMax());
          if (lane == 0) short_keys[kWave] = best;
        }
      }
      __syncthreads();
      lo = short_keys[kWave];
      break;
    }
    tau = __uint_as_float(lo);
  }

  // compaction in slot order: wave totals first, then per-vector wave scans
  // (tau > 0 below p = 1, so W >= tau already excludes W = 0 and the -1 of non-candidates;
  // with no positive W and p < 1 nothing is kept)
  const float thr = keep_all ? 0.f : (kmax != 0 ? tau : INFINITY);
  auto kept_w = [&](float w) { return w >= thr; };
  uint32_t nk = 0;
  for_each_w([&](int, const float(&w)[VW]) {
#pragma unroll
    for (int j = 0; j < VW; ++j) nk += kept_w(w[j]) ? 1u : 0u;
  });
  nk = wave_reduce(nk, OpSum());
  if (lane == 0) wave_tot[wv] = nk;
  __syncthreads();
  uint32_t run = 0, total = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const uint32_t c = wave_tot[i];
    run += i < wv ? c : 0u;
    total += c;
  }
  int32_t* out = kept + unit * n_slots;
  // register vectors reuse the tokens found while forming W; LDS vectors look them up
  auto emit = [&](int v, const float(&w)[VW], int t0_known) {
    uint32_t c = 0;
#pragma unroll
    for (int j = 0; j < VW; ++j) c += kept_w(w[j]) ? 1u : 0u;
    const uint32_t incl = wave_incl_scan(c);
    if (c != 0) {
      const int s0 = wbase + v * kWave * VW + lane * VW;
      const int t0 = t0_known != kNoToken
                         ? t0_known
                         : page_token(cand_row, cnt, max_pages, s0,
                                      page_id_of(cand_row, cand_stride_pages, s0));
      uint32_t pos = run + incl - c;
#pragma unroll
      for (int j = 0; j < VW; ++j)
        if (kept_w(w[j])) out[pos++] = t0 + j;
    }
    run += readlane(incl, kWave - 1);
  };
#pragma unroll
  for (int v = 0; v < NR; ++v) emit(v, W[v], kKeepT0 ? T0[v] : kNoToken);
  if constexpr (NL > 0) {
#pragma unroll 2
    for (int v = 0; v < NL; ++v) {
      const f32x4 t = w_lds[v * NT + threadIdx.x];
      float w[VW];
#pragma unroll
      for (int j = 0; j < VW; ++j) w[j] = t[j];
      emit(NR + v, w, kNoToken);
    }
  }
  if (threadIdx.x == 0) {
    kept_count[unit] = static_cast<int32_t>(total);
    if (tau_out) tau_out[unit] = tau;
  }
}

// Everything a launch needs besides the kernel's template arguments.
struct ToppArgs {
  const Layout* L;
  const float* weights;
  const int32_t* cand_pages;
  const int32_t* cand_count;
  int stride;
  float p;
  int32_t* kept;
  int32_t* kept_count;
  float* tau;
  float* stage;
  hipStream_t s;
  const float2* norm;  // non-null: weights hold logits, normalised in the top-p kernel
  int norm_chunks;
};

template <int NT, int G, int SPT>
void launch_main(const ToppArgs& a, const float* src) {
  topp_kernel<NT, G, SPT><<<dim3(a.L->units(), a.L->B), NT, 0, a.s>>>(
      src, a.cand_pages, a.cand_count, a.stride, a.L->seq_lens, a.L->units(),
      a.L->headwise ? a.L->G() : 1, a.L->max_pages, a.p, a.kept, a.kept_count, a.tau,
      src == a.weights ? a.norm : nullptr, a.norm_chunks);
}

template <int G>
void launch_mean(const ToppArgs& a) {
  const int n_slots = a.stride * kPage;
  const dim3 grid((n_slots + kMeanSlots - 1) / kMeanSlots, a.L->Hkv, a.L->B);
  topp_mean_kernel<G><<<grid, kMeanThreads, 0, a.s>>>(a.weights, a.cand_pages, a.cand_count,
                                                      a.stride, a.L->seq_lens, a.L->Hkv,
                                                      a.L->max_pages, a.stage, a.norm,
                                                      a.norm_chunks);
}

// Units of up to 4096 slots take 512-thread blocks: four fit a CU, so a large batch of
// small units runs in one round (estimate + top-p 90.2 -> 88.8 us on the B = 32 ragged MHA
// step, 4096 slots per unit).
int block_threads(int n_slots) { return n_slots <= 4096 ? 512 : 1024; }

int slots_per_thread(int n_slots) {
  const int nt = block_threads(n_slots);
  int spt = 1;
  while (spt * nt < n_slots) spt *= 2;
  return spt;
}

bool uses_mean_pass(int G, int n_slots) {
  const int direct = ToppShape<1024>::kDirectLoads;  // (the same for 512-thread blocks)
  return G > 1 && G * slots_per_thread(n_slots) > direct;
}

template <int NT, int SPT>
void launch_spt(const ToppArgs& a) {
  const int G = a.L->unit_G();
  if (uses_mean_pass(G, a.stride * kPage)) {
    if (G == 2) launch_mean<2>(a);
    else if (G == 4) launch_mean<4>(a);
    else launch_mean<8>(a);
    launch_main<NT, 1, SPT>(a, a.stage);
    return;
  }
  constexpr int kDirect = ToppShape<NT>::kDirectLoads;
  if (G == 1) {
    launch_main<NT, 1, SPT>(a, a.weights);
  } else if (G == 2) {
    if constexpr (2 * SPT <= kDirect) launch_main<NT, 2, SPT>(a, a.weights);
  } else if (G == 4) {
    if constexpr (4 * SPT <= kDirect) launch_main<NT, 4, SPT>(a, a.weights);
  } else {
    if constexpr (8 * SPT <= kDirect) launch_main<NT, 8, SPT>(a, a.weights);
  }
}

}  // namespace

size_t topp_workspace_bytes(const Layout& L, int cand_stride_pages) {
  const long n_slots = static_cast<long>(cand_stride_pages) * kPage;
  if (!uses_mean_pass(L.unit_G(), static_cast<int>(n_slots))) return 0;
  return align_up(static_cast<size_t>(L.B) * L.Hkv * n_slots * sizeof(float), 256);
}

hipError_t launch_topp(const Layout& L, const float* weights, const int32_t* cand_pages,
                       const int32_t* cand_count, int cand_stride_pages, float p,
                       int32_t* kept, int32_t* kept_count, float* tau, void* ws,
                       hipStream_t s, const float2* norm, int norm_chunks,
                       size_t stage_offset) {
  const ToppArgs a{&L, weights, cand_pages, cand_count, cand_stride_pages, p, kept,
                   kept_count, tau,
                   reinterpret_cast<float*>(static_cast<char*>(stage_scratch(ws, L)) +
                                            stage_offset),
                   s, norm, norm_chunks};
  const int n_slots = cand_stride_pages * kPage;
  if (block_threads(n_slots) == 512) {
    switch (slots_per_thread(n_slots)) {
      case 1: launch_spt<512, 1>(a); break;
      case 2: launch_spt<512, 2>(a); break;
      case 4: launch_spt<512, 4>(a); break;
      default: launch_spt<512, 8>(a); break;
    }
    return hipGetLastError();
  }
  switch (slots_per_thread(n_slots)) {
    case 1: launch_spt<1024, 1>(a); break;
    case 2: launch_spt<1024, 2>(a); break;
    case 4: launch_spt<1024, 4>(a); break;
    case 8: launch_spt<1024, 8>(a); break;
    case 16: launch_spt<1024, 16>(a); break;
    case 32: launch_spt<1024, 32>(a); break;
    default: launch_spt<1024, 64>(a); break;
  }
  return hipGetLastError();
}

}  // namespace twl
