// Twilight's attention-weight estimate over the candidate tokens from the int4 key cache
// (Twilight pages, atlas.scime.ai summary "Approach": top-p runs on estimated weights of
// the pre-selected tokens, computed from a 4-bit quantized key cache; "Limitations": the
// estimate's own cost matters when token loading is not the bottleneck). The 2-bit key
// cache of the pages' ablation runs through the same kernel with BITS = 2.
//
// Per candidate token j and query head h of the group:
//   s_hj = sm_scale * sum_groups [zero * Q_grp,h + scale * sum_{c in grp} q_hc * code_c],
// with Q_grp,h = sum_{c in grp} q_hc, the same value as q_h . dequant(k_j). Then a softmax
// over the unit's valid candidates, done as per-chunk (max, sum of exp) partials followed
// by a normalization pass (or, in the fused estimate + top-p call, normalised by the top-p
// kernel as it reads the logits). The logits are kept in log2 units (s_hj * log2 e), so
// that every exponential is one exp2.
#include <utility>

#include "twl_device.h"
#include "twl_launch.h"

namespace twl {
namespace {


constexpr int kEstWaves = kEstChunk / kWave;  // 4
constexpr int kEstBatch = 4;                  // candidate pages per wave per batch
constexpr int kNormThreads = 256;
constexpr int kNormSlots = kNormThreads * 16;  // weights per normalization work-group
#ifndef TWL_EST_TARGET_BLOCKS
#define TWL_EST_TARGET_BLOCKS 1024
#endif
#ifndef TWL_EST_MAX_CHUNK_PAGES
#define TWL_EST_MAX_CHUNK_PAGES 256
#endif

// The dot products run on the matrix cores, one 16-token tile (a candidate page) at a time,
// with v_mfma_f32_16x16x16_f16 (lane l supplies A[l%16][4(l/16)..+3] and
// B[4(l/16)..+3][l%16] and receives D[4(l/16)..+3][l%16]):
//  * B = channels x tokens: the codes as exact fp16 integers. Lane group c4 = l/16
//    supplies "virtual group" c4, the c4-th quarter of the channels (D/4 of them, one
//    contiguous run of the token's code row), four channels per instruction.
//  * A = rows (c4, h) = virtual group x query head, block-diagonal: row (c4, h) carries
//    q_h on the channels of virtual group c4 and 0 elsewhere.
//  * Over the D/16 instructions D[(c4, h)][t] accumulates the dot product of q_h with the
//    codes of virtual group c4 of token t, for up to 4 heads (a second set of instructions
//    covers heads 4..7).
// Lane (t, c4) scales its group's dot products (scale, plus zero * Q_grp once per real
// group), the four lane groups' terms are summed across rows, and lane (t, c4) keeps head
// c4 (and c4 + 4). A dot product is invariant to a common permutation of both operands, so
// the channel slots are ordered for cheap unpacking. With 4-bit codes a word holds 8
// channels; its even and odd nibbles are spread into bytes and converted two at a time
// (code_pairs_fp8), so instruction pair (2w, 2w+1) takes its slots {0,2,1,3} and
// {4,6,5,7}. With 2-bit codes a mask of the same bits of both 16-bit halves of a word yields
// two codes at once; a word holds 16 channels and instructions 4w..4w+3 take {0,8,1,9},
// {2,10,3,11}, {4,12,5,13}, {6,14,7,15}. Every product of an fp16 q and a code is exact in
// fp32.
template <int BITS>
__device__ __forceinline__ int mfma_channel(int c4, int vg_channels, int m, int e) {
  if constexpr (BITS == 4) {
    constexpr int kPerm[2][4] = {{0, 2, 1, 3}, {4, 6, 5, 7}};
    return c4 * vg_channels + 8 * (m / 2) + kPerm[m % 2][e];
  } else {
    const int mm = m % 4;
    return c4 * vg_channels + 16 * (m / 4) + 2 * mm + (e % 2) * 8 + e / 2;
  }
}

// (2-bit codes; 4-bit codes go through code_pairs_fp8 below.) Codes K of both 16-bit
// halves of a code word (bits [p + BITS - 1 : p] of each half, p = BITS * K) as two exact
// fp16 integers. A field that lies inside the fp16 significand
// (p + BITS <= 10) is converted where it stands: with the exponent of 2^(10 - p) or-ed in,
// the half reads 2^(10 - p) + n exactly (its ulp is 1 there), and subtracting 2^(10 - p)
// leaves n. Higher fields are first shifted down by 8 bits, one shift that serves all of
// them. The values are those of the plain shift-mask-convert, at fewer instructions.
// The exponent patterns for fields at p = 0, 2, 4, 6, 8 (index p / 2), both halves. The
// caller keeps them in VGPRs, so that mask and or go out as one v_and_or_b32 (whose one
// scalar operand is then the mask).
constexpr uint32_t code_exp(int p) {
  return (static_cast<uint32_t>(25 - p) << 10) | (static_cast<uint32_t>(25 - p) << 26);
}
template <int BITS, int K>
__device__ __forceinline__ uint32_t code_pair(uint32_t w, uint32_t w_hi,
                                              const uint32_t (&exp_v)[5]) {
  constexpr uint32_t kMask = BITS == 4 ? 0x000f000fu : 0x00030003u;
  constexpr int p0 = BITS * K;
  constexpr bool kLow = p0 + BITS <= 10;
  constexpr int p = kLow ? p0 : p0 - 8;
  const uint32_t x = ((kLow ? w : w_hi) & (kMask << p)) | exp_v[p / 2];
  const f16 off = static_cast<f16>(static_cast<float>(1 << (10 - p)));
  const f16x2 r = __builtin_bit_cast(f16x2, x) - f16x2{off, off};
  return __builtin_bit_cast(uint32_t, r);
}
template <int BITS, int... K>
__device__ __forceinline__ void code_pairs(uint32_t w, uint32_t (&bw)[16 / BITS],
                                           const uint32_t (&exp_v)[5],
                                           std::integer_sequence<int, K...>) {
  const uint32_t w_hi = w >> 8;
  ((bw[K] = code_pair<BITS, K>(w, w_hi, exp_v)), ...);
}

// The eight 4-bit codes of a word as four pairs of exact fp16 integers: the even and the
// odd nibbles are spread into bytes of their own, and a byte holding n in [0, 15] is, read
// as an fp8 e4m3 number, exactly n * 2^-9 (the subnormals and the first binade of e4m3 are
// evenly spaced). gfx950 converts two such bytes to fp16 at once, times a power-of-two
// scale, here 2^9, which makes them n again. Pairs: nibbles {0, 2}, {1, 3}, {4, 6},
// {5, 7}. 7 instructions per word instead of 9.
__device__ __forceinline__ void code_pairs_fp8(uint32_t w, uint32_t (&bw)[4]) {
  constexpr float kScale = 512.f;
  const uint32_t ev = w & 0x0f0f0f0fu;         // nibbles 0, 2, 4, 6 in bytes 0..3
  const uint32_t od = (w >> 4) & 0x0f0f0f0fu;  // nibbles 1, 3, 5, 7
  bw[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, kScale, false));
  bw[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, kScale, false));
  bw[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(ev, kScale, true));
  bw[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(od, kScale, true));
}

// *(p + off bytes) with p wave-uniform and off a 32-bit vector offset: the load takes the
// global_load form with a scalar base, so a wave-uniform address costs no 64-bit vector
// arithmetic, and it stays a vector-memory load (completed in order). The offset gets a
// fresh opaque zero added at each call, so that the compiler cannot hoist a vector copy of
// p + off out of a loop and form the addresses from it.
template <typename T>
__device__ __forceinline__ T load_at(const T* p, uint32_t off) {
  const uint32_t o = off + static_cast<uint32_t>(vgpr_zero());
  return *reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + o);
}

template <int NG>
struct CodeWords {
  uint32_t w[NG];
};
template <int NG>
__device__ __forceinline__ CodeWords<NG> load_words(const uint32_t* p, uint32_t off) {
  CodeWords<NG> r;
  if constexpr (NG == 4) {
    const u32x4 v = load_at(reinterpret_cast<const u32x4*>(p), off);
    r.w[0] = v[0];
    r.w[1] = v[1];
    r.w[2] = v[2];
    r.w[3] = v[3];
  } else if constexpr (NG == 1) {
    r.w[0] = load_at(p, off);
  } else {
    const u32x2 v = load_at(reinterpret_cast<const u32x2*>(p), off);
    r.w[0] = v[0];
    r.w[1] = v[1];
  }
  return r;
}

// One block per chunk of chunk_pages candidate pages of a (sequence, KV head). Wave w takes
// batches of kEstBatch pages (pages (j * 4 + w) * kEstBatch .. of the chunk, batch j), one
// MFMA tile per page. Each page goes through three dependent loads (candidate page id, page
// table, codes and metadata), pipelined across batches: ids two batches ahead, page-table
// entries and codes one ahead. The chunk's (max, sum exp) per head is kept online per lane.
template <int D, int G, int BITS>
__global__ __launch_bounds__(kEstChunk) void estimate_logits_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint32_t* __restrict__ meta, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cand_pages,
    const int32_t* __restrict__ cand_count, int cand_stride_pages, int Hkv, int max_pages,
    int num_phys, float scale_log2, float* __restrict__ logits, float2* __restrict__ partials,
    int chunk_pages, int n_chunks) {
  constexpr int NG = D / 32;
  constexpr int VG = D / 4;           // channels per virtual group (lane group)
  constexpr int MPT = D / 16;         // instructions per tile and head set
  constexpr int NHB = (G + 3) / 4;    // head sets of up to 4 heads
  constexpr int PB = kEstBatch;
  constexpr int NW = VG * BITS / 32;  // code words per lane and token
  constexpr int RB = D * BITS / 8;    // code bytes per token row
  static_assert(G <= 8, "at most 8 query heads per KV head");
  __shared__ __attribute__((aligned(16))) f16 qs[G][D];
  __shared__ float qsum[G][NG];
  __shared__ float red_m[kEstWaves][G], red_l[kEstWaves][G];
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int chunk = blockIdx.x;
  const int Hq = Hkv * G;
  const long unit = static_cast<long>(b) * Hkv + g;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int tok_in_page = lane % 16;
  const int c4 = lane / 16;
  // the sequence length comes on the vector path (made scalar after the q staging, where it
  // is first needed), so that no kernel-argument wait also waits for it
  const int n_lane = load_uniform_vec(seq_lens + b);
  int n = 0;  // set after the q staging
  const int n_slots = cand_stride_pages * kPage;
  const int page0 = chunk * chunk_pages;
  const int page_end = min(cand_stride_pages, page0 + chunk_pages);
  const int n_batches = (page_end - page0 + kEstWaves * PB - 1) / (kEstWaves * PB);
  const int32_t* crow = cand_pages ? cand_pages + unit * cand_stride_pages : nullptr;

  auto rank_of = [&](int j, int i) { return page0 + (j * kEstWaves + wave) * PB + i; };
  // Page ids of batch j, read before the candidate count is known (from inside the row).
  // The loads are unconditional (without a page list they read page-table entry 0 and are
  // replaced by the rank), and the tests below use no short-circuit branches, so that the
  // compiler issues a batch's loads together instead of one per branch. Page ids and
  // page-table entries are the same for the whole wave but are loaded on the vector path
  // (load_at, an opaque zero in the offset): vector loads complete in order, so a wait for this
  // batch's entries does not also wait for the ids already requested for the batch after
  // next, as a wait on a scalar load would, and the pipeline below stays three deep.
  // Once such a value has arrived it is made scalar (readfirstlane), so that the checks and
  // address arithmetic that follow run on the scalar unit. The loaded word is kept as it
  // came; the rank replaces it only where it is used (load_phys), since a select right after
  // the load would make the wave wait for it there, two batches early.
  const int32_t* id_src = crow != nullptr ? crow : page_table;
  auto load_ids = [&](int j, int (&pid)[PB]) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int r = rank_of(j, i);
      pid[i] = load_at(id_src + (crow != nullptr ? (r < page_end ? r : page0) : 0), 0u);
    }
  };
  int ids0[PB], ids1[PB];
  load_ids(0, ids0);
  load_ids(1, ids1);
  // the candidate count, loaded unconditionally as well (entry 0 of the page table stands in
  // for a missing count array), on the vector path; it is first needed after the q staging
  // below, whose barrier waits for it anyway
  const int cnt_lane = load_uniform_vec((cand_count != nullptr ? cand_count : page_table) +
                                        (cand_count != nullptr ? unit : 0));
  int cnt = cand_stride_pages;  // set after the q staging
  // validated page ids and their page-table entries
  const int32_t* pt_row = page_table + static_cast<long>(b) * max_pages;
  auto load_phys = [&](int j, int (&pid)[PB], int (&phys)[PB]) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int r = rank_of(j, i);
      const int ps = crow == nullptr ? r : __builtin_amdgcn_readfirstlane(pid[i]);
      const bool ok = (r < page_end) & (r < cnt) & (ps >= 0) & (ps < max_pages) &
                      (ps * kPage < n);
      pid[i] = ok ? ps : -1;
      phys[i] = load_at(pt_row + (ok ? ps : 0), 0u);
    }
  };
  // this lane's codes (virtual group c4 of its token's row) and its group's {scale, zero}:
  // the page's first row is a scalar base, the lane's part a small byte offset
  const uint32_t code_off = static_cast<uint32_t>(tok_in_page * RB + c4 * NW * 4);
  const uint32_t meta_off = static_cast<uint32_t>((tok_in_page * NG + c4 * VG / 32) * 4);
  auto load_codes = [&](int (&pid)[PB], const int (&phys)[PB], CodeWords<NW> (&cw)[PB],
                        uint32_t (&mw)[PB]) {
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int phs = __builtin_amdgcn_readfirstlane(phys[i]);
      const int pis = __builtin_amdgcn_readfirstlane(pid[i]);
      const bool ok = (pis >= 0) & (phs >= 0) & (phs < num_phys);
      pid[i] = ok ? pis : -1;
      // rows of an invalid page read page 0 of head 0 (always present) and are discarded
      const long row0 = ok ? (static_cast<long>(phs) * Hkv + g) * kPage : 0;
      cw[i] = load_words<NW>(reinterpret_cast<const uint32_t*>(codes + row0 * RB), code_off);
      mw[i] = load_at(meta + row0 * NG, meta_off);
    }
  };
  // the group's queries and their per-group sums, staged while the first ids are in flight:
  // a block barrier waits for every load the wave has issued, so it comes before the page
  // entries and codes are requested
  // (every thread copies one 16-byte piece, several threads the same one with the same
  // bytes, so that no branch holds the id loads back)
  static_assert(kEstChunk % (G * D / 8) == 0, "whole copies of q per block");
  {
    const int piece = threadIdx.x % (G * D / 8);
    const int h = piece / (D / 8), c = (piece % (D / 8)) * 8;
    *reinterpret_cast<u32x4*>(&qs[h][c]) =
        *reinterpret_cast<const u32x4*>(q + (static_cast<long>(b) * Hq + g * G + h) * D + c);
  }
  __syncthreads();
  if (threadIdx.x < G * NG) {
    const int h = threadIdx.x / NG, grp = threadIdx.x % NG;
    float acc = 0.f;
    for (int c = 0; c < 32; ++c) acc += static_cast<float>(qs[h][grp * 32 + c]);
    qsum[h][grp] = acc;
  }
  __syncthreads();
  {
    const int nv = __builtin_amdgcn_readfirstlane(n_lane);
    n = nv < 0 ? 0 : (nv > max_pages * kPage ? max_pages * kPage : nv);
    const int cnt_v = __builtin_amdgcn_readfirstlane(cnt_lane);
    const int cnt_list = cand_count != nullptr ? cnt_v : (n + kPage - 1) / kPage;
    cnt = crow == nullptr ? cand_stride_pages : min(cnt_list, cand_stride_pages);
  }
  int phys0[PB], phys1[PB];
  CodeWords<NW> cw0[PB];
  uint32_t mw0[PB];
  load_phys(0, ids0, phys0);

  // A operands: row (vg, h) = (lane%16 / 4, lane%16 % 4 + 4 hb), nonzero only on the
  // channels of virtual group vg and for h < G
  f16x4 qa[NHB][MPT];
  {
    const int vg = (lane % 16) / 4;
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      const int h = (lane % 16) % 4 + 4 * hb;
#pragma unroll
      for (int m = 0; m < MPT; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qa[hb][m][e] = (vg == c4 && h < G) ? qs[h < G ? h : 0][mfma_channel<BITS>(c4, VG, m, e)]
                                             : static_cast<f16>(0.f);
    }
  }
  // Q_grp * zero enters once per real group: by the lane group holding its first channels
  const bool adds_zero = (c4 * VG) % 32 == 0;
  float qg[NHB][4];  // Q of this lane's group for heads r + 4 hb
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = r + 4 * hb;
      qg[hb][r] = (h < G && adds_zero) ? qsum[h < G ? h : 0][c4 * VG / 32] : 0.f;
    }
  // every page entry of the batch is in hand before the code loads go out (the compiler
  // would otherwise interleave them, one round trip per page)
#pragma unroll
  for (int i = 0; i < PB; ++i) keep_loaded(phys0[i]);
  load_codes(ids0, phys0, cw0, mw0);

  uint32_t code_exp_v[5];  // code_exp(2i), held in VGPRs (vz is an opaque zero)
  const int vz = vgpr_zero();
#pragma unroll
  for (int i = 0; i < 5; ++i) code_exp_v[i] = static_cast<uint32_t>(vz) + code_exp(2 * i);
  float run_m[NHB], run_l[NHB];  // online max and sum of exp of this lane's head(s)
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    run_m[hb] = -INFINITY;
    run_l[hb] = 0.f;
  }
  // Batch j: the tiles of its pages (codes in cw0, {scale, zero} in mw0, ids in ids0), their
  // logits written and folded into the online (max, sum of exp).
  auto batch = [&](int j) {
    float s[PB][NHB];
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      // B operands of the tile: 32 / (4 BITS) instructions per 32-bit word of codes
      f16x4 bq[MPT];
#pragma unroll
      for (int wi = 0; wi < NW; ++wi) {
        const uint32_t w = cw0[i].w[wi];
        constexpr int kPairs = 16 / BITS;  // code pairs per word
        uint32_t bw[kPairs];
        if constexpr (BITS == 4) {
          code_pairs_fp8(w, bw);
        } else {
          code_pairs<BITS>(w, bw, code_exp_v, std::make_integer_sequence<int, kPairs>());
        }
#pragma unroll
        for (int m = 0; m < kPairs / 2; ++m)
          bq[wi * (kPairs / 2) + m] = __builtin_bit_cast(f16x4, u32x2{bw[2 * m], bw[2 * m + 1]});
      }
      const float scale = h2f(static_cast<uint16_t>(mw0[i] & 0xffffu));
      const float zero = h2f(static_cast<uint16_t>(mw0[i] >> 16));
      const bool valid = (ids0[i] >= 0) & (tok_in_page < n - ids0[i] * kPage);
#pragma unroll
      for (int hb = 0; hb < NHB; ++hb) {
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < MPT; ++m)
          d = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[hb][m], bq[m], d, 0, 0, 0);
        // this lane group's terms for heads r + 4 hb, summed over the four lane groups so
        // that lane group c4 ends with head c4 + 4 hb (a reduce-scatter: each swap moves two
        // different values, and no lane forms a total it does not keep)
        float v[4], tot[1];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = fmaf(scale, d[r], zero * qg[hb][r]);
        sum_rows_scatter<4>(v, tot);
        const float mine = tot[0];
        s[i][hb] = (valid && c4 + 4 * hb < G) ? scale_log2 * mine : -INFINITY;
      }
      // logits row entries (every slot of the chunk is written, -inf when not a candidate)
      const int slot = rank_of(j, i) * kPage + tok_in_page;
      if (rank_of(j, i) < page_end) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
          const int h = c4 + 4 * hb;
          if (h < G) logits[(static_cast<long>(b) * Hq + g * G + h) * n_slots + slot] = s[i][hb];
        }
      }
    }
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
      float bm = s[0][hb];
#pragma unroll
      for (int i = 1; i < PB; ++i) bm = fmaxf(bm, s[i][hb]);
      const float mn = fmaxf(run_m[hb], bm);
      if (mn > -INFINITY) {
        // mn is finite here, so the -inf old max and -inf scores give exactly 0
        float l = run_l[hb] * exp2_unit(run_m[hb] - mn);
#pragma unroll
        for (int i = 0; i < PB; ++i) l += exp2_unit(s[i][hb] - mn);
        run_l[hb] = l;
        run_m[hb] = mn;
      }
    }
  };
  // Pipeline: page ids two batches ahead, page-table entries and codes one ahead. The
  // steady-state loop runs while batch j + 2 exists, so that it issues the same loads on
  // every path: the compiler's wait before a batch's codes then covers the page-table
  // entries alone. (Issuing the loads only while needed, inside the loop, made it wait for
  // the page ids just requested, a round trip per batch.) The last two batches are peeled.
  if (n_batches >= 2) {
    load_phys(1, ids1, phys1);
    for (int j = 0; j + 2 < n_batches; ++j) {
      int ids2[PB];
      load_ids(j + 2, ids2);
      CodeWords<NW> cw1[PB];
      uint32_t mw1[PB];
      load_codes(ids1, phys1, cw1, mw1);
      batch(j);
      // rotate: batch j + 1 (codes in flight) becomes current, then batch j + 2 (page ids
      // in hand) gets its page-table entries
#pragma unroll
      for (int i = 0; i < PB; ++i) {
        ids0[i] = ids1[i];
        cw0[i] = cw1[i];
        mw0[i] = mw1[i];
      }
      load_phys(j + 2, ids2, phys1);
#pragma unroll
      for (int i = 0; i < PB; ++i) ids1[i] = ids2[i];
    }
    CodeWords<NW> cw1[PB];
    uint32_t mw1[PB];
    load_codes(ids1, phys1, cw1, mw1);
    batch(n_batches - 2);
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      ids0[i] = ids1[i];
      cw0[i] = cw1[i];
      mw0[i] = mw1[i];
    }
  }
  batch(n_batches - 1);
  // (max, sum exp) per head: over the row's 16 tokens, then over the waves
#pragma unroll
  for (int hb = 0; hb < NHB; ++hb) {
    const float M = group_reduce<16>(run_m[hb], OpMax());
    const float l = run_m[hb] > -INFINITY ? run_l[hb] * exp2_unit(run_m[hb] - M) : 0.f;
    const float L = group_reduce<16>(l, OpSum());
    const int h = c4 + 4 * hb;
    if (h < G && tok_in_page == 0) {
      red_m[wave][h] = M;
      red_l[wave][h] = L;
    }
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float M = red_m[0][h];
#pragma unroll
    for (int w2 = 1; w2 < kEstWaves; ++w2) M = fmaxf(M, red_m[w2][h]);
    float L = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < kEstWaves; ++w2)
      L += red_m[w2][h] > -INFINITY ? red_l[w2][h] * exp2_unit(red_m[w2][h] - M) : 0.f;
    partials[(static_cast<long>(b) * Hq + g * G + h) * n_chunks + chunk] = make_float2(M, L);
  }
}

// w = exp(s - M) / L with (M, L) merged from the row's chunk partials; invalid slots hold
// s = -inf and come out as exactly 0. Each thread takes 16 consecutive weights; wave 0
// merges the partials while every thread's loads are in flight.
__global__ __launch_bounds__(kNormThreads) void estimate_normalize_kernel(
    float* __restrict__ weights, const float2* __restrict__ partials, int n_chunks, int n_slots) {
  __shared__ float s_ml[2];
  const long hrow = blockIdx.y;
  const int first = blockIdx.x * kNormSlots + threadIdx.x * 16;
  float* w = weights + hrow * n_slots;
  f32x4 v[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int sl = first + 4 * k;  // n_slots is a multiple of 16
    v[k] = *reinterpret_cast<const f32x4*>(w + (sl < n_slots ? sl : 0));
  }
  if (threadIdx.x < kWave) {
    const float2 ml = merge_max_sum_wave(partials + hrow * n_chunks, n_chunks);
    if (threadIdx.x == 0) {
      s_ml[0] = ml.x;
      s_ml[1] = softmax_inv_sum(ml.y);  // once per row, not per thread
    }
  }
  __syncthreads();
  const float M = s_ml[0], inv_l = s_ml[1];
  if (first >= n_slots) return;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = softmax_weight(v[k][e], M, inv_l);
    *reinterpret_cast<f32x4*>(w + first + 4 * k) = o;
  }
}

template <int D, int G, int BITS>
void logits_launch(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                   const int32_t* cand_pages, const int32_t* cand_count, int stride,
                   float sm_scale, float* weights, float2* partials, int chunk_pages,
                   int n_chunks, hipStream_t s) {
  estimate_logits_kernel<D, G, BITS><<<dim3(n_chunks, L.Hkv, L.B), kEstChunk, 0, s>>>(
      static_cast<const uint16_t*>(q), codes, static_cast<const uint32_t*>(meta), L.page_table,
      L.seq_lens, cand_pages, cand_count, stride, L.Hkv, L.max_pages, L.num_phys, sm_scale,
      weights, partials, chunk_pages, n_chunks);
}

template <int D, int BITS>
void logits_dispatch_g(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                       const int32_t* cand_pages, const int32_t* cand_count, int stride,
                       float sm_scale, float* weights, float2* partials, int chunk_pages,
                       int n_chunks, hipStream_t s) {
  switch (L.G()) {
    case 1: logits_launch<D, 1, BITS>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, chunk_pages, n_chunks, s); break;
    case 2: logits_launch<D, 2, BITS>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, chunk_pages, n_chunks, s); break;
    case 4: logits_launch<D, 4, BITS>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, chunk_pages, n_chunks, s); break;
    default: logits_launch<D, 8, BITS>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, chunk_pages, n_chunks, s); break;
  }
}

template <int D>
void logits_dispatch_bits(const Layout& L, const void* q, const uint8_t* codes,
                          const void* meta, const int32_t* cand_pages,
                          const int32_t* cand_count, int stride, float sm_scale,
                          float* weights, float2* partials, int chunk_pages, int n_chunks,
                          hipStream_t s) {
  if (L.bits == 2) {
    logits_dispatch_g<D, 2>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale,
                            weights, partials, chunk_pages, n_chunks, s);
  } else {
    logits_dispatch_g<D, 4>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale,
                            weights, partials, chunk_pages, n_chunks, s);
  }
}

// Candidate pages per logits work-group: about TWL_EST_TARGET_BLOCKS work-groups over all
// candidate pages, at least one batch per wave and at most TWL_EST_MAX_CHUNK_PAGES.
int estimate_chunk_pages(const Layout& L, int cand_stride_pages) {
  const long total = static_cast<long>(L.B) * L.Hkv * cand_stride_pages;
  const long want = (total + TWL_EST_TARGET_BLOCKS - 1) / TWL_EST_TARGET_BLOCKS;
  long c = kEstWaves * kEstBatch;
  while (c < want && c < TWL_EST_MAX_CHUNK_PAGES) c <<= 1;
  return static_cast<int>(c);
}

}  // namespace

size_t estimate_workspace_bytes(const Layout& L, int cand_stride_pages) {
  const int cp = estimate_chunk_pages(L, cand_stride_pages);
  const long n_chunks = (static_cast<long>(cand_stride_pages) + cp - 1) / cp;
  return align_up(static_cast<size_t>(L.B) * L.Hq * n_chunks * sizeof(float2), 256);
}

int estimate_chunks(const Layout& L, int cand_stride_pages) {
  const int cp = estimate_chunk_pages(L, cand_stride_pages);
  return (cand_stride_pages + cp - 1) / cp;
}

hipError_t launch_estimate(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                           const int32_t* cand_pages, const int32_t* cand_count,
                           int cand_stride_pages, float sm_scale, float* weights, void* ws,
                           hipStream_t s, bool normalize) {
  const int n_slots = cand_stride_pages * kPage;
  const int cp = estimate_chunk_pages(L, cand_stride_pages);
  const int n_chunks = estimate_chunks(L, cand_stride_pages);
  float2* partials = static_cast<float2*>(stage_scratch(ws, L));
  const float scale_log2 = sm_scale * 1.4426950408889634f;  // logits in log2 units
  if (L.d == 128) {
    logits_dispatch_bits<128>(L, q, codes, meta, cand_pages, cand_count, cand_stride_pages,
                              scale_log2, weights, partials, cp, n_chunks, s);
  } else {
    logits_dispatch_bits<64>(L, q, codes, meta, cand_pages, cand_count, cand_stride_pages,
                             scale_log2, weights, partials, cp, n_chunks, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !normalize) return e;
  const dim3 grid((n_slots + kNormSlots - 1) / kNormSlots, L.B * L.Hq);
  estimate_normalize_kernel<<<grid, kNormThreads, 0, s>>>(weights, partials, n_chunks, n_slots);
  return hipGetLastError();
}

}  // namespace twl
