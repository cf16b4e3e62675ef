// Sparse paged decode attention over the kept tokens (Twilight pages, atlas.scime.ai
// summary "Key results": the Twilight sparse self-attention operator, which attends only to
// the tokens that survive pruning).
//
// For each query head h of KV head g: o_h = sum_{j in kept} softmax_j(sm_scale q_h . k_j) v_j
// on the fp16 cache, the softmax over the kept set only.
//
// Split-KV: each work-group takes a chunk of a KV head's kept list and leaves (max, sum,
// unnormalized o) in log2 units in the workspace; a merge kernel combines the chunks and
// writes the fp16 output. A list that fits one chunk is finished in place. Chunks are one to
// sixteen batches of rows: short enough that every row's chain of dependent loads is in
// flight at once across the chip when lists are short, long enough that long lists leave few
// partials. (Merging in the last work-group to finish, found with an atomic ticket, needs
// device-scope fences that write back and invalidate whole L2s on this multi-XCD part;
// measured, it costs far more than the second launch.)
//
// Layout on the device: V rows (and K rows in the dot2 form) take D/8 lanes per kept token,
// 8 channels (16 B) per lane, so one wave gathers 64/(D/8) token rows per load instruction,
// each row one contiguous 2*D-byte stretch of the paged cache. For d = 128 and groups of
// four or more heads, q . k runs on the matrix cores with K rows in the MFMA operand layout
// and the weights broadcast back into the V layout; otherwise it uses v_dot2_f32_f16 on fp16
// pairs reduced across the row's lanes with DPP. Products are exact and sums fp32 either
// way; softmax and p * v run in fp32.
#include "twl_device.h"
#include "twl_launch.h"

namespace twl {
namespace {

// Tuning constants (compile-time; the defaults are the measured choice on MI355X).
#ifndef TWL_DEC_THREADS
#define TWL_DEC_THREADS 256
#endif
#ifndef TWL_DEC_UNROLL
#define TWL_DEC_UNROLL 4
#endif
#ifndef TWL_DEC_TARGET_BLOCKS
#define TWL_DEC_TARGET_BLOCKS 512
#endif
#ifndef TWL_DEC_MAX_BATCHES
#define TWL_DEC_MAX_BATCHES 16
#endif
// A full-length kept list still splits into at least this many chunks, or, in a step of
// at most TWL_DEC_FEW_UNITS (sequence, KV head) units, TWL_DEC_MIN_CHUNKS_FEW.
#ifndef TWL_DEC_MIN_CHUNKS
#define TWL_DEC_MIN_CHUNKS 16
#endif
#ifndef TWL_DEC_MIN_CHUNKS_FEW
#define TWL_DEC_MIN_CHUNKS_FEW 64
#endif
#ifndef TWL_DEC_FEW_UNITS
#define TWL_DEC_FEW_UNITS 64
#endif
constexpr int kDecThreads = TWL_DEC_THREADS;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecUnroll = TWL_DEC_UNROLL;
#ifndef TWL_MERGE_SLICE
#define TWL_MERGE_SLICE 32
#endif
constexpr int kMergeSlice = TWL_MERGE_SLICE;  // channels per merge work-group

// Kept tokens one work-group takes per batch: every wave takes kDecUnroll rows per lane
// group, 64 / (D/8) lane groups per wave.
__host__ __device__ constexpr int decode_batch_tokens(int d) {
  return kDecWaves * kDecUnroll * (kWave / (d / 8));
}

__device__ __forceinline__ float rescale(float m, float M) {
  return m == -INFINITY ? 0.f : exp2_unit(m - M);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

// Each work-group takes chunk_tokens consecutive entries of a KV head's kept list, in
// batches of decode_batch_tokens(D). A lane's rows go through three dependent loads (kept
// id, page-table entry, K/V row), pipelined across batches: ids two batches ahead, page
// entries one ahead. Every load is issued unconditionally (entries past the list or the
// sequence read a valid stand-in and are masked afterwards), so no load waits behind a
// branch; the kept count is read alongside the first ids. kSingle is the form for chunks
// of exactly one batch: with no next batch to prefetch, the pipeline's second set of rows
// and registers is compiled out, which leaves room for twice the resident work-groups.
template <int D, int G, bool kSingle>
__global__ __launch_bounds__(kDecThreads)
__attribute__((amdgpu_waves_per_eu(kSingle && G <= 4 ? 4 : 1))) void sparse_decode_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, int kept_stride, int units, int Hkv, int max_pages,
    int num_phys, float scale_log2, float* __restrict__ part_o, float2* __restrict__ part_ml,
    int n_chunks, int chunk_tokens, uint16_t* __restrict__ out) {
  constexpr int LPT = D / 8;        // lanes per token row
  constexpr int TPW = kWave / LPT;  // token rows per wave per load
  constexpr int U = kDecUnroll;
  constexpr int STEP = TPW * U;     // tokens per wave per batch
  constexpr int BSTEP = decode_batch_tokens(D);
  // per wave: each head's max, then the token-group sums of (l, acc[0..7]) per head,
  // [value][channel slice] (one padding column against bank conflicts)
  constexpr int kRedQ = (G * 9 + 3) / 4;
  __shared__ float s_m[kDecWaves][G];
  __shared__ float s_red[kDecWaves][4 * kRedQ][LPT + 1];

  // work-groups are numbered chunk-major (every KV head's first chunk, then every second
  // chunk, ...), so that chunks past a short kept list, which exit at once, are dispatched
  // last instead of holding slots ahead of useful work
  // a unit is a KV head and its G query heads, or (head-wise, G = 1) one query head, whose
  // K/V rows are those of KV head g / (units / Hkv)
  const int b = blockIdx.y;
  const int g = blockIdx.x % units;
  const int chunk = blockIdx.x / units;
  const long unit = static_cast<long>(b) * units + g;
  const int kvh = g / (units / Hkv);
  const int Hq = units * G;
  const long head0 = static_cast<long>(b) * Hq + g * G;
  const int t0 = chunk * chunk_tokens;
  const int tend = min(kept_stride, t0 + chunk_tokens);  // the chunk's slots in the list
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int sub = lane % LPT;
  const int tk = lane / LPT;
  const int c0 = sub * 8;
  const int32_t* krow = kept + unit * kept_stride;
  const int32_t* trow = page_table + static_cast<long>(b) * max_pages;

  // q . k on the matrix cores when a wave's batch is one 16-token tile (d = 128) and the group
  // has at least 4 query heads: K rows then come in the MFMA operand layout, lane l holding
  // channels 8 (l / 16) + 32 jj + [0, 8), jj = 0..3, of tile token l % 16, which is the token
  // of row u = (l % 16) % 4 of token group (l % 16) / 4 in the V layout below. Each lane then
  // has one more row (index U) to look up besides its U V rows. (That layout reads 64-byte
  // pieces of 16 rows per load instead of whole rows; for one or two heads, where the dot2
  // form costs few instructions, the whole-row loads are faster.)
  constexpr bool kMfma = D == 128 && STEP == 16 && G >= 4;
  constexpr int NU = U + (kMfma ? 1 : 0);
  constexpr int KX = kMfma ? 4 : U;  // K registers per lane
  const int mrow = lane % 16;        // the lane's MFMA row: its tile token

  // slot of this lane's row u of batch j (u = U: the MFMA row)
  auto slot_of = [&](int j, int u) {
    const int uu = u < U ? u : mrow % 4;
    const int gg = u < U ? tk : mrow / 4;
    return t0 + j * BSTEP + wave * STEP + uu * TPW + gg;
  };
  auto load_ids = [&](int j, int (&id)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int sl = slot_of(j, u);
      id[u] = krow[sl < tend ? sl : t0];
    }
  };
  // Everything the first K/V loads depend on goes out at once, before any branch: the
  // kept ids, the kept count, the sequence length and q, then batch 0's page entries
  // (masked by the chunk's slot range; the list end is applied once the count is known).
  int ids0[NU], ids1[NU];
  load_ids(0, ids0);
  if constexpr (!kSingle) load_ids(1, ids1);
  int K = kept_count[unit];
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  // q: per head, this lane's 8 channels (dot2 form), or the MFMA B operand: column
  // mrow < G is head mrow, with the same channels as the lane's K operand
  uint32_t qw[kMfma ? 4 : G][4];
  if constexpr (kMfma) {
    const int hq = mrow < G ? mrow : 0;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const u32x4 v =
          *reinterpret_cast<const u32x4*>(q + (head0 + hq) * D + 32 * jj + 8 * (lane / 16));
#pragma unroll
      for (int e = 0; e < 4; ++e) qw[jj][e] = mrow < G ? v[e] : 0u;
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(q + (head0 + h) * D + c0);
#pragma unroll
      for (int e = 0; e < 4; ++e) qw[h][e] = v[e];
    }
  }

  // page entries of batch j: the token's page id (or a stand-in) and its in-page offset;
  // slots at or past `last` are masked
  auto load_rows = [&](int j, int last, const int (&id)[NU], int (&phys)[NU], int (&tok)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int sl = slot_of(j, u);
      const int t = id[u];
      const bool ok = sl < last && t >= 0 && t < n;
      tok[u] = ok ? t : -1;
      phys[u] = trow[ok ? t / kPage : 0];
    }
  };
  int phys0[NU], tok0[NU], phys1[NU], tok1[NU];
  load_rows(0, tend, ids0, phys0, tok0);
  // the page entries stay ahead of the exit tests below (the compiler would otherwise sink
  // them past the branches, behind a wait on every load in flight)
#pragma unroll
  for (int u = 0; u < NU; ++u) keep_loaded(phys0[u]);

  K = K < 0 ? 0 : (K > kept_stride ? kept_stride : K);
  if (K == 0) {
    // empty kept set: o = 0, written by the first work-group
    if (chunk == 0)
      for (int i = threadIdx.x; i < G * D; i += kDecThreads) out[head0 * D + i] = 0;
    return;
  }
  if (t0 >= K) return;
  const int t1 = min(K, t0 + chunk_tokens);
  const int nc = (K + chunk_tokens - 1) / chunk_tokens;
  // (a single-batch chunk that reached this point holds at least one slot of the list)
  const int n_batches = kSingle ? 1 : (t1 - t0 + BSTEP - 1) / BSTEP;
#pragma unroll
  for (int u = 0; u < NU; ++u)
    if (slot_of(0, u) >= t1) tok0[u] = -1;

  auto row_of = [&](int phys, int tok) -> long {
    if (tok < 0 || !phys_ok(phys, num_phys)) return -1;
    return ((static_cast<long>(phys) * Hkv + kvh) * kPage + tok % kPage) * D;
  };
  // V rows (and in the dot2 form K rows) at the lane's channels; in the MFMA form the K
  // operand of the lane's tile token. Dead rows read row 0 and are masked afterwards. A
  // step reads each kept row once: non-temporal loads (measured 13.4 -> 12.9 us for decode
  // + merge at the 128k GQA layer, 299 -> 285 us at the B = 8 64k full-attention step).
  auto load_kv = [&](const int (&phys)[NU], const int (&tok)[NU], bool (&live)[U],
                     u32x4 (&kx)[KX], u32x4 (&vv)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long row = row_of(phys[u], tok[u]);
      live[u] = row >= 0;
      const long r = row >= 0 ? row : 0;
      if constexpr (!kMfma)
        kx[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(k_cache + r + c0));
      vv[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(v_cache + r + c0));
    }
    if constexpr (kMfma) {
      const long row = row_of(phys[U], tok[U]);
      const uint16_t* kr = k_cache + (row >= 0 ? row : 0) + 8 * (lane / 16);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj)
        kx[jj] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kr + 32 * jj));
    }
  };

  // running softmax state: l and acc per head in the V layout; the max per head is uniform
  // over the wave (dot2 form: m[h] in every lane; MFMA form: mh, lane column mrow = head)
  float m[G], l[G], acc[G][8];
  float mh = -INFINITY;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }

  // pipeline: K/V of batch 0, then the page entries of batch 1
  bool live0[U];
  u32x4 kx0[KX], vv0[U];
  load_kv(phys0, tok0, live0, kx0, vv0);

  // batch j: scores of the lane's rows (K in kx0), their weights and the running softmax
  // state, and p.v into acc (V in vv0)
  auto batch = [&](int j) {
    // weights pr[u][h] of the lane's V rows and the rescale alpha[h] of the old state.
    // Exponentials are taken against the new max, or against 0 while a head has no live
    // token yet, which gives exactly 0 for -inf scores and a -inf old max.
    float pr[U][G], alpha[G];
    if constexpr (kMfma) {
      // S = K_tile q^T: lane l ends with the scores of tile rows 4 (l / 16) + r, r = 0..3
      // (tokens u = r of token group l / 16, i.e. the lane's own V rows), for head l % 16
      f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const f16x4 a = __builtin_bit_cast(
              f16x4, u32x2{kx0[jj][2 * hf], kx0[jj][2 * hf + 1]});
          const f16x4 bq = __builtin_bit_cast(f16x4, u32x2{qw[jj][2 * hf], qw[jj][2 * hf + 1]});
          sacc = __builtin_amdgcn_mfma_f32_16x16x16f16(a, bq, sacc, 0, 0, 0);
        }
      }
      float sc[U];
#pragma unroll
      for (int r = 0; r < U; ++r) sc[r] = live0[r] ? sacc[r] * scale_log2 : -INFINITY;
      float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
      mb = across_groups<16>(mb, OpMax());
      const float mn = fmaxf(mh, mb);
      const float mref = mn == -INFINITY ? 0.f : mn;
      const float al = j == 0 ? 0.f : exp2_unit(mh - mref);
      float pm[U];
#pragma unroll
      for (int r = 0; r < U; ++r) pm[r] = exp2_unit(sc[r] - mref);
      mh = mn;
      // to the V layout: lane (group tk, slice sub) takes head h's values from lane h of its
      // row, which holds the same four tokens
#pragma unroll
      for (int h = 0; h < G; ++h) {
        alpha[h] = j == 0 ? 0.f : row_bcast_f32(al, h);
#pragma unroll
        for (int u = 0; u < U; ++u) pr[u][h] = row_bcast_f32(pm[u], h);
      }
    } else {
      float s[U][G];
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float d = 0.f;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj)
            d = __builtin_amdgcn_fdot2(as_h2(qw[h][jj]), as_h2(kx0[u][jj]), d, false);
          d = group_sum<LPT>(d);
          s[u][h] = live0[u] ? d * scale_log2 : -INFINITY;
        }
      }
      // one running max per head for the whole wave: the token groups' batch maxima are
      // combined across groups, so every group's (l, acc) stays on the same scale
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float mb = s[0][h];
#pragma unroll
        for (int u = 1; u < U; ++u) mb = fmaxf(mb, s[u][h]);
        mb = across_groups<LPT>(mb, OpMax());
        const float mn = fmaxf(m[h], mb);
        const float mref = mn == -INFINITY ? 0.f : mn;
        alpha[h] = j == 0 ? 0.f : exp2_unit(m[h] - mref);
#pragma unroll
        for (int u = 0; u < U; ++u) pr[u][h] = exp2_unit(s[u][h] - mref);
        m[h] = mn;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float lsum = l[h] * alpha[h];
#pragma unroll
      for (int u = 0; u < U; ++u) lsum += pr[u][h];
      l[h] = lsum;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= alpha[h];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[8];
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const f16x2 p2 = as_h2(vv0[u][jj]);
        vf[2 * jj] = static_cast<float>(p2[0]);
        vf[2 * jj + 1] = static_cast<float>(p2[1]);
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(pr[u][h], vf[c], acc[h][c]);
      }
    }
  };
  if constexpr (kSingle) {
    batch(0);
  } else {
    // The pipeline (ids two batches ahead, page entries and K/V one ahead) runs its
    // steady state while batch j + 2 exists, issuing the same loads on every path: the
    // compiler's wait before a batch's K/V then covers its page entries alone. (Loads issued
    // only while needed, inside one loop, made it wait for the ids just requested, a round
    // trip per batch.) The last two batches are peeled.
    if (n_batches > 1) {
      load_rows(1, t1, ids1, phys1, tok1);
      for (int j = 0; j + 2 < n_batches; ++j) {
        int ids2[NU];
        bool live1[U];
        u32x4 kx1[KX], vv1[U];
        load_ids(j + 2, ids2);
        load_kv(phys1, tok1, live1, kx1, vv1);
        batch(j);
        int phys2[NU], tok2[NU];
        load_rows(j + 2, t1, ids2, phys2, tok2);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          phys1[u] = phys2[u];
          tok1[u] = tok2[u];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          live0[u] = live1[u];
          vv0[u] = vv1[u];
        }
#pragma unroll
        for (int u = 0; u < KX; ++u) kx0[u] = kx1[u];
      }
      bool live1[U];
      u32x4 kx1[KX], vv1[U];
      load_kv(phys1, tok1, live1, kx1, vv1);
      batch(n_batches - 2);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        live0[u] = live1[u];
        vv0[u] = vv1[u];
      }
#pragma unroll
      for (int u = 0; u < KX; ++u) kx0[u] = kx1[u];
    }
    batch(n_batches - 1);
  }
  if constexpr (kMfma) {
#pragma unroll
    for (int h = 0; h < G; ++h) m[h] = row_bcast_f32(mh, h);
  }
  // Sum the token groups of each channel slice (same scale: m is shared by the wave). The
  // values are (l, acc[0..7]) per head; for d = 64 the two groups of a row are added first,
  // then the four rows are summed scattered, so each row ends with a quarter of the values
  // and writes them to LDS.
  float x[4 * kRedQ];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    x[h * 9] = l[h];
#pragma unroll
    for (int c = 0; c < 8; ++c) x[h * 9 + 1 + c] = acc[h][c];
  }
#pragma unroll
  for (int k = G * 9; k < 4 * kRedQ; ++k) x[k] = 0.f;
  if constexpr (LPT == 8) {
#pragma unroll
    for (int k = 0; k < G * 9; ++k) x[k] += dpp_f32<kRowRor8>(x[k]);
  }
  float y[kRedQ];
  sum_rows_scatter<4 * kRedQ>(x, y);
  {
    const int row = lane / 16, col = lane % 16;
    if (col < LPT) {
#pragma unroll
      for (int i = 0; i < kRedQ; ++i) s_red[wave][row * kRedQ + i][col] = y[i];
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) s_m[wave][h] = m[h];
    }
  }
  __syncthreads();
  // this chunk's (M, L, A) per head, merged over the waves
  for (int i = threadIdx.x; i < G * D; i += kDecThreads) {
    const int h = i / D, c = i % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, s_m[w][h]);
    const float mref = M == -INFINITY ? 0.f : M;
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = exp2_unit(s_m[w][h] - mref);
      L += s_red[w][h * 9][0] * f;
      A += s_red[w][h * 9 + 1 + c % 8][c / 8] * f;
    }
    if (nc == 1) {
      const float o = L > 0.f ? A / L : 0.f;
      out[(head0 + h) * D + c] = __builtin_bit_cast(uint16_t, static_cast<f16>(o));
    } else {
      const long pidx = (head0 + h) * n_chunks + chunk;
      if (c == 0) part_ml[pidx] = make_float2(M, L);
      part_o[pidx * D + c] = A;
    }
  }
}

// Merge of the chunk partials when they are more than one: one wave per (sequence, query
// head, 32-channel slice: a whole 128-byte line of each chunk's record). Lane i takes
// chunks i, i + 64, ... with a running (max, sum, o) of its own; the lanes are then
// combined on the common maximum. The (max, sum) pairs sit
// in their own compact array and each chunk's o in a 512-byte record, so every byte of the
// partials is fetched once.
template <int D>
__global__ __launch_bounds__(kWave) void decode_merge_kernel(
    const float* __restrict__ part_o, const float2* __restrict__ part_ml,
    const int32_t* __restrict__ kept_count, int kept_stride, int units, int G, int n_chunks,
    int chunk_tokens, uint16_t* __restrict__ out) {
  __shared__ float s_acc[kWave][kMergeSlice + 1];
  const int slice = blockIdx.x;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int Hq = units * G;
  const long unit = static_cast<long>(b) * units + h / G;
  int K = kept_count[unit];
  K = K < 0 ? 0 : (K > kept_stride ? kept_stride : K);
  const int nc = (K + chunk_tokens - 1) / chunk_tokens;
  if (nc <= 1) return;  // finished by the partial kernel
  const int lane = lane_id();
  const long hrow = static_cast<long>(b) * Hq + h;
  const float2* ml = part_ml + hrow * n_chunks;
  const float* po = part_o + hrow * n_chunks * D + slice * kMergeSlice;
  float M = -INFINITY, L = 0.f;
  float acc[kMergeSlice];
#pragma unroll
  for (int c = 0; c < kMergeSlice; ++c) acc[c] = 0.f;
  for (int i = lane; i < nc; i += kWave) {
    const float2 mi = ml[i];
    f32x4 a[kMergeSlice / 4];
#pragma unroll
    for (int v = 0; v < kMergeSlice / 4; ++v)
      a[v] = *reinterpret_cast<const f32x4*>(po + static_cast<long>(i) * D + 4 * v);
    const float Mn = fmaxf(M, mi.x);
    const float fo = rescale(M, Mn), fi = rescale(mi.x, Mn);
    L = L * fo + mi.y * fi;
#pragma unroll
    for (int v = 0; v < kMergeSlice / 4; ++v) {
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[4 * v + j] = acc[4 * v + j] * fo + a[v][j] * fi;
    }
    M = Mn;
  }
  const float Mw = wave_max(M);
  const float f = rescale(M, Mw);
  L = wave_sum(L * f);
#pragma unroll
  for (int c = 0; c < kMergeSlice; ++c) s_acc[lane][c] = acc[c] * f;
  __syncthreads();
  if (lane < kMergeSlice) {
    float t = 0.f;
    for (int r = 0; r < kWave; ++r) t += s_acc[r][lane];
    const float o = L > 0.f ? t / L : 0.f;
    out[hrow * D + slice * kMergeSlice + lane] = __builtin_bit_cast(uint16_t, static_cast<f16>(o));
  }
}

template <int D, int G>
void decode_launch(const Layout& L, const void* q, const void* k, const void* v,
                   const int32_t* kept, const int32_t* kept_count, int kept_stride,
                   float scale_log2, float* part_o, float2* part_ml, int n_chunks, int ch,
                   void* out, hipStream_t s) {
  const dim3 grid(n_chunks * L.units(), L.B);
  if (ch == decode_batch_tokens(D)) {
    sparse_decode_kernel<D, G, true><<<grid, kDecThreads, 0, s>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), L.page_table, L.seq_lens, kept, kept_count,
        kept_stride, L.units(), L.Hkv, L.max_pages, L.num_phys, scale_log2, part_o, part_ml,
        n_chunks, ch, static_cast<uint16_t*>(out));
  } else {
    sparse_decode_kernel<D, G, false><<<grid, kDecThreads, 0, s>>>(
        static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
        static_cast<const uint16_t*>(v), L.page_table, L.seq_lens, kept, kept_count,
        kept_stride, L.units(), L.Hkv, L.max_pages, L.num_phys, scale_log2, part_o, part_ml,
        n_chunks, ch, static_cast<uint16_t*>(out));
  }
}

template <int D>
void decode_dispatch_g(const Layout& L, const void* q, const void* k, const void* v,
                       const int32_t* kept, const int32_t* kept_count, int kept_stride,
                       float scale_log2, float* part_o, float2* part_ml, int n_chunks, int ch,
                       void* out, hipStream_t s) {
  switch (L.unit_G()) {
    case 1: decode_launch<D, 1>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, part_o, part_ml, n_chunks, ch, out, s); break;
    case 2: decode_launch<D, 2>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, part_o, part_ml, n_chunks, ch, out, s); break;
    case 4: decode_launch<D, 4>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, part_o, part_ml, n_chunks, ch, out, s); break;
    default: decode_launch<D, 8>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, part_o, part_ml, n_chunks, ch, out, s); break;
  }
}

}  // namespace

int decode_chunk_tokens(const Layout& L, int kept_stride) {
  // about TWL_DEC_TARGET_BLOCKS work-groups over the largest possible kept lists: one to
  // TWL_DEC_MAX_BATCHES batches per work-group, but a full-length list still in at least
  // TWL_DEC_MIN_CHUNKS chunks (TWL_DEC_MIN_CHUNKS_FEW when the step has few units), so that
  // lists only partly full (short sequences, strong pruning) keep several work-groups each.
  // Long lists then take long chunks: fewer partials to write and merge. (Measured: the
  // 128k GQA step's 8 units take 128-token chunks, 1.2 us faster than 64; the 32k MHA
  // step's 32 units keep 64-token chunks, 0.4 us faster than 128.)
  const long units = static_cast<long>(L.B) * L.units();
  const long want =
      (static_cast<long>(kept_stride) * units + TWL_DEC_TARGET_BLOCKS - 1) / TWL_DEC_TARGET_BLOCKS;
  const long min_chunks = units <= TWL_DEC_FEW_UNITS ? TWL_DEC_MIN_CHUNKS_FEW : TWL_DEC_MIN_CHUNKS;
  const int batch = decode_batch_tokens(L.d);
  long c = batch;
  while (c < want && c < static_cast<long>(batch) * TWL_DEC_MAX_BATCHES &&
         2 * c * min_chunks <= kept_stride)
    c <<= 1;
  return static_cast<int>(c);
}

size_t decode_workspace_bytes(const Layout& L, int kept_stride) {
  const int ch = decode_chunk_tokens(L, kept_stride);
  const long n_chunks = (static_cast<long>(kept_stride) + ch - 1) / ch;
  // o records [B * Hq, n_chunks, d], then (max, sum) pairs [B * Hq, n_chunks]
  return align_up(static_cast<size_t>(L.B) * L.Hq * n_chunks * (L.d + 2) * sizeof(float), 256);
}

hipError_t launch_sparse_decode(const Layout& L, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* kept,
                                const int32_t* kept_count, int kept_stride, float sm_scale,
                                void* out, void* ws, hipStream_t s) {
  const int ch = decode_chunk_tokens(L, kept_stride);
  const int n_chunks = (kept_stride + ch - 1) / ch;
  auto* part_o = static_cast<float*>(stage_scratch(ws, L));
  auto* part_ml = reinterpret_cast<float2*>(part_o + static_cast<long>(L.B) * L.Hq * n_chunks * L.d);
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (L.d == 128) {
    decode_dispatch_g<128>(L, q, k_cache, v_cache, kept, kept_count, kept_stride, scale_log2,
                           part_o, part_ml, n_chunks, ch, out, s);
  } else {
    decode_dispatch_g<64>(L, q, k_cache, v_cache, kept, kept_count, kept_stride, scale_log2,
                          part_o, part_ml, n_chunks, ch, out, s);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto* o = static_cast<uint16_t*>(out);
  const dim3 grid(L.d / kMergeSlice, L.Hq, L.B);
  if (L.d == 128) {
    decode_merge_kernel<128><<<grid, kWave, 0, s>>>(part_o, part_ml, kept_count, kept_stride,
                                                    L.units(), L.unit_G(), n_chunks, ch, o);
  } else {
    decode_merge_kernel<64><<<grid, kWave, 0, s>>>(part_o, part_ml, kept_count, kept_stride,
                                                    L.units(), L.unit_G(), n_chunks, ch, o);
  }
  return hipGetLastError();
}

}  // namespace twl
