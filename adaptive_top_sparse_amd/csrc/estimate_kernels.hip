// Twilight's attention-weight estimate over the candidate tokens from the int4 key cache
// (Twilight pages, atlas.scime.ai summary "Approach": top-p runs on estimated weights of
// the pre-selected tokens, computed from a 4-bit quantized key cache; "Limitations": the
// estimate's own cost matters when token loading is not the bottleneck).
//
// Per candidate token j and query head h of the group:
//   s_hj = sm_scale * sum_groups [zero * Q_grp,h + scale * sum_{c in grp} q_hc * code_c],
// with Q_grp,h = sum_{c in grp} q_hc, the same value as q_h . dequant(k_j). Then a softmax
// over the unit's valid candidates, done as per-chunk (max, sum of exp) partials followed
// by a normalization pass.
#include "twl_device.h"
#include "twl_launch.h"

TWL_PHASE_STORAGE(estimate)

namespace twl {
namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

constexpr int kEstWaves = kEstChunk / kWave;             // 4
constexpr int kPagesPerWave = kEstChunk / kPage / kEstWaves;  // candidate pages per wave

// The per-group dot products on the matrix cores: one v_mfma_f32_16x16x16_f16 takes a
// 16-token tile (one candidate page) and 16 channels of a 32-channel group, with
//   A = the group's query heads (rows, padded to 16 with zeros) x channels,
//   B = channels x the tile's tokens (the 4-bit codes as exact fp16 integers),
// and leaves D[head][token] in fp32: lane l holds heads 4(l/16)..+3 of token l%16. Lane l
// feeds channel slots 4(l/16)..+3, which are permuted so that the codes unpack cheaply:
// lane group c4 = l/16 covers channels 8 c4 .. 8 c4 + 7 of the group (one 32-bit word of
// codes), slot order {0,4,1,5} in the first and {2,6,3,7} in the second instruction. A dot
// product is invariant to a common permutation of both operands, and every product of an
// fp16 q and a code is exact in fp32.
__device__ __forceinline__ int mfma_channel(int c4, int m, int e) {
  constexpr int kPerm[2][4] = {{0, 4, 1, 5}, {2, 6, 3, 7}};
  return 8 * c4 + kPerm[m][e];
}

// Two fp16 codes from the nibble pair at bits [3:0] and [19:16]: 1024 + n is exact in fp16
// (its ulp is 1), so or-ing n into the significand of 1024 and subtracting 1024 gives n.
__device__ __forceinline__ uint32_t codes_to_f16x2(uint32_t pair_bits) {
  const f16x2 v = __builtin_bit_cast(f16x2, pair_bits | 0x64006400u);
  const f16x2 r = v - f16x2{static_cast<f16>(1024.f), static_cast<f16>(1024.f)};
  return __builtin_bit_cast(uint32_t, r);
}

// One block per kEstChunk candidate slots (16 pages) of a (sequence, KV head); wave w takes
// pages 4w..4w+3 of the chunk, one MFMA tile each.
template <int D, int G>
__global__ __launch_bounds__(kEstChunk) void estimate_logits_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint32_t* __restrict__ meta, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cand_pages,
    const int32_t* __restrict__ cand_count, int cand_stride_pages, int Hkv, int max_pages,
    int num_phys, float sm_scale, float* __restrict__ logits, float2* __restrict__ partials,
    int n_chunks) {
  constexpr int NG = D / 32;
  constexpr int HR = G < 4 ? G : 4;  // heads per lane (rows 4(l/16)..+3 that exist)
  static_assert(G <= 8, "at most 8 query heads per KV head");
  __shared__ f16 qs[G][D];
  __shared__ float qsum[G][NG];
  __shared__ float red_m[kEstWaves][G], red_l[kEstWaves][G];
  TWL_PHASE(0);
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int chunk = blockIdx.x;
  const int Hq = Hkv * G;
  const long unit = static_cast<long>(b) * Hkv + g;
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int tok_in_page = lane % 16;
  const int c4 = lane / 16;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int n_slots = cand_stride_pages * kPage;

  // this wave's pages: candidate rank -> page id -> physical page (wave-uniform loads; the
  // page ids are read before the candidate count is known, from inside the row)
  int rank[kPagesPerWave], pid[kPagesPerWave], phys[kPagesPerWave];
#pragma unroll
  for (int i = 0; i < kPagesPerWave; ++i) {
    rank[i] = (chunk * kEstWaves + wave) * kPagesPerWave + i;
    if (cand_pages == nullptr) {
      pid[i] = rank[i];
    } else {
      const int r = rank[i] < cand_stride_pages ? rank[i] : 0;
      pid[i] = cand_pages[unit * cand_stride_pages + r];
    }
  }
  int cnt = cand_stride_pages;
  if (cand_pages != nullptr) {
    cnt = cand_count ? cand_count[unit] : (n + kPage - 1) / kPage;
    cnt = cnt < cand_stride_pages ? cnt : cand_stride_pages;
  }
#pragma unroll
  for (int i = 0; i < kPagesPerWave; ++i) {
    const bool ok = rank[i] < cnt && pid[i] >= 0 && pid[i] < max_pages && pid[i] * kPage < n;
    pid[i] = ok ? pid[i] : -1;
    phys[i] = page_table[static_cast<long>(b) * max_pages + (ok ? pid[i] : 0)];
  }
  // codes (one word per group) and {scale, zero} of this lane's token in each page
  uint32_t cw[kPagesPerWave][NG], mw[kPagesPerWave][NG];
#pragma unroll
  for (int i = 0; i < kPagesPerWave; ++i) {
    const bool ok = pid[i] >= 0 && phys_ok(phys[i], num_phys);
    const long row = ok ? (static_cast<long>(phys[i]) * Hkv + g) * kPage + tok_in_page : 0;
    const uint32_t* crow = reinterpret_cast<const uint32_t*>(codes + row * (D / 2));
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      cw[i][grp] = crow[grp * 4 + c4];
      mw[i][grp] = meta[row * NG + grp];
    }
    if (!ok) pid[i] = -1;
  }

  // the group's queries and their per-group sums
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D, c = i % D;
    qs[h][c] = __builtin_bit_cast(f16, q[(static_cast<long>(b) * Hq + g * G + h) * D + c]);
  }
  __syncthreads();
  if (threadIdx.x < G * NG) {
    const int h = threadIdx.x / NG, grp = threadIdx.x % NG;
    float acc = 0.f;
    for (int c = 0; c < 32; ++c) acc += static_cast<float>(qs[h][grp * 32 + c]);
    qsum[h][grp] = acc;
  }
  __syncthreads();
  // A operands: row = head lane%16 (zero past G), channel slots as in mfma_channel
  f16x4 qa[NG][2];
  const int qh = lane % 16;
#pragma unroll
  for (int grp = 0; grp < NG; ++grp)
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qa[grp][m][e] = qh < G ? qs[qh < G ? qh : 0][grp * 32 + mfma_channel(c4, m, e)]
                               : static_cast<f16>(0.f);
  float qg[NG][HR];  // Q_grp of this lane's output heads 4 c4 + r
#pragma unroll
  for (int grp = 0; grp < NG; ++grp)
#pragma unroll
    for (int r = 0; r < HR; ++r) {
      const int h = 4 * c4 + r;
      qg[grp][r] = h < G ? qsum[h < G ? h : 0][grp] : 0.f;
    }
  TWL_PHASE(1);

  const int wave_slot0 = (chunk * kEstWaves + wave) * kPagesPerWave * kPage;
  float s[kPagesPerWave][HR];
#pragma unroll
  for (int i = 0; i < kPagesPerWave; ++i) {
    float acc[HR];
#pragma unroll
    for (int r = 0; r < HR; ++r) acc[r] = 0.f;
#pragma unroll
    for (int grp = 0; grp < NG; ++grp) {
      const uint32_t w = cw[i][grp];
      uint32_t bw[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) bw[k] = codes_to_f16x2((w >> (4 * k)) & 0x000f000fu);
      const f16x4 b0 = __builtin_bit_cast(f16x4, u32x2{bw[0], bw[1]});
      const f16x4 b1 = __builtin_bit_cast(f16x4, u32x2{bw[2], bw[3]});
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      d = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[grp][0], b0, d, 0, 0, 0);
      d = __builtin_amdgcn_mfma_f32_16x16x16f16(qa[grp][1], b1, d, 0, 0, 0);
      const float scale = h2f(static_cast<uint16_t>(mw[i][grp] & 0xffffu));
      const float zero = h2f(static_cast<uint16_t>(mw[i][grp] >> 16));
#pragma unroll
      for (int r = 0; r < HR; ++r) acc[r] = fmaf(scale, d[r], fmaf(zero, qg[grp][r], acc[r]));
    }
    const int t = pid[i] * kPage + tok_in_page;
    const bool valid = pid[i] >= 0 && t < n;
#pragma unroll
    for (int r = 0; r < HR; ++r) s[i][r] = valid ? sm_scale * acc[r] : -INFINITY;
  }
  TWL_PHASE(2);
  // logits rows, then (max, sum exp) of this chunk per head
  const bool head_lane = 4 * c4 < G;
#pragma unroll
  for (int i = 0; i < kPagesPerWave; ++i) {
    const int slot = wave_slot0 + i * kPage + tok_in_page;
    if (head_lane && slot < n_slots) {
#pragma unroll
      for (int r = 0; r < HR; ++r) {
        const int h = 4 * c4 + r;
        if (h < G) logits[(static_cast<long>(b) * Hq + g * G + h) * n_slots + slot] = s[i][r];
      }
    }
  }
  // per head: max over this wave's 64 slots (4 pages in registers, 16 tokens across the row)
  float wm[HR];
#pragma unroll
  for (int r = 0; r < HR; ++r) {
    float v = s[0][r];
#pragma unroll
    for (int i = 1; i < kPagesPerWave; ++i) v = fmaxf(v, s[i][r]);
    wm[r] = group_reduce<16>(v, OpMax());
  }
  if (head_lane && tok_in_page == 0) {
#pragma unroll
    for (int r = 0; r < HR; ++r)
      if (4 * c4 + r < G) red_m[wave][4 * c4 + r] = wm[r];
  }
  __syncthreads();
  float e_sum[HR];
  float M[HR];
#pragma unroll
  for (int r = 0; r < HR; ++r) {
    const int h = 4 * c4 + r < G ? 4 * c4 + r : 0;
    float m = red_m[0][h];
#pragma unroll
    for (int w2 = 1; w2 < kEstWaves; ++w2) m = fmaxf(m, red_m[w2][h]);
    M[r] = m;
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < kPagesPerWave; ++i)
      acc += (s[i][r] > -INFINITY && m > -INFINITY) ? expf(s[i][r] - m) : 0.f;
    e_sum[r] = group_reduce<16>(acc, OpSum());
  }
  if (head_lane && tok_in_page == 0) {
#pragma unroll
    for (int r = 0; r < HR; ++r)
      if (4 * c4 + r < G) red_l[wave][4 * c4 + r] = e_sum[r];
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float m = red_m[0][h], l = 0.f;
#pragma unroll
    for (int w2 = 1; w2 < kEstWaves; ++w2) m = fmaxf(m, red_m[w2][h]);
#pragma unroll
    for (int w2 = 0; w2 < kEstWaves; ++w2) l += red_l[w2][h];
    partials[(static_cast<long>(b) * Hq + g * G + h) * n_chunks + chunk] = make_float2(m, l);
  }
  (void)M;
  TWL_PHASE(3);
}

// w = exp(s - M) / L with (M, L) merged from the row's chunk partials; invalid slots hold
// s = -inf and come out as exactly 0.
__global__ __launch_bounds__(kEstChunk) void estimate_normalize_kernel(
    float* __restrict__ weights, const float2* __restrict__ partials, int n_chunks, int n_slots) {
  __shared__ float red[kEstChunk / kWave];
  const long hrow = static_cast<long>(blockIdx.y) * gridDim.z + blockIdx.z;
  const int slot = blockIdx.x * kEstChunk + threadIdx.x;
  float* w = weights + hrow * n_slots + slot;
  const float s = slot < n_slots ? *w : -INFINITY;  // issued before the partials
  const float2* pr = partials + hrow * n_chunks;
  float m = -INFINITY, l = 0.f;
  // this thread's share of the chunk partials, merged on the fly
  for (int i = threadIdx.x; i < n_chunks; i += blockDim.x) {
    const float2 v = pr[i];
    if (v.x > -INFINITY) {
      const float mn = fmaxf(m, v.x);
      l = (m > -INFINITY ? l * expf(m - mn) : 0.f) + v.y * expf(v.x - mn);
      m = mn;
    }
  }
  const float M = block_max<kEstChunk>(m, red);
  const float L = block_sum<kEstChunk>(m > -INFINITY ? l * expf(m - M) : 0.f, red);
  if (slot >= n_slots) return;
  *w = (L > 0.f && s > -INFINITY) ? expf(s - M) / L : 0.f;
}

template <int D, int G>
void logits_launch(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                   const int32_t* cand_pages, const int32_t* cand_count, int stride,
                   float sm_scale, float* weights, float2* partials, int n_chunks,
                   hipStream_t s) {
  estimate_logits_kernel<D, G><<<dim3(n_chunks, L.Hkv, L.B), kEstChunk, 0, s>>>(
      static_cast<const uint16_t*>(q), codes, static_cast<const uint32_t*>(meta), L.page_table,
      L.seq_lens, cand_pages, cand_count, stride, L.Hkv, L.max_pages, L.num_phys, sm_scale,
      weights, partials, n_chunks);
}

template <int D>
void logits_dispatch_g(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                       const int32_t* cand_pages, const int32_t* cand_count, int stride,
                       float sm_scale, float* weights, float2* partials, int n_chunks,
                       hipStream_t s) {
  switch (L.G()) {
    case 1: logits_launch<D, 1>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, n_chunks, s); break;
    case 2: logits_launch<D, 2>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, n_chunks, s); break;
    case 4: logits_launch<D, 4>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, n_chunks, s); break;
    default: logits_launch<D, 8>(L, q, codes, meta, cand_pages, cand_count, stride, sm_scale, weights, partials, n_chunks, s); break;
  }
}

}  // namespace

size_t estimate_workspace_bytes(const Layout& L, int cand_stride_pages) {
  const long n_slots = static_cast<long>(cand_stride_pages) * kPage;
  const long n_chunks = (n_slots + kEstChunk - 1) / kEstChunk;
  return align_up(static_cast<size_t>(L.B) * L.Hq * n_chunks * sizeof(float2), 256);
}

hipError_t launch_estimate(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                           const int32_t* cand_pages, const int32_t* cand_count,
                           int cand_stride_pages, float sm_scale, float* weights, void* ws,
                           hipStream_t s) {
  const int n_slots = cand_stride_pages * kPage;
  const int n_chunks = (n_slots + kEstChunk - 1) / kEstChunk;
  float2* partials = static_cast<float2*>(stage_scratch(ws, L));
  if (L.d == 128) {
    logits_dispatch_g<128>(L, q, codes, meta, cand_pages, cand_count, cand_stride_pages,
                           sm_scale, weights, partials, n_chunks, s);
  } else {
    logits_dispatch_g<64>(L, q, codes, meta, cand_pages, cand_count, cand_stride_pages,
                          sm_scale, weights, partials, n_chunks, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  estimate_normalize_kernel<<<dim3(n_chunks, L.B, L.Hq), kEstChunk, 0, s>>>(weights, partials,
                                                                          n_chunks, n_slots);
  return hipGetLastError();
}

}  // namespace twl
