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

// One lane per candidate slot, kEstChunk slots per block. The query group (G x D) and its
// per-group sums sit in LDS as fp32 and are read as broadcasts.
template <int D, int G>
__global__ __launch_bounds__(kEstChunk) void estimate_logits_kernel(
    const uint16_t* __restrict__ q, const uint8_t* __restrict__ codes,
    const uint32_t* __restrict__ meta, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ cand_pages,
    const int32_t* __restrict__ cand_count, int cand_stride_pages, int Hkv, int max_pages,
    int num_phys, float sm_scale, float* __restrict__ logits, float2* __restrict__ partials,
    int n_chunks) {
  constexpr int NG = D / 32;
  constexpr int Hq_per = G;
  __shared__ float qs[G][D];
  __shared__ float qsum[G][NG];
  TWL_PHASE(0);
  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int chunk = blockIdx.x;
  const int Hq = Hkv * G;
  const long unit = static_cast<long>(b) * Hkv + g;

  for (int i = threadIdx.x; i < G * D; i += blockDim.x) {
    const int h = i / D, c = i % D;
    qs[h][c] = h2f(q[(static_cast<long>(b) * Hq + g * Hq_per + h) * D + c]);
  }
  __syncthreads();
  if (threadIdx.x < G * NG) {
    const int h = threadIdx.x / NG, grp = threadIdx.x % NG;
    float acc = 0.f;
    for (int c = 0; c < 32; ++c) acc += qs[h][grp * 32 + c];
    qsum[h][grp] = acc;
  }
  __syncthreads();

  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int n_slots = cand_stride_pages * kPage;
  const int slot = chunk * kEstChunk + threadIdx.x;
  int tok = -1;
  if (slot < n_slots) {
    if (cand_pages == nullptr) {
      tok = slot;
    } else {
      int cnt = cand_count ? cand_count[unit] : (n + kPage - 1) / kPage;
      cnt = cnt < cand_stride_pages ? cnt : cand_stride_pages;
      const int r = slot / kPage;
      if (r < cnt) {
        const int pg = cand_pages[unit * cand_stride_pages + r];
        tok = pg >= 0 ? pg * kPage + slot % kPage : -1;
      }
    }
  }
  TWL_PHASE(1);
  bool valid = tok >= 0 && tok < n;
  float s[G];
#pragma unroll
  for (int h = 0; h < G; ++h) s[h] = -INFINITY;
  if (valid) {
    const int phys = page_table[static_cast<long>(b) * max_pages + tok / kPage];
    valid = phys_ok(phys, num_phys);
    if (valid) {
      const long row = (static_cast<long>(phys) * Hkv + g) * kPage + tok % kPage;
      const u32x4* crow = reinterpret_cast<const u32x4*>(codes + row * (D / 2));
      u32x4 cw[NG];
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) cw[grp] = crow[grp];
      uint32_t mw[NG];
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) mw[grp] = meta[row * NG + grp];
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
      for (int grp = 0; grp < NG; ++grp) {
        float dot[G];
#pragma unroll
        for (int h = 0; h < G; ++h) dot[h] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t word = cw[grp][w];
          const uint32_t lo = word & 0x0f0f0f0fu;         // channels 0,2,4,6 of the word
          const uint32_t hi = (word >> 4) & 0x0f0f0f0fu;  // channels 1,3,5,7
          float cv[8];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            cv[2 * j] = static_cast<float>((lo >> (8 * j)) & 0xffu);
            cv[2 * j + 1] = static_cast<float>((hi >> (8 * j)) & 0xffu);
          }
          const int cbase = grp * 32 + w * 8;
#pragma unroll
          for (int h = 0; h < G; ++h) {
#pragma unroll
            for (int j = 0; j < 8; ++j) dot[h] = fmaf(qs[h][cbase + j], cv[j], dot[h]);
          }
        }
        const float scale = h2f(static_cast<uint16_t>(mw[grp] & 0xffffu));
        const float zero = h2f(static_cast<uint16_t>(mw[grp] >> 16));
#pragma unroll
        for (int h = 0; h < G; ++h) acc[h] = fmaf(scale, dot[h], fmaf(zero, qsum[h][grp], acc[h]));
      }
#pragma unroll
      for (int h = 0; h < G; ++h) s[h] = sm_scale * acc[h];
    }
  }
  // logits row, then (max, sum exp) of this chunk per head: one max pass and one sum pass
  // for all G heads
  __shared__ float red_m[kEstChunk / kWave][G], red_l[kEstChunk / kWave][G];
  const int wave = threadIdx.x / kWave;
  TWL_PHASE(2);
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const long hrow = static_cast<long>(b) * Hq + g * G + h;
    if (slot < n_slots) logits[hrow * n_slots + slot] = s[h];
    const float wm = wave_max(s[h]);
    if (lane_id() == 0) red_m[wave][h] = wm;
  }
  __syncthreads();
  float e[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float m = red_m[0][h];
#pragma unroll
    for (int w = 1; w < kEstChunk / kWave; ++w) m = fmaxf(m, red_m[w][h]);
    e[h] = (valid && m > -INFINITY) ? expf(s[h] - m) : 0.f;
    const float ws = wave_sum(e[h]);
    if (lane_id() == 0) red_l[wave][h] = ws;
  }
  __syncthreads();
  if (threadIdx.x < G) {
    const int h = threadIdx.x;
    float m = red_m[0][h], l = 0.f;
#pragma unroll
    for (int w = 1; w < kEstChunk / kWave; ++w) m = fmaxf(m, red_m[w][h]);
#pragma unroll
    for (int w = 0; w < kEstChunk / kWave; ++w) l += red_l[w][h];
    const long hrow = static_cast<long>(b) * Hq + g * G + h;
    partials[hrow * n_chunks + chunk] = make_float2(m, l);
  }
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
