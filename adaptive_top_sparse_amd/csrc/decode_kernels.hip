// Sparse paged decode attention over the kept tokens (Twilight pages, atlas.scime.ai
// summary "Key results": the Twilight sparse self-attention operator, which attends only to
// the tokens that survive pruning).
//
// For each query head h of KV head g: o_h = sum_{j in kept} softmax_j(sm_scale q_h . k_j) v_j
// on the fp16 cache, the softmax over the kept set only. Split-KV: each work-group takes a
// chunk of the kept list and leaves (max, sum, unnormalized o) in log2 units; a merge kernel
// combines the chunks and rounds to fp16.
//
// Layout on the device: D/8 lanes per kept token, 8 channels (16 B of K, 16 B of V) per lane,
// so one wave gathers 64/(D/8) token rows per load instruction, each row one contiguous
// 2*D-byte stretch of the paged cache. q . k uses v_dot2_f32_f16 on fp16 pairs (exact
// products, fp32 sums); the softmax and p * v run in fp32.
#include "twl_device.h"
#include "twl_launch.h"

namespace twl {
namespace {

constexpr int kDecThreads = 256;
constexpr int kDecWaves = kDecThreads / kWave;
constexpr int kDecUnroll = 4;

__device__ __forceinline__ float rescale(float m, float M) {
  return m == -INFINITY ? 0.f : exp2f(m - M);
}

__device__ __forceinline__ f16x2 as_h2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }

template <int D, int G>
__global__ __launch_bounds__(kDecThreads) void decode_partial_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ kept,
    const int32_t* __restrict__ kept_count, int kept_stride, int Hkv, int max_pages,
    int num_phys, float scale_log2, float* __restrict__ partials, int n_chunks,
    int chunk_tokens) {
  constexpr int LPT = D / 8;      // lanes per token row
  constexpr int TPW = kWave / LPT;  // token rows per wave per load
  constexpr int STEP = TPW * kDecUnroll;
  __shared__ float s_m[kDecWaves][G], s_l[kDecWaves][G];
  __shared__ float s_acc[kDecWaves][G][D];

  const int b = blockIdx.z;
  const int g = blockIdx.y;
  const int chunk = blockIdx.x;
  const long unit = static_cast<long>(b) * Hkv + g;
  int K = kept_count[unit];
  K = K < 0 ? 0 : (K > kept_stride ? kept_stride : K);
  const int t0 = chunk * chunk_tokens;
  if (t0 >= K) return;
  const int t1 = min(K, t0 + chunk_tokens);
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int Hq = Hkv * G;
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int sub = lane % LPT;
  const int tk = lane / LPT;
  const int c0 = sub * 8;

  uint32_t qw[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(q + (static_cast<long>(b) * Hq + g * G + h) * D + c0);
#pragma unroll
    for (int j = 0; j < 4; ++j) qw[h][j] = v[j];
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[h][c] = 0.f;
  }
  const int32_t* krow = kept + unit * kept_stride;
  const int32_t* trow = page_table + static_cast<long>(b) * max_pages;

  for (int base = t0 + wave * STEP; base < t1; base += kDecWaves * STEP) {
    u32x4 kv[kDecUnroll], vv[kDecUnroll];
    bool ok[kDecUnroll];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
      const int t = base + u * TPW + tk;
      int tok = t < t1 ? krow[t] : -1;
      bool good = tok >= 0 && tok < n;
      const int phys = good ? trow[tok / kPage] : -1;
      good = good && phys_ok(phys, num_phys);
      ok[u] = good;
      if (good) {
        const long row = ((static_cast<long>(phys) * Hkv + g) * kPage + tok % kPage) * D + c0;
        kv[u] = *reinterpret_cast<const u32x4*>(k_cache + row);
        vv[u] = *reinterpret_cast<const u32x4*>(v_cache + row);
      } else {
        kv[u] = u32x4{0u, 0u, 0u, 0u};
        vv[u] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    float s[kDecUnroll][G];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float d = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j)
          d = __builtin_amdgcn_fdot2(as_h2(qw[h][j]), as_h2(kv[u][j]), d, false);
#pragma unroll
        for (int o = LPT / 2; o > 0; o >>= 1) d += __shfl_xor(d, o);
        s[u][h] = ok[u] ? d * scale_log2 : -INFINITY;
      }
    }
    float vf[kDecUnroll][8];
#pragma unroll
    for (int u = 0; u < kDecUnroll; ++u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 p2 = as_h2(vv[u][j]);
        vf[u][2 * j] = static_cast<float>(p2[0]);
        vf[u][2 * j + 1] = static_cast<float>(p2[1]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mb = s[0][h];
#pragma unroll
      for (int u = 1; u < kDecUnroll; ++u) mb = fmaxf(mb, s[u][h]);
      const float mn = fmaxf(m[h], mb);
      if (mn == -INFINITY) continue;
      const float alpha = rescale(m[h], mn);
      l[h] *= alpha;
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[h][c] *= alpha;
#pragma unroll
      for (int u = 0; u < kDecUnroll; ++u) {
        const float pr = rescale(s[u][h], mn);
        l[h] += pr;
#pragma unroll
        for (int c = 0; c < 8; ++c) acc[h][c] = fmaf(pr, vf[u][c], acc[h][c]);
      }
      m[h] = mn;
    }
  }

  // merge the TPW token lanes of each channel slice inside the wave
#pragma unroll
  for (int o = LPT; o < kWave; o <<= 1) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float mo = __shfl_xor(m[h], o);
      const float lo = __shfl_xor(l[h], o);
      const float M = fmaxf(m[h], mo);
      const float a = rescale(m[h], M), bb = rescale(mo, M);
      l[h] = l[h] * a + lo * bb;
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        const float ao = __shfl_xor(acc[h][c], o);
        acc[h][c] = acc[h][c] * a + ao * bb;
      }
      m[h] = M;
    }
  }
  if (tk == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      if (sub == 0) {
        s_m[wave][h] = m[h];
        s_l[wave][h] = l[h];
      }
#pragma unroll
      for (int c = 0; c < 8; ++c) s_acc[wave][h][c0 + c] = acc[h][c];
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < G * D; i += kDecThreads) {
    const int h = i / D, c = i % D;
    float M = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = rescale(s_m[w][h], M);
      L += s_l[w][h] * f;
      A += s_acc[w][h][c] * f;
    }
    float* dst = partials + ((static_cast<long>(b) * Hq + g * G + h) * n_chunks + chunk) * (D + 2);
    if (c == 0) {
      dst[0] = M;
      dst[1] = L;
    }
    dst[2 + c] = A;
  }
}

// One work-group of D threads per (sequence, query head): lane c merges channel c.
template <int D>
__global__ __launch_bounds__(D) void decode_merge_kernel(
    const float* __restrict__ partials, const int32_t* __restrict__ kept_count, int kept_stride,
    int Hkv, int G, int n_chunks, int chunk_tokens, uint16_t* __restrict__ out) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int Hq = Hkv * G;
  const long unit = static_cast<long>(b) * Hkv + h / G;
  int K = kept_count[unit];
  K = K < 0 ? 0 : (K > kept_stride ? kept_stride : K);
  const int nc = (K + chunk_tokens - 1) / chunk_tokens;
  const int c = threadIdx.x;
  const float* pr = partials + (static_cast<long>(b) * Hq + h) * n_chunks * (D + 2);
  float M = -INFINITY;
  for (int i = 0; i < nc; ++i) M = fmaxf(M, pr[i * (D + 2)]);
  float L = 0.f, A = 0.f;
  for (int i = 0; i < nc; ++i) {
    const float f = rescale(pr[i * (D + 2)], M);
    L += pr[i * (D + 2) + 1] * f;
    A += pr[i * (D + 2) + 2 + c] * f;
  }
  const float o = L > 0.f ? A / L : 0.f;
  out[(static_cast<long>(b) * Hq + h) * D + c] = __builtin_bit_cast(uint16_t, static_cast<f16>(o));
}

template <int D, int G>
void partial_launch(const Layout& L, const void* q, const void* k, const void* v,
                    const int32_t* kept, const int32_t* kept_count, int kept_stride,
                    float scale_log2, float* partials, int n_chunks, int ch, hipStream_t s) {
  decode_partial_kernel<D, G><<<dim3(n_chunks, L.Hkv, L.B), kDecThreads, 0, s>>>(
      static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
      static_cast<const uint16_t*>(v), L.page_table, L.seq_lens, kept, kept_count, kept_stride,
      L.Hkv, L.max_pages, L.num_phys, scale_log2, partials, n_chunks, ch);
}

template <int D>
void partial_dispatch_g(const Layout& L, const void* q, const void* k, const void* v,
                        const int32_t* kept, const int32_t* kept_count, int kept_stride,
                        float scale_log2, float* partials, int n_chunks, int ch, hipStream_t s) {
  switch (L.G()) {
    case 1: partial_launch<D, 1>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, partials, n_chunks, ch, s); break;
    case 2: partial_launch<D, 2>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, partials, n_chunks, ch, s); break;
    case 4: partial_launch<D, 4>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, partials, n_chunks, ch, s); break;
    default: partial_launch<D, 8>(L, q, k, v, kept, kept_count, kept_stride, scale_log2, partials, n_chunks, ch, s); break;
  }
}

}  // namespace

int decode_chunk_tokens(const Layout& L, int kept_stride) {
  // aim at about 2048 work-groups over the largest possible kept lists
  const long units = static_cast<long>(L.B) * L.Hkv;
  long ch = (static_cast<long>(kept_stride) * units + 2047) / 2048;
  long c = 64;
  while (c < ch && c < 2048) c <<= 1;
  return static_cast<int>(c);
}

size_t decode_workspace_bytes(const Layout& L, int kept_stride) {
  const int ch = decode_chunk_tokens(L, kept_stride);
  const long n_chunks = (static_cast<long>(kept_stride) + ch - 1) / ch;
  return align_up(static_cast<size_t>(L.B) * L.Hq * n_chunks * (L.d + 2) * sizeof(float), 256);
}

hipError_t launch_sparse_decode(const Layout& L, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* kept,
                                const int32_t* kept_count, int kept_stride, float sm_scale,
                                void* out, void* ws, hipStream_t s) {
  const int ch = decode_chunk_tokens(L, kept_stride);
  const int n_chunks = (kept_stride + ch - 1) / ch;
  float* partials = static_cast<float*>(ws);
  const float scale_log2 = sm_scale * 1.4426950408889634f;
  if (L.d == 128) {
    partial_dispatch_g<128>(L, q, k_cache, v_cache, kept, kept_count, kept_stride, scale_log2,
                            partials, n_chunks, ch, s);
  } else {
    partial_dispatch_g<64>(L, q, k_cache, v_cache, kept, kept_count, kept_stride, scale_log2,
                           partials, n_chunks, ch, s);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  auto* o = static_cast<uint16_t*>(out);
  if (L.d == 128) {
    decode_merge_kernel<128><<<dim3(L.Hq, L.B), 128, 0, s>>>(partials, kept_count, kept_stride,
                                                             L.Hkv, L.G(), n_chunks, ch, o);
  } else {
    decode_merge_kernel<64><<<dim3(L.Hq, L.B), 64, 0, s>>>(partials, kept_count, kept_stride,
                                                           L.Hkv, L.G(), n_chunks, ch, o);
  }
  return hipGetLastError();
}

}  // namespace twl
