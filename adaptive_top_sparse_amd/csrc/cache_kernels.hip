// Cache maintenance: the int4 key cache used by Twilight's weight estimate and Quest's
// per-page channelwise key bounds (Twilight pages, atlas.scime.ai summary: "Approach" for
// the 4-bit key cache, "Surprising findings" for Quest's per-page max-pooled layout).
// Neither runs inside a decode step's hot loop; both run at prefill and then once per
// appended token (token_begin).
#include "twl_device.h"
#include "twl_launch.h"

namespace twl {
namespace {

// One lane per (token, 32-channel group). A wave covers one (page, KV head) block of
// 16 tokens x d channels when d = 128 (64 lanes = 16 tokens x 4 groups), so its loads are
// one contiguous 4 KiB stretch.
//
// zero = min (the first occurrence of the minimum's bit pattern), scale = the fp16 nearest
// to (max - min) / 15 (fp64 quotient, one RNE rounding to fp16), and
// code = clamp(rint((x - zero) / scale), 0, 15) in fp64. fp64 decides every code exactly:
// (x - zero) and scale are multiples of 2^-24 below 2^17, so a quotient that is not a
// half-integer lies at least 2^-41 away from one, far beyond the fp64 quotient's error;
// half-integers are exact and rint sends them to the even code.
template <int D>
__global__ __launch_bounds__(256) void quantize_keys_kernel(
    const uint16_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ token_begin, int Hkv,
    int max_pages, int num_phys, uint8_t* __restrict__ codes, uint32_t* __restrict__ meta) {
  constexpr int NG = D / 32;
  const int b = blockIdx.y;
  const long item = static_cast<long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int g = static_cast<int>(item % NG);
  const int slot = static_cast<int>((item / NG) % kPage);
  const int kvh = static_cast<int>((item / (NG * kPage)) % Hkv);
  const long page = item / (static_cast<long>(NG) * kPage * Hkv);
  if (page >= max_pages) return;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int tok = static_cast<int>(page) * kPage + slot;
  const int begin = token_begin ? token_begin[b] : 0;
  if (tok >= n || tok < begin) return;
  const int phys = page_table[static_cast<long>(b) * max_pages + page];
  if (!phys_ok(phys, num_phys)) return;
  const long row = (static_cast<long>(phys) * Hkv + kvh) * kPage + slot;

  const u32x4* src = reinterpret_cast<const u32x4*>(k_cache + row * D + g * 32);
  uint16_t x[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const u32x4 v = src[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[i * 8 + j * 2] = static_cast<uint16_t>(v[j] & 0xffffu);
      x[i * 8 + j * 2 + 1] = static_cast<uint16_t>(v[j] >> 16);
    }
  }
  float mn = h2f(x[0]), mx = mn;
  uint16_t mn_bits = x[0];
#pragma unroll
  for (int c = 1; c < 32; ++c) {
    const float v = h2f(x[c]);
    if (v < mn) {
      mn = v;
      mn_bits = x[c];
    }
    mx = fmaxf(mx, v);
  }
  const double zero = static_cast<double>(mn);
  const uint16_t s_bits = f64_to_f16_bits_nonneg((static_cast<double>(mx) - zero) / 15.0);
  const double s = static_cast<double>(h2f(s_bits));
  uint32_t packed[4] = {0u, 0u, 0u, 0u};
  if (s > 0.0) {
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      double code = rint((static_cast<double>(h2f(x[c])) - zero) / s);
      code = code > 15.0 ? 15.0 : code;
      packed[c / 8] |= static_cast<uint32_t>(code) << (4 * (c % 8));
    }
  }
  u32x4 out = {packed[0], packed[1], packed[2], packed[3]};
  *reinterpret_cast<u32x4*>(codes + row * (D / 2) + g * 16) = out;
  meta[row * NG + g] = static_cast<uint32_t>(s_bits) | (static_cast<uint32_t>(mn_bits) << 16);
}

// One wave per (sequence, logical page, KV head); each lane owns D/64 channels and walks
// the page's valid tokens in order, so the first occurrence of a tied min/max is kept. The
// bounds go to the page's logical slot [b, kvh, page], so that one KV head's bounds form a
// contiguous stretch for the scorer.
template <int D>
__global__ __launch_bounds__(256) void page_bounds_kernel(
    const uint16_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ token_begin, int Hkv,
    int max_pages, int num_phys, uint16_t* __restrict__ minmax) {
  constexpr int CPL = D / 64;
  const int b = blockIdx.y;
  const long wv = static_cast<long>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int kvh = static_cast<int>(wv % Hkv);
  const long page = wv / Hkv;
  if (page >= max_pages) return;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int t0 = static_cast<int>(page) * kPage;
  if (t0 >= n) return;
  const int begin = token_begin ? token_begin[b] : 0;
  if (t0 + kPage <= begin) return;
  const int phys = page_table[static_cast<long>(b) * max_pages + page];
  if (!phys_ok(phys, num_phys)) return;
  const int nv = n - t0 < kPage ? n - t0 : kPage;
  const long blk = static_cast<long>(phys) * Hkv + kvh;
  const uint16_t* src = k_cache + blk * kPage * D + lane_id() * CPL;
  uint16_t lo[CPL], hi[CPL];
  float flo[CPL], fhi[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    lo[c] = hi[c] = src[c];
    flo[c] = fhi[c] = h2f(src[c]);
  }
  for (int t = 1; t < nv; ++t) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const uint16_t x = src[t * D + c];
      const float v = h2f(x);
      if (v < flo[c]) {
        flo[c] = v;
        lo[c] = x;
      }
      if (v > fhi[c]) {
        fhi[c] = v;
        hi[c] = x;
      }
    }
  }
  uint16_t* dst =
      minmax + ((static_cast<long>(b) * Hkv + kvh) * max_pages + page) * 2 * D + lane_id() * CPL;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    dst[c] = lo[c];
    dst[D + c] = hi[c];
  }
}

}  // namespace

hipError_t launch_quantize_keys(const Layout& L, const void* k_cache, const int32_t* token_begin,
                                uint8_t* codes, void* meta, hipStream_t s) {
  const long items = static_cast<long>(L.max_pages) * L.Hkv * kPage * (L.d / 32);
  const dim3 grid(static_cast<unsigned>((items + 255) / 256), L.B);
  const auto* k = static_cast<const uint16_t*>(k_cache);
  auto* m = static_cast<uint32_t*>(meta);
  if (L.d == 128) {
    quantize_keys_kernel<128><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, token_begin,
                                                    L.Hkv, L.max_pages, L.num_phys, codes, m);
  } else {
    quantize_keys_kernel<64><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, token_begin,
                                                   L.Hkv, L.max_pages, L.num_phys, codes, m);
  }
  return hipGetLastError();
}

hipError_t launch_page_bounds(const Layout& L, const void* k_cache, const int32_t* token_begin,
                              void* minmax, hipStream_t s) {
  const long waves = static_cast<long>(L.max_pages) * L.Hkv;
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4), L.B);
  const auto* k = static_cast<const uint16_t*>(k_cache);
  auto* mm = static_cast<uint16_t*>(minmax);
  if (L.d == 128) {
    page_bounds_kernel<128><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, token_begin,
                                                  L.Hkv, L.max_pages, L.num_phys, mm);
  } else {
    page_bounds_kernel<64><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, token_begin,
                                                 L.Hkv, L.max_pages, L.num_phys, mm);
  }
  return hipGetLastError();
}

}  // namespace twl
