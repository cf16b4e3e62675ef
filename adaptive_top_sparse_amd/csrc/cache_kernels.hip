// Cache maintenance: the int4 key cache used by Twilight's weight estimate and Quest's
// per-page channelwise key bounds (Twilight pages, atlas.scime.ai summary: "Approach" for
// the 4-bit key cache, "Surprising findings" for Quest's per-page max-pooled layout).
// Neither runs inside a decode step's hot loop; both run at prefill and then once per
// appended token (token_begin).
#include "twl_device.h"
#include "twl_launch.h"

namespace twl {
namespace {

// Codes of one 32-channel group, BITS (4, or 2 for the ablated variant) per channel:
// zero = min (the first occurrence of the minimum's bit pattern), scale = the fp16 nearest
// to (max - min) / Lv with Lv = 2^BITS - 1 (fp64 quotient, one RNE rounding to fp16), and
// code = clamp(rint((x - zero) / scale), 0, Lv) in fp64. fp64 decides every code exactly:
// (x - zero) and scale are multiples of 2^-24 below 2^17, so a quotient that is not a
// half-integer lies at least 2^-41 away from one, far beyond the fp64 quotient's error;
// half-integers are exact and rint sends them to the even code.
// Quantizes the group g of token `slot` of physical page `phys` (KV head kvh).
template <int D, int BITS>
__device__ __forceinline__ void quantize_group(const uint16_t* __restrict__ k_cache, int Hkv,
                                               int phys, int kvh, int slot, int g,
                                               uint8_t* __restrict__ codes,
                                               uint32_t* __restrict__ meta) {
  constexpr int NG = D / 32;
  constexpr int kLevels = (1 << BITS) - 1;
  constexpr int kWords = BITS;  // 32 codes of BITS bits
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
  const uint16_t s_bits =
      f64_to_f16_bits_nonneg((static_cast<double>(mx) - zero) / static_cast<double>(kLevels));
  const double s = static_cast<double>(h2f(s_bits));
  uint32_t packed[kWords];
#pragma unroll
  for (int i = 0; i < kWords; ++i) packed[i] = 0u;
  if (s > 0.0) {
#pragma unroll
    for (int c = 0; c < 32; ++c) {
      double code = rint((static_cast<double>(h2f(x[c])) - zero) / s);
      code = code > kLevels ? kLevels : code;
      packed[c * BITS / 32] |= static_cast<uint32_t>(code) << (BITS * c % 32);
    }
  }
  uint8_t* dst = codes + row * (D * BITS / 8) + g * (4 * BITS);
  if constexpr (BITS == 4) {
    *reinterpret_cast<u32x4*>(dst) = u32x4{packed[0], packed[1], packed[2], packed[3]};
  } else {
    *reinterpret_cast<u32x2*>(dst) = u32x2{packed[0], packed[1]};
  }
  meta[row * NG + g] = static_cast<uint32_t>(s_bits) | (static_cast<uint32_t>(mn_bits) << 16);
}

// Whole-cache (prefill) form: one lane per (token, 32-channel group). A wave covers one
// (page, KV head) block of 16 tokens x d channels when d = 128 (64 lanes = 16 tokens x 4
// groups), so its loads are one contiguous 4 KiB stretch.
template <int D, int BITS>
__global__ __launch_bounds__(256) void quantize_keys_kernel(
    const uint16_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int Hkv, int max_pages, int num_phys,
    uint8_t* __restrict__ codes, uint32_t* __restrict__ meta) {
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
  if (tok >= n) return;
  const int phys = page_table[static_cast<long>(b) * max_pages + page];
  if (!phys_ok(phys, num_phys)) return;
  quantize_group<D, BITS>(k_cache, Hkv, phys, kvh, slot, g, codes, meta);
}

// The 16 rows of one (physical page, KV head) block, D / 64 channels per lane (lane l owns
// channels l * D/64 ...). Rows at or past nv are not loaded from their own address: they
// repeat row 0 and every consumer ignores them. All loads are issued before any is used.
template <int D>
struct PageRows {
  static constexpr int CPL = D / 64;
  uint16_t x[kPage][CPL];

  __device__ __forceinline__ void load(const uint16_t* __restrict__ k_cache, int Hkv, int phys,
                                       int kvh, int nv) {
    const long blk = static_cast<long>(phys) * Hkv + kvh;
    const uint16_t* src = k_cache + blk * kPage * D + lane_id() * CPL;
#pragma unroll
    for (int t = 0; t < kPage; ++t)
#pragma unroll
      for (int c = 0; c < CPL; ++c) x[t][c] = src[(t < nv ? t : 0) * D + c];
  }
};

// Channelwise min/max over the first nv rows, walking the rows in order so that the first
// occurrence of a tied min/max is kept; written at the page's logical slot [b, kvh, page],
// so that one KV head's bounds form a contiguous stretch for the scorer.
template <int D>
__device__ __forceinline__ void store_page_bounds(const PageRows<D>& r, int Hkv, int max_pages,
                                                  int b, int kvh, long page, int nv,
                                                  uint16_t* __restrict__ minmax) {
  constexpr int CPL = D / 64;
  uint16_t lo[CPL], hi[CPL];
  float flo[CPL], fhi[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    lo[c] = hi[c] = r.x[0][c];
    flo[c] = fhi[c] = h2f(r.x[0][c]);
  }
#pragma unroll
  for (int t = 1; t < kPage; ++t) {
    if (t >= nv) break;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const float v = h2f(r.x[t][c]);
      if (v < flo[c]) {
        flo[c] = v;
        lo[c] = r.x[t][c];
      }
      if (v > fhi[c]) {
        fhi[c] = v;
        hi[c] = r.x[t][c];
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

// Image of a finite fp16 value as an unsigned key that orders like the value itself, with
// -0 and +0 mapped to the same key.
__device__ __forceinline__ uint32_t f16_order_key(uint16_t bits) {
  const uint32_t mag = bits & 0x7fffu;
  return (bits & 0x8000u) && mag != 0 ? 0x7fffu - mag : 0x8000u + mag;
}

// Codes of one token row held across the wave (the same rule as quantize_group, so both
// forms write identical bytes): the lanes of each 32-channel group find the group's first
// minimum (smallest key, then smallest channel) and its maximum together, then each lane
// codes its own channels and the lanes sharing a byte combine theirs. `row` is the row
// index [phys, kvh, slot].
template <int D, int BITS>
__device__ __forceinline__ void quantize_row_wave(const uint16_t (&x)[D / 64], long row,
                                                  uint8_t* __restrict__ codes,
                                                  uint32_t* __restrict__ meta) {
  constexpr int CPL = D / 64;
  constexpr int LPG = 32 / CPL;              // lanes per 32-channel group
  constexpr int LPB = 8 / (CPL * BITS);      // lanes per code byte
  constexpr int NG = D / 32;
  constexpr int kLevels = (1 << BITS) - 1;
  const int lane = lane_id();
  float v[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) v[c] = h2f(x[c]);
  float mx = v[0];
  int mi = 0;
#pragma unroll
  for (int c = 1; c < CPL; ++c) {
    if (v[c] < v[mi]) mi = c;
    mx = fmaxf(mx, v[c]);
  }
  uint16_t mine = x[0];
#pragma unroll
  for (int c = 1; c < CPL; ++c) mine = mi == c ? x[c] : mine;
  // key = order of the value above the channel index within the group (0..31)
  uint32_t key = (f16_order_key(mine) << 8) | static_cast<uint32_t>((lane % LPG) * CPL + mi);
#pragma unroll
  for (int off = 1; off < LPG; off <<= 1) {
    const uint32_t k2 = static_cast<uint32_t>(__shfl_xor(static_cast<int>(key), off));
    key = k2 < key ? k2 : key;
    mx = fmaxf(mx, __shfl_xor(mx, off));
  }
  // the winner's own bit pattern (the key does not tell -0 from +0)
  const int ch = static_cast<int>(key & 0xffu);
  uint32_t both = x[0];
  if constexpr (CPL > 1) both |= static_cast<uint32_t>(x[1]) << 16;
  const uint32_t w = static_cast<uint32_t>(
      __shfl(static_cast<int>(both), (lane / LPG) * LPG + ch / CPL));
  const uint16_t mn_bits = static_cast<uint16_t>(CPL > 1 && (ch & 1) ? w >> 16 : w & 0xffffu);
  const double zero = static_cast<double>(h2f(mn_bits));
  const uint16_t s_bits =
      f64_to_f16_bits_nonneg((static_cast<double>(mx) - zero) / static_cast<double>(kLevels));
  const double s = static_cast<double>(h2f(s_bits));
  uint32_t bits = 0;  // this lane's CPL codes, lowest channel in the lowest bits
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    double q = 0.0;
    if (s > 0.0) {
      q = rint((static_cast<double>(v[c]) - zero) / s);
      q = q > kLevels ? kLevels : q;
    }
    bits |= static_cast<uint32_t>(q) << (BITS * c);
  }
  uint32_t byte = bits;
#pragma unroll
  for (int i = 1; i < LPB; ++i)
    byte |= static_cast<uint32_t>(__shfl(static_cast<int>(bits), (lane & ~(LPB - 1)) + i))
            << (i * CPL * BITS);
  if (lane % LPB == 0) codes[row * (D * BITS / 8) + lane / LPB] = static_cast<uint8_t>(byte);
  if (lane % LPG == 0)
    meta[row * NG + lane / LPG] = static_cast<uint32_t>(s_bits) | (static_cast<uint32_t>(mn_bits) << 16);
}

// Whole-cache (prefill) form: one wave per (sequence, logical page, KV head).
template <int D>
__global__ __launch_bounds__(256) void page_bounds_kernel(
    const uint16_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, int Hkv, int max_pages, int num_phys,
    uint16_t* __restrict__ minmax) {
  const int b = blockIdx.y;
  const long wv = static_cast<long>(blockIdx.x) * (blockDim.x / kWave) + threadIdx.x / kWave;
  const int kvh = static_cast<int>(wv % Hkv);
  const long page = wv / Hkv;
  if (page >= max_pages) return;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  const int t0 = static_cast<int>(page) * kPage;
  if (t0 >= n) return;
  const int phys = page_table[static_cast<long>(b) * max_pages + page];
  if (!phys_ok(phys, num_phys)) return;
  const int nv = n - t0 < kPage ? n - t0 : kPage;
  PageRows<D> r;
  r.load(k_cache, Hkv, phys, kvh, nv);
  store_page_bounds<D>(r, Hkv, max_pages, b, kvh, page, nv, minmax);
}

// Append form (token_begin given): one wave per (sequence, KV head) walks the pages holding
// tokens at or after token_begin[b] (one page for a one-token append). Each page's rows are
// loaded once and serve both its bounds (kBounds) and the codes of its tokens at or after
// token_begin (kCodes), so a decode step's cache maintenance is a single short launch.
template <int D, int BITS, bool kCodes, bool kBounds>
__global__ __launch_bounds__(kWave) void append_keys_kernel(
    const uint16_t* __restrict__ k_cache, const int32_t* __restrict__ page_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ token_begin, int Hkv,
    int max_pages, int num_phys, uint8_t* __restrict__ codes, uint32_t* __restrict__ meta,
    uint16_t* __restrict__ minmax) {
  const int kvh = blockIdx.x;
  const int b = blockIdx.y;
  const int n = seq_len_clamped(seq_lens, b, max_pages);
  int begin = token_begin[b];
  begin = begin < 0 ? 0 : begin;
  for (int page = begin / kPage; page * kPage < n; ++page) {
    const int phys = page_table[static_cast<long>(b) * max_pages + page];
    if (!phys_ok(phys, num_phys)) continue;
    const int t0 = page * kPage;
    const int nv = n - t0 < kPage ? n - t0 : kPage;
    PageRows<D> r;
    r.load(k_cache, Hkv, phys, kvh, nv);
    if constexpr (kBounds) store_page_bounds<D>(r, Hkv, max_pages, b, kvh, page, nv, minmax);
    if constexpr (kCodes) {
      const int first = begin > t0 ? begin - t0 : 0;
      const long row0 = (static_cast<long>(phys) * Hkv + kvh) * kPage;
      for (int slot = first; slot < nv; ++slot) {
        uint16_t x[D / 64];
#pragma unroll
        for (int c = 0; c < D / 64; ++c) {
          x[c] = r.x[0][c];
#pragma unroll
          for (int t = 1; t < kPage; ++t) x[c] = slot == t ? r.x[t][c] : x[c];
        }
        quantize_row_wave<D, BITS>(x, row0 + slot, codes, meta);
      }
    }
  }
}

template <int D, bool kCodes, bool kBounds>
void launch_append_d(const Layout& L, const uint16_t* k, const int32_t* token_begin,
                     uint8_t* codes, uint32_t* meta, uint16_t* mm, hipStream_t s) {
  const dim3 grid(L.Hkv, L.B);
  if (L.bits == 2) {
    append_keys_kernel<D, 2, kCodes, kBounds><<<grid, kWave, 0, s>>>(
        k, L.page_table, L.seq_lens, token_begin, L.Hkv, L.max_pages, L.num_phys, codes, meta, mm);
  } else {
    append_keys_kernel<D, 4, kCodes, kBounds><<<grid, kWave, 0, s>>>(
        k, L.page_table, L.seq_lens, token_begin, L.Hkv, L.max_pages, L.num_phys, codes, meta, mm);
  }
}

template <bool kCodes, bool kBounds>
void launch_append(const Layout& L, const uint16_t* k, const int32_t* token_begin,
                   uint8_t* codes, uint32_t* meta, uint16_t* mm, hipStream_t s) {
  if (L.d == 128) {
    launch_append_d<128, kCodes, kBounds>(L, k, token_begin, codes, meta, mm, s);
  } else {
    launch_append_d<64, kCodes, kBounds>(L, k, token_begin, codes, meta, mm, s);
  }
}

template <int D>
void launch_quantize_d(const Layout& L, const uint16_t* k, uint8_t* codes, uint32_t* m,
                       hipStream_t s) {
  const long items = static_cast<long>(L.max_pages) * L.Hkv * kPage * (D / 32);
  const dim3 grid(static_cast<unsigned>((items + 255) / 256), L.B);
  if (L.bits == 2) {
    quantize_keys_kernel<D, 2><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, L.Hkv,
                                                    L.max_pages, L.num_phys, codes, m);
  } else {
    quantize_keys_kernel<D, 4><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, L.Hkv,
                                                    L.max_pages, L.num_phys, codes, m);
  }
}

}  // namespace

hipError_t launch_quantize_keys(const Layout& L, const void* k_cache, const int32_t* token_begin,
                                uint8_t* codes, void* meta, hipStream_t s) {
  const auto* k = static_cast<const uint16_t*>(k_cache);
  auto* m = static_cast<uint32_t*>(meta);
  if (token_begin != nullptr) {
    launch_append<true, false>(L, k, token_begin, codes, m, nullptr, s);
    return hipGetLastError();
  }
  if (L.d == 128) {
    launch_quantize_d<128>(L, k, codes, m, s);
  } else {
    launch_quantize_d<64>(L, k, codes, m, s);
  }
  return hipGetLastError();
}

hipError_t launch_page_bounds(const Layout& L, const void* k_cache, const int32_t* token_begin,
                              void* minmax, hipStream_t s) {
  const auto* k = static_cast<const uint16_t*>(k_cache);
  auto* mm = static_cast<uint16_t*>(minmax);
  if (token_begin != nullptr) {
    launch_append<false, true>(L, k, token_begin, nullptr, nullptr, mm, s);
    return hipGetLastError();
  }
  const long waves = static_cast<long>(L.max_pages) * L.Hkv;
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4), L.B);
  if (L.d == 128) {
    page_bounds_kernel<128><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, L.Hkv,
                                                  L.max_pages, L.num_phys, mm);
  } else {
    page_bounds_kernel<64><<<grid, 256, 0, s>>>(k, L.page_table, L.seq_lens, L.Hkv,
                                                 L.max_pages, L.num_phys, mm);
  }
  return hipGetLastError();
}

}  // namespace twl

namespace twl {

hipError_t launch_append_keys(const Layout& L, const void* k_cache, const int32_t* token_begin,
                              uint8_t* codes, void* meta, void* minmax, hipStream_t s) {
  const auto* k = static_cast<const uint16_t*>(k_cache);
  auto* m = static_cast<uint32_t*>(meta);
  if (minmax != nullptr) {
    launch_append<true, true>(L, k, token_begin, codes, m, static_cast<uint16_t*>(minmax), s);
  } else {
    launch_append<true, false>(L, k, token_begin, codes, m, nullptr, s);
  }
  return hipGetLastError();
}

}  // namespace twl
