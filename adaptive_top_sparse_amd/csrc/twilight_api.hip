// C ABI of libtwilight.so: argument validation on the host, then kernel launches on the
// caller's stream. Every host-checkable error is reported before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "../../include/twilight.h"
#include "twl_launch.h"

namespace {

using twl::Layout;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Validates the layout. On success fills *out and returns TWL_OK. *empty is set when the
// batch is empty (every call is then a no-op).
int check_layout(const twl_layout_t* L, Layout* out, bool* empty) {
  if (L == nullptr) return TWL_ERR_INVALID_ARG;
  *empty = false;
  if (L->batch < 0 || L->num_q_heads < 1 || L->num_kv_heads < 1 || L->max_pages_per_seq < 1 ||
      L->num_phys_pages < 1 || L->page_size < 1 || L->head_dim < 1)
    return TWL_ERR_INVALID_ARG;
  if (L->num_q_heads % L->num_kv_heads != 0) return TWL_ERR_INVALID_ARG;
  const int G = L->num_q_heads / L->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return TWL_ERR_UNSUPPORTED;
  if (L->head_dim != 64 && L->head_dim != 128) return TWL_ERR_UNSUPPORTED;
  if (L->page_size != twl::kPage) return TWL_ERR_UNSUPPORTED;
  if (L->batch > 65535) return TWL_ERR_UNSUPPORTED;
  // every flat index of the caches and tables must fit the kernels' 64-bit arithmetic and
  // every token position an int
  if (static_cast<int64_t>(L->max_pages_per_seq) * twl::kPage > INT32_MAX / 2)
    return TWL_ERR_UNSUPPORTED;
  if (L->batch == 0) {
    *empty = true;
  } else if (L->page_table == nullptr || L->seq_lens == nullptr || !aligned4(L->page_table) ||
             !aligned4(L->seq_lens)) {
    return TWL_ERR_INVALID_ARG;
  }
  if (L->key_bits != 0 && L->key_bits != 4 && L->key_bits != 2) return TWL_ERR_UNSUPPORTED;
  *out = Layout{L->batch,     L->num_q_heads,     L->num_kv_heads,  L->head_dim,
                L->max_pages_per_seq, L->num_phys_pages, L->page_table, L->seq_lens};
  out->bits = L->key_bits == 2 ? 2 : 4;
  return TWL_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? TWL_OK : TWL_ERR_LAUNCH; }

size_t workspace_mode(const Layout& L, int cand_stride_pages) {
  size_t need = twl::quest_workspace_bytes(L);
  const size_t e = twl::estimate_workspace_bytes(L, cand_stride_pages);
  const size_t d = twl::decode_workspace_bytes(L, cand_stride_pages * twl::kPage);
  const size_t t = twl::topp_workspace_bytes(L, cand_stride_pages);
  if (e > need) need = e;
  if (e + t > need) need = e + t;  // the fused estimate + top-p holds both at once
  if (d > need) need = d;
  return need;
}

// Large enough for every call in either mode (group-wise or head-wise units).
size_t workspace_for(Layout L, int cand_stride_pages) {
  L.headwise = false;
  const size_t group = workspace_mode(L, cand_stride_pages);
  L.headwise = true;
  const size_t head = workspace_mode(L, cand_stride_pages);
  return group > head ? group : head;
}

int topp_select(bool headwise, const twl_layout_t* L, const float* weights,
                const int32_t* cand_pages, const int32_t* cand_count, int32_t cand_stride_pages,
                float p, int32_t* kept, int32_t* kept_count, float* tau, void* workspace,
                size_t workspace_bytes, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  lay.headwise = headwise;
  if (weights == nullptr || kept == nullptr || kept_count == nullptr) return TWL_ERR_INVALID_ARG;
  if (!aligned16(weights) || !aligned4(kept) || !aligned4(kept_count)) return TWL_ERR_INVALID_ARG;
  if (cand_pages != nullptr && !aligned4(cand_pages)) return TWL_ERR_INVALID_ARG;
  if (cand_count != nullptr && !aligned4(cand_count)) return TWL_ERR_INVALID_ARG;
  if (tau != nullptr && !aligned4(tau)) return TWL_ERR_INVALID_ARG;
  if (cand_stride_pages < 1 || !(p > 0.0f && p <= 1.0f)) return TWL_ERR_INVALID_ARG;
  if (cand_pages == nullptr && cand_stride_pages < lay.max_pages) return TWL_ERR_INVALID_ARG;
  if (static_cast<int64_t>(cand_stride_pages) * twl::kPage > twl::kToppMaxSlots)
    return TWL_ERR_UNSUPPORTED;
  if (empty) return TWL_OK;
  const size_t need = twl::topp_workspace_bytes(lay, cand_stride_pages);
  if (need > 0 && (workspace == nullptr || !aligned16(workspace) ||
                   workspace_bytes < need))
    return TWL_ERR_WORKSPACE;
  return launch_status(twl::launch_topp(lay, weights, cand_pages, cand_count, cand_stride_pages,
                                        p, kept, kept_count, tau, workspace, stream));
}

// Host checks of a decode call's arguments other than its workspace.
int check_decode(bool headwise, const twl_layout_t* L, const void* q, const void* k_cache,
                 const void* v_cache, const int32_t* kept, const int32_t* kept_count,
                 int32_t kept_stride, float sm_scale, const void* out, Layout* lay,
                 bool* empty) {
  int st = check_layout(L, lay, empty);
  if (st != TWL_OK) return st;
  lay->headwise = headwise;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || kept == nullptr ||
      kept_count == nullptr || out == nullptr)
    return TWL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned4(kept) ||
      !aligned4(kept_count) || !aligned4(out))
    return TWL_ERR_INVALID_ARG;
  if (kept_stride < 1 || !std::isfinite(sm_scale)) return TWL_ERR_INVALID_ARG;
  if (static_cast<int64_t>(kept_stride) > twl::kToppMaxSlots * 64) return TWL_ERR_UNSUPPORTED;
  return TWL_OK;
}

int sparse_decode(bool headwise, const twl_layout_t* L, const void* q, const void* k_cache,
                  const void* v_cache, const int32_t* kept, const int32_t* kept_count,
                  int32_t kept_stride, float sm_scale, void* out, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  const int st = check_decode(headwise, L, q, k_cache, v_cache, kept, kept_count, kept_stride,
                              sm_scale, out, &lay, &empty);
  if (st != TWL_OK) return st;
  if (empty) return TWL_OK;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < twl::decode_workspace_bytes(lay, kept_stride))
    return TWL_ERR_WORKSPACE;
  return launch_status(twl::launch_sparse_decode(lay, q, k_cache, v_cache, kept, kept_count,
                                                 kept_stride, sm_scale, out, workspace, stream));
}

// Fixed device scratch of twilight_sparse_decode_noalloc, for callers that cannot
// allocate. In host code `scratch` is only a stand-in for the symbol: its device address is
// looked up once per device (with that device current) and kept in scratch_ptr.
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::once_flag scratch_once[kMaxDevices];
void* scratch_ptr[kMaxDevices];

// The current device's copy of the scratch array, or nullptr when it cannot be found.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(scratch_once[dev], [dev]() {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) scratch_ptr[dev] = p;
  });
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* twilight_status_string(int status) {
  switch (status) {
    case TWL_OK: return "ok";
    case TWL_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size or value)";
    case TWL_ERR_UNSUPPORTED: return "unsupported shape (head_dim, group size, page size or extent)";
    case TWL_ERR_WORKSPACE: return "workspace missing or too small";
    case TWL_ERR_LAUNCH: return "kernel launch failed";
    case TWL_ERR_SCRATCH: return "the call needs more than the fixed 16 MiB no-allocation scratch";
    default: return "unknown status";
  }
}

size_t twilight_workspace_size(const twl_layout_t* L, int32_t cand_stride_pages) {
  Layout lay{};
  bool empty = false;
  if (check_layout(L, &lay, &empty) != TWL_OK || cand_stride_pages < 1) return 0;
  if (static_cast<int64_t>(cand_stride_pages) * twl::kPage > twl::kToppMaxSlots * 64) return 0;
  if (empty) return 256;
  return workspace_for(lay, cand_stride_pages);
}

int twilight_quantize_keys(const twl_layout_t* L, const void* k_cache,
                           const int32_t* token_begin, uint8_t* k_codes, void* k_meta,
                           hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (k_cache == nullptr || k_codes == nullptr || k_meta == nullptr) return TWL_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(k_codes) || !aligned4(k_meta)) return TWL_ERR_INVALID_ARG;
  if (token_begin != nullptr && !aligned4(token_begin)) return TWL_ERR_INVALID_ARG;
  if (empty) return TWL_OK;
  return launch_status(twl::launch_quantize_keys(lay, k_cache, token_begin, k_codes, k_meta, stream));
}

int quest_page_bounds(const twl_layout_t* L, const void* k_cache, const int32_t* token_begin,
                      void* page_minmax, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (k_cache == nullptr || page_minmax == nullptr) return TWL_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned16(page_minmax)) return TWL_ERR_INVALID_ARG;
  if (token_begin != nullptr && !aligned4(token_begin)) return TWL_ERR_INVALID_ARG;
  if (empty) return TWL_OK;
  return launch_status(twl::launch_page_bounds(lay, k_cache, token_begin, page_minmax, stream));
}

int twilight_append_keys(const twl_layout_t* L, const void* k_cache, const int32_t* token_begin,
                         uint8_t* k_codes, void* k_meta, void* page_minmax, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (k_cache == nullptr || token_begin == nullptr || k_codes == nullptr || k_meta == nullptr)
    return TWL_ERR_INVALID_ARG;
  if (!aligned16(k_cache) || !aligned4(token_begin) || !aligned16(k_codes) || !aligned4(k_meta))
    return TWL_ERR_INVALID_ARG;
  if (page_minmax != nullptr && !aligned16(page_minmax)) return TWL_ERR_INVALID_ARG;
  if (empty) return TWL_OK;
  return launch_status(
      twl::launch_append_keys(lay, k_cache, token_begin, k_codes, k_meta, page_minmax, stream));
}

int quest_select_pages(const twl_layout_t* L, const void* q, const void* page_minmax,
                       int32_t budget_pages, int32_t* sel_pages, int32_t* sel_count,
                       void* workspace, size_t workspace_bytes, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (q == nullptr || page_minmax == nullptr || sel_pages == nullptr || sel_count == nullptr)
    return TWL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(page_minmax) || !aligned4(sel_pages) || !aligned4(sel_count))
    return TWL_ERR_INVALID_ARG;
  if (budget_pages < 1) return TWL_ERR_INVALID_ARG;
  if (lay.max_pages > twl::kQuestMaxPages) return TWL_ERR_UNSUPPORTED;
  if (empty) return TWL_OK;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < twl::quest_workspace_bytes(lay))
    return TWL_ERR_WORKSPACE;
  return launch_status(twl::launch_quest_select(lay, q, page_minmax, budget_pages, sel_pages,
                                                sel_count, workspace, stream));
}

int64_t quest_score_stride(int32_t max_pages_per_seq) {
  if (max_pages_per_seq < 1) return -1;
  return twl::quest_score_stride(max_pages_per_seq);
}

int quest_page_scores(const twl_layout_t* L, const void* q, const void* page_minmax,
                      double* scores, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (q == nullptr || page_minmax == nullptr || scores == nullptr) return TWL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(page_minmax) || !aligned16(scores)) return TWL_ERR_INVALID_ARG;
  if (empty) return TWL_OK;
  return launch_status(twl::launch_quest_scores(lay, q, page_minmax, scores, stream));
}

int quest_top_pages(const twl_layout_t* L, const double* scores, int32_t budget_pages,
                    int32_t* sel_pages, int32_t* sel_count, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (scores == nullptr || sel_pages == nullptr || sel_count == nullptr) return TWL_ERR_INVALID_ARG;
  if (!aligned16(scores) || !aligned4(sel_pages) || !aligned4(sel_count)) return TWL_ERR_INVALID_ARG;
  if (budget_pages < 1) return TWL_ERR_INVALID_ARG;
  if (lay.max_pages > twl::kQuestMaxPages) return TWL_ERR_UNSUPPORTED;
  if (empty) return TWL_OK;
  return launch_status(
      twl::launch_quest_top(lay, scores, budget_pages, sel_pages, sel_count, stream));
}

int twilight_estimate_weights(const twl_layout_t* L, const void* q, const uint8_t* k_codes,
                              const void* k_meta, const int32_t* cand_pages,
                              const int32_t* cand_count, int32_t cand_stride_pages,
                              float sm_scale, float* weights, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  if (q == nullptr || k_codes == nullptr || k_meta == nullptr || weights == nullptr)
    return TWL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned4(k_meta) || !aligned16(weights))
    return TWL_ERR_INVALID_ARG;
  if (cand_pages != nullptr && !aligned4(cand_pages)) return TWL_ERR_INVALID_ARG;
  if (cand_count != nullptr && !aligned4(cand_count)) return TWL_ERR_INVALID_ARG;
  if (cand_stride_pages < 1 || !std::isfinite(sm_scale)) return TWL_ERR_INVALID_ARG;
  if (cand_pages == nullptr && cand_stride_pages < lay.max_pages) return TWL_ERR_INVALID_ARG;
  if (static_cast<int64_t>(cand_stride_pages) * twl::kPage > twl::kToppMaxSlots * 64)
    return TWL_ERR_UNSUPPORTED;
  if (empty) return TWL_OK;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < twl::estimate_workspace_bytes(lay, cand_stride_pages))
    return TWL_ERR_WORKSPACE;
  return launch_status(twl::launch_estimate(lay, q, k_codes, k_meta, cand_pages, cand_count,
                                            cand_stride_pages, sm_scale, weights, workspace,
                                            stream));
}

int estimate_topp(bool headwise, const twl_layout_t* L, const void* q, const uint8_t* k_codes,
                  const void* k_meta, const int32_t* cand_pages, const int32_t* cand_count,
                  int32_t cand_stride_pages, float sm_scale, float p, float* weights,
                  int32_t* kept, int32_t* kept_count, float* tau, void* workspace,
                  size_t workspace_bytes, hipStream_t stream) {
  Layout lay{};
  bool empty = false;
  int st = check_layout(L, &lay, &empty);
  if (st != TWL_OK) return st;
  lay.headwise = headwise;
  if (q == nullptr || k_codes == nullptr || k_meta == nullptr || weights == nullptr ||
      kept == nullptr || kept_count == nullptr)
    return TWL_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_codes) || !aligned4(k_meta) || !aligned16(weights) ||
      !aligned4(kept) || !aligned4(kept_count))
    return TWL_ERR_INVALID_ARG;
  if (cand_pages != nullptr && !aligned4(cand_pages)) return TWL_ERR_INVALID_ARG;
  if (cand_count != nullptr && !aligned4(cand_count)) return TWL_ERR_INVALID_ARG;
  if (tau != nullptr && !aligned4(tau)) return TWL_ERR_INVALID_ARG;
  if (cand_stride_pages < 1 || !std::isfinite(sm_scale) || !(p > 0.0f && p <= 1.0f))
    return TWL_ERR_INVALID_ARG;
  if (cand_pages == nullptr && cand_stride_pages < lay.max_pages) return TWL_ERR_INVALID_ARG;
  if (static_cast<int64_t>(cand_stride_pages) * twl::kPage > twl::kToppMaxSlots)
    return TWL_ERR_UNSUPPORTED;
  if (empty) return TWL_OK;
  // the estimate's chunk pairs at the start of the workspace, any group-mean stage after
  const size_t pairs = twl::estimate_workspace_bytes(lay, cand_stride_pages);
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < pairs + twl::topp_workspace_bytes(lay, cand_stride_pages))
    return TWL_ERR_WORKSPACE;
  hipError_t e = twl::launch_estimate(lay, q, k_codes, k_meta, cand_pages, cand_count,
                                      cand_stride_pages, sm_scale, weights, workspace, stream,
                                      false);
  if (e != hipSuccess) return TWL_ERR_LAUNCH;
  return launch_status(twl::launch_topp(
      lay, weights, cand_pages, cand_count, cand_stride_pages, p, kept, kept_count, tau,
      workspace, stream, static_cast<const float2*>(workspace),
      twl::estimate_chunks(lay, cand_stride_pages), pairs));
}

int twilight_topp_select(const twl_layout_t* L, const float* weights, const int32_t* cand_pages,
                         const int32_t* cand_count, int32_t cand_stride_pages, float p,
                         int32_t* kept, int32_t* kept_count, float* tau, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return topp_select(false, L, weights, cand_pages, cand_count, cand_stride_pages, p, kept,
                     kept_count, tau, workspace, workspace_bytes, stream);
}

int twilight_estimate_topp(const twl_layout_t* L, const void* q, const uint8_t* k_codes,
                           const void* k_meta, const int32_t* cand_pages,
                           const int32_t* cand_count, int32_t cand_stride_pages,
                           float sm_scale, float p, float* weights, int32_t* kept,
                           int32_t* kept_count, float* tau, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return estimate_topp(false, L, q, k_codes, k_meta, cand_pages, cand_count, cand_stride_pages,
                       sm_scale, p, weights, kept, kept_count, tau, workspace, workspace_bytes,
                       stream);
}

int twilight_estimate_topp_headwise(const twl_layout_t* L, const void* q,
                                    const uint8_t* k_codes, const void* k_meta,
                                    const int32_t* cand_pages, const int32_t* cand_count,
                                    int32_t cand_stride_pages, float sm_scale, float p,
                                    float* weights, int32_t* kept, int32_t* kept_count,
                                    float* tau, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream) {
  return estimate_topp(true, L, q, k_codes, k_meta, cand_pages, cand_count, cand_stride_pages,
                       sm_scale, p, weights, kept, kept_count, tau, workspace, workspace_bytes,
                       stream);
}

int twilight_topp_select_headwise(const twl_layout_t* L, const float* weights,
                                  const int32_t* cand_pages, const int32_t* cand_count,
                                  int32_t cand_stride_pages, float p, int32_t* kept,
                                  int32_t* kept_count, float* tau, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  return topp_select(true, L, weights, cand_pages, cand_count, cand_stride_pages, p, kept,
                     kept_count, tau, workspace, workspace_bytes, stream);
}

int twilight_sparse_decode(const twl_layout_t* L, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* kept, const int32_t* kept_count,
                           int32_t kept_stride, float sm_scale, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  return sparse_decode(false, L, q, k_cache, v_cache, kept, kept_count, kept_stride, sm_scale,
                       out, workspace, workspace_bytes, stream);
}

int twilight_sparse_decode_noalloc(const twl_layout_t* L, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* kept,
                                   const int32_t* kept_count, int32_t kept_stride,
                                   float sm_scale, void* out, hipStream_t stream) {
  // every host check, the size limit included, comes before the device query
  Layout lay{};
  bool empty = false;
  const int st = check_decode(false, L, q, k_cache, v_cache, kept, kept_count, kept_stride,
                              sm_scale, out, &lay, &empty);
  if (st != TWL_OK) return st;
  if (empty) return TWL_OK;
  if (twl::decode_workspace_bytes(lay, kept_stride) > kNoAllocScratchBytes)
    return TWL_ERR_SCRATCH;
  void* ws = device_scratch();
  if (ws == nullptr) return TWL_ERR_LAUNCH;
  return launch_status(twl::launch_sparse_decode(lay, q, k_cache, v_cache, kept, kept_count,
                                                 kept_stride, sm_scale, out, ws, stream));
}

int twilight_sparse_decode_headwise(const twl_layout_t* L, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* kept,
                                    const int32_t* kept_count, int32_t kept_stride,
                                    float sm_scale, void* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream) {
  return sparse_decode(true, L, q, k_cache, v_cache, kept, kept_count, kept_stride, sm_scale,
                       out, workspace, workspace_bytes, stream);
}

}  // extern "C"
