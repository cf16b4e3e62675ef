// Host-side launchers of the Twilight kernels (internal to libtwilight.so). Arguments are
// validated by the C ABI layer before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace twl {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Tokens per KV-cache page.
constexpr int kPage = 16;

struct Layout {
  int B, Hq, Hkv, d, max_pages, num_phys;
  const int32_t* page_table;
  const int32_t* seq_lens;
  int bits = 4;  // width of the estimate's key codes: 4 or 2
  // Top-p and decode units: one kept set per KV head, shared by its G query heads
  // (group-wise), or one per query head (head-wise).
  bool headwise = false;
  int G() const { return Hq / Hkv; }
  int units() const { return headwise ? Hq : Hkv; }   // units per sequence
  int unit_G() const { return headwise ? 1 : Hq / Hkv; }  // query heads per unit
};

// Rows of candidate slots are processed in chunks of this many slots by the estimate.
constexpr int kEstChunk = 256;

// Kept tokens per decode work-group for a given kept stride and unit count.
int decode_chunk_tokens(const Layout& L, int kept_stride);

size_t quest_workspace_bytes(const Layout& L);
size_t estimate_workspace_bytes(const Layout& L, int cand_stride_pages);
size_t decode_workspace_bytes(const Layout& L, int kept_stride);
size_t topp_workspace_bytes(const Layout& L, int cand_stride_pages);

hipError_t launch_quantize_keys(const Layout& L, const void* k_cache, const int32_t* token_begin,
                                uint8_t* codes, void* meta, hipStream_t s);
hipError_t launch_page_bounds(const Layout& L, const void* k_cache, const int32_t* token_begin,
                              void* minmax, hipStream_t s);
hipError_t launch_append_keys(const Layout& L, const void* k_cache, const int32_t* token_begin,
                              uint8_t* codes, void* meta, void* minmax, hipStream_t s);
// Quest page scores into rows of quest_score_stride(max_pages) doubles, then the top pages
// from such rows; launch_quest_select runs both with the scores in the workspace.
long quest_score_stride(int max_pages);
hipError_t launch_quest_scores(const Layout& L, const void* q, const void* minmax, double* scores,
                               hipStream_t s);
hipError_t launch_quest_top(const Layout& L, const double* scores, int budget,
                            int32_t* sel_pages, int32_t* sel_count, hipStream_t s);
hipError_t launch_quest_select(const Layout& L, const void* q, const void* minmax, int budget,
                               int32_t* sel_pages, int32_t* sel_count, void* ws, hipStream_t s);
// With normalize false the weights are left as logits (-inf off the candidates) and the
// per-chunk (max, sum of exp) pairs stay at the start of ws, estimate_chunks per query head.
hipError_t launch_estimate(const Layout& L, const void* q, const uint8_t* codes, const void* meta,
                           const int32_t* cand_pages, const int32_t* cand_count,
                           int cand_stride_pages, float sm_scale, float* weights, void* ws,
                           hipStream_t s, bool normalize = true);
int estimate_chunks(const Layout& L, int cand_stride_pages);
// With norm given, weights hold the estimate's logits (log2 units) and norm its per-chunk
// (max, sum of exp2) pairs (norm_chunks per query head); the top-p kernels normalise them
// themselves. The group-mean stage, when one is needed, starts stage_offset bytes into ws
// (past the pairs, when they live there too).
hipError_t launch_topp(const Layout& L, const float* weights, const int32_t* cand_pages,
                       const int32_t* cand_count, int cand_stride_pages, float p,
                       int32_t* kept, int32_t* kept_count, float* tau, void* ws,
                       hipStream_t s, const float2* norm = nullptr, int norm_chunks = 0,
                       size_t stage_offset = 0);
hipError_t launch_sparse_decode(const Layout& L, const void* q, const void* k_cache,
                                const void* v_cache, const int32_t* kept,
                                const int32_t* kept_count, int kept_stride, float sm_scale,
                                void* out, void* ws, hipStream_t s);

// Every call uses the workspace as scratch for its own duration only; nothing in it needs
// to survive between calls or be initialised by the caller.
inline void* stage_scratch(void* ws, const Layout&) { return ws; }

// Largest slot count per unit the top-p kernel holds on chip.
constexpr int kToppMaxSlots = 65536;
// Largest page count per sequence the Quest selector holds on chip.
constexpr int kQuestMaxPages = 32768;


}  // namespace twl
