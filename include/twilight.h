/*
 * twilight.h -- C ABI of libtwilight.so: Twilight hierarchical top-p sparse decode
 * attention for AMD Instinct MI355X (gfx950).
 *
 * The method (Twilight: Adaptive Attention Sparsity with Hierarchical Top-p Pruning;
 * atlas.scime.ai summary, "Approach" and "Surprising findings"): a base sparse-attention
 * selector pre-selects tokens (here Quest: page-level top-k over per-page key bounds);
 * Twilight then estimates the attention weights of those candidates from a 4-bit
 * quantized key cache and keeps the smallest set whose weight mass reaches p (top-p,
 * nucleus thresholding), so the budget adapts per head and per query; attention then runs
 * over the kept tokens only. Under GQA the kept set is shared by the KV-head group
 * ("Limitations").
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers, except the layout struct itself, which is a
 *    host struct read during the call only.
 *  - Every call is asynchronous on `stream`. None allocates, frees or synchronizes; none
 *    keeps state between calls, so calls on different streams with different buffers may
 *    run concurrently.
 *  - The caller owns every buffer, including the workspace.
 *  - Host-checkable errors return a negative status with NOTHING enqueued: null pointers,
 *    pointers not 16-byte aligned where a row is read with 16-byte loads, unsupported
 *    shapes, p outside (0, 1], budget < 1, too small a workspace.
 *  - A launch failure returns TWL_ERR_LAUNCH.
 *  - Device-side data cannot be checked synchronously, so its edge cases are defined:
 *    seq_len <= 0 is an empty sequence (nothing selected, nothing kept, zero output);
 *    seq_len is clamped to max_pages_per_seq * page_size; a page id outside
 *    [0, num_phys_pages), a candidate page outside the sequence and a kept token id
 *    outside [0, seq_len) are skipped as if absent. No input makes a kernel read or write
 *    outside the buffers described here.
 *  - fp16 means IEEE binary16. Values must be finite.
 *
 * Shapes: B = batch, Hq / Hkv = query / KV heads (Hq % Hkv == 0, G = Hq / Hkv in
 * {1, 2, 4, 8}; query head h reads KV head h / G), d = head_dim in {64, 128},
 * page_size = 16, P_b = ceil(seq_len_b / 16) pages of sequence b.
 *
 * Paged cache layout (one contiguous block per (physical page, KV head)):
 *   k_cache, v_cache : fp16  [num_phys_pages, Hkv, 16, d]
 *   page_minmax      : fp16  [B, Hkv, max_pages_per_seq, 2, d] in LOGICAL page order of
 *                      each sequence, row 0 = min, row 1 = max (so one KV head's bounds are
 *                      one contiguous stretch that the page scorer streams)
 *   k_codes          : uint8 [num_phys_pages, Hkv, 16, d * key_bits / 8]; 4-bit: byte i
 *                      = channel 2i in the low nibble, channel 2i+1 in the high nibble;
 *                      2-bit: byte i = channels 4i .. 4i+3 from the low bits up
 *   k_meta           : fp16  [num_phys_pages, Hkv, 16, d/32, 2] {scale, zero} per group
 *   page_table       : int32 [B, max_pages_per_seq] logical page -> physical page
 *   seq_lens         : int32 [B]
 */
#ifndef TWILIGHT_H_
#define TWILIGHT_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TWL_OK = 0,
  TWL_ERR_INVALID_ARG = -1, /* null or misaligned pointer, bad size or value */
  TWL_ERR_UNSUPPORTED = -2, /* a shape the library has no kernel for */
  TWL_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  TWL_ERR_LAUNCH = -4,      /* the HIP runtime rejected a kernel launch */
  TWL_ERR_SCRATCH = -5      /* the call needs more scratch than the fixed device buffer of
                               twilight_sparse_decode_noalloc holds */
} twl_status_t;

typedef struct twl_layout {
  int32_t batch;             /* B >= 0; B == 0 is a no-op */
  int32_t num_q_heads;       /* Hq */
  int32_t num_kv_heads;      /* Hkv */
  int32_t head_dim;          /* d in {64, 128} */
  int32_t page_size;         /* must be 16 */
  int32_t max_pages_per_seq; /* row stride of page_table, >= 1 */
  int32_t num_phys_pages;    /* leading extent of the paged caches, >= 1 */
  const int32_t* page_table; /* device [B, max_pages_per_seq] */
  const int32_t* seq_lens;   /* device [B] */
  int32_t key_bits;          /* width of the estimate's key codes: 4 (0 also means 4), or
                                2, the variant the pages ablate (atlas.scime.ai ablation
                                table: 4-bit keeps the estimated weights more stable) */
} twl_layout_t;

/* Int4 key cache for the weight estimate (atlas.scime.ai "Approach": weights are
 * estimated from a 4-bit quantized key cache; "Limitations": it costs about 1/8 of the
 * KV cache, which is what the codes take at 4 of fp16 K+V's 32 bits per channel).
 * Per token, KV head and group of 32 channels, with Lv = 2^key_bits - 1 (15, or 3 for
 * 2-bit codes): zero = min, scale = the fp16 value nearest (ties to even) to
 * (max - min) / Lv, code = the c in 0..Lv whose zero + c*scale is nearest to x (ties to
 * the even code); every code is 0 when scale is 0. Quantizes tokens
 * [token_begin[b], seq_len_b) of each sequence (token_begin NULL means 0), so a decode
 * step can append one token. Writes k_codes and k_meta at those tokens only. */
int twilight_quantize_keys(const twl_layout_t* L, const void* k_cache,
                           const int32_t* token_begin, uint8_t* k_codes, void* k_meta,
                           hipStream_t stream);

/* Quest per-page channelwise key bounds (atlas.scime.ai "Surprising findings": Quest
 * keeps per-page max-pooled key information). For every page holding a token at or after
 * token_begin[b] (NULL means 0), min and max of each channel over the page's valid tokens
 * (a partial last page uses only its seq_len-bounded tokens), written at the page's
 * logical position. Pages whose physical id is invalid are left untouched. */
int quest_page_bounds(const twl_layout_t* L, const void* k_cache,
                      const int32_t* token_begin, void* page_minmax, hipStream_t stream);

/* Per-step cache maintenance for a decode loop (the pages' setting is decode with a KV
 * cache that grows by one token per step, atlas.scime.ai "Approach"): for every sequence,
 * the int4 codes of tokens [token_begin[b], seq_len_b), exactly as twilight_quantize_keys
 * writes them, and, when page_minmax is not NULL, the bounds of every page holding such a
 * token, exactly as quest_page_bounds writes them. One launch of one wave per (sequence, KV
 * head) that reads each touched page's rows once, for an append of a few tokens per step.
 * token_begin (device, int32[B]) is required; values below 0 mean 0. k_cache, k_codes and
 * page_minmax must be 16-byte aligned, token_begin and k_meta 4-byte aligned; otherwise
 * TWL_ERR_INVALID_ARG and nothing is enqueued. The caller owns every buffer. */
int twilight_append_keys(const twl_layout_t* L, const void* k_cache, const int32_t* token_begin,
                         uint8_t* k_codes, void* k_meta, void* page_minmax, hipStream_t stream);

/* Quest base selector, the first (page-level top-k) stage of the hierarchy (atlas.scime.ai
 * "Approach" and "Surprising findings"). score(page) = sum over the KV head's G query heads
 * h and channels c of max(q_hc * min_c, q_hc * max_c), the largest value of q_h . k over
 * the page's bounding box, summed over the group; computed exactly (fp16 products are exact
 * in fp32 and the sums in fp64 are exact for finite fp16 inputs of ordinary range), so ties
 * are real ties. The min(budget_pages, P_b) pages with the highest score (ties: lower page
 * index) are written in ascending page order.
 *   q         : fp16 [B, Hq, d]
 *   sel_pages : int32 [B, Hkv, budget_pages] (entries past sel_count are left untouched)
 *   sel_count : int32 [B, Hkv]
 * Supports max_pages_per_seq <= 32768. Workspace: twilight_workspace_size(). */
int quest_select_pages(const twl_layout_t* L, const void* q, const void* page_minmax,
                       int32_t budget_pages, int32_t* sel_pages, int32_t* sel_count,
                       void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The two halves of quest_select_pages, for callers that want the page scores themselves.
 * quest_page_scores writes score(page) as defined above, exact in fp64, for pages
 * [0, P_b) of every (sequence, KV head); entries at and past P_b are left untouched.
 *   scores : fp64 [B, Hkv, quest_score_stride(max_pages_per_seq)], 16-byte aligned
 * quest_top_pages then writes what quest_select_pages writes, from such scores (entries at
 * and past P_b are ignored). Same limits and errors as quest_select_pages, without a
 * workspace. The caller owns every buffer. */
int64_t quest_score_stride(int32_t max_pages_per_seq); /* max_pages rounded up to 64; -1 if < 1 */
int quest_page_scores(const twl_layout_t* L, const void* q, const void* page_minmax,
                      double* scores, hipStream_t stream);
int quest_top_pages(const twl_layout_t* L, const double* scores, int32_t budget_pages,
                    int32_t* sel_pages, int32_t* sel_count, hipStream_t stream);

/* Twilight's weight estimate over the candidates (atlas.scime.ai "Approach": top-p is
 * applied to the estimated attention weights of the pre-selected tokens, estimated with
 * the 4-bit key cache). Candidate slot j = r * 16 + o is offset o of the r-th candidate
 * page; it is valid when r < cand_count[b, kvh] and its token r-th-page * 16 + o is below
 * seq_len_b. With cand_pages == NULL every page is a candidate (slot j is token j; then
 * cand_stride_pages must be >= max_pages_per_seq). For each query head h:
 * s_hj = sm_scale * q_h . dequant(k_j); weights = softmax of s_h over the valid slots;
 * invalid slots get exactly 0. Weights are fp32 and carry full precision down to 2^-126,
 * the bottom of fp32's normal range: a weight whose exact value is below 2^-126 (a logit
 * more than about 87 nats below its head's largest) comes out as some value in
 * [0, 2^-126), 0 included, since the exponentials run on the transcendental unit, which
 * returns 0 for results below the normal range. Top-p does not depend on such weights
 * beyond its mass tolerance, and at p = 1 it keeps their tokens all the same.
 *   cand_pages : int32 [B, Hkv, cand_stride_pages] ascending page ids, or NULL
 *   cand_count : int32 [B, Hkv], or NULL (then min(P_b, cand_stride_pages))
 *   weights    : fp32 [B, Hq, cand_stride_pages * 16] */
int twilight_estimate_weights(const twl_layout_t* L, const void* q, const uint8_t* k_codes,
                              const void* k_meta, const int32_t* cand_pages,
                              const int32_t* cand_count, int32_t cand_stride_pages,
                              float sm_scale, float* weights, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* Top-p pruning, the second (token-level) stage (atlas.scime.ai "Approach": top-p
 * thresholding found with binary-search top-p kernels; "Limitations": one budget per GQA
 * group). W_j = mean over the group's G heads of weights[h, j] on the valid slots. tau is
 * the largest threshold whose kept mass sum_{W_j >= tau} W_j reaches p * sum_j W_j
 * (masses summed exactly in fixed point, in units of 2^-40 of the largest W's binade);
 * p == 1 prunes nothing: every valid slot is kept, whatever its W (0 included). Below
 * p = 1, a unit with no positive W keeps nothing, and W below 2^-126 (fp32 subnormals)
 * carry no mass; a unit whose largest W is itself below 2^-126 has no fixed-point
 * resolution left and may keep every valid slot (tau 0). Softmax weights never come near
 * that case (their largest W is at least 1 / slots). The kept slots are compacted into
 * ascending logical token ids.
 *   kept       : int32 [B, Hkv, cand_stride_pages * 16] (entries past kept_count untouched)
 *   kept_count : int32 [B, Hkv]
 *   tau        : fp32 [B, Hkv] or NULL; at p == 1 the smallest positive W (0 if none)
 * Supports cand_stride_pages * 16 <= 65536 slots per unit. */
int twilight_topp_select(const twl_layout_t* L, const float* weights,
                         const int32_t* cand_pages, const int32_t* cand_count,
                         int32_t cand_stride_pages, float p, int32_t* kept,
                         int32_t* kept_count, float* tau, void* workspace,
                         size_t workspace_bytes, hipStream_t stream);

/* twilight_estimate_weights followed by twilight_topp_select (or, for the _headwise form,
 * twilight_topp_select_headwise), as one call with identical kept sets, counts and tau.
 * The top-p kernel normalises the estimate's logits itself from their per-chunk
 * (max, sum of exp) pairs, with the same arithmetic as the estimate's normalising pass, so
 * that pass (a launch and a round trip of the weights) drops out of the decode step
 * (atlas.scime.ai "Limitations": the estimate's own cost is what limits the gain when
 * loading tokens is not the bottleneck). Where top-p first forms group means over many
 * work-groups (large GQA units), that pass normalises instead.
 *   weights : fp32 [B, Hq, cand_stride_pages * 16], scratch for the call; afterwards it
 *             holds either the logits or the normalised weights, so read it only through
 *             twilight_estimate_weights.
 * The other arguments are those of the two calls; the workspace must be as large as both
 * need (twilight_workspace_size covers it). */
int twilight_estimate_topp(const twl_layout_t* L, const void* q, const uint8_t* k_codes,
                           const void* k_meta, const int32_t* cand_pages,
                           const int32_t* cand_count, int32_t cand_stride_pages,
                           float sm_scale, float p, float* weights, int32_t* kept,
                           int32_t* kept_count, float* tau, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);
int twilight_estimate_topp_headwise(const twl_layout_t* L, const void* q,
                                    const uint8_t* k_codes, const void* k_meta,
                                    const int32_t* cand_pages, const int32_t* cand_count,
                                    int32_t cand_stride_pages, float sm_scale, float p,
                                    float* weights, int32_t* kept, int32_t* kept_count,
                                    float* tau, void* workspace, size_t workspace_bytes,
                                    hipStream_t stream);

/* Head-wise top-p under GQA (atlas.scime.ai "Limitations": under GQA the pages' dynamic
 * budgets are per group, not per head, which costs adaptivity; this is the per-head form).
 * Each query head h is its own unit: the rule of twilight_topp_select with G = 1, applied to
 * weights[h] over the candidates of its KV head h / G. Same arguments, except:
 *   kept       : int32 [B, Hq, cand_stride_pages * 16]
 *   kept_count : int32 [B, Hq]
 *   tau        : fp32 [B, Hq] or NULL
 * Needs no workspace; accepts the same workspace arguments. */
int twilight_topp_select_headwise(const twl_layout_t* L, const float* weights,
                                  const int32_t* cand_pages, const int32_t* cand_count,
                                  int32_t cand_stride_pages, float p, int32_t* kept,
                                  int32_t* kept_count, float* tau, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* Sparse paged decode attention over the kept tokens (atlas.scime.ai "Key results": the
 * Twilight sparse self-attention operator). For each query head h of KV head g:
 * o_h = sum_{j in kept} softmax_j(sm_scale * q_h . k_j) v_j over the fp16 K/V cache, the
 * softmax taken over the kept set only; fp32 accumulation, fp16 output (round to nearest
 * even). An empty kept set gives o_h = 0.
 *   kept       : int32 [B, Hkv, kept_stride] logical token ids
 *   kept_count : int32 [B, Hkv] (clamped to kept_stride)
 *   out        : fp16 [B, Hq, d] */
int twilight_sparse_decode(const twl_layout_t* L, const void* q, const void* k_cache,
                           const void* v_cache, const int32_t* kept, const int32_t* kept_count,
                           int32_t kept_stride, float sm_scale, void* out, void* workspace,
                           size_t workspace_bytes, hipStream_t stream);

/* Sparse decode with one kept set per query head (the head-wise form above): o_h is the
 * attention of q_h over its own kept tokens, whose K/V rows are those of KV head h / G.
 * Same arguments as twilight_sparse_decode, except:
 *   kept       : int32 [B, Hq, kept_stride] logical token ids
 *   kept_count : int32 [B, Hq] (clamped to kept_stride) */
int twilight_sparse_decode_headwise(const twl_layout_t* L, const void* q, const void* k_cache,
                                    const void* v_cache, const int32_t* kept,
                                    const int32_t* kept_count, int32_t kept_stride,
                                    float sm_scale, void* out, void* workspace,
                                    size_t workspace_bytes, hipStream_t stream);

/* twilight_sparse_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the same kernels
 * and results, with the split-KV partials in a fixed 16 MiB device buffer that the library
 * owns (one per GPU, held until the process ends) instead of a caller's workspace. The call
 * allocates and frees nothing. Its partials need B * Hq * chunks * (d + 2) * 4 bytes, with
 * chunks = ceil(kept_stride / chunk tokens) as the decode splits the lists (for example
 * 2.1 MB for B = 1, Hq = 32, d = 128, kept_stride = 8192); a call that needs more returns
 * TWL_ERR_SCRATCH with nothing enqueued. Every call on one GPU shares that GPU's buffer:
 * calls that overlap on one GPU (other streams, other host threads) race and must be
 * ordered by the caller. Other arguments and errors as twilight_sparse_decode. */
int twilight_sparse_decode_noalloc(const twl_layout_t* L, const void* q, const void* k_cache,
                                   const void* v_cache, const int32_t* kept,
                                   const int32_t* kept_count, int32_t kept_stride,
                                   float sm_scale, void* out, hipStream_t stream);

/* Workspace bytes that every call above needs for this layout when candidate and kept
 * lists have cand_stride_pages pages (kept_stride = cand_stride_pages * 16). One
 * allocation of this size may be shared by calls issued in order on one stream. Returns 0
 * for an invalid layout. */
size_t twilight_workspace_size(const twl_layout_t* L, int32_t cand_stride_pages);

/* Static description of a status code (never NULL). */
const char* twilight_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* TWILIGHT_H_ */
