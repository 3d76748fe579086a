/*
 * sd.h - C ABI of the sparse-KV self-speculative decoding hot path (gfx950).
 *
 * The method is MagicDec's self-speculation with a compressed draft KV cache
 * ("MagicDec: Breaking the Latency-Throughput Tradeoff for Long Context
 * Generation with Speculative Decoding", deep notes on papercache.org) plus the
 * modified rejection sampling round described in "Wann beschleunigt
 * spekulatives Decoding das LLM-Serving?" (slavadubrov.com). Per round the
 * draft attends over a budget of K selected cached tokens for gamma steps, the
 * target verifies the gamma+1 candidate positions against the full cache in one
 * batched pass, and acceptance keeps a prefix of the drafts plus one
 * correction or bonus token.
 *
 * Conventions shared by every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. Shapes are listed
 *    row-major; every tensor is dense in the layout given.
 *  - Each call validates its arguments on the host, then enqueues kernels on
 *    `stream` (a hipStream_t passed as void*, NULL = the null stream) and
 *    returns without synchronising. A failed validation returns a non-zero
 *    status before any launch and before any write.
 *  - The library allocates no memory. Its mutable global state is a
 *    per-device cache of resident-wave counts (an occupancy query made once
 *    per kernel and device; a race stores the same value), which sets launch
 *    sizes and the split-KV schedule only, so a device always computes the
 *    same bits; and the per-device scratch array of sd_spec_accept_noalloc
 *    (see there). Calls are thread-safe and re-entrant. Scratch space is the
 *    caller's `workspace` of at least the size its *_workspace_size function
 *    returns; concurrent calls need distinct workspaces.
 *  - Device-resident integers (page_table, kv_lens, idx, sel_lens,
 *    draft_tokens) are the caller's responsibility and are not validated;
 *    kernels clamp them into range so that bad values give wrong numbers,
 *    not out-of-bounds accesses.
 *  - Random numbers are inputs: the library draws none.
 *  - Results are bitwise reproducible for a given input and shape.
 *  - Errors from the HIP runtime at launch return SD_ERR_HIP; faults inside
 *    kernels surface at the caller's next synchronisation.
 */
#ifndef SD_H_
#define SD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SD_OK = 0,
  SD_ERR_INVALID_ARG = 1, /* null pointer, negative or inconsistent size */
  SD_ERR_UNSUPPORTED = 2, /* valid but not implemented (head_dim, dtype, rows) */
  SD_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required */
  SD_ERR_HIP = 4          /* the HIP runtime reported an error at launch */
} sd_status;

typedef enum { SD_BF16 = 0, SD_F32 = 1 } sd_dtype;

/*
 * One layer's paged KV cache, read-only for every call here.
 * k_pages, v_pages: [num_pages, num_kv_heads, page_size, head_dim] of dtype;
 *   each (page, head) block of page_size * head_dim elements is contiguous.
 * page_table: int32 [batch, max_pages]; token t of sequence b lives in page
 *   page_table[b*max_pages + t/page_size] at slot t % page_size.
 * kv_lens: int32 [batch] valid tokens per sequence (for verify this count
 *   includes the n_q tokens being verified).
 * page_size must be a multiple of 16; head_dim 64 or 128.
 * k_pages and v_pages must be 16-byte aligned, and so must every query and
 *   attention output array below (the kernels move rows in 16-byte pieces):
 *   else SD_ERR_INVALID_ARG.
 */
typedef struct {
  const void *k_pages;
  const void *v_pages;
  const int32_t *page_table;
  const int32_t *kv_lens;
  int32_t num_pages;
  int32_t page_size;
  int32_t max_pages;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t dtype; /* sd_dtype */
} sd_kv_cache;

/*
 * Verify attention (MagicDec notes, §3.1-§3.2: the target scores the gamma
 * drafted positions plus one in a single batched pass over the full KV cache,
 * so verification and decoding share the same KV loading cost).
 *
 * q: [batch, n_q, num_q_heads, head_dim] of kv->dtype, n_q = gamma + 1; the
 *   n_q verify tokens are the last n_q tokens of each sequence's cache and
 *   query i (0-based) attends causally to positions 0 .. kv_len - n_q + i.
 * GQA: query head h reads KV head h / (num_q_heads / num_kv_heads).
 * softmax_scale multiplies q.k (pass 1.0 when the scale is folded into q); it
 *   must be finite and > 0 (softmax_scale * log2(e) finite), else
 *   SD_ERR_INVALID_ARG.
 * max_kv_len: an upper bound on kv_lens (sizes the split-KV plan; must not
 *   exceed max_pages * page_size).
 * out: [batch, n_q, num_q_heads, head_dim] of kv->dtype (bf16 results are
 *   rounded to nearest even). lse: [batch, n_q, num_q_heads] float32 natural-
 *   log log-sum-exp of the scaled scores, or NULL. A row that sees no key gets
 *   out = 0 and lse = -inf.
 * Limits: (num_q_heads / num_kv_heads) * n_q <= 64; batch * ceil(max_kv_len / 16)
 *   < 2^31 (else SD_ERR_UNSUPPORTED).
 */
sd_status sd_verify_attn(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                         int32_t num_q_heads, int32_t max_kv_len, float softmax_scale,
                         void *out, float *lse, void *workspace, size_t workspace_bytes,
                         void *stream);

size_t sd_verify_attn_workspace_size(int32_t batch, int32_t n_q, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim,
                                     int32_t max_kv_len);

/*
 * Draft attention over a compressed KV budget (MagicDec notes, §3.3 and §4.1:
 * the self-speculative draft is the target model attending to a sparse subset
 * of its own KV cache, at a cost that grows with the budget K, not with the
 * context).
 *
 * idx: int32 [batch, idx_heads, max_sel] cached positions; idx_heads is 1 (one
 *   set for all KV heads, as StreamingLLM selects), num_kv_heads (one set per
 *   KV head, as SnapKV selects) or num_q_heads (one set per query head, as
 *   sd_topk_select selects). Sequence b, KV head g uses the first sel_lens[b]
 *   entries of idx[b, idx_heads > 1 ? g : 0, :]; with one set per query head
 *   (and num_q_heads > num_kv_heads), query head h uses idx[b, h, :].
 * Every query row attends to every selected position (q: [batch, n_q,
 *   num_q_heads, head_dim], normally n_q = 1). softmax_scale, out and lse as
 *   for verify.
 * Limits: (num_q_heads / num_kv_heads) * n_q <= 64; batch * ceil(max_sel / 16)
 *   < 2^31 (else SD_ERR_UNSUPPORTED).
 */
sd_status sd_draft_attn_sparse(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t n_q,
                               int32_t num_q_heads, const int32_t *idx, const int32_t *sel_lens,
                               int32_t idx_heads, int32_t max_sel, float softmax_scale, void *out,
                               float *lse, void *workspace, size_t workspace_bytes, void *stream);

size_t sd_draft_attn_sparse_workspace_size(int32_t batch, int32_t n_q, int32_t num_q_heads,
                                           int32_t num_kv_heads, int32_t head_dim,
                                           int32_t max_sel);

/*
 * Draft attention over the selection plus the tokens appended since it was
 * made (MagicDec notes, §3.3 and §4.1: the static compressed cache is chosen
 * once at prefill; each draft step then also reads the tokens generated after
 * that, the drafts of the current round included).
 *
 * As sd_draft_attn_sparse, and sequence b, KV head g then also reads
 * positions tail_begin[b] .. kv->kv_lens[b] - 1 in order (an empty range when
 * kv_lens[b] <= tail_begin[b]). tail_begin: int32 [batch], device. max_tail
 *   bounds kv_lens[b] - tail_begin[b] (longer tails are cut to it).
 * Workspace: sd_draft_attn_sparse_workspace_size.
 * Limits: as sd_draft_attn_sparse, with batch * ceil((max_sel + max_tail) / 16)
 *   < 2^31; 0 <= max_tail <= max_pages * page_size.
 */
sd_status sd_draft_attn_sparse_tail(const sd_kv_cache *kv, const void *q, int32_t batch,
                                    int32_t n_q, int32_t num_q_heads, const int32_t *idx,
                                    const int32_t *sel_lens, int32_t idx_heads, int32_t max_sel,
                                    const int32_t *tail_begin, int32_t max_tail,
                                    float softmax_scale, void *out, float *lse, void *workspace,
                                    size_t workspace_bytes, void *stream);

/*
 * StreamingLLM draft set (named as a static KV selection in the MagicDec
 * notes, §4.4 and §5.2): the first `sink` positions and the last `recent`
 * positions of each sequence, ascending, without duplicates:
 *   [0, min(sink, L)) U [max(sink, L - recent), L).
 * idx: int32 [batch, 1, sink + recent] (entries past sel_lens[b] are -1);
 * sel_lens: int32 [batch] = min(L, sink + recent).
 * Errors: SD_ERR_INVALID_ARG for null pointers, batch <= 0, negative sink or
 * recent, or sink + recent == 0; SD_ERR_UNSUPPORTED for sink + recent >= 2^30.
 */
sd_status sd_streaming_select(const int32_t *kv_lens, int32_t batch, int32_t sink,
                              int32_t recent, int32_t *idx, int32_t *sel_lens, void *stream);

/*
 * SnapKV draft set (named as the best static KV selection in the MagicDec
 * notes, §4.4 and §5.2; built once at prefill and reused for drafting,
 * Appendix A.1). Per (sequence b, KV head g) with L = kv_lens[b]:
 *  1. the last `window` prompt positions are the observation window;
 *     q_obs[b, w, h] (w < window, h in g's query-head group) attends causally
 *     to keys 0 .. L - window + w with softmax weights p;
 *  2. vote_j = sum over the group's heads and the window rows of p, j < L - window;
 *  3. votes are max-pooled with odd kernel `pool_kernel`, stride 1, clipped;
 *  4. the budget - window prefix positions with the largest pooled value are
 *     kept, ties toward the lower position;
 *  5. idx[b, g, :] = ascending union of those and the window (budget entries).
 *  If L <= budget every position 0..L-1 is kept (rest -1).
 * q_obs: [batch, window, num_q_heads, head_dim] of kv->dtype. softmax_scale
 *   multiplies q_obs.k inside the softmax of step 1 (1.0 when the scale is
 *   folded into q_obs); finite and > 0 as for verify, else SD_ERR_INVALID_ARG.
 * idx: int32 [batch, num_kv_heads, budget]; sel_lens: int32 [batch] = min(L, budget).
 * Limits: budget > window >= 1; (num_q_heads / num_kv_heads) * window <= 128;
 *   pool_kernel odd and >= 1; max_kv_len bounds kv_lens; batch *
 *   ceil(max_kv_len / 16) < 2^31 (else SD_ERR_UNSUPPORTED).
 */
sd_status sd_snapkv_select(const sd_kv_cache *kv, const void *q_obs, int32_t batch,
                           int32_t window, int32_t num_q_heads, int32_t pool_kernel,
                           int32_t budget, int32_t max_kv_len, float softmax_scale,
                           int32_t *idx, int32_t *sel_lens, void *workspace,
                           size_t workspace_bytes, void *stream);

size_t sd_snapkv_select_workspace_size(int32_t batch, int32_t window, int32_t num_q_heads,
                                       int32_t num_kv_heads, int32_t max_kv_len);

/*
 * The observation window's softmax normalisers, step 1 of sd_snapkv_select
 * alone (MagicDec notes, Appendix A.1: the SnapKV set is built at prefill,
 * where the attention of the window queries is computed anyway; a prefill
 * attention kernel returns these values as its log-sum-exp).
 * lse: float32 [batch, window, num_q_heads], device: for sequence b with
 *   L = kv_lens[b], lse[b, w, h] = ln sum_j exp(softmax_scale * q_obs[b, w, h] . k_j)
 *   over j = 0 .. L - window + w of KV head h / (num_q_heads / num_kv_heads);
 *   -inf for a row that sees no key (L - window + w < 0). Every sequence is
 *   scored, whatever its length.
 * q_obs, softmax_scale, max_kv_len and the limits are those of
 * sd_snapkv_select (no budget or pool kernel). Workspace:
 * sd_snapkv_select_workspace_size. One pass over K.
 */
sd_status sd_snapkv_window_lse(const sd_kv_cache *kv, const void *q_obs, int32_t batch,
                               int32_t window, int32_t num_q_heads, int32_t max_kv_len,
                               float softmax_scale, float *lse, void *workspace,
                               size_t workspace_bytes, void *stream);

/*
 * sd_snapkv_select with the window normalisers of step 1 given instead of
 * computed (MagicDec notes, §4.4 and Appendix A.1: the window's attention
 * comes from the prefill): obs_lse float32 [batch, window, num_q_heads],
 * device, as written by sd_snapkv_window_lse, with p = exp(softmax_scale *
 * q.k - obs_lse) in step 2. One pass over K instead of two. With the values
 * sd_snapkv_window_lse returns the selection equals sd_snapkv_select's up to
 * the fp32 rounding of the normalisers (votes within a few units in the last
 * place), so only near ties at the cut can differ. Finite values are the
 * caller's to supply (-inf marks a row that sees no key). Other arguments,
 * outputs, limits and workspace: as sd_snapkv_select.
 */
sd_status sd_snapkv_select_lse(const sd_kv_cache *kv, const void *q_obs, const float *obs_lse,
                               int32_t batch, int32_t window, int32_t num_q_heads,
                               int32_t pool_kernel, int32_t budget, int32_t max_kv_len,
                               float softmax_scale, int32_t *idx, int32_t *sel_lens,
                               void *workspace, size_t workspace_bytes, void *stream);

/*
 * SnapKV with one budget per sequence (MagicDec notes, §4.3: the best draft
 * budget depends on batch size and context length, so a ragged batch may give
 * each sequence its own): as sd_snapkv_select, with sequence b selected on
 * budgets[b] (int32 [batch], device; values are clamped into
 * [window + 1, max_budget]). idx: int32 [batch, num_kv_heads, max_budget], rows
 * padded with -1 past min(L, budgets[b]); sel_lens[b] = min(L, budgets[b]).
 * Workspace: sd_snapkv_select_workspace_size. Limits: as sd_snapkv_select with
 * budget = max_budget.
 */
sd_status sd_snapkv_select_budgets(const sd_kv_cache *kv, const void *q_obs, int32_t batch,
                                   int32_t window, int32_t num_q_heads, int32_t pool_kernel,
                                   const int32_t *budgets, int32_t max_budget, int32_t max_kv_len,
                                   float softmax_scale, int32_t *idx, int32_t *sel_lens,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * Top-K attention selection for one draft step (MagicDec notes, §4.4: dynamic
 * selection searches the cache again for every query; exact top-K attention
 * keeps acceptance high at a small budget but pays its search at every draft
 * step, and §4.1 counts that search in the draft cost).
 *
 * q: [batch, 1, num_q_heads, head_dim] bf16, the draft query. For sequence b
 *   and query head h, s_j = <q_h, k_j> over the kv_lens[b] cached keys of KV
 *   head h / (num_q_heads / num_kv_heads); the `budget` positions with the
 *   largest s_j are kept, ties to the lower position, ascending (a positive
 *   softmax scale does not change the order, so none is taken). A sequence
 *   not longer than the budget keeps every position.
 * idx: int32 [batch, num_q_heads, budget]: the kept positions, then -1.
 * sel_lens: int32 [batch] = min(kv_len, budget). Feed both to
 *   sd_draft_attn_sparse with idx_heads = num_q_heads.
 * Scores are fp32 sums of exact bf16 products; where two scores lie within
 *   fp32 rounding of each other at the cut, either may be kept.
 * Limits: bf16 caches; num_q_heads / num_kv_heads <= 16; batch *
 *   ceil(max_kv_len / 16) < 2^31 (else SD_ERR_UNSUPPORTED). max_kv_len bounds
 *   kv_lens as for verify. Workspace: sd_topk_select_workspace_size (about
 *   8 * batch * num_q_heads * max_kv_len bytes: room for a 32-bit key and a
 *   position per cached token of every row; a call writes only the keys at
 *   or above a sampled per-row threshold, and recomputes a row in full when
 *   the threshold proves too high, so the result never depends on it).
 */
sd_status sd_topk_select(const sd_kv_cache *kv, const void *q, int32_t batch, int32_t num_q_heads,
                         int32_t budget, int32_t max_kv_len, int32_t *idx, int32_t *sel_lens,
                         void *workspace, size_t workspace_bytes, void *stream);

size_t sd_topk_select_workspace_size(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t max_kv_len);

/*
 * Modified rejection sampling for one verification round ("Wann beschleunigt
 * spekulatives Decoding das LLM-Serving?", section on a verification round):
 * per sequence, with p_i = softmax(target_logits[b, i] / temperature) and
 * q_i = softmax(draft_logits[b, i] / temperature):
 *  - for i = 0..gamma-1, draft token x_i is accepted iff
 *    u_accept[b, i] * q_i(x_i) < p_i(x_i); stop at the first rejection; n = count;
 *  - the emitted token y is drawn from max(0, p_n - q_n) normalised (or from
 *    p_n if that is identically zero) when n < gamma, else from p_gamma (bonus):
 *    y = smallest t with cumulative weight > u_sample[b, n] * total.
 * target_logits: float32 [batch, gamma+1, vocab]; draft_logits: float32
 *   [batch, gamma, vocab]; draft_tokens: int32 [batch, gamma];
 *   u_accept: float32 [batch, gamma], u_sample: float32 [batch, gamma+1],
 *   uniforms in [0, 1).
 * n_accepted: int32 [batch]; out_tokens: int32 [batch, gamma+1] =
 *   [x_0 .. x_{n-1}, y, -1 ...].
 * Softmax exponentials are float32; normalisers and cumulative sums are
 *   accumulated in float64. The residual weights are formed as
 *   p (1 - q/p) from the logit difference and the difference of the two
 *   normalisers (itself from a float64 sum of p-weighted expm1 of the logit
 *   differences), so they keep float32's relative accuracy when q is close
 *   to p.
 * Limits: gamma >= 0, vocab >= 1, 0 < temperature < inf, null pointers
 *   (draft_* and u_accept may be null only when gamma = 0): else
 *   SD_ERR_INVALID_ARG; gamma <= 64, vocab < 2^30,
 *   batch * (gamma + 1) * vocab < 2^40 and batch * (2 gamma + 1) < 2^31: else
 *   SD_ERR_UNSUPPORTED; a workspace smaller than
 *   sd_spec_accept_workspace_size: SD_ERR_WORKSPACE.
 */
sd_status sd_spec_accept(const float *target_logits, const float *draft_logits,
                         const int32_t *draft_tokens, const float *u_accept,
                         const float *u_sample, int32_t batch, int32_t gamma, int32_t vocab,
                         float temperature, int32_t *n_accepted, int32_t *out_tokens,
                         void *workspace, size_t workspace_bytes, void *stream);

size_t sd_spec_accept_workspace_size(int32_t batch, int32_t gamma, int32_t vocab);

/*
 * Allocation-free acceptance, for callers that cannot allocate device memory
 * or pass a workspace: code under HIP graph capture, tight serving loops and
 * harnesses that forbid allocation. Same arguments and results as
 * sd_spec_accept, bit for bit, without the workspace: the scratch comes from a
 * fixed array of SD_SPEC_ACCEPT_SCRATCH_BYTES inside the library's device
 * memory (one copy per GPU, held until the process ends; its device address
 * is looked up once per device on the first call there). The call allocates
 * nothing and needs no cleared memory (every scratch byte is written before
 * it is read).
 * All calls on one GPU share that GPU's array: calls that overlap in time on
 * one GPU (different streams, or other host threads) race and may return
 * wrong results; serialise them on one stream.
 * stream must belong to the current device (else SD_ERR_INVALID_ARG).
 * Limits: as sd_spec_accept, and sd_spec_accept_workspace_size(batch, gamma,
 *   vocab) <= SD_SPEC_ACCEPT_SCRATCH_BYTES, else SD_ERR_UNSUPPORTED (about
 *   864 sequences at gamma = 4 over a 128256-token vocabulary).
 */
#define SD_SPEC_ACCEPT_SCRATCH_BYTES (4u << 20)

sd_status sd_spec_accept_noalloc(const float *target_logits, const float *draft_logits,
                                 const int32_t *draft_tokens, const float *u_accept,
                                 const float *u_sample, int32_t batch, int32_t gamma, int32_t vocab,
                                 float temperature, int32_t *n_accepted, int32_t *out_tokens,
                                 void *stream);

/*
 * Draft-token sampling is sd_spec_accept with gamma = 0: draft_logits,
 * draft_tokens and u_accept may be NULL, n_accepted is 0 and out_tokens[b, 0]
 * is drawn from softmax(target_logits[b, 0] / temperature) by inverse CDF with
 * u_sample[b, 0].
 */

/*
 * Append n_new tokens' K/V at the end of every sequence (MagicDec notes,
 * §3.1-§3.3: each draft step and the verification pass add the K/V of the
 * tokens they process to the cache).
 *
 * k_new, v_new: [batch, n_new, num_kv_heads, head_dim] of kv->dtype, device,
 *   16-byte aligned (else SD_ERR_INVALID_ARG).
 * Token j of sequence b goes to position p = kv->kv_lens[b] + j: page
 *   kv->page_table[b, p / page_size], slot p % page_size, of the pools kv
 *   points at. THIS CALL WRITES kv->k_pages and kv->v_pages (the only entry
 *   point that does); it does not change kv_lens (see sd_kv_advance).
 * The caller provides the pages; positions at or past max_pages * page_size
 *   are not written, and page ids are clamped into [0, num_pages).
 */
sd_status sd_kv_append(const sd_kv_cache *kv, const void *k_new, const void *v_new,
                       int32_t batch, int32_t n_new, void *stream);

/*
 * kv_lens[b] <- max(0, kv_lens[b] + add + (n_accepted ? n_accepted[b] : 0)),
 * on the device. After appending a round's gamma + 1 tokens and accepting n
 * drafts: add = -gamma keeps the round's first token and the accepted drafts
 * (MagicDec notes, §3.1: rejected drafts are discarded).
 * kv_lens: int32 [batch], device, updated in place; n_accepted: int32 [batch]
 *   or NULL.
 */
sd_status sd_kv_advance(int32_t *kv_lens, const int32_t *n_accepted, int32_t batch, int32_t add,
                        void *stream);

/*
 * The draft's compressed cache as a cache of its own (MagicDec notes, §4.4
 * and Appendix A.1: the draft reads a static compressed KV cache built once
 * at prefill). Copies the K and V rows of each selection, in list order, into
 * caller-owned pools, so that the draft steps become dense decodes
 * (sd_verify_attn with n_q = 1) over contiguous pages instead of gathers.
 * idx: int32 [batch, idx_heads, max_sel], idx_heads = 1 (one set for every KV
 *   head) or num_kv_heads; sel_lens: int32 [batch] (entries past
 *   min(sel_lens[b], max_sel) are not read); both device, as for
 *   sd_draft_attn_sparse.
 * k_out, v_out: [batch * pages_per_seq, num_kv_heads, page_size, head_dim] of
 *   kv->dtype, 16-byte aligned, device. List entry t of sequence b and KV
 *   head h goes to page b * pages_per_seq + t / page_size, head h, slot
 *   t % page_size; slots past the selection are left as they were.
 *   pages_per_seq >= ceil(max_sel / page_size) (more leaves room for tokens
 *   appended later with sd_kv_append).
 * The compact cache is then {k_out, v_out, page_table[b][j] =
 *   b * pages_per_seq + j, kv_lens = the selection lengths, num_pages =
 *   batch * pages_per_seq, max_pages = pages_per_seq, the source's page size,
 *   heads, head_dim and dtype}; its dense decode equals the draft over the
 *   selection up to the fp32 summation order.
 * Errors: SD_ERR_INVALID_ARG for null or misaligned pointers, batch <= 0,
 *   max_sel < 1, idx_heads not 1 or num_kv_heads, pages_per_seq too small;
 *   SD_ERR_UNSUPPORTED when the compact pool would exceed the cache limits.
 */
sd_status sd_kv_compact(const sd_kv_cache *kv, const int32_t *idx, const int32_t *sel_lens,
                        int32_t batch, int32_t idx_heads, int32_t max_sel, int32_t pages_per_seq,
                        void *k_out, void *v_out, void *stream);

/*
 * Analytic speedup model, host only (no GPU call; safe on any thread). The
 * MagicDec summary (jarxiv.com) gives the speedup of speculative decoding as
 * T_T * Omega(gamma, alpha) / (gamma * T_D + T_V(gamma)), where with a
 * compressed draft cache gamma * T_D becomes T_select(K) + gamma * T_D(K)
 * (MagicDec notes, §3.1 and §4.1). Times are in any one unit.
 *
 * sd_expected_tokens: Omega = sum_{i=0..gamma} alpha^i, the expected tokens
 *   of one round for a constant per-token acceptance rate alpha in [0, 1];
 *   NaN for gamma < 0 or alpha outside [0, 1].
 * sd_speedup: t_target * Omega / (t_select_fixed + gamma * t_select_step +
 *   gamma * t_draft + t_verify). t_select_fixed is the selection cost charged
 *   to one round by a static selection (made once), t_select_step that of a
 *   dynamic selection searched at every draft step. NaN for a negative or
 *   non-finite time, t_target <= 0, or a round time of 0.
 * sd_best_gamma: the gamma in 1..max_gamma with the lowest expected time per
 *   token (round time / Omega; ties to the smaller gamma), t_verify[g - 1]
 *   being T_V(g); writes it and its speedup. SD_ERR_INVALID_ARG for null
 *   pointers, max_gamma < 1, or any argument sd_speedup rejects.
 */
double sd_expected_tokens(int32_t gamma, double alpha);

double sd_speedup(double t_target, double t_draft, double t_verify, int32_t gamma, double alpha,
                  double t_select_fixed, double t_select_step);

sd_status sd_best_gamma(double t_target, double t_draft, const double *t_verify, int32_t max_gamma,
                        double alpha, double t_select_fixed, double t_select_step, int32_t *gamma_out,
                        double *speedup_out);

/*
 * Streaming-read probe: the attainable HBM read bandwidth, the ceiling the
 * attention kernels are measured against next to the nominal figure (MagicDec
 * notes, §3.2: at long context verification and drafting are bound by loading
 * the KV cache). Not a step of the method: a measurement tool.
 *
 * Reads `bytes` bytes at `buf` once with 16-byte loads (with the nontemporal
 * hint when nontemporal = 1, plain loads when 0), each wave of `blocks`
 * 256-thread workgroups streaming one contiguous slice (blocks = 0: as many
 * as the chip keeps resident), and ADDS the sum of its 32-bit words, modulo
 * 2^32, to *checksum: the caller zeroes *checksum first (it is never cleared
 * here). The best launch size depends on the chip and the access pattern, so
 * a measurement sweeps `blocks` and keeps the fastest.
 * buf: device, 16-byte aligned, bytes > 0 and a multiple of 16;
 * checksum: device, one uint32, 4-byte aligned. Read-only on buf.
 * SD_ERR_INVALID_ARG for null pointers, a misaligned buffer, a size that is
 * zero or not a multiple of 16, nontemporal not 0 or 1, or blocks outside
 * [0, 65536].
 */
sd_status sd_hbm_read_probe(const void *buf, size_t bytes, int32_t nontemporal, int32_t blocks,
                            uint32_t *checksum, void *stream);

/* Static string for a status code (never NULL). */
const char *sd_status_string(sd_status status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t sd_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SD_H_ */
