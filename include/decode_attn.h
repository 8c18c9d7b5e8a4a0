/*
 * decode_attn.h -- C ABI of libdecode_attn.so: folded-GQA single-token decode
 * attention and the Quest query-aware sparse variant, for AMD MI355X (gfx950).
 *
 * Sources, cited by page and section:
 *   [CoreML-GQA]   "Core ML Decode Optimization: Removing the 1.9 GiB Per-Token
 *                  Copy Caused by GQA repeat_kv" (OptAI engineering blog).
 *   [Quest-review] jaehun.me review of "Quest: Query-Aware Sparsity for
 *                  Efficient Long-Context LLM Inference" (paper sections 3.3-3.5,
 *                  Algorithm 1 as the review cites them).
 *
 * Conventions for every entry point
 *   - Pointers marked (device) are HIP device pointers; (host) are host memory.
 *   - fp16 means IEEE binary16; every tensor is contiguous, row-major, last
 *     axis fastest.  fp16 is the only element type for Q, K, V and outputs.
 *   - Query head h belongs to KV head h / G with G = Hq / Hkv, i.e. the heads
 *     of one group are contiguous (h = G*kv + g).  [CoreML-GQA] section 3 "Why
 *     Reshape Replaces Integer Division"; interleaved head orders (section 5)
 *     are outside the contract and cannot be detected.
 *   - seqlens (device, int32 [B]) holds the valid length L_b of each sequence,
 *     *including* the token appended this step.  Values are clamped on the
 *     device to [0, capacity]; L_b = 0 yields an all-zero output row.
 *   - The caller owns every buffer, including the workspace.  The library never
 *     allocates, frees or synchronises, and keeps no pointer after returning.
 *     All work is enqueued on `stream` (a hipStream_t; NULL = null stream) and
 *     is complete after the caller synchronises that stream.
 *   - Workspace: size it with da_workspace_size / da_quest_workspace_size.
 *     It holds per-split partial results, for one call a page choice, and a
 *     work counter that the paged attention launch takes its chunks from
 *     (the call clears it first).  It needs no initialisation, nothing a call
 *     leaves in it changes a later call's result, and it must not be shared
 *     between calls that may run concurrently.
 *   - Return value: DA_OK or a negative DA_ERR_* code.  All argument checks run
 *     before anything is enqueued; only DA_ERR_HIP can follow a partial enqueue.
 *     The library never prints and never aborts.
 */
#ifndef DECODE_ATTN_H
#define DECODE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum da_status {
  DA_OK = 0,
  DA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  DA_ERR_SHAPE = -2,       /* inconsistent sizes (Hq % Hkv != 0, capacity < 1, ...) */
  DA_ERR_UNSUPPORTED = -3, /* D not in {64,128}, G not in {1,2,4,8}, S not in {8,16,32,64} */
  DA_ERR_BUDGET = -4,      /* token budget not a positive multiple of S          */
  DA_ERR_WORKSPACE = -5,   /* workspace too small                                */
  DA_ERR_HIP = -6,         /* a HIP launch or query failed (e.g. no device)      */
  DA_ERR_TOO_LARGE = -7    /* gqa_decode_attn_noalloc: the call needs more than
                              DA_NOALLOC_SCRATCH_BYTES of split partials        */
};

/* Size of the library's static per-device scratch used by
 * gqa_decode_attn_noalloc (32 MiB). */
#define DA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * A KV cache, described on the host (the struct itself is host memory).
 *
 * Contiguous (page_table == NULL):
 *   k, v      (device) fp16 [batch, num_kv_heads, capacity, head_dim].
 *   page_size  Quest metadata page size S (only read by the quest_* calls).
 * Paged (page_table != NULL):
 *   k, v      (device) fp16 pool [num_pages, num_kv_heads, page_size, head_dim].
 *   page_table (device) int32 [batch, max_pages]: token t of sequence b is row
 *              (t mod S) of pool page page_table[b][t / S].  Entries for pages
 *              that hold a valid token must lie in [0, num_pages); this is a
 *              precondition the device cannot check.
 *   capacity   is ignored; the per-sequence capacity is max_pages * page_size.
 * k and v are written only by calls that append a row (k_new/v_new != NULL).
 */
typedef struct da_kv_cache {
  void* k;
  void* v;
  const int32_t* page_table;
  int32_t batch;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t capacity;
  int32_t page_size;
  int32_t max_pages;
  int64_t num_pages;
} da_kv_cache;

/* Human-readable name of a status code (static storage; never NULL). */
const char* da_status_string(int status);

/*
 * Workspace bytes for gqa_decode_attn (budget_tokens == 0) or
 * quest_sparse_decode_attn (budget_tokens > 0, the token budget K*S) on this
 * cache with num_q_heads query heads and the given num_splits (0 = automatic).
 * Writes the size to *bytes_out (host).  The split heuristic depends only on
 * these arguments, so a workspace sized once can be reused for every call with
 * the same shapes.  With a budget it also covers the choice [B, Hkv, K] int32
 * that quest_select_sparse_decode_attn keeps there above 16384 pages per unit
 * when it is given no page_idx.
 */
int da_workspace_size(const da_kv_cache* kv, int32_t num_q_heads, int32_t budget_tokens,
                      int32_t num_splits, size_t* bytes_out);

/*
 * Folded GQA decode attention.  [CoreML-GQA] section 3 "Fold Q Instead of
 * Expanding KV" / "Implementation": Q [B, Hq, D] is read as [B, Hkv, G, D], so
 * every K/V row is read from HBM once for the G query heads that share it (no
 * repeat_kv copy); scores = scale * q.k over t < L_b, softmax over the context
 * axis, out = prob . V, written back as [B, Hq, D].
 *
 *   q          (device) fp16 [B, Hq, D]
 *   kv         (host)   cache description (contiguous or paged)
 *   seqlens    (device) int32 [B]
 *   num_q_heads Hq; Hq % Hkv == 0 and G = Hq / Hkv in {1, 2, 4, 8}
 *   scale      multiplier on q.k (1/sqrt(D) for standard attention)
 *   k_new, v_new (device) fp16 [B, Hkv, D] or both NULL.  When given, the row
 *              is first stored at slot L_b - 1 of the cache ([CoreML-GQA]
 *              section 1: one position per token) and attention covers
 *              [0, L_b) including it.  Skipped for sequences with L_b = 0.
 *   out        (device) fp16 [B, Hq, D]
 *   workspace  (device) >= da_workspace_size(kv, Hq, 0, num_splits) bytes
 *   num_splits 0 = automatic; otherwise the number of context chunks per
 *              (b, kv) unit for the longest possible sequence.
 */
int gqa_decode_attn(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                    int32_t num_q_heads, float scale, const void* k_new, const void* v_new,
                    void* out, void* workspace, size_t workspace_bytes, int32_t num_splits,
                    void* stream);

/*
 * gqa_decode_attn for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments and result as gqa_decode_attn, without the workspace: the
 * split partials go to a static device array inside the library
 * (DA_NOALLOC_SCRATCH_BYTES per GPU, held by every GPU the library runs on
 * until the process ends).  The call allocates and frees nothing; the caller
 * still passes every input and output buffer.
 *
 *   arguments as gqa_decode_attn (workspace omitted).
 *   Returns DA_ERR_TOO_LARGE, before anything is enqueued, when
 *   da_workspace_size(kv, num_q_heads, 0, num_splits) exceeds
 *   DA_NOALLOC_SCRATCH_BYTES; otherwise as gqa_decode_attn.
 * Every call on one GPU shares that GPU's scratch: calls that may overlap on
 * one GPU (different streams, concurrent host threads) race on it and must be
 * ordered by the caller.  The scratch needs no clearing between calls (each
 * call writes every partial it reads).  Its device address is looked up on
 * the first call on each device (the device current at the call).
 */
int gqa_decode_attn_noalloc(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                            int32_t num_q_heads, float scale, const void* k_new,
                            const void* v_new, void* out, int32_t num_splits, void* stream);

/*
 * Folded GQA attention for q_len > 1 query positions per head (chunked
 * prefill, speculative verify).  [CoreML-GQA] section 5 "Limitations and Next
 * Steps" ("Prefill Needs Separate Design"): the group and sequence axes are
 * merged into one row axis, and the causal mask is aligned per row.  Q
 * [B, Hq, q_len, D] is read as [B, Hkv, G * q_len, D]; every K/V row is read
 * once for all G * q_len rows.  The q_len queries are the last q_len positions
 * of each sequence: query i of sequence b attends to keys
 * t <= L_b - q_len + i (their own K/V rows must already be in the cache);
 * a query with no such key (L_b - q_len + i < 0) yields zeros.
 *
 *   q          (device) fp16 [B, Hq, q_len, D]
 *   q_len      1 <= q_len; G * q_len must be in {1, 2, 4, 8}
 *   out        (device) fp16 [B, Hq, q_len, D]
 *   workspace  >= da_workspace_size(kv, Hq * q_len, 0, num_splits) bytes
 *   other arguments as gqa_decode_attn (no append: write the new rows first).
 * With q_len = 1 the result equals gqa_decode_attn without an append.
 */
int gqa_decode_attn_multi(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                          int32_t num_q_heads, int32_t q_len, float scale, void* out,
                          void* workspace, size_t workspace_bytes, int32_t num_splits,
                          void* stream);

/*
 * Materialised repeat_kv, the copy the fold removes; for A/B comparison only.
 * [CoreML-GQA] section 2 "Why Does GQA Replicate KV?" (and "expand Is a View,
 * but reshape Introduces a Copy"): the GQA reference path copies each KV head
 * to the G query heads that read it.  This call builds that tensor so that
 * gqa_decode_attn can run on it with num_kv_heads = Hq (G = 1), the baseline
 * of the page's section 4 comparison.
 *
 *   kv         (host)   cache description (contiguous or paged)
 *   num_q_heads Hq; G = Hq / Hkv in {1, 2, 4, 8}
 *   seqlens    (device) int32 [B]; clamped to [0, capacity] on the device
 *   k_out, v_out (device) fp16 [B, Hq, cap, D], cap = kv->capacity (contiguous)
 *              or kv->max_pages * page_size (paged): row t of head h is row t
 *              of KV head h / G for t < L_b.  Rows t >= L_b, and rows of a
 *              paged sequence whose page-table entry is outside the pool, are
 *              not written.  The outputs must not overlap the cache.
 * Reads every valid cache byte once and writes it G times.
 */
int gqa_repeat_kv(const da_kv_cache* kv, int32_t num_q_heads, const int32_t* seqlens,
                  void* k_out, void* v_out, void* stream);

/*
 * Quest metadata update.  [Quest-review] "the page score is not an exact
 * attention probability" (paper section 3.4): per page p and channel i keep
 * the Key minimum m_{p,i} and maximum M_{p,i}, updated as new Keys arrive.
 *
 *   kv         (host)   cache description; S = kv->page_size in {8,16,32,64}
 *   meta       (device) fp16 [B, Hkv, meta_max_pages, 2, D]; [...,0,:] = min,
 *              [...,1,:] = max.  meta_max_pages * S >= per-sequence capacity;
 *              meta_max_pages <= 2^28 in every quest_* call (DA_ERR_SHAPE).
 *   seqlens    (device) int32 [B] (lengths after this update)
 *   n_new      keys [L_b - n_new, L_b) are folded in, in order.  A key at a
 *              page start (t mod S == 0) resets that page to (k, k); any other
 *              key lowers the min and raises the max.  n_new = 1 is the decode
 *              step; n_new >= capacity rebuilds every page from the cache.
 *   k_new, v_new (device) fp16 [B, Hkv, D] or both NULL.  When given, n_new
 *              must be 1 and the row is also stored at slot L_b - 1 of the
 *              cache (so a following sparse attention call sees it).
 * The update is exact (min/max of fp16 values) and idempotent for n_new = 1.
 */
int quest_meta_append(const da_kv_cache* kv, void* meta, int32_t meta_max_pages,
                      const int32_t* seqlens, int32_t n_new, const void* k_new,
                      const void* v_new, void* stream);

/*
 * Quest workspace bytes for quest_page_score_topk (page scores of every
 * (b, kv) unit when the caller passes page_scores = NULL).
 */
int da_quest_workspace_size(int32_t batch, int32_t num_kv_heads, int32_t meta_max_pages,
                            size_t* bytes_out);

/*
 * Quest page scores and top-K pages.  [Quest-review] (paper section 3.4,
 * Algorithm 1): U(p, q) = sum_i max(q_i m_{p,i}, q_i M_{p,i}); keep the K pages
 * with the highest U.  With G > 1 query heads per KV head the score of a page
 * is the sum of U over the G heads of the group, and one page set per (b, kv)
 * serves all of them.  No softmax scale is applied (the ranking is invariant
 * to a common positive scale).
 *
 *   q          (device) fp16 [B, Hq, D]
 *   meta       (device) fp16 [B, Hkv, meta_max_pages, 2, D] (quest_meta_append)
 *   seqlens    (device) int32 [B]; pages p < ceil(L_b / S) exist
 *   page_size  S in {8, 16, 32, 64}
 *   budget_tokens  B = K * S tokens ([Quest-review] "distinguish page count
 *              from token budget"); must be a positive multiple of S.
 *   page_idx   (device) int32 [B, Hkv, K] out: the min(K, P_b) chosen pages in
 *              ascending page order, then -1.  Ties in U go to the lower index.
 *              NULL: scores only (no top-K launch); page_scores is then
 *              required, e.g. for quest_select_sparse_decode_attn.
 *   page_scores (device) fp32 [B, Hkv, meta_max_pages] out, or NULL to keep the
 *              scores in the workspace.  Entries p >= P_b are not written.
 *   workspace  (device) >= da_quest_workspace_size(...) bytes when
 *              page_scores is NULL (may be NULL otherwise)
 * Up to 16384 pages per (b, kv) the top-K launch holds the unit's scores in
 * registers; above that a streaming top-K launch (1,024 threads per unit)
 * re-reads the score row once per radix pass.  Same choice either way.
 */
int quest_page_score_topk(const void* q, const void* meta, int32_t meta_max_pages,
                          const int32_t* seqlens, int32_t batch, int32_t num_q_heads,
                          int32_t num_kv_heads, int32_t head_dim, int32_t page_size,
                          int32_t budget_tokens, int32_t* page_idx, float* page_scores,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step's cache and metadata update fused into page scoring:
 * the effect of quest_meta_append(kv, meta, meta_max_pages, seqlens, 1, k_new,
 * v_new) followed by quest_page_score_topk(q, meta, ...) in one score launch
 * plus the top-K launch, with bit-identical results.  [Quest-review] (paper
 * section 3.4): the metadata is updated as each new Key arrives, then the
 * query scores the pages; [CoreML-GQA] section 5 names the update path as the
 * next thing to fuse.  The workgroup that scores page (L_b - 1) / S folds
 * k_new into that page's min/max (reset at a page start) before scoring it,
 * writes the page's metadata back and stores k_new / v_new at slot L_b - 1 of
 * the cache.
 *
 *   q          (device) fp16 [B, Hq, D]
 *   kv         (host)   cache description (contiguous or paged); S =
 *              kv->page_size in {8, 16, 32, 64}; D and Hkv from kv
 *   meta       (device) fp16 [B, Hkv, meta_max_pages, 2, D], updated in place;
 *              meta_max_pages * S >= per-sequence capacity
 *   seqlens    (device) int32 [B], lengths after this step (L_b >= 1 appends;
 *              L_b = 0 appends nothing)
 *   k_new, v_new (device) fp16 [B, Hkv, D], both required
 *   budget_tokens, page_idx, page_scores, workspace: as quest_page_score_topk
 *   (the workspace size is da_quest_workspace_size(B, Hkv, meta_max_pages);
 *   page_idx NULL with page_scores given: the append and the scores only).
 */
int quest_append_score_topk(const void* q, const da_kv_cache* kv, void* meta,
                            int32_t meta_max_pages, const int32_t* seqlens, int32_t num_q_heads,
                            int32_t budget_tokens, const void* k_new, const void* v_new,
                            int32_t* page_idx, float* page_scores, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * Attention over the chosen pages only.  [Quest-review] flowchart and worked
 * example (paper sections 3.3-3.5): exact attention over the real K/V of the
 * tokens in the chosen pages, [p*S, min(p*S + S, L_b)) for every p in
 * page_idx[b][kv], folded across the G query heads of the group; the softmax
 * renormalises over those tokens.
 *
 *   page_idx   (device) int32 [B, Hkv, K] as written by quest_page_score_topk
 *              (ascending, -1 padded); K = budget_tokens / kv->page_size
 *   other arguments as gqa_decode_attn (no append: use quest_meta_append's
 *   k_new/v_new for the step's row).  A paged cache must use the same page
 *   size as the metadata.
 */
int quest_sparse_decode_attn(const void* q, const da_kv_cache* kv, const int32_t* seqlens,
                             const int32_t* page_idx, int32_t budget_tokens,
                             int32_t num_q_heads, float scale, void* out, void* workspace,
                             size_t workspace_bytes, int32_t num_splits, void* stream);

/*
 * Top-K page selection fused into the attention over the chosen pages: the
 * effect of the top-K half of quest_page_score_topk followed by
 * quest_sparse_decode_attn, with bit-identical choice and output, in one
 * attention launch (plus the split merge) instead of two.  [Quest-review]
 * (paper section 3.4 and the flowchart of section 3.3): keep the K pages
 * with the highest score, then attend over their tokens only.  Every
 * workgroup of a (b, kv) unit selects from the unit's scores itself and
 * attends over its share of the choice.
 *
 *   page_scores (device) fp32 [B, Hkv, meta_max_pages] as written by
 *              quest_page_score_topk or quest_append_score_topk (with page_idx
 *              NULL, for the scores alone); entries p >= P_b are ignored.
 *   meta_max_pages  row width of page_scores; meta_max_pages * S >= the
 *              per-sequence capacity.  Above 16384 pages per (b, kv) the call
 *              runs the streaming top-K launch of quest_page_score_topk
 *              first and the attention over its choice second (written to
 *              page_idx, or to the workspace without it): the same choice
 *              and output, one launch more.
 *   page_idx   (device) int32 [B, Hkv, K] out: the choice, as
 *              quest_page_score_topk writes it; or NULL
 *   budget_tokens, q, kv, seqlens, num_q_heads, scale, out, workspace
 *              (da_workspace_size(kv, Hq, budget_tokens, num_splits) bytes),
 *              num_splits, stream: as quest_sparse_decode_attn.
 * Returns DA_ERR_NULL if page_scores is NULL (B > 0), DA_ERR_SHAPE if
 * meta_max_pages does not cover the capacity (or, above 16384 pages, B or Hkv
 * exceeds 65535), otherwise as quest_sparse_decode_attn.
 */
int quest_select_sparse_decode_attn(const void* q, const da_kv_cache* kv,
                                    const int32_t* seqlens, const float* page_scores,
                                    int32_t meta_max_pages, int32_t budget_tokens,
                                    int32_t num_q_heads, float scale, int32_t* page_idx,
                                    void* out, void* workspace, size_t workspace_bytes,
                                    int32_t num_splits, void* stream);

/*
 * Debugging aid, not part of the method: reports the device-side inputs that
 * the other calls clamp or mask silently instead of failing on (they cannot
 * see device memory at call time).  Run it on the same cache and lengths,
 * on the same stream, when results look wrong.
 *
 *   kv         (host)   cache description (contiguous or paged)
 *   seqlens    (device) int32 [B]
 *   report     (device) int32 [4] out, written by one small kernel:
 *              [0] sequences with L_b < 0 or L_b > capacity (they are clamped
 *                  to [0, capacity] by every call);
 *              [1] paged caches: page-table entries of pages that hold a
 *                  valid token (p < ceil(min(L_b, capacity) / S)) that lie
 *                  outside [0, num_pages) (every call masks those tokens);
 *                  0 for a contiguous cache;
 *              [2] the lowest sequence index with such an input, or -1;
 *              [3] 0.
 * Asynchronous on `stream`; reads seqlens and the page table only.
 * Returns DA_OK (and writes nothing) for B = 0, DA_ERR_NULL / DA_ERR_SHAPE /
 * DA_ERR_UNSUPPORTED for bad arguments as the attention calls check them,
 * or DA_ERR_HIP.
 */
int da_check_cache(const da_kv_cache* kv, const int32_t* seqlens, int32_t* report, void* stream);

/*
 * Measurement helper, not part of the method: the HBM read rate a plain
 * streaming kernel reaches, the practical ceiling next to the nominal peak
 * for kernels that stream K/V or page metadata.  Reads the `bytes` bytes at
 * `buf` once with coalesced 16-byte non-temporal loads and folds them with
 * XOR; `sink` receives one uint32 only if the fold equals a fixed constant
 * (so the reads cannot be elided), and is otherwise left untouched.
 *   buf   (device) any contents, 16-byte aligned
 *   bytes > 0, a multiple of 16
 *   sink  (device) uint32 [1]
 * Asynchronous on `stream`; time it with events on that stream.
 * Returns DA_ERR_NULL (buf or sink NULL), DA_ERR_SHAPE (bytes not a positive
 * multiple of 16, or buf misaligned) or DA_ERR_HIP.
 */
int da_read_calibration(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DECODE_ATTN_H */
