/*
 * spd.h -- C ABI of a sparse paged decode-attention step for AMD gfx950.
 *
 * One decode step, per (request b, KV head h) "row":
 *   1. page_meta_build      per-page channel-wise key min / max
 *                           (LServe summary, "Hierarchical Paging" -- logical page
 *                           statistics k_min / k_max -- and "Key statistics storage and
 *                           updating": refreshed as tokens are appended); or
 *      page_stats_build     per-page channel-wise key mean / variance (Moira, section 3.1)
 *   2. page_score           Quest-style page bound S_j = sum_i max(q_i kmax_i, q_i kmin_i)
 *                           (LServe, "Hierarchical Paging", page importance score), combined
 *                           over the query-head group; in coverage mode turned into Moira's
 *                           group-mean page share pi_bar (Moira, section 3.2, Eq. 3), from the
 *                           bound or from the mvar estimate of each page's mass (Eq. 2)
 *   3. page_select          page list per row: forced sink + local pages plus either the
 *                           best pages under a page budget (LServe, "Token budget and
 *                           physical page selection") or the smallest share-threshold set
 *                           reaching gamma (Moira, section 3.2, Eq. 3 and Algorithm 1);
 *                           streaming heads take only the static sink + local table
 *                           (LServe, "Decoding Stage: Kernel Implementation with Two-Level
 *                           Indexing")
 *   4. sparse_paged_decode  grouped-query decode attention over the listed pages through the
 *                           native block table (PersistentKV, sections 3.1-3.3), split over a
 *                           device-side self-planned grid (Moira, section 3.3, Eq. 4 and
 *                           Algorithm 2)
 *   5. lse_merge            exact log-sum-exp merge of the split states (PersistentKV,
 *                           section 3.3; Moira, section 3.3 "Merge")
 *
 * Hierarchical paging (LServe summary, "Hierarchical Paging"; spd_desc.page_size = 64): physical
 * pages of N_P = 64 tokens hold 4 logical pages of N_L = 16 tokens.  Key statistics are kept per
 * logical page; a physical page's score is the largest score of its logical pages ("Physical page
 * importance aggregation"); under the coverage rule a physical page's share is the sum of its
 * logical pages' shares (mass is additive); the budget, the sink and local windows and the lists
 * count physical pages ("Token budget and physical page selection": K = ceil(token budget / N_P)),
 * and attention reads every valid token of each listed physical page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers marked (device) are device memory owned by the caller; pointers marked (host)
 *    are host memory read during the call only.  The library never allocates, frees or
 *    synchronises, and never reads device memory from the host, so every call can be
 *    captured into a hipGraph.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Work is only
 *    enqueued; results are ready when the stream reaches the enqueued work.
 *  - Every call returns SPD_OK (0) or a negative spd_status.  Argument checks happen on the
 *    host before anything is enqueued; on an error nothing is launched.  SPD_ERR_LAUNCH
 *    reports a HIP launch failure.  No exceptions cross the ABI and, apart from the per-device
 *    address of spd_sparse_paged_decode_noalloc's array, there is no global mutable state, so calls
 *    from several host threads are safe.
 *  - Layouts are dense row-major C arrays:
 *      q            [B, Hq, d]                 f32 or f16 (spd_desc.q_dtype)
 *    P = spd_desc.page_size (tokens of a physical page), g = P / 16 (logical pages per
 *    physical page: 1, or 4 with hierarchical paging)
 *      k_pool,v_pool [num_pool_pages, Hkv, P, d]  f32, f16 or fp8 E4M3FN bytes
 *      k_scale,v_scale [num_pool_pages, Hkv, P]  fp16 bits (fp8 pools only; value =
 *                                              E4M3FN(code) * scale)
 *      page_meta    [B, Hkv, max_pages_per_seq * g, 2, d] per request, in logical page
 *                                              order: entry [b, h, p] is logical page p of
 *                                              request b (tokens 16 p .. 16 p + 15); index 0 =
 *                                              channel min, 1 = channel max; f32 for f32 pools,
 *                                              f16 otherwise (for fp8 pools rounded outward:
 *                                              min down, max up).  The key statistics are
 *                                              request state, like the request's block-table
 *                                              row: a caller that moves a request to another
 *                                              batch position moves its rows with it
 *      page_stats   [B, Hkv, max_pages_per_seq * g, 2, d] bf16 bits, per request in logical
 *                                              page order as page_meta: index 0 = channel mean, 1 =
 *                                              channel variance (mean squared deviation) of
 *                                              the page's valid keys, each rounded to nearest
 *                                              even (Moira, section 3.1 "Page summaries and the
 *                                              mvar estimate"; bf16 as in "Memory for page
 *                                              summaries").  Scorers with the MVAR estimator
 *                                              take it in the page_meta argument.
 *      block_table  [B, max_pages_per_seq]     int32 physical page holding tokens
 *                                              [P j, P j + P) of the request, j = 0, 1, ...
 *      seq_lens     [B]                        int32 tokens of each request
 *      head_kind    [Hkv]                      uint8 (host) SPD_HEAD_DYNAMIC or _STREAMING
 *      scores       [B, Hkv, max_pages_per_seq] f32, per block-table slot j
 *      page_list    [B, Hkv, max_list]         int32 block-table slots j, ascending
 *      list_len     [B, Hkv]                   int32
 *      out          [B, Hq, d]                 f32; out_lse [B, Hq] f32 (natural log of the
 *                                              softmax denominator of the scaled logits)
 *      part_o       [B, Hkv, J, G, d] f32 and part_lse [B, Hkv, J, G] f32, J from
 *                                              spd_plan_grid
 *  - Request b has n_b = ceil(seq_lens[b] / P) pages (block-table slots) and ceil(seq_lens[b] /
 *    16) logical pages; logical page p holds min(16, seq_lens[b] - 16 p) valid tokens, in
 *    physical page block_table[b, p / g] at token slots 16 (p mod g) .. 16 (p mod g) + 15
 *    (PersistentKV, section 3.3: bounds follow the row's own length).  With P = 16 a page and a
 *    logical page are the same thing, and "page" below means either; otherwise rows, scores,
 *    budgets, forced windows and lists count pages (slots of P tokens) and statistics count
 *    logical pages.  Only valid tokens enter the statistics and the attention; the remaining
 *    slots of a partial page may hold anything, NaN included.
 *  - Robustness: n_b is clamped to max_pages_per_seq, negative lengths count as 0, list
 *    entries outside [0, n_b) and block-table entries outside [0, num_pool_pages) are
 *    treated as empty pages (never dereferenced).
 */
#ifndef SPD_H_
#define SPD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPD_ABI_VERSION 18
#define SPD_PAGE_SIZE 16       /* logical page, and the plain physical page */
#define SPD_HIER_PAGE_SIZE 64  /* physical page of hierarchical paging (4 logical pages) */
#define SPD_MAX_KV_HEADS 64

typedef enum spd_status {
  SPD_OK = 0,
  SPD_ERR_INVALID_ARG = -1,  /* null pointer, inconsistent sizes, bad enum value */
  SPD_ERR_UNSUPPORTED = -2,  /* valid but not compiled: head dim, group size, dtype combo */
  SPD_ERR_LAUNCH = -3,       /* a HIP launch failed (hipGetLastError) */
  SPD_ERR_WORKSPACE = -4     /* workspace null or smaller than spd_workspace_bytes */
} spd_status;

typedef enum spd_dtype {
  SPD_DTYPE_F32 = 0,
  SPD_DTYPE_F16 = 1,
  SPD_DTYPE_FP8_E4M3FN = 2   /* OCP 8-bit E4M3, no infinities, 0x7F / 0xFF are NaN */
} spd_dtype;

typedef enum spd_select_mode {
  SPD_SELECT_TOPK = 0,       /* fixed page budget */
  SPD_SELECT_COVERAGE = 1    /* smallest share-threshold set reaching gamma */
} spd_select_mode;

/* How COVERAGE estimates the attention mass of a page: */
typedef enum spd_estimator {
  SPD_ESTIMATOR_BOUND = 0,   /* from the key box: l = sm_scale * S + ln(valid tokens) */
  SPD_ESTIMATOR_MVAR = 1     /* from the page summary (Moira, section 3.1, Eq. 2):
                              * l_g = s q_g . mu + (1/2) (s q_g)^2 . sigma^2 + ln(valid tokens),
                              * s = sm_scale; the row's first page and its last page are not
                              * estimated but computed exactly, l_g = log sum_k exp(s q_g . k)
                              * over their valid keys read from k_pool */
} spd_estimator;

typedef enum spd_head_kind {
  SPD_HEAD_DYNAMIC = 0,
  SPD_HEAD_STREAMING = 1
} spd_head_kind;

/* What the scorers do with the last logical page of each dynamic row (the page the newest
 * token is in): */
typedef enum spd_tail_mode {
  SPD_TAIL_NONE = 0,     /* score it from page_meta like every other page */
  SPD_TAIL_REBUILD = 1,  /* rebuild its key min / max from k_pool first (written to page_meta),
                          * then score it (LServe, "Key statistics storage and updating") */
  SPD_TAIL_SKIP = 2      /* do not score it: TOPK with n_local >= 1 only (the local window keeps
                          * the page whatever its score); its score (and its sel_scores entry) is
                          * written as -inf and page_meta is not read for it, so
                          * spd_page_meta_build may refresh it concurrently */
} spd_tail_mode;

typedef enum spd_op {
  SPD_OP_PAGE_SCORE = 0,
  SPD_OP_PAGE_SELECT = 1,
  SPD_OP_PAGE_SCORE_SELECT = 2
} spd_op;

/* Shapes of one step.  Supported: page_size 16 or 64; head_dim 64 or 128; Hq / Hkv = 4;
 * (q_dtype, kv_dtype) in {(f32, f32), (f16, f16), (f16, fp8)}.  page_size 64 (hierarchical
 * paging) supports both rules and both estimators (summaries and estimates per 16-token logical
 * page), tail modes NONE and SKIP, and the unfused entry points; f32 pools need head_dim 64 there.  Others return SPD_ERR_UNSUPPORTED so
 * a caller can route them elsewhere. */
typedef struct spd_desc {
  int32_t batch;              /* B >= 0 */
  int32_t num_q_heads;        /* Hq */
  int32_t num_kv_heads;       /* Hkv, 1..SPD_MAX_KV_HEADS, divides Hq */
  int32_t head_dim;           /* d */
  int32_t page_size;          /* 16, or 64 (hierarchical paging) */
  int32_t max_pages_per_seq;  /* block-table row stride, >= 1 */
  int32_t num_pool_pages;     /* pool pages, >= 1 */
  int32_t max_list;           /* page_list row stride, >= 1 */
  int32_t q_dtype;            /* spd_dtype */
  int32_t kv_dtype;           /* spd_dtype */
} spd_desc;

/* Selection rule.  Forced pages of a dynamic row are 0..n_sink-1 and n_b-n_local..n_b-1;
 * a streaming row keeps exactly 0..n_sink_stream-1 and n_b-n_local_stream..n_b-1 (each
 * page once).  TOPK: the list holds the forced pages plus the best budget_pages - |forced|
 * other pages by (score desc, page asc); all pages when n_b <= budget_pages; only the
 * forced pages when they fill the budget.  COVERAGE: t = gamma - sum of forced shares;
 * the list holds the forced pages plus every other page whose share is >= tau, the
 * largest share value whose at-or-above mass reaches t (Moira, Eq. 3); t <= 0 keeps the
 * forced pages only, and all pages are kept when the other pages cannot reach t. */
typedef struct spd_select_params {
  int32_t mode;               /* spd_select_mode */
  int32_t budget_pages;       /* TOPK budget (pages, forced included), >= 1 */
  float gamma;                /* COVERAGE target in (0, 1] */
  float sm_scale;             /* COVERAGE log-mass scale s (usually 1/sqrt(d)), > 0 */
  int32_t n_sink;
  int32_t n_local;
  int32_t n_sink_stream;
  int32_t n_local_stream;
  int32_t estimator;          /* spd_estimator; MVAR needs COVERAGE */
  void* topk_state;           /* (device, nullable) TOPK with the BOUND estimator and page_size 16 only: the
                               * LiteTopK gate state of every (token) row, spd_topk_state_bytes(rows)
                               * bytes, zero-filled before its first use and then left to the library.
                               * When set, spd_page_select / spd_page_select_mq predict each row's gate
                               * from its previous selection (LiteTopK, section 3.3 "Predictive Gating":
                               * the lower edge where 1.5 K' free pages are reached) and, on the next call,
                               * rank only the free pages scoring at or above it when they number at
                               * least the K' = budget - |forced| pages the rule takes and at most 2048
                               * (then they hold the top K' and every page tied with the K'-th; LiteTopK,
                               * section 3.2 "Top-k Selection"), else the whole row.  Lists are those of
                               * the ungated selection exactly.  Calls on one state must not overlap.
                               * Ignored by the scorers and spd_page_list_refresh. */
} spd_select_params;

/* Self-planned split (Moira, section 3.3, Eq. 4): J = max(min_blocks_per_row,
 * ceil(min_grid_blocks / (B * Hkv))) blocks per row; row with n listed pages is cut into
 * chunks of c = max(min_chunk, ceil(n / J)) pages, m = ceil(n / c) of them; block j >= m
 * exits at once.  J is fixed by (B, Hkv) so a captured graph serves every list length.
 *
 * balanced != 0 plans the whole step at once instead (for skewed list lengths): with T the
 * total listed pages of all rows, n_max the longest list and z the number of rows with a
 * non-empty list, every chunk holds c = max(min_chunk, ceil(T / N'), ceil(n_max / 1024))
 * pages, where N' = N_T - z when N_T > z and N' = N_T otherwise; row r has m_r = ceil(n_r / c)
 * chunks, chunks are numbered row by row, and block k of the N_T + B * Hkv blocks processes
 * chunk k (sum m_r < N_T when N_T > z, and sum m_r <= N_T + B * Hkv always).  Every block derives the plan from the list lengths on
 * the device, so a captured graph still serves every list length.  min_blocks_per_row is
 * not used; N_T >= 1. */
typedef struct spd_plan_params {
  int32_t min_chunk;          /* C >= 1 */
  int32_t min_blocks_per_row; /* N_J >= 1 */
  int32_t min_grid_blocks;    /* N_T >= 0 (>= 1 when balanced) */
  int32_t balanced;           /* 0: per-row split (Eq. 4); 1: step-wide split */
} spd_plan_params;

/* ------------------------------------------------------------------ entry points */

/* Channel-wise min / max of the valid keys of logical pages p of each request, for every KV
 * head, read through the block table and written to page_meta at [b, h, p].  first_page and
 * span_pages count logical pages.  first_page (device, [B], may be
 * NULL): when set, pages first_page[b] .. min(n_b, first_page[b] + span_pages) - 1 are built
 * (span_pages >= 1).  When NULL, span_pages = 0 builds every page 0..n_b-1 (the bulk build at
 * prefill) and span_pages >= 1 builds the last span_pages pages of each request, read from
 * seq_lens on the device -- span_pages = 1 is the refresh of the page the newest token is in.
 * k_scale (device) is required for fp8 pools and ignored otherwise.  Other entries of page_meta,
 * and those of pages whose block-table entry is outside [0, num_pool_pages), are not touched. */
int spd_page_meta_build(const spd_desc* desc, const void* k_pool, const uint16_t* k_scale,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* first_page, int32_t span_pages, void* page_meta,
                        void* stream);

/* Moira page summaries (section 3.1, "Page summaries and the mvar estimate"): channel mean and
 * variance of the valid keys of logical pages of each request, every KV head, written to
 * page_stats (bf16, layout above) at [b, h, p].  Pages, arguments and errors as
 * in spd_page_meta_build. */
int spd_page_stats_build(const spd_desc* desc, const void* k_pool, const uint16_t* k_scale,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* first_page, int32_t span_pages, void* page_stats,
                         void* stream);

/* Page scores of every dynamic row (streaming rows are skipped, their scores untouched).
 * TOPK: scores[b,h,p] = max over the G query heads of the row of S_{g,p} (LServe page
 * importance, computed from page_meta); with page_size 64, the largest of these over the logical
 * pages of page p that hold valid tokens (LServe, "Physical page importance aggregation"), and
 * SPD_TAIL_SKIP skips the row's last page (all its logical pages); COVERAGE takes l, head_lse and
 * the shares over logical pages and writes scores[b,h,p] = the sum of the shares of page p's
 * logical pages.  COVERAGE: l_{g,p} = sm_scale * S_{g,p} +
 * ln(valid tokens of p); head_lse[b, h*G+g] = logsumexp_p l_{g,p}; scores[b,h,p] =
 * (1/G) sum_g exp(l_{g,p} - head_lse) (Moira's group-mean share, section 3.2, Eq. 3).
 * The key boxes are read from page_meta at [b, h, p] alone; block_table (device) only marks the
 * pages whose entry lies outside [0, num_pool_pages): they score -inf (TOPK) or carry no mass.
 * tail_mode (spd_tail_mode) says how each dynamic row's last logical page is treated;
 * SPD_TAIL_REBUILD reads k_pool (and k_scale for fp8 pools) and writes the entries of page_meta
 * of each request's last page for every KV head, streaming heads included (what
 * spd_page_meta_build does for that page), which page_meta is otherwise only read for;
 * SPD_TAIL_SKIP is valid in TOPK mode only.  head_lse
 * (device, [B, Hq]) may be NULL in TOPK mode.  workspace (device) of spd_workspace_bytes(desc,
 * sel, SPD_OP_PAGE_SCORE) bytes (0 in TOPK mode).
 * With the MVAR estimator page_meta holds page_stats; k_pool (and k_scale for fp8 pools) is
 * always read, for the exact first and last pages; SPD_TAIL_NONE leaves page_stats untouched and
 * SPD_TAIL_REBUILD also writes the last page's summary (what spd_page_stats_build does for that
 * page), for the steps after this one -- the page itself is computed exactly either way. */
int spd_page_score(const spd_desc* desc, const spd_select_params* sel, const void* q,
                   void* page_meta, const void* k_pool, const uint16_t* k_scale,
                   int32_t tail_mode, const int32_t* block_table, const int32_t* seq_lens,
                   const uint8_t* head_kind, float* scores, float* head_lse, void* workspace,
                   size_t workspace_bytes, void* stream);

/* Page list of every row from its scores (selection rule: spd_select_params).  Lists are
 * ascending pages (block-table slots).  page_phys (device, [B, Hkv, max_list], may be NULL) receives the
 * physical page of each listed page, read from block_table (device, required when page_phys
 * is set), so spd_sparse_paged_decode need not read the block table.  When page_meta (device,
 * may be NULL) is set, workgroups beside the selection also rebuild the key min / max of each
 * request's last logical page (the one the newest token is in), every KV head, from k_pool (and k_scale for fp8 pools) into
 * page_meta -- what spd_page_meta_build does with first_page = that page and span 1 (LServe,
 * "Key statistics storage and updating"); block_table is then required, and the scores must
 * not depend on those statistics (the scorer ran with SPD_TAIL_SKIP).  sel_scores (device,
 * [B, Hkv, max_list], may be NULL) receives the score of each listed page of a dynamic row
 * (streaming rows: untouched).  With the MVAR estimator page_meta is page_stats and the last
 * page's summary is rebuilt by a second launch on the same stream, after the selection.  Returns
 * SPD_ERR_INVALID_ARG when max_list cannot hold the
 * longest possible list: TOPK needs max_list >= max(budget, n_sink + n_local) and
 * >= n_sink_stream + n_local_stream; COVERAGE needs max_list >= max_pages_per_seq.  Rows of
 * more than 65536 pages return SPD_ERR_UNSUPPORTED. */
int spd_page_select(const spd_desc* desc, const spd_select_params* sel, const float* scores,
                    const int32_t* seq_lens, const uint8_t* head_kind, const int32_t* block_table,
                    const void* k_pool, const uint16_t* k_scale, void* page_meta, int32_t* page_list,
                    int32_t* page_phys, int32_t* list_len, float* sel_scores, void* stream);

/* spd_page_score followed by spd_page_select in one launch, for both rules (LiteTopK,
 * section 3.2, "Extension to Decoding": selection fused into score computation).  The
 * workgroups of a row score into the workspace; the last one to finish selects the row.
 * tail_mode as in spd_page_score.  scores (device,
 * [B, Hkv, max_pages_per_seq], may be NULL) receives the TOPK scores or COVERAGE shares of
 * dynamic rows; head_lse (device, [B, Hq], may be NULL) the COVERAGE per-head log-sum-exp.
 * page_list, page_phys, list_len, sel_scores as in spd_page_select (block_table is
 * required).  workspace (device) of spd_workspace_bytes(desc, sel, SPD_OP_PAGE_SCORE_SELECT)
 * bytes must be zero-filled before its first use; every call leaves its counters zero
 * again.  Calls that share one workspace must not overlap.  The MVAR estimator returns
 * SPD_ERR_UNSUPPORTED. */
int spd_page_score_select(const spd_desc* desc, const spd_select_params* sel, const void* q,
                          void* page_meta, const void* k_pool, const uint16_t* k_scale,
                          int32_t tail_mode, const int32_t* block_table, const int32_t* seq_lens,
                          const uint8_t* head_kind, int32_t* page_list, int32_t* page_phys,
                          int32_t* list_len, float* sel_scores, float* scores, float* head_lse,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Reusable page selection (LServe, "Reusable Page Selection": the selector runs on the first
 * step of each chunk of decoding steps and its lists serve the rest of the chunk).  Called on
 * each later step of a chunk, after the requests have grown: a dynamic row keeps its list and
 * gets the pages of the current forced set (n_sink sink pages, n_local local pages) that lie past
 * its last entry appended in ascending order; a streaming row's list is rewritten as its static
 * sink + local table for the current length.  Lengths must not shrink between the selection and
 * this call.  max_list must leave room for the pages a chunk can add (one per 16 tokens
 * appended, plus one); entries that do not fit are dropped.  page_phys (device, may be NULL)
 * receives the physical page of every appended entry; block_table is required.  When page_meta is
 * set, workgroups beside the rows also rebuild the key min / max of each request's last page (with
 * the MVAR estimator: its summary), as in spd_page_select.  Same ownership and errors as
 * spd_page_select. */
int spd_page_list_refresh(const spd_desc* desc, const spd_select_params* sel, const int32_t* seq_lens,
                          const uint8_t* head_kind, const int32_t* block_table, const void* k_pool,
                          const uint16_t* k_scale, void* page_meta, int32_t* page_list,
                          int32_t* page_phys, int32_t* list_len, void* stream);

/* Grouped-query decode attention of every row over its listed pages.  Block (b, h, j)
 * processes chunk j of row (b, h) (spd_plan_params; with page_size 64 the plan counts 16-token
 * units, four per listed page, so list_len n plans as 4 n); rows with one chunk write out /
 * out_lse directly, rows with more write their chunk states to part_o / part_lse for
 * spd_lse_merge.  A row with no listed pages writes out = 0 and out_lse = -inf.
 * page_phys (device, may be NULL) holds the physical page of each list entry (as written by
 * the selectors); when NULL they are read from block_table.  k_scale / v_scale (device) are
 * required for fp8 pools. */
int spd_sparse_paged_decode(const spd_desc* desc, const spd_plan_params* plan, const void* q,
                            const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                            const uint16_t* v_scale, const int32_t* block_table,
                            const int32_t* seq_lens, const int32_t* page_list,
                            const int32_t* page_phys, const int32_t* list_len, float sm_scale,
                            float* out, float* out_lse, float* part_o, float* part_lse,
                            void* stream);

/* spd_sparse_paged_decode with the merge in the same launch (a fused decode + merge): each block
 * of a row with more than one chunk writes its chunk state, makes it visible device-wide and takes
 * a ticket on its row in counters (device, [B, Hkv] uint32); the block that takes the row's last
 * ticket merges the row's chunk states exactly (as spd_lse_merge) into out / out_lse and sets the
 * ticket back to 0.  No block waits for another.  counters must be zero-filled before the first
 * call and is left zero by every call; calls that share counters must not overlap.  part_o /
 * part_lse are still needed (the chunk states pass through them).  No spd_lse_merge follows. */
int spd_sparse_paged_decode_merged(const spd_desc* desc, const spd_plan_params* plan, const void* q,
                                   const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                                   const uint16_t* v_scale, const int32_t* block_table,
                                   const int32_t* seq_lens, const int32_t* page_list,
                                   const int32_t* page_phys, const int32_t* list_len, float sm_scale,
                                   float* out, float* out_lse, float* part_o, float* part_lse,
                                   uint32_t* counters, void* stream);

/* Exact merge of the chunk states of every row with more than one chunk:
 * out_lse = log sum_j exp(lse_j), out = sum_j exp(lse_j - out_lse) * o_j.  Rows with at
 * most one chunk are left as spd_sparse_paged_decode wrote them.  Must see the same
 * list_len and plan as the decode call it follows. */
int spd_lse_merge(const spd_desc* desc, const spd_plan_params* plan, const float* part_o,
                  const float* part_lse, const int32_t* list_len, float* out, float* out_lse,
                  void* stream);

/* spd_sparse_paged_decode followed by spd_lse_merge, for callers that cannot allocate memory (code
 * under graph capture, tight serving loops, harnesses that forbid allocation): the chunk partials
 * live in a device array inside the library, SPD_NOALLOC_SCRATCH_BYTES bytes, one per GPU, held
 * until the process ends; the caller passes only inputs and outputs, with the meaning, layouts and
 * results of spd_sparse_paged_decode + spd_lse_merge.  Nothing is allocated or freed.  The first call
 * on a device looks the array's address up for that device (not a stream operation; make that call
 * before capturing the entry point into a graph).  Returns SPD_ERR_WORKSPACE when the partials of
 * the descriptor and plan (spd_partials_size: part_o elements, then part_lse elements after rounding
 * up to 256 bytes, 4 bytes each) exceed SPD_NOALLOC_SCRATCH_BYTES, SPD_ERR_LAUNCH when the device or
 * the array's address cannot be found; other errors as spd_sparse_paged_decode.  Every call on a GPU
 * uses that GPU's one array: calls that overlap on one GPU (other streams, other host threads) race
 * and must be serialised by the caller. */
#define SPD_NOALLOC_SCRATCH_BYTES (32u << 20)
int spd_sparse_paged_decode_noalloc(const spd_desc* desc, const spd_plan_params* plan, const void* q,
                                    const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                                    const uint16_t* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* page_list, const int32_t* page_phys, const int32_t* list_len,
                                    float sm_scale, float* out, float* out_lse, void* stream);

/* ------------------------------------------------------------------ several query tokens per request
 *
 * One step for T <= SPD_MQ_MAX_TOKENS query tokens per request -- the draft tokens that
 * speculative decoding verifies at once -- with their page lists shared as one scan (LiteTopK,
 * section 3.4, LiteDSA: "Candidate Union and Membership Masks", "Grouped Sparse Attention").
 * Request b's cache holds seq_lens[b] = L keys, the draft tokens' included; query token t sits at
 * position L - T + t and attends to positions < L - T + 1 + t.  The caller scores every token's
 * pages in one scan with spd_page_score_mq and selects them with spd_page_select_mq (row b T + t:
 * token t's queries, request b's block-table row, length L - T + 1 + t derived on the device, key
 * statistics covering all L keys), then merges them with spd_page_list_union and attends with spd_sparse_paged_decode_mq
 * and spd_lse_merge_mq.  Supported: page_size 16, max_pages_per_seq <= SPD_MQ_MAX_PAGES; decode
 * and merge need f16 queries, f16 or fp8 pools, head_dim 128 and the per-row plan (balanced = 0). */
#define SPD_MQ_MAX_TOKENS 4
#define SPD_MQ_ROWS 16          /* chunk-state rows per (request, KV head): 4 tokens x G = 4 */
#define SPD_MQ_MAX_PAGES 32768

/* Page scores of the T token rows of every request in one scan (top-K, bound estimator): each
 * (page, KV head) key box is read once and bounded against the T query groups (LServe summary,
 * "Hierarchical Paging", page importance; LiteTopK, section 3.4, one candidate list per query
 * token).  desc describes the B requests; seq_lens (device, [B]) holds L; q (device, [B, T, Hq, d],
 * the query dtype of desc); page_meta and block_table as for spd_page_score; head_kind (host, [Hkv])
 * as for spd_page_score: streaming heads are not scored.  Writes scores (device,
 * [B * T, Hkv, max_pages_per_seq] f32; row b T + t) for the pages of token t's length
 * L - T + 1 + t, bit for bit what spd_page_score with SPD_TAIL_NONE writes on a descriptor of B * T
 * rows whose block-table rows and page_meta rows repeat each request's T times; later entries are
 * not written.  tail_mode SPD_TAIL_NONE scores every page: the statistics of the pages the draft
 * tokens are in must then be current (spd_page_meta_build over the last pages first).
 * SPD_TAIL_SKIP (needs sel->n_local >= 2, else SPD_ERR_INVALID_ARG) reads no statistics of the
 * request's last two pages and writes -inf for them in every token row that holds them: with at
 * most 4 draft tokens each token's last page is one of the two, so both are in every token's local
 * window or past its length, and the selection takes them without their scores; their statistics
 * may then be rebuilt beside the selection (spd_page_select_mq with page_meta).  Other tail modes
 * return SPD_ERR_INVALID_ARG.  sel must be top-K with the bound estimator (else
 * SPD_ERR_UNSUPPORTED); errors otherwise as spd_page_score and spd_page_list_union. */
int spd_page_score_mq(const spd_desc* desc, int32_t num_tokens, const spd_select_params* sel, const void* q,
                      const void* page_meta, int32_t tail_mode, const int32_t* block_table,
                      const int32_t* seq_lens, const uint8_t* head_kind, float* scores, void* stream);

/* Page lists of the T token rows of every request (top-K, bound estimator): row (b T + t, h) is
 * token t of request b, selected as a single query of length L - T + 1 + t would be (forced sink and
 * local pages of that length, then the best pages by (score desc, page asc) under the budget; LServe,
 * "Token budget and physical page selection"), where L = seq_lens[b] is read on the device, so a
 * captured call follows lengths that change between replays.  desc describes the B requests
 * (block_table [B, max_pages_per_seq] is request b's row for all of its tokens); scores (device,
 * [B * T, Hkv, max_pages_per_seq] f32) as spd_page_score_mq writes them; token_list (device,
 * [B * T, Hkv, token_max_list]) and token_len (device, [B * T, Hkv]) receive the lists, ascending;
 * token_phys (device, same shape as token_list, may be NULL) the physical page of each entry, read
 * from block_table (then required).  head_kind (host): streaming heads get their static table for
 * the token's length.  When page_meta (device, may be NULL) is set, workgroups beside the selection
 * rebuild the key min / max of each request's last two logical pages (the ones the draft tokens are
 * in), every KV head, from k_pool (and k_scale for fp8 pools) into page_meta -- what
 * spd_page_meta_build does with span 2 (LServe, "Key statistics storage and updating"); block_table
 * is then required, and the scores must not depend on those statistics (spd_page_score_mq with
 * SPD_TAIL_SKIP).  Returns SPD_ERR_INVALID_ARG when token_max_list cannot hold the longest list
 * (as spd_page_select's max_list), SPD_ERR_UNSUPPORTED for COVERAGE or MVAR; otherwise errors as
 * spd_page_select. */
int spd_page_select_mq(const spd_desc* desc, int32_t num_tokens, int32_t token_max_list,
                       const spd_select_params* sel, const float* scores, const int32_t* seq_lens,
                       const uint8_t* head_kind, const int32_t* block_table, const void* k_pool,
                       const uint16_t* k_scale, void* page_meta, int32_t* token_list, int32_t* token_phys,
                       int32_t* token_len, void* stream);

/* Union of the T token lists of every (request, KV head) row (LiteDSA's candidate union).
 * desc describes the B requests (max_list: the union's capacity, at least
 * min(T * token_max_list, max_pages_per_seq)).  token_list (device, [B * T, Hkv, token_max_list])
 * and token_len (device, [B * T, Hkv]) are the tokens' lists as spd_page_select writes them; entries
 * outside [0, n_b) of the request are ignored.  Writes page_list (device, [B, Hkv, max_list]) in
 * ascending page order, page_mask (device, same shape, uint32: bit t set when token t listed the
 * page), list_len (device, [B, Hkv]) and, when page_phys (device, may be NULL) is set, the
 * physical page of each entry from block_table.  Two methods give the same union: block tables of
 * at least 16,384 pages whose token lists are ascending and hold at most 1,024 entries in all merge
 * the lists by rank, the others collect them in a byte map over the request's pages; union_path
 * (device, may be NULL, [B, Hkv]) receives 1 for a row merged by rank and 0 for a byte-map row.
 * Errors as elsewhere; num_tokens outside [1, SPD_MQ_MAX_TOKENS] is SPD_ERR_INVALID_ARG. */
int spd_page_list_union(const spd_desc* desc, int32_t num_tokens, int32_t token_max_list,
                        const int32_t* token_list, const int32_t* token_len, const int32_t* block_table,
                        const int32_t* seq_lens, int32_t* page_list, int32_t* page_phys,
                        uint32_t* page_mask, int32_t* list_len, int32_t* union_path, void* stream);

/* Decode attention of the T query tokens of every row over the union list: q (device,
 * [B, T, Hq, d] f16), out (device, [B, T, Hq, d] f32), out_lse (device, [B, T, Hq] f32);
 * k_scale / v_scale (device) are required for fp8 pools and ignored otherwise.  Each
 * union page is read once for all T x G query rows; row (t, g) keeps the page only when bit t of
 * its mask is set, and only positions < L - T + 1 + t.  Split as spd_sparse_paged_decode's per-row
 * plan over the union lengths; rows with more than one chunk write part_o (device,
 * [B, Hkv, J, SPD_MQ_ROWS, d] f32) and part_lse ([B, Hkv, J, SPD_MQ_ROWS] f32) for
 * spd_lse_merge_mq.  A row with an empty union, or a token with no kept key, writes out = 0 and
 * out_lse = -inf.  page_phys may be NULL (then block_table is read). */
int spd_sparse_paged_decode_mq(const spd_desc* desc, int32_t num_tokens, const spd_plan_params* plan,
                               const void* q, const void* k_pool, const void* v_pool,
                               const uint16_t* k_scale, const uint16_t* v_scale,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* page_list, const int32_t* page_phys,
                               const uint32_t* page_mask, const int32_t* list_len, float sm_scale,
                               float* out, float* out_lse, float* part_o, float* part_lse, void* stream);

/* spd_lse_merge for spd_sparse_paged_decode_mq's chunk states (same plan and list_len). */
int spd_lse_merge_mq(const spd_desc* desc, int32_t num_tokens, const spd_plan_params* plan,
                     const float* part_o, const float* part_lse, const int32_t* list_len, float* out,
                     float* out_lse, void* stream);

/* ------------------------------------------------------------------ host helpers */

/* J, the blocks per row of spd_sparse_paged_decode (Moira, Eq. 4); for a balanced plan, the
 * decode grid N_T + B * Hkv. */
int spd_plan_grid(const spd_desc* desc, const spd_plan_params* plan, int32_t* blocks_per_row);

/* Chunk size c and chunk count m of a row with n_pages listed pages under J blocks per
 * row and minimum chunk min_chunk (Moira, Eq. 4 and Algorithm 2); n_pages = 0 gives 0 / 0. */
int spd_plan_chunks(int32_t n_pages, int32_t blocks_per_row, int32_t min_chunk,
                    int32_t* chunk_pages, int32_t* chunks);

/* Element counts of part_o and part_lse for spd_sparse_paged_decode / spd_lse_merge. */
int spd_partials_size(const spd_desc* desc, const spd_plan_params* plan, size_t* part_o_elems,
                      size_t* part_lse_elems);

/* Workspace bytes an op needs (0 when it needs none); (size_t)-1 on invalid arguments or an
 * op that the arguments do not support. */
size_t spd_workspace_bytes(const spd_desc* desc, const spd_select_params* sel, int32_t op);

/* Bytes of a LiteTopK gate state (spd_select_params.topk_state) for `rows` rows: B * Hkv for a
 * single-query step, B * T * Hkv for spd_page_select_mq.  Per row 32 bytes: {float gate, float largest
 * free score of the last selection, uint32 valid, uint32 path of the last selection (1: from the
 * candidates, 0: whole row), uint32 candidates it counted, 3 x uint32 reserved}.  (size_t)-1 for
 * rows < 0. */
size_t spd_topk_state_bytes(int32_t rows);

/* Static description of a status code. */
const char* spd_error_string(int status);

/* SPD_ABI_VERSION of the built library. */
int spd_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPD_H_ */
