// Kernel argument blocks and launchers (internal to the library; the public surface is
// include/spd.h).  Launchers return 0 or SPD_ERR_UNSUPPORTED and only enqueue work.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spd.h"

namespace spd {

// Scoring workgroups: NW waves, each with ITERS groups of pages (score_common.h).
constexpr int kScoreWaves = 4;  // standalone scorer
// Page groups per lane of the standalone scorer: 2 for short scans, 4 once the step scans at least
// kScoreLongItems (page, dynamic head) pairs -- more meta bytes in flight per lane pays off only
// when the scan is long enough to be bandwidth- rather than latency-bound.
constexpr int kScoreItersShort = 2, kScoreItersLong = 4;
constexpr long long kScoreLongItems = 65536;
inline int score_iters(long long items) { return items >= kScoreLongItems ? kScoreItersLong : kScoreItersShort; }

// Selection workgroup shape for rows of up to max_pages pages (select_row.h): NW waves with
// KPL key slots per lane; the fused score + select kernel scores with the same workgroup and
// `iters` page groups per lane.  Returns false when rows are too long to select.
struct SelectGeometry {
  int nw, kpl, iters;
};
inline bool select_geometry(int max_pages, SelectGeometry& g) {
  // 16 waves: a row's selection is a chain of short dependent steps per key slot, so four waves
  // per SIMD hide each other's latencies; the scoring part covers 128 pages per workgroup (f16 d128)
  if (max_pages <= 16 * 64 * 2) g = {16, 2, 2};
  else if (max_pages <= 16 * 64 * 8) g = {16, 8, 2};
  else if (max_pages <= 16 * 64 * 32) g = {16, 32, 2};
  else if (max_pages <= 16 * 64 * 64) g = {16, 64, 4};
  else return false;
  return true;
}

struct MetaArgs {
  const void* k_pool;
  const uint16_t* k_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* first_page;
  void* meta;
  int batch, num_kv_heads, max_pages, num_pool_pages;
  int span;            // pages after first_page (when first_page is set)
  int blocks_per_req;  // workgroups per request (4 (page, head) items each)
  int head_dim, kv_dtype;
  int stats;           // 0: key min / max (page meta); 1: key mean / variance, bf16 (page summaries)
  int lgs;             // log2 of logical pages per physical page (hierarchical paging; 0: 16-token pages)
};
int launch_page_meta_build(const MetaArgs& a, int head_dim, int kv_dtype, hipStream_t stream);

// KV heads of one kind, listed in ascending order (dynamic heads for the scorer).
struct HeadList {
  uint8_t head[SPD_MAX_KV_HEADS];  // ascending
  int count;
  uint64_t mask;  // bit h set for every listed head
  // head[k] from the mask alone (k-th set bit): a kernel finds its head with bit operations instead of
  // a dependent read of the argument block before its first loads
  __device__ __forceinline__ int at(int k) const {
    uint64_t m = mask;
    for (int i = 0; i < k; ++i) m &= m - 1;
    return __builtin_ctzll(m);
  }
};

// LiteTopK gate state of top-K rows (LiteTopK, section 3.2 "Sampling" and "Top-k Selection", section 3.3
// "Predictive Gating"): per (token row, KV head) a gate predicted from the row's previous selection.  The
// selector ranks only the free pages scoring at or above it when they hold the top K'.
struct TopkGateRow {
  float lo;        // gate: free pages scoring >= lo are candidates
  float top;       // largest free score of the previous selection (range of the sample)
  uint32_t valid;  // nonzero once a selection has predicted a gate
  uint32_t path;   // how the last selection ran: 1 from the candidates, 0 over the whole row
  uint32_t seen;   // candidates (free pages at or above the gate) the last selection counted
  uint32_t pad[3];
};
constexpr int kGateCap = 2048;  // candidates the selector ranks; more send it to the whole row
struct TopkGate {
  TopkGateRow* rows;  // [B * T * Hkv]; null: no gate
};

struct ScoreArgs {
  const void* q;
  const void* meta;
  void* meta_out;            // tail refresh target (the same buffer as meta)
  const void* k_pool;        // tail refresh source
  const uint16_t* k_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  float* scores;             // top-K: [B, Hkv, max_pages]; coverage: shares (nullable when fused)
  float4* ell;               // coverage: [B, Hkv, max_pages] log-masses of the G heads
  float2* partials;          // coverage: [B, Hkv, partial_stride, G] (max, sum of exp)
  float* head_lse;           // coverage: [B, Hq] (nullable when fused)
  HeadList dyn;
  int batch, num_q_heads, num_kv_heads, max_pages, num_pool_pages;
  int blocks_per_row;        // page-scanning workgroups per (request, dynamic head)
  int partial_stride;        // partial slots per row: blocks_per_row + 1 (the tail workgroup's)
  int pages_per_block;
  float sm_scale;
  int tail_mode;             // spd_tail_mode: last page of each dynamic row scored / rebuilt / skipped
  int lgs;                   // log2 of logical pages per physical page; > 0: scores are per physical page
};
int launch_page_score(const ScoreArgs& a, int head_dim, int kv_dtype, bool coverage, hipStream_t stream);
// Coverage shares from the log-masses in a.ell (the scorers' second and third kernels).
void launch_coverage_shares(const ScoreArgs& a, hipStream_t stream);
// Coverage log-masses from the Moira page summaries (mvar), then the shares.
int launch_page_score_mvar(const ScoreArgs& a, int head_dim, int kv_dtype, hipStream_t stream);

struct SelectArgs {
  const float* scores;      // [B, Hkv, max_pages] (top-K scores or coverage shares)
  const int32_t* seq_lens;
  const int32_t* block_table;  // read when page_phys is set
  int32_t* page_list;       // [B, Hkv, max_list]
  int32_t* page_phys;       // [B, Hkv, max_list] physical pages of the list (nullable)
  int32_t* list_len;        // [B, Hkv]
  float* sel_scores;        // nullable
  uint64_t streaming_mask;  // bit h set: KV head h is a streaming head
  int batch, num_kv_heads, max_pages, max_list;
  int mode, budget;
  unsigned long long gamma_fx;  // gamma in 2^-40 fixed point
  int n_sink, n_local, n_sink_stream, n_local_stream;
  int lgs;                  // log2 of logical pages per physical page: rows, lists and budget count physical pages
  int num_tokens;           // query tokens per request (>= 1): rows are (b T + t, h); token t of request b sees
                            // seq_lens[b] - T + 1 + t keys and request b's block-table row
  TopkGate gate;            // top-K: select from the scorer's gated candidates when they hold the top K'
                            // pages, then predict the next gate (rows.null: no gate)
  MetaArgs tail;            // tail.meta set: also rebuild each request's last logical page, all KV heads
};
int launch_page_select(const SelectArgs& a, hipStream_t stream);
int launch_page_list_refresh(const SelectArgs& a, hipStream_t stream);

struct FusedArgs {
  ScoreArgs score;         // score.scores / score.ell / score.partials -> workspace
  SelectArgs sel;          // sel.scores unused; shares are written to score_out when set
  float* score_out;        // optional copy of the row scores (top-K) or shares (coverage) [B, Hkv, max_pages]
  HeadList stream_heads;   // streaming heads: one extra block per (request, head)
  unsigned int* counters;  // [B, Hkv] finished-block tickets (workspace, zero between calls)
};
int launch_page_score_select(const FusedArgs& a, int head_dim, int kv_dtype, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const uint16_t* k_scale;
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* page_list;
  const int32_t* page_phys;  // nullable: physical pages of the lists (block_table is then not read)
  const int32_t* list_len;
  float* out;
  float* out_lse;
  float* part_o;
  float* part_lse;
  int batch, num_q_heads, num_kv_heads, max_pages, num_pool_pages, max_list;
  int blocks_per_row, min_chunk;
  int spec_chunk;  // per-row plan: the chunk of a full list (max_list entries), where the list reads are guessed
  int balanced, grid_target;  // step-wide split over grid_target (N_T) + rows blocks
  float sm_scale_log2;  // softmax scale times log2(e)
  int lgs;              // log2 of logical pages per physical page: each list entry is 2^lgs work units
  unsigned int* counters;  // [B, Hkv] row tickets (zero between calls): set = merge in the same launch
};
int launch_sparse_paged_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype,
                               hipStream_t stream);

struct MergeArgs {
  const float* part_o;
  const float* part_lse;
  const int32_t* list_len;
  float* out;
  float* out_lse;
  int batch, num_q_heads, num_kv_heads, max_list, blocks_per_row, min_chunk;
  int balanced, grid_target;
  int lgs;  // as in DecodeArgs
  int rows_per_head;  // chunk-state rows per (request, KV head): G, or 16 for several query tokens
  int num_tokens;     // query tokens per request (outputs [B, T, Hq, d]); rows r >= T * G are not merged
};
int launch_lse_merge(const MergeArgs& a, int head_dim, hipStream_t stream);

// Several query tokens per request (mq_decode.hip).
struct UnionArgs {
  const int32_t* token_list;  // [B * T, Hkv, token_max_list]
  const int32_t* token_len;   // [B * T, Hkv]
  const int32_t* block_table;
  const int32_t* seq_lens;    // [B] keys in each request's cache
  int32_t* page_list;         // [B, Hkv, max_list]
  int32_t* page_phys;         // nullable
  uint32_t* page_mask;        // [B, Hkv, max_list]
  int32_t* list_len;          // [B, Hkv]
  int32_t* path;              // nullable [B, Hkv]: 1 where the rank merge built the row's union, 0 the byte map
  int batch, num_kv_heads, max_pages, max_list, num_tokens, token_max_list;
};
int launch_page_list_union(const UnionArgs& a, hipStream_t stream);

struct MqDecodeArgs {
  const void* q;              // [B, T, Hq, d]
  const void* k_pool;
  const void* v_pool;
  const uint16_t* k_scale;    // fp8 pools
  const uint16_t* v_scale;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* page_list;
  const int32_t* page_phys;   // nullable
  const uint32_t* page_mask;
  const int32_t* list_len;
  float* out;                 // [B, T, Hq, d]
  float* out_lse;             // [B, T, Hq]
  float* part_o;              // [B, Hkv, J, 16, d]
  float* part_lse;            // [B, Hkv, J, 16]
  int batch, num_q_heads, num_kv_heads, max_pages, num_pool_pages, max_list, num_tokens;
  int blocks_per_row, min_chunk;
  float sm_scale_log2;
};
int launch_mq_decode(const MqDecodeArgs& a, int head_dim, int kv_dtype, hipStream_t stream);

// Moira Eq. 4: chunk size and count of a row of n listed pages.
__host__ __device__ inline void plan_chunks(int n, int J, int C, int& c, int& m) {
  if (n <= 0) { c = 0; m = 0; return; }
  int per = (n + J - 1) / J;
  c = per > C ? per : C;
  m = (n + c - 1) / c;
}

}  // namespace spd
