// Host side of the C ABI: argument checks, shape / dtype dispatch, grid sizing.  Nothing
// here allocates, synchronises or reads device memory; every entry point only enqueues
// kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/spd.h"
#include "mq_score.h"
#include "score_common.h"
#include "spd_launch.h"

namespace {

// pages per scoring workgroup (fixed by the compiled work layouts)
int meta_bytes_of(const spd_desc* d) { return d->kv_dtype == SPD_DTYPE_F32 ? 4 : 2; }

bool is_mvar(const spd_select_params* s) { return s->estimator == SPD_ESTIMATOR_MVAR; }

// log2 of the 16-token logical pages per physical page (hierarchical paging): 0 for 16-token pages, 2 for 64.
int lgs_of(const spd_desc* d) { return d->page_size == 64 ? 2 : 0; }
bool is_hier(const spd_desc* d) { return lgs_of(d) > 0; }

// Pages per scorer workgroup (the standalone scorer's page groups per lane depend on the scan's size;
// the mvar page summaries are bf16 whatever the pool type).
int score_ppb(const spd_desc* d, const spd_select_params* s, int dyn_heads) {
  const int iters = spd::score_iters((long long)d->batch * dyn_heads * ((long long)d->max_pages_per_seq << lgs_of(d)));
  return spd::score_pages_per_block(d->head_dim, is_mvar(s) ? 2 : meta_bytes_of(d), spd::kScoreWaves, iters);
}

int fused_ppb(const spd_desc* d, const spd::SelectGeometry& g) {
  return spd::score_pages_per_block(d->head_dim, meta_bytes_of(d), g.nw, g.iters);
}

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_dtype(int v) { return v == SPD_DTYPE_F32 || v == SPD_DTYPE_F16 || v == SPD_DTYPE_FP8_E4M3FN; }


int check_desc(const spd_desc* d) {
  if (!d) return SPD_ERR_INVALID_ARG;
  if (d->batch < 0 || d->num_kv_heads < 1 || d->num_kv_heads > SPD_MAX_KV_HEADS || d->num_q_heads < 1 ||
      d->num_q_heads % d->num_kv_heads != 0 || d->head_dim < 1 || d->page_size < 1 ||
      d->max_pages_per_seq < 1 || d->num_pool_pages < 1 || d->max_list < 1)
    return SPD_ERR_INVALID_ARG;
  if (!is_dtype(d->q_dtype) || !is_dtype(d->kv_dtype) || d->q_dtype == SPD_DTYPE_FP8_E4M3FN)
    return SPD_ERR_INVALID_ARG;
  // index arithmetic stays within 64-bit sizes; grids within 2^31 blocks
  if (((int64_t)d->batch * d->num_kv_heads * d->max_pages_per_seq << lgs_of(d)) > ((int64_t)1 << 40)) return SPD_ERR_INVALID_ARG;
  // logical pages and decode work units (4 per list entry) fit in int32
  if (is_hier(d) && (d->max_pages_per_seq > (1 << 28) || d->max_list > (1 << 28))) return SPD_ERR_INVALID_ARG;
  if (d->page_size != SPD_PAGE_SIZE && d->page_size != SPD_HIER_PAGE_SIZE) return SPD_ERR_UNSUPPORTED;
  // hierarchical scoring folds a physical page's logical pages inside one wave instruction: a
  // logical page's key box may span at most 16 lanes of 16 bytes (f32 at d = 128 spans 32)
  if (d->page_size == SPD_HIER_PAGE_SIZE && d->kv_dtype == SPD_DTYPE_F32 && d->head_dim > 64) return SPD_ERR_UNSUPPORTED;
  if (d->num_q_heads / d->num_kv_heads != 4) return SPD_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return SPD_ERR_UNSUPPORTED;
  const bool ok = (d->q_dtype == SPD_DTYPE_F32 && d->kv_dtype == SPD_DTYPE_F32) ||
                  (d->q_dtype == SPD_DTYPE_F16 && d->kv_dtype == SPD_DTYPE_F16) ||
                  (d->q_dtype == SPD_DTYPE_F16 && d->kv_dtype == SPD_DTYPE_FP8_E4M3FN && d->head_dim == 128);
  return ok ? SPD_OK : SPD_ERR_UNSUPPORTED;
}

int check_sel(const spd_desc* d, const spd_select_params* s) {
  if (!s) return SPD_ERR_INVALID_ARG;
  if (s->n_sink < 0 || s->n_local < 0 || s->n_sink_stream < 0 || s->n_local_stream < 0) return SPD_ERR_INVALID_ARG;
  if (s->mode == SPD_SELECT_TOPK) {
    if (s->budget_pages < 1) return SPD_ERR_INVALID_ARG;
  } else if (s->mode == SPD_SELECT_COVERAGE) {
    if (!(s->gamma > 0.f && s->gamma <= 1.f)) return SPD_ERR_INVALID_ARG;
    if (!(s->sm_scale > 0.f) || !std::isfinite(s->sm_scale)) return SPD_ERR_INVALID_ARG;
  } else {
    return SPD_ERR_INVALID_ARG;
  }
  if (s->estimator != SPD_ESTIMATOR_BOUND && s->estimator != SPD_ESTIMATOR_MVAR) return SPD_ERR_INVALID_ARG;
  if (s->estimator == SPD_ESTIMATOR_MVAR && s->mode != SPD_SELECT_COVERAGE) return SPD_ERR_INVALID_ARG;
  // the LiteTopK gate serves the top-K rule with the bound estimator over 16-token pages
  if (s->topk_state && (s->mode != SPD_SELECT_TOPK || s->estimator != SPD_ESTIMATOR_BOUND)) return SPD_ERR_INVALID_ARG;
  if (s->topk_state && d->page_size != SPD_PAGE_SIZE) return SPD_ERR_UNSUPPORTED;
  return SPD_OK;
}

// The LiteTopK gate state of `rows` rows in the caller's buffer (layout in spd.h).
constexpr size_t kGateRowBytes = sizeof(spd::TopkGateRow);
static_assert(kGateRowBytes == 32, "the gate header is 32 bytes");
size_t gate_state_bytes(int64_t rows) { return (size_t)rows * kGateRowBytes; }
spd::TopkGate gate_of(const spd_select_params* s, int64_t) {
  spd::TopkGate g{};
  g.rows = static_cast<spd::TopkGateRow*>(s->topk_state);
  return g;
}

// Tail mode: a known value; a rebuild needs the K pool (and its scales for fp8); skipping the
// last page is only for TOPK with a local window, which always keeps that page.
int check_tail(const spd_desc* d, const spd_select_params* s, int32_t mode, const void* k_pool,
               const uint16_t* k_scale) {
  if (mode != SPD_TAIL_NONE && mode != SPD_TAIL_REBUILD && mode != SPD_TAIL_SKIP) return SPD_ERR_INVALID_ARG;
  if (mode == SPD_TAIL_REBUILD && (!k_pool || (d->kv_dtype == SPD_DTYPE_FP8_E4M3FN && !k_scale)))
    return SPD_ERR_INVALID_ARG;
  if (mode == SPD_TAIL_SKIP && (s->mode != SPD_SELECT_TOPK || s->n_local < 1)) return SPD_ERR_INVALID_ARG;
  if (mode == SPD_TAIL_REBUILD && is_hier(d)) return SPD_ERR_UNSUPPORTED;
  return SPD_OK;
}

// Longest list a row can produce under the rule; max_list must hold it.
int check_list_capacity(const spd_desc* d, const spd_select_params* s) {
  const int64_t stream_len = std::min<int64_t>((int64_t)s->n_sink_stream + s->n_local_stream, d->max_pages_per_seq);
  int64_t dyn_len;
  if (s->mode == SPD_SELECT_TOPK)
    dyn_len = std::min<int64_t>(std::max<int64_t>(s->budget_pages, (int64_t)s->n_sink + s->n_local), d->max_pages_per_seq);
  else
    dyn_len = d->max_pages_per_seq;
  return (d->max_list >= dyn_len && d->max_list >= stream_len) ? SPD_OK : SPD_ERR_INVALID_ARG;
}

int head_lists(const spd_desc* d, const uint8_t* head_kind, spd::HeadList& dyn, spd::HeadList& strm, uint64_t& mask) {
  if (!head_kind) return SPD_ERR_INVALID_ARG;
  dyn.count = strm.count = 0;
  dyn.mask = strm.mask = 0;
  mask = 0;
  for (int h = 0; h < d->num_kv_heads; ++h) {
    if (head_kind[h] == SPD_HEAD_DYNAMIC) { dyn.head[dyn.count++] = (uint8_t)h; dyn.mask |= 1ull << h; }
    else if (head_kind[h] == SPD_HEAD_STREAMING) { strm.head[strm.count++] = (uint8_t)h; mask |= 1ull << h; }
    else return SPD_ERR_INVALID_ARG;
  }
  strm.mask = mask;
  return SPD_OK;
}

// J of the per-row plan (blocks per row), or the grid N_T + rows of the balanced plan.
int plan_j(const spd_desc* d, const spd_plan_params* p, int32_t& J) {
  if (!p || p->min_chunk < 1 || p->min_blocks_per_row < 1 || p->min_grid_blocks < 0) return SPD_ERR_INVALID_ARG;
  if (p->balanced != 0 && p->balanced != 1) return SPD_ERR_INVALID_ARG;
  const int64_t rows = (int64_t)d->batch * d->num_kv_heads;
  if (p->balanced) {
    if (p->min_grid_blocks < 1) return SPD_ERR_INVALID_ARG;
    const int64_t grid = (int64_t)p->min_grid_blocks + rows;
    if (grid > ((int64_t)1 << 31) - 1) return SPD_ERR_INVALID_ARG;
    J = (int32_t)grid;
    return SPD_OK;
  }
  int64_t j = p->min_blocks_per_row;
  if (rows > 0) j = std::max<int64_t>(j, (p->min_grid_blocks + rows - 1) / rows);
  if (j > 1024 || rows * j > ((int64_t)1 << 31) - 1) return SPD_ERR_INVALID_ARG;  // merge holds <= 1024 chunks
  J = (int32_t)j;
  return SPD_OK;
}

int launched(int rc) {
  if (rc != 0) return rc;
  return hipGetLastError() == hipSuccess ? SPD_OK : SPD_ERR_LAUNCH;
}

// Standalone coverage scorer: the per-page log-masses [B, Hkv, max_pages, G] and the per-block
// (max, sum exp) pairs [B, Hkv, ceil(max_pages / 1024), G] between its kernels.
struct ScoreWs {
  size_t ell_off, part_off, total;
};

ScoreWs score_ws(const spd_desc* d) {
  const size_t rows = (size_t)d->batch * d->num_kv_heads;
  const int G = d->num_q_heads / d->num_kv_heads;
  const size_t logical = (size_t)d->max_pages_per_seq << lgs_of(d);  // log-masses per logical page
  const size_t parts = (logical + 1023) / 1024;
  ScoreWs w;
  w.ell_off = 0;
  w.part_off = align_up(rows * logical * G * sizeof(float));
  w.total = w.part_off + align_up(rows * parts * G * 2 * sizeof(float));
  return w;
}

struct FusedWs {
  size_t scores_off, part_off, counters_off, total;
  int ppb;
};

// Fused workspace: top-K scores (or coverage log-masses of the G heads), coverage workgroup
// partials, one ticket counter per row.
bool fused_ws(const spd_desc* d, const spd_select_params* s, FusedWs& w) {
  spd::SelectGeometry g;
  if (!spd::select_geometry(d->max_pages_per_seq, g)) return false;
  const size_t rows = (size_t)d->batch * d->num_kv_heads;
  const int G = d->num_q_heads / d->num_kv_heads;
  const bool cov = s->mode == SPD_SELECT_COVERAGE;
  w.ppb = fused_ppb(d, g);
  const size_t bpr = (d->max_pages_per_seq + w.ppb - 1) / w.ppb;
  w.scores_off = 0;
  w.part_off = align_up(rows * d->max_pages_per_seq * (cov ? G : 1) * sizeof(float));
  w.counters_off = w.part_off + (cov ? align_up(rows * (bpr + 1) * G * 2 * sizeof(float)) : 0);
  w.total = w.counters_off + align_up(rows * sizeof(uint32_t));
  return true;
}

spd::ScoreArgs score_args(const spd_desc* d, const spd_select_params* s, const void* q, const void* meta,
                          const int32_t* bt, const int32_t* sl, const spd::HeadList& dyn, int ppb) {
  spd::ScoreArgs a{};
  a.q = q;
  a.meta = meta;
  a.block_table = bt;
  a.seq_lens = sl;
  a.dyn = dyn;
  a.batch = d->batch;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages = d->max_pages_per_seq;
  a.num_pool_pages = d->num_pool_pages;
  a.pages_per_block = ppb;
  a.lgs = lgs_of(d);
  a.blocks_per_row = (int)((((int64_t)d->max_pages_per_seq << a.lgs) + ppb - 1) / ppb);
  a.partial_stride = a.blocks_per_row + 1;
  a.sm_scale = s->sm_scale;
  return a;
}

spd::SelectArgs select_args(const spd_desc* d, const spd_select_params* s, const int32_t* sl, const int32_t* bt,
                            int32_t* list, int32_t* phys, int32_t* len, float* sel_scores, uint64_t mask) {
  spd::SelectArgs a{};
  a.seq_lens = sl;
  a.block_table = bt;
  a.page_list = list;
  a.page_phys = phys;
  a.list_len = len;
  a.sel_scores = sel_scores;
  a.streaming_mask = mask;
  a.batch = d->batch;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages = d->max_pages_per_seq;
  a.max_list = d->max_list;
  a.mode = s->mode;
  a.budget = s->budget_pages;
  a.gamma_fx = (unsigned long long)std::floor((double)s->gamma * 1099511627776.0);
  a.n_sink = s->n_sink;
  a.n_local = s->n_local;
  a.n_sink_stream = s->n_sink_stream;
  a.n_local_stream = s->n_local_stream;
  a.lgs = lgs_of(d);
  a.num_tokens = 1;
  a.gate = gate_of(s, (int64_t)d->batch * d->num_kv_heads);
  return a;
}

spd::MetaArgs meta_args(const spd_desc* d, const void* k_pool, const uint16_t* k_scale, const int32_t* bt,
                        const int32_t* sl, void* meta) {
  spd::MetaArgs a{};
  a.k_pool = k_pool;
  a.k_scale = k_scale;
  a.block_table = bt;
  a.seq_lens = sl;
  a.meta = meta;
  a.batch = d->batch;
  a.num_kv_heads = d->num_kv_heads;
  a.max_pages = d->max_pages_per_seq;
  a.num_pool_pages = d->num_pool_pages;
  a.head_dim = d->head_dim;
  a.kv_dtype = d->kv_dtype;
  a.lgs = lgs_of(d);
  return a;
}

// spd_page_meta_build and spd_page_stats_build: the pages to build and the launch.
int build_summaries(const spd_desc* desc, const void* k_pool, const uint16_t* k_scale, const int32_t* block_table,
                    const int32_t* seq_lens, const int32_t* first_page, int32_t span_pages, void* out, int stats,
                    void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (desc->batch == 0) return SPD_OK;
  if (!k_pool || !block_table || !seq_lens || !out) return SPD_ERR_INVALID_ARG;
  if (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && !k_scale) return SPD_ERR_INVALID_ARG;
  if ((first_page && span_pages < 1) || span_pages < 0) return SPD_ERR_INVALID_ARG;
  spd::MetaArgs a = meta_args(desc, k_pool, k_scale, block_table, seq_lens, out);
  a.first_page = first_page;
  a.stats = stats;
  // logical pages per request: the span (from first_page, or the last span pages), or every page
  const int max_logical = desc->max_pages_per_seq << lgs_of(desc);
  const int span = (first_page || span_pages > 0) ? std::min(span_pages, max_logical) : max_logical;
  a.span = span;
  a.blocks_per_req = (span * desc->num_kv_heads + 3) / 4;
  return launched(spd::launch_page_meta_build(a, desc->head_dim, desc->kv_dtype, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int spd_abi_version(void) { return SPD_ABI_VERSION; }

size_t spd_topk_state_bytes(int32_t rows) { return rows < 0 ? (size_t)-1 : gate_state_bytes(rows); }

const char* spd_error_string(int status) {
  switch (status) {
    case SPD_OK: return "ok";
    case SPD_ERR_INVALID_ARG: return "invalid argument";
    case SPD_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case SPD_ERR_LAUNCH: return "kernel launch failed";
    case SPD_ERR_WORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int spd_plan_grid(const spd_desc* desc, const spd_plan_params* plan, int32_t* blocks_per_row) {
  int rc = check_desc(desc);
  if (rc == SPD_ERR_INVALID_ARG) return rc;
  if (!blocks_per_row) return SPD_ERR_INVALID_ARG;
  int32_t J;
  rc = plan_j(desc, plan, J);
  if (rc) return rc;
  *blocks_per_row = J;
  return SPD_OK;
}

int spd_plan_chunks(int32_t n_pages, int32_t blocks_per_row, int32_t min_chunk, int32_t* chunk_pages,
                    int32_t* chunks) {
  if (!chunk_pages || !chunks || n_pages < 0 || blocks_per_row < 1 || min_chunk < 1) return SPD_ERR_INVALID_ARG;
  int c, m;
  spd::plan_chunks(n_pages, blocks_per_row, min_chunk, c, m);
  *chunk_pages = c;
  *chunks = m;
  return SPD_OK;
}

int spd_partials_size(const spd_desc* desc, const spd_plan_params* plan, size_t* part_o_elems,
                      size_t* part_lse_elems) {
  int rc = check_desc(desc);
  if (rc == SPD_ERR_INVALID_ARG) return rc;
  if (!part_o_elems || !part_lse_elems) return SPD_ERR_INVALID_ARG;
  int32_t J;
  rc = plan_j(desc, plan, J);
  if (rc) return rc;
  // rows * J * G chunk states, or (balanced) one per chunk of the N_T + rows grid, times G
  const size_t slots = plan->balanced ? (size_t)J * (desc->num_q_heads / desc->num_kv_heads)
                                      : (size_t)desc->batch * desc->num_q_heads * J;
  *part_lse_elems = slots;
  *part_o_elems = slots * desc->head_dim;
  return SPD_OK;
}

size_t spd_workspace_bytes(const spd_desc* desc, const spd_select_params* sel, int32_t op) {
  if (check_desc(desc) == SPD_ERR_INVALID_ARG || check_sel(desc, sel) != SPD_OK) return (size_t)-1;
  switch (op) {
    case SPD_OP_PAGE_SCORE: return sel->mode == SPD_SELECT_COVERAGE ? score_ws(desc).total : 0;
    case SPD_OP_PAGE_SELECT: return 0;
    case SPD_OP_PAGE_SCORE_SELECT: {
      FusedWs w;
      return !is_mvar(sel) && !is_hier(desc) && fused_ws(desc, sel, w) ? w.total : (size_t)-1;
    }
    default: return (size_t)-1;
  }
}

int spd_page_meta_build(const spd_desc* desc, const void* k_pool, const uint16_t* k_scale,
                        const int32_t* block_table, const int32_t* seq_lens, const int32_t* first_page,
                        int32_t span_pages, void* page_meta, void* stream) {
  return build_summaries(desc, k_pool, k_scale, block_table, seq_lens, first_page, span_pages, page_meta, 0, stream);
}

int spd_page_stats_build(const spd_desc* desc, const void* k_pool, const uint16_t* k_scale,
                         const int32_t* block_table, const int32_t* seq_lens, const int32_t* first_page,
                         int32_t span_pages, void* page_stats, void* stream) {
  return build_summaries(desc, k_pool, k_scale, block_table, seq_lens, first_page, span_pages, page_stats, 1,
                         stream);
}

int spd_page_score(const spd_desc* desc, const spd_select_params* sel, const void* q, void* page_meta,
                   const void* k_pool, const uint16_t* k_scale, int32_t tail_mode, const int32_t* block_table,
                   const int32_t* seq_lens, const uint8_t* head_kind, float* scores, float* head_lse,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if ((rc = check_sel(desc, sel))) return rc;
  spd::HeadList dyn, strm;
  uint64_t mask;
  if ((rc = head_lists(desc, head_kind, dyn, strm, mask))) return rc;
  if (desc->batch == 0 || dyn.count == 0) return SPD_OK;
  if (!q || !page_meta || !block_table || !seq_lens || !scores) return SPD_ERR_INVALID_ARG;
  if ((rc = check_tail(desc, sel, tail_mode, k_pool, k_scale))) return rc;
  // the mvar estimator computes the first and current pages exactly, from the K pool
  if (is_mvar(sel) && (!k_pool || (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && !k_scale))) return SPD_ERR_INVALID_ARG;
  spd::ScoreArgs a = score_args(desc, sel, q, page_meta, block_table, seq_lens, dyn, score_ppb(desc, sel, dyn.count));
  a.scores = scores;
  a.meta_out = page_meta;
  a.k_pool = k_pool;
  a.k_scale = k_scale;
  a.tail_mode = tail_mode;
  const bool coverage = sel->mode == SPD_SELECT_COVERAGE;
  if (coverage) {
    if (!head_lse) return SPD_ERR_INVALID_ARG;
    const ScoreWs w = score_ws(desc);
    if (!workspace || workspace_bytes < w.total) return SPD_ERR_WORKSPACE;
    a.ell = reinterpret_cast<float4*>(static_cast<char*>(workspace) + w.ell_off);
    a.partials = reinterpret_cast<float2*>(static_cast<char*>(workspace) + w.part_off);
    a.head_lse = head_lse;
  }
  if (is_mvar(sel)) return launched(spd::launch_page_score_mvar(a, desc->head_dim, desc->kv_dtype, (hipStream_t)stream));
  return launched(spd::launch_page_score(a, desc->head_dim, desc->kv_dtype, coverage, (hipStream_t)stream));
}

int spd_page_select(const spd_desc* desc, const spd_select_params* sel, const float* scores,
                    const int32_t* seq_lens, const uint8_t* head_kind, const int32_t* block_table,
                    const void* k_pool, const uint16_t* k_scale, void* page_meta, int32_t* page_list,
                    int32_t* page_phys, int32_t* list_len, float* sel_scores, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if ((rc = check_sel(desc, sel))) return rc;
  if ((rc = check_list_capacity(desc, sel))) return rc;
  spd::SelectGeometry g;
  if (!spd::select_geometry(desc->max_pages_per_seq, g)) return SPD_ERR_UNSUPPORTED;
  spd::HeadList dyn, strm;
  uint64_t mask;
  if ((rc = head_lists(desc, head_kind, dyn, strm, mask))) return rc;
  if (desc->batch == 0) return SPD_OK;
  if (!seq_lens || !page_list || !list_len || (dyn.count > 0 && !scores)) return SPD_ERR_INVALID_ARG;
  if (page_phys && !block_table) return SPD_ERR_INVALID_ARG;
  if (page_meta && (!block_table || !k_pool || (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && !k_scale)))
    return SPD_ERR_INVALID_ARG;
  spd::SelectArgs a = select_args(desc, sel, seq_lens, block_table, page_list, page_phys, list_len, sel_scores, mask);
  a.scores = scores;
  if (page_meta && !is_mvar(sel)) a.tail = meta_args(desc, k_pool, k_scale, block_table, seq_lens, page_meta);
  if ((rc = launched(spd::launch_page_select(a, (hipStream_t)stream)))) return rc;
  // page summaries (mvar): a launch of their own, which keeps the selector's registers unchanged
  if (page_meta && is_mvar(sel))
    return build_summaries(desc, k_pool, k_scale, block_table, seq_lens, nullptr, 1, page_meta, 1, stream);
  return SPD_OK;
}

int spd_page_list_refresh(const spd_desc* desc, const spd_select_params* sel, const int32_t* seq_lens,
                          const uint8_t* head_kind, const int32_t* block_table, const void* k_pool,
                          const uint16_t* k_scale, void* page_meta, int32_t* page_list, int32_t* page_phys,
                          int32_t* list_len, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if ((rc = check_sel(desc, sel))) return rc;
  if ((rc = check_list_capacity(desc, sel))) return rc;
  spd::HeadList dyn, strm;
  uint64_t mask;
  if ((rc = head_lists(desc, head_kind, dyn, strm, mask))) return rc;
  if (desc->batch == 0) return SPD_OK;
  if (!seq_lens || !page_list || !list_len || !block_table) return SPD_ERR_INVALID_ARG;
  if (page_meta && (!k_pool || (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && !k_scale))) return SPD_ERR_INVALID_ARG;
  spd::SelectArgs a = select_args(desc, sel, seq_lens, block_table, page_list, page_phys, list_len, nullptr, mask);
  a.gate = spd::TopkGate{};  // the refresh selects nothing
  if (page_meta && !is_mvar(sel)) a.tail = meta_args(desc, k_pool, k_scale, block_table, seq_lens, page_meta);
  if ((rc = launched(spd::launch_page_list_refresh(a, (hipStream_t)stream)))) return rc;
  if (page_meta && is_mvar(sel))
    return build_summaries(desc, k_pool, k_scale, block_table, seq_lens, nullptr, 1, page_meta, 1, stream);
  return SPD_OK;
}

int spd_page_score_select(const spd_desc* desc, const spd_select_params* sel, const void* q, void* page_meta,
                          const void* k_pool, const uint16_t* k_scale, int32_t tail_mode,
                          const int32_t* block_table, const int32_t* seq_lens, const uint8_t* head_kind,
                          int32_t* page_list, int32_t* page_phys, int32_t* list_len, float* sel_scores, float* scores,
                          float* head_lse, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if ((rc = check_sel(desc, sel))) return rc;
  if ((rc = check_list_capacity(desc, sel))) return rc;
  FusedWs w;
  if (is_mvar(sel) || is_hier(desc) || !fused_ws(desc, sel, w) || sel->topk_state) return SPD_ERR_UNSUPPORTED;
  spd::HeadList dyn, strm;
  uint64_t mask;
  if ((rc = head_lists(desc, head_kind, dyn, strm, mask))) return rc;
  if (desc->batch == 0) return SPD_OK;
  if (!seq_lens || !page_list || !list_len || !block_table) return SPD_ERR_INVALID_ARG;
  if (dyn.count > 0 && (!q || !page_meta)) return SPD_ERR_INVALID_ARG;
  if ((rc = check_tail(desc, sel, tail_mode, k_pool, k_scale))) return rc;
  if (!workspace || workspace_bytes < w.total) return SPD_ERR_WORKSPACE;
  const bool cov = sel->mode == SPD_SELECT_COVERAGE;
  char* ws = static_cast<char*>(workspace);
  spd::FusedArgs f{};
  f.score = score_args(desc, sel, q, page_meta, block_table, seq_lens, dyn, w.ppb);
  f.score.meta_out = page_meta;
  f.score.k_pool = k_pool;
  f.score.k_scale = k_scale;
  f.score.tail_mode = tail_mode;
  if (cov) {
    f.score.ell = reinterpret_cast<float4*>(ws + w.scores_off);
    f.score.partials = reinterpret_cast<float2*>(ws + w.part_off);
    f.score.head_lse = head_lse;
    f.score_out = scores;
  } else {
    f.score.scores = scores ? scores : reinterpret_cast<float*>(ws + w.scores_off);
  }
  f.sel = select_args(desc, sel, seq_lens, block_table, page_list, page_phys, list_len, sel_scores, mask);
  f.stream_heads = strm;
  f.counters = reinterpret_cast<unsigned int*>(ws + w.counters_off);
  return launched(spd::launch_page_score_select(f, desc->head_dim, desc->kv_dtype, (hipStream_t)stream));
}

static int decode_impl(const spd_desc* desc, const spd_plan_params* plan, const void* q, const void* k_pool,
                       const void* v_pool, const uint16_t* k_scale, const uint16_t* v_scale,
                       const int32_t* block_table, const int32_t* seq_lens, const int32_t* page_list,
                       const int32_t* page_phys, const int32_t* list_len, float sm_scale, float* out,
                       float* out_lse, float* part_o, float* part_lse, uint32_t* counters, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  int32_t J;
  if ((rc = plan_j(desc, plan, J))) return rc;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return SPD_ERR_INVALID_ARG;
  if (desc->batch == 0) return SPD_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !page_list || !list_len || !out || !out_lse ||
      !part_o || !part_lse)
    return SPD_ERR_INVALID_ARG;
  if (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && (!k_scale || !v_scale)) return SPD_ERR_INVALID_ARG;
  spd::DecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.page_list = page_list;
  a.page_phys = page_phys;
  a.list_len = list_len;
  a.out = out;
  a.out_lse = out_lse;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_pages = desc->max_pages_per_seq;
  a.num_pool_pages = desc->num_pool_pages;
  a.max_list = desc->max_list;
  a.blocks_per_row = J;
  a.min_chunk = plan->min_chunk;
  {  // the chunk the decode guesses its list reads from: the plan's for a full list
    int sc = 0, sm = 0;
    spd::plan_chunks(desc->max_list << lgs_of(desc), J, plan->min_chunk, sc, sm);
    a.spec_chunk = sc;
  }
  a.balanced = plan->balanced;
  a.grid_target = plan->min_grid_blocks;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  a.lgs = lgs_of(desc);
  a.counters = counters;
  return launched(spd::launch_sparse_paged_decode(a, desc->head_dim, desc->q_dtype, desc->kv_dtype,
                                                  (hipStream_t)stream));
}

int spd_sparse_paged_decode(const spd_desc* desc, const spd_plan_params* plan, const void* q, const void* k_pool,
                            const void* v_pool, const uint16_t* k_scale, const uint16_t* v_scale,
                            const int32_t* block_table, const int32_t* seq_lens, const int32_t* page_list,
                            const int32_t* page_phys, const int32_t* list_len, float sm_scale, float* out,
                            float* out_lse, float* part_o, float* part_lse, void* stream) {
  return decode_impl(desc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, page_list, page_phys,
                     list_len, sm_scale, out, out_lse, part_o, part_lse, nullptr, stream);
}

int spd_sparse_paged_decode_merged(const spd_desc* desc, const spd_plan_params* plan, const void* q,
                                   const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                                   const uint16_t* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* page_list, const int32_t* page_phys, const int32_t* list_len,
                                   float sm_scale, float* out, float* out_lse, float* part_o, float* part_lse,
                                   uint32_t* counters, void* stream) {
  if (!counters && desc && desc->batch > 0) return SPD_ERR_INVALID_ARG;
  return decode_impl(desc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, page_list, page_phys,
                     list_len, sm_scale, out, out_lse, part_o, part_lse, counters, stream);
}

int spd_lse_merge(const spd_desc* desc, const spd_plan_params* plan, const float* part_o, const float* part_lse,
                  const int32_t* list_len, float* out, float* out_lse, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  int32_t J;
  if ((rc = plan_j(desc, plan, J))) return rc;
  if (desc->batch == 0) return SPD_OK;
  if (!part_o || !part_lse || !list_len || !out || !out_lse) return SPD_ERR_INVALID_ARG;
  spd::MergeArgs a{};
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.list_len = list_len;
  a.out = out;
  a.out_lse = out_lse;
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_list = desc->max_list;
  a.blocks_per_row = J;
  a.min_chunk = plan->min_chunk;
  a.balanced = plan->balanced;
  a.grid_target = plan->min_grid_blocks;
  a.lgs = lgs_of(desc);
  a.rows_per_head = desc->num_q_heads / desc->num_kv_heads;
  a.num_tokens = 1;
  return launched(spd::launch_lse_merge(a, desc->head_dim, (hipStream_t)stream));
}

// ------------------------------------------------------------------ decode without allocation

// Chunk partials of spd_sparse_paged_decode_noalloc: a file-scope array in device memory, one copy per
// GPU, held until the process ends.  In host code `scratch` only names the symbol; kernels get the
// device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[SPD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
static std::atomic<void*> g_scratch_addr[kMaxDevices];  // per device, resolved on its first call

// The current device's address of `scratch` (looked up once per device, with that device current).
static int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPD_ERR_LAUNCH;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPD_ERR_LAUNCH;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return SPD_OK;
}

int spd_sparse_paged_decode_noalloc(const spd_desc* desc, const spd_plan_params* plan, const void* q,
                                    const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                                    const uint16_t* v_scale, const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* page_list, const int32_t* page_phys, const int32_t* list_len,
                                    float sm_scale, float* out, float* out_lse, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  size_t n_po, n_pl;
  if ((rc = spd_partials_size(desc, plan, &n_po, &n_pl))) return rc;
  const size_t lse_off = align_up(n_po * sizeof(float));
  if (lse_off + n_pl * sizeof(float) > (size_t)SPD_NOALLOC_SCRATCH_BYTES) return SPD_ERR_WORKSPACE;
  if (desc->batch == 0) return SPD_OK;
  void* base = nullptr;
  if ((rc = scratch_address(&base))) return rc;
  float* part_o = static_cast<float*>(base);
  float* part_lse = reinterpret_cast<float*>(static_cast<char*>(base) + lse_off);
  if ((rc = decode_impl(desc, plan, q, k_pool, v_pool, k_scale, v_scale, block_table, seq_lens, page_list,
                        page_phys, list_len, sm_scale, out, out_lse, part_o, part_lse, nullptr, stream)))
    return rc;
  return spd_lse_merge(desc, plan, part_o, part_lse, list_len, out, out_lse, stream);
}

// ------------------------------------------------------------------ several query tokens per request

static int check_mq(const spd_desc* d, int32_t num_tokens) {
  int rc = check_desc(d);
  if (rc) return rc;
  if (num_tokens < 1 || num_tokens > SPD_MQ_MAX_TOKENS) return SPD_ERR_INVALID_ARG;
  if (is_hier(d) || d->max_pages_per_seq > SPD_MQ_MAX_PAGES) return SPD_ERR_UNSUPPORTED;
  return SPD_OK;
}

int spd_page_score_mq(const spd_desc* desc, int32_t num_tokens, const spd_select_params* sel, const void* q,
                      const void* page_meta, int32_t tail_mode, const int32_t* block_table, const int32_t* seq_lens,
                      const uint8_t* head_kind, float* scores, void* stream) {
  int rc = check_mq(desc, num_tokens);
  if (rc) return rc;
  if ((rc = check_sel(desc, sel))) return rc;
  if (sel->mode != SPD_SELECT_TOPK || is_mvar(sel)) return SPD_ERR_UNSUPPORTED;
  // skipping the last two pages needs them forced for every token: a local window of two pages
  if (tail_mode != SPD_TAIL_NONE && (tail_mode != SPD_TAIL_SKIP || sel->n_local < 2)) return SPD_ERR_INVALID_ARG;
  spd::HeadList dyn, strm;
  uint64_t mask;
  if ((rc = head_lists(desc, head_kind, dyn, strm, mask))) return rc;
  if (desc->batch == 0 || dyn.count == 0) return SPD_OK;
  if (!q || !page_meta || !block_table || !seq_lens || !scores) return SPD_ERR_INVALID_ARG;
  spd::ScoreArgs a = score_args(desc, sel, q, page_meta, block_table, seq_lens, dyn, score_ppb(desc, sel, dyn.count));
  a.scores = scores;
  a.tail_mode = tail_mode;
  return launched(spd::launch_mq_page_score(a, num_tokens, desc->head_dim, desc->kv_dtype, (hipStream_t)stream));
}

int spd_page_select_mq(const spd_desc* desc, int32_t num_tokens, int32_t token_max_list,
                       const spd_select_params* sel, const float* scores, const int32_t* seq_lens,
                       const uint8_t* head_kind, const int32_t* block_table, const void* k_pool,
                       const uint16_t* k_scale, void* page_meta, int32_t* token_list, int32_t* token_phys,
                       int32_t* token_len, void* stream) {
  int rc = check_mq(desc, num_tokens);
  if (rc) return rc;
  if (token_max_list < 1) return SPD_ERR_INVALID_ARG;
  if ((rc = check_sel(desc, sel))) return rc;
  if (sel->mode != SPD_SELECT_TOPK || is_mvar(sel)) return SPD_ERR_UNSUPPORTED;
  // the token lists' capacity must hold the longest list the rule can produce
  spd_desc tok = *desc;
  tok.max_list = token_max_list;
  if ((rc = check_list_capacity(&tok, sel))) return rc;
  spd::SelectGeometry g;
  if (!spd::select_geometry(desc->max_pages_per_seq, g)) return SPD_ERR_UNSUPPORTED;
  spd::HeadList dyn, strm;
  uint64_t mask;
  if ((rc = head_lists(desc, head_kind, dyn, strm, mask))) return rc;
  if (desc->batch == 0) return SPD_OK;
  if (!seq_lens || !token_list || !token_len || (dyn.count > 0 && !scores)) return SPD_ERR_INVALID_ARG;
  if (token_phys && !block_table) return SPD_ERR_INVALID_ARG;
  if (page_meta && (!block_table || !k_pool || (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && !k_scale)))
    return SPD_ERR_INVALID_ARG;
  spd::SelectArgs a = select_args(&tok, sel, seq_lens, block_table, token_list, token_phys, token_len, nullptr, mask);
  a.scores = scores;
  a.num_tokens = num_tokens;
  if (page_meta) {  // the last two pages of every request, all KV heads, beside the selection
    a.tail = meta_args(desc, k_pool, k_scale, block_table, seq_lens, page_meta);
    a.tail.span = 2;
  }
  a.gate = gate_of(sel, (int64_t)desc->batch * num_tokens * desc->num_kv_heads);  // rows of the token rows
  return launched(spd::launch_page_select(a, (hipStream_t)stream));
}

int spd_page_list_union(const spd_desc* desc, int32_t num_tokens, int32_t token_max_list, const int32_t* token_list,
                        const int32_t* token_len, const int32_t* block_table, const int32_t* seq_lens,
                        int32_t* page_list, int32_t* page_phys, uint32_t* page_mask, int32_t* list_len,
                        int32_t* union_path, void* stream) {
  int rc = check_mq(desc, num_tokens);
  if (rc) return rc;
  if (token_max_list < 1) return SPD_ERR_INVALID_ARG;
  // the union of T lists of at most token_max_list pages each, within the request's pages
  if ((int64_t)desc->max_list < std::min<int64_t>((int64_t)num_tokens * token_max_list, desc->max_pages_per_seq))
    return SPD_ERR_INVALID_ARG;
  if (desc->batch == 0) return SPD_OK;
  if (!token_list || !token_len || !seq_lens || !page_list || !page_mask || !list_len) return SPD_ERR_INVALID_ARG;
  if (page_phys && !block_table) return SPD_ERR_INVALID_ARG;
  spd::UnionArgs a{};
  a.token_list = token_list;
  a.token_len = token_len;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.page_list = page_list;
  a.page_phys = page_phys;
  a.page_mask = page_mask;
  a.list_len = list_len;
  a.path = union_path;
  a.batch = desc->batch;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_pages = desc->max_pages_per_seq;
  a.max_list = desc->max_list;
  a.num_tokens = num_tokens;
  a.token_max_list = token_max_list;
  return launched(spd::launch_page_list_union(a, (hipStream_t)stream));
}

int spd_sparse_paged_decode_mq(const spd_desc* desc, int32_t num_tokens, const spd_plan_params* plan, const void* q,
                               const void* k_pool, const void* v_pool, const uint16_t* k_scale,
                               const uint16_t* v_scale, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* page_list, const int32_t* page_phys,
                               const uint32_t* page_mask, const int32_t* list_len, float sm_scale, float* out,
                               float* out_lse, float* part_o, float* part_lse, void* stream) {
  int rc = check_mq(desc, num_tokens);
  if (rc) return rc;
  int32_t J;
  if ((rc = plan_j(desc, plan, J))) return rc;
  if (plan->balanced) return SPD_ERR_UNSUPPORTED;
  if (desc->q_dtype != SPD_DTYPE_F16 || desc->head_dim != 128) return SPD_ERR_UNSUPPORTED;
  if (!(sm_scale > 0.f) || !std::isfinite(sm_scale)) return SPD_ERR_INVALID_ARG;
  if (desc->batch == 0) return SPD_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !page_list || !page_mask || !list_len || !out ||
      !out_lse || !part_o || !part_lse)
    return SPD_ERR_INVALID_ARG;
  if (desc->kv_dtype == SPD_DTYPE_FP8_E4M3FN && (!k_scale || !v_scale)) return SPD_ERR_INVALID_ARG;
  spd::MqDecodeArgs a{};
  a.q = q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.page_list = page_list;
  a.page_phys = page_phys;
  a.page_mask = page_mask;
  a.list_len = list_len;
  a.out = out;
  a.out_lse = out_lse;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_pages = desc->max_pages_per_seq;
  a.num_pool_pages = desc->num_pool_pages;
  a.max_list = desc->max_list;
  a.num_tokens = num_tokens;
  a.blocks_per_row = J;
  a.min_chunk = plan->min_chunk;
  a.sm_scale_log2 = sm_scale * 1.4426950408889634f;
  return launched(spd::launch_mq_decode(a, desc->head_dim, desc->kv_dtype, (hipStream_t)stream));
}

int spd_lse_merge_mq(const spd_desc* desc, int32_t num_tokens, const spd_plan_params* plan, const float* part_o,
                     const float* part_lse, const int32_t* list_len, float* out, float* out_lse, void* stream) {
  int rc = check_mq(desc, num_tokens);
  if (rc) return rc;
  int32_t J;
  if ((rc = plan_j(desc, plan, J))) return rc;
  if (plan->balanced) return SPD_ERR_UNSUPPORTED;
  if (desc->head_dim != 128) return SPD_ERR_UNSUPPORTED;
  if (desc->batch == 0) return SPD_OK;
  if (!part_o || !part_lse || !list_len || !out || !out_lse) return SPD_ERR_INVALID_ARG;
  spd::MergeArgs a{};
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.list_len = list_len;
  a.out = out;
  a.out_lse = out_lse;
  a.batch = desc->batch;
  a.num_q_heads = desc->num_q_heads;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_list = desc->max_list;
  a.blocks_per_row = J;
  a.min_chunk = plan->min_chunk;
  a.rows_per_head = SPD_MQ_ROWS;
  a.num_tokens = num_tokens;
  return launched(spd::launch_lse_merge(a, desc->head_dim, (hipStream_t)stream));
}

}  // extern "C"
