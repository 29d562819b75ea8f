// Page lists from page scores: one workgroup per (request, KV head) row.  The selection rules
// and their sources are described in select_row.h.  With hierarchical paging the rows, scores,
// forced pages, budget and lists are physical pages, and the rebuilt statistics those of the
// newest token's 16-token logical page.  Optionally, workgroups after the rows
// rebuild the key statistics of each request's last page, one wave per KV head (LServe, "Key
// statistics storage and updating"), beside the selection: where the scorer skipped that page
// (the local window keeps it), the rebuild leaves the critical path of the step.
#include "meta_build.h"
#include "select_row.h"

namespace spd {

// Keys (and physical pages, when the list of physical pages is wanted) of the row's pages in
// the slot layout of select_row_keys.  `sc` holds top-K scores or coverage shares.  The row's length
// (len_src[0] - len_off, at least 0), its scores over the whole row stride (max_pages: they need no
// length) and its LiteTopK gate (gate_src, nullable) are requested together and waited for once; then
// slots at or past the row's n pages are cleared (coverage), or every slot that is not a free page
// (top-K: the sinks of n_sink and the window of n_local are taken without their keys).  A row with a
// valid gate leaves the physical pages of its slots to the selection (phys_later): the gated cut
// requests only its candidates'.
template <int NW, int KPL, bool COV>
__device__ __forceinline__ void load_row_keys(const float* sc, const int32_t* len_src, int len_off, int max_pages,
                                              int lgs, int n_sink, int n_local, const TopkGateRow* gate_src,
                                              TopkGateRow& gr, uint32_t (&key)[KPL], SlotPhys<KPL>& phys, int& n,
                                              bool& phys_later) {
  const int wbase = (int)(threadIdx.x / kWave) * kWave * KPL + (int)(threadIdx.x % kWave);
  const int raw_len = *len_src;
  // the gate's threshold and validity, read without a branch (no gate: both read 0)
  const __amdgpu_buffer_rsrc_t gate_r = make_rsrc(gate_src, gate_src ? (uint32_t)sizeof(TopkGateRow) : 0u);
  gr.lo = buf_load_f32(gate_r, (uint32_t)offsetof(TopkGateRow, lo));
  gr.valid = (uint32_t)buf_load_i32(gate_r, (uint32_t)offsetof(TopkGateRow, valid));
  const __amdgpu_buffer_rsrc_t sc_r = make_rsrc(sc, (uint32_t)max_pages * 4u);  // slots past the row read 0
  float v[KPL];
#pragma unroll
  for (int i = 0; i < KPL; ++i) v[i] = buf_load_f32(sc_r, (uint32_t)(wbase + i * kWave) * 4u);
  n = row_phys_pages(max(raw_len - len_off, 0), max_pages, lgs);
  phys_later = !COV && KPL <= 32 && gate_src && gr.valid;
  if (!phys_later) {
#pragma unroll
    for (int i = 0; i < KPL; ++i) phys.load(i, wbase + i * kWave, max_pages);
  }
  const RowShape r = row_shape(n, n_sink, n_local);
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int p = wbase + i * kWave;
    if constexpr (COV) key[i] = p < n ? coverage_key(v[i]) : 0u;
    else key[i] = (unsigned)(p - r.sink_end) < (unsigned)(r.local_begin - r.sink_end) ? score_key(v[i]) : 0u;
  }
}

// Tail workgroup k: wave w rebuilds (request, KV head, page) item k * NW + w: the request's last
// logical page, or its last tail.span pages when span > 1 (several query tokens per step).
__device__ __forceinline__ int tail_span(const SelectArgs& a) { return a.tail.span > 1 ? a.tail.span : 1; }

template <int NW>
__device__ __forceinline__ void rebuild_tail_pages(const SelectArgs& a, int k) {
  const int span = tail_span(a);
  const int item = k * NW + (int)(threadIdx.x / kWave);
  if (item >= a.batch * a.num_kv_heads * span) return;
  const int s = item % span, bh = item / span;
  const int b = bh / a.num_kv_heads, h = bh % a.num_kv_heads;
  const int len = a.seq_lens[b];
  const int n = row_logical_pages(len, a.max_pages, a.tail.lgs);  // the newest token's logical page
  if (n - 1 - s >= 0) build_page_meta_rt(a.tail, b, n - 1 - s, h, len);
}

// Row blockIdx.x = (b T + t) Hkv + h of a step with T = a.num_tokens query tokens per request: token t of
// request b sees the first seq_lens[b] - T + 1 + t keys (T = 1: the request's own length) and reads
// request b's block-table row.  Returns the token row's length; b is the request.
__device__ __forceinline__ int token_row_length(const SelectArgs& a, int token_row, int& b) {
  const int T = a.num_tokens;
  b = token_row / T;
  const int len = a.seq_lens[b] - (T - 1 - token_row % T);
  return len > 0 ? len : 0;
}

template <int NW, int KPL, bool COV>
__global__ __launch_bounds__(NW * kWave) void page_select_kernel(SelectArgs a) {
  __shared__ SelectSmem<NW, KPL, COV> sm;
  const int rows = a.batch * a.num_tokens * a.num_kv_heads;
  if ((int)blockIdx.x >= rows) {
    rebuild_tail_pages<NW>(a, blockIdx.x - rows);
    return;
  }
  const int token_row = blockIdx.x / a.num_kv_heads;
  const int h = blockIdx.x % a.num_kv_heads;
  const size_t row = (size_t)token_row * a.num_kv_heads + h;
  const int T = a.num_tokens;
  const int b = token_row / T;
  const int32_t* bt_row = a.page_phys ? a.block_table + (size_t)b * a.max_pages : nullptr;
  if ((a.streaming_mask >> h) & 1ull) {
    int b_;
    select_streaming_row(a, row_phys_pages(token_row_length(a, token_row, b_), a.max_pages, a.lgs), row, bt_row);
    return;
  }
  TopkGateRow gr{};
  uint32_t key[KPL];
  SlotPhys<KPL> phys;
  phys.bt_row = bt_row;
  // token t of request b sees seq_lens[b] - (T - 1 - t) keys (T = 1: the request's length)
  int n;
  bool phys_later;
  load_row_keys<NW, KPL, COV>(a.scores + row * a.max_pages, a.seq_lens + b, T - 1 - token_row % T, a.max_pages, a.lgs,
                              a.n_sink, a.n_local, COV ? nullptr : a.gate.rows ? a.gate.rows + row : nullptr, gr, key,
                              phys, n, phys_later);
  if constexpr (COV) {
    select_row_keys<NW, KPL, COV>(a, key, phys, row_shape(n, a.n_sink, a.n_local), row, sm);
  } else {
    __shared__ GateSmem gs;
    select_row_keys<NW, KPL, COV>(a, key, phys, row_shape(n, a.n_sink, a.n_local), row, sm, &gr, &gs, phys_later);
  }
}

// Reusable page selection (LServe, "Reusable Page Selection"): between two selections the lists
// of the chunk's first step are reused, while the requests grow.  A dynamic row keeps its list
// and gets every page of the current forced set (sink + local window) that lies past its last
// entry appended in order -- the local window only moves right, so the list stays ascending; a
// streaming row's static table is rewritten for the current length.  Workgroups after the rows
// rebuild each request's newest page statistics, as in the selector.
constexpr int kRefreshThreads = 256;

__global__ __launch_bounds__(kRefreshThreads) void page_list_refresh_kernel(SelectArgs a) {
  const int rows = a.batch * a.num_kv_heads;
  if ((int)blockIdx.x >= rows) {
    rebuild_tail_pages<kRefreshThreads / kWave>(a, blockIdx.x - rows);
    return;
  }
  const int b = blockIdx.x / a.num_kv_heads;
  const int h = blockIdx.x % a.num_kv_heads;
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const int n = row_phys_pages(a.seq_lens[b], a.max_pages, a.lgs);
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  if ((a.streaming_mask >> h) & 1ull) {
    select_streaming_row(a, n, row, bt_row);
    return;
  }
  int32_t* out = a.page_list + row * a.max_list;
  const int len = min(max(a.list_len[row], 0), a.max_list);
  const int last = len > 0 ? out[len - 1] : -1;
  const RowShape r = row_shape(n, a.n_sink, a.n_local);
  // forced pages past `last`: sinks [last + 1, sink_end), then locals [max(last + 1, local_begin), n)
  const int s0 = last + 1;
  const int n_sink_new = max(0, r.sink_end - s0);
  const int l0 = max(s0, r.local_begin);
  const int n_local_new = max(0, n - l0);
  const int add = n_sink_new + n_local_new;
  for (int i = threadIdx.x; i < add && len + i < a.max_list; i += blockDim.x) {
    const int p = i < n_sink_new ? s0 + i : l0 + (i - n_sink_new);
    out[len + i] = p;
    if (a.page_phys) a.page_phys[row * a.max_list + len + i] = bt_row[p];
  }
  if (threadIdx.x == 0) a.list_len[row] = min(len + add, a.max_list);
}

int launch_page_list_refresh(const SelectArgs& a, hipStream_t stream) {
  const int rows = a.batch * a.num_kv_heads;
  const int waves = kRefreshThreads / kWave;
  const int tail_blocks = a.tail.meta ? (rows + waves - 1) / waves : 0;
  hipLaunchKernelGGL(page_list_refresh_kernel, dim3((unsigned)(rows + tail_blocks)), dim3(kRefreshThreads), 0, stream, a);
  return 0;
}

int launch_page_select(const SelectArgs& a, hipStream_t stream) {
  SelectGeometry g;
  if (!select_geometry(a.max_pages, g)) return SPD_ERR_UNSUPPORTED;
  const int rows = a.batch * a.num_tokens * a.num_kv_heads;
  const int tail_blocks = a.tail.meta ? (a.batch * a.num_kv_heads * (a.tail.span > 1 ? a.tail.span : 1) + g.nw - 1) / g.nw : 0;
  const dim3 grid((unsigned)(rows + tail_blocks)), block(g.nw * kWave);
  const bool cov = a.mode == SPD_SELECT_COVERAGE;
#define SPD_SEL_CASE(NW, KPL)                                                                          \
  if (g.nw == NW && g.kpl == KPL) {                                                                    \
    if (cov) hipLaunchKernelGGL((page_select_kernel<NW, KPL, true>), grid, block, 0, stream, a);       \
    else hipLaunchKernelGGL((page_select_kernel<NW, KPL, false>), grid, block, 0, stream, a);          \
    return 0;                                                                                          \
  }
  SPD_SEL_CASE(16, 2)
  SPD_SEL_CASE(16, 8)
  SPD_SEL_CASE(16, 32)
  SPD_SEL_CASE(16, 64)
#undef SPD_SEL_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
