// Page lists from page scores: one workgroup per (request, KV head) row.  The selection rules
// and their sources are described in select_row.h.  Optionally, workgroups after the rows
// rebuild the key statistics of each request's last page, one wave per KV head (LServe, "Key
// statistics storage and updating"), beside the selection: where the scorer skipped that page
// (the local window keeps it), the rebuild leaves the critical path of the step.
#include "meta_build.h"
#include "select_row.h"

namespace spd {

// Keys (and physical pages, when the list of physical pages is wanted) of the row's pages in
// the slot layout of select_row_keys.  `sc` holds top-K scores or coverage shares.
template <int NW, int KPL, bool COV>
__device__ __forceinline__ void load_row_keys(const float* sc, int n, uint32_t (&key)[KPL], SlotPhys<KPL>& phys) {
  const int wbase = (int)(threadIdx.x / kWave) * kWave * KPL + (int)(threadIdx.x % kWave);
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const int p = wbase + i * kWave;
    const float v = p < n ? sc[p] : 0.f;
    key[i] = COV ? coverage_key(v) : score_key(v);
    phys.load(i, p, n);
  }
}

// Tail workgroup k: wave w rebuilds (request, KV head) item k * NW + w.
template <int NW>
__device__ __forceinline__ void rebuild_tail_pages(const SelectArgs& a, int k) {
  const int item = k * NW + (int)(threadIdx.x / kWave);
  if (item >= a.batch * a.num_kv_heads) return;
  const int b = item / a.num_kv_heads, h = item % a.num_kv_heads;
  const int len = a.seq_lens[b];
  const int n = row_pages(len, a.max_pages);
  if (n > 0) build_page_meta_rt(a.tail, b, n - 1, h, len);
}

template <int NW, int KPL, bool COV>
__global__ __launch_bounds__(NW * kWave) void page_select_kernel(SelectArgs a) {
  __shared__ SelectSmem<NW, KPL, COV> sm;
  const int rows = a.batch * a.num_kv_heads;
  if ((int)blockIdx.x >= rows) {
    rebuild_tail_pages<NW>(a, blockIdx.x - rows);
    return;
  }
  const int b = blockIdx.x / a.num_kv_heads;
  const int h = blockIdx.x % a.num_kv_heads;
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const int32_t* bt_row = a.page_phys ? a.block_table + (size_t)b * a.max_pages : nullptr;
  if ((a.streaming_mask >> h) & 1ull) {
    select_streaming_row(a, n, row, bt_row);
    return;
  }
  uint32_t key[KPL];
  SlotPhys<KPL> phys;
  phys.bt_row = bt_row;
  load_row_keys<NW, KPL, COV>(a.scores + row * a.max_pages, n, key, phys);
  select_row_keys<NW, KPL, COV>(a, key, phys, row_shape(n, a.n_sink, a.n_local), row, sm);
}

int launch_page_select(const SelectArgs& a, hipStream_t stream) {
  SelectGeometry g;
  if (!select_geometry(a.max_pages, g)) return SPD_ERR_UNSUPPORTED;
  const int rows = a.batch * a.num_kv_heads;
  const int tail_blocks = a.tail.meta ? (rows + g.nw - 1) / g.nw : 0;
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
