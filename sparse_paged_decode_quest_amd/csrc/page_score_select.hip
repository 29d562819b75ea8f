// Fused page scoring and selection in one launch (LiteTopK, section 3.2, "Extension to
// Decoding": in decode the score write-back is small, so selection is fused into score
// computation and finished over the aggregated per-block results), for both selection rules.
//
// The workgroups of a dynamic row score their pages into the workspace (top-K scores, or the
// coverage log-masses and per-workgroup (max, sum exp) pairs) and publish them by taking a
// ticket from the row's counter with a device-scope release.  The workgroup that
// takes the last ticket acquires, builds the row's keys (coverage: the per-head log-sum-exp
// and Moira's group-mean shares, section 3.2, Eq. 3), selects the row's pages
// (select_row.h) and returns the counter to zero, so the workspace is ready for the next call
// (and for graph replay) without a clearing step.  With SPD_TAIL_REBUILD one more workgroup per
// dynamic row rebuilds the key statistics of the row's last page from the K pool and scores it
// (LServe, "Key statistics storage and updating"); it takes a ticket like the others.  With
// SPD_TAIL_SKIP (top-K) that page is not scored: the local window keeps it.  Extra workgroups
// write the static lists of streaming rows.
#include "score_common.h"
#include "select_row.h"

namespace spd {

template <int D, int KVD, int NW, int ITERS, int KPL, bool COV>
__global__ __launch_bounds__(NW * kWave) void page_score_select_kernel(FusedArgs f) {
  __shared__ SelectSmem<NW, KPL, COV> sm;
  __shared__ int last;
  const ScoreArgs& a = f.score;
  const int per_row = a.blocks_per_row + tail_blocks(a);  // + the tail workgroup
  const int dyn_blocks = a.batch * a.dyn.count * per_row;
  if ((int)blockIdx.x >= dyn_blocks) {
    const int k = blockIdx.x - dyn_blocks;
    const int b = k / f.stream_heads.count;
    const int h = f.stream_heads.at(k % f.stream_heads.count);
    const size_t row = (size_t)b * a.num_kv_heads + h;
    const int len = a.seq_lens[b];
    const int n = row_pages(len, a.max_pages);
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
    select_streaming_row(f.sel, n, row, bt_row);
    if (a.tail_mode == SPD_TAIL_REBUILD && n > 0) rebuild_tail_page<D, KVD>(a, bt_row, n, len, b, h);
    return;
  }
  const int row_dyn = blockIdx.x / per_row;
  const int blk = blockIdx.x % per_row;
  const bool tail_block = blk == a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.at(row_dyn % a.dyn.count);
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  const int p_begin = blk * a.pages_per_block;
  const int len = a.seq_lens[b];
  int raw[ITERS];
  if (!tail_block) load_block_table<D, KVD, NW, ITERS>(bt_row, a.max_pages, p_begin, raw);
  const int n = row_pages(len, a.max_pages);
  if (n == 0) {
    if (blk == 0 && threadIdx.x == 0) f.sel.list_len[row] = 0;
    if (COV && blk == 0 && threadIdx.x < kG && a.head_lse)
      a.head_lse[(size_t)b * a.num_q_heads + (size_t)h * kG + threadIdx.x] = -INFINITY;
    return;
  }
  const int n_scan = scan_pages(a, n);
  // Page-scanning workgroups, then the tail workgroup; when the only page is a skipped last
  // page, workgroup 0 still takes the one ticket.
  int used = (n_scan + a.pages_per_block - 1) / a.pages_per_block;
  if (used + tail_blocks(a) == 0) used = 1;
  const int tickets = used + tail_blocks(a);
  if (tail_block) {
    score_tail<D, KVD, COV>(a, bt_row, n, len, b, h, used);
  } else {
    if (blk >= used) return;
    if (!COV && a.tail_mode == SPD_TAIL_SKIP && blk == 0 && threadIdx.x == 0) a.scores[row * a.max_pages + n - 1] = -INFINITY;
    if (p_begin < n_scan) {
      if constexpr (COV) score_block_coverage<D, KVD, NW, ITERS>(a, raw, n_scan, len, b, h, p_begin, blk);
      else score_block_topk<D, KVD, NW, ITERS>(a, raw, n_scan, b, h, p_begin, a.scores + row * a.max_pages);
    }
  }
  // Publish: every wave waits for its own score stores, the workgroup barrier orders them before
  // the ticket, and the ticket is a release at device scope (one L2 write-back per workgroup;
  // a fence in every wave would write back and invalidate the L2 once per wave).  The workgroup
  // that takes the last ticket acquires with one fence (the L1 it invalidates is the CU's, shared
  // by all its waves) before any wave reads the other workgroups' scores.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(&f.counters[row], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(tickets - 1);
  __syncthreads();
  if (!last) return;
  if (threadIdx.x < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  __syncthreads();

  const int wbase = (int)(threadIdx.x / kWave) * kWave * KPL + (int)(threadIdx.x % kWave);  // select_row.h slots
  uint32_t key[KPL];
  SlotPhys<KPL> phys;
  phys.bt_row = f.sel.page_phys ? bt_row : nullptr;
  if constexpr (COV) {
    float lse[kG];
    row_head_lse(a.partials + row * a.partial_stride * kG, tickets, lse);  // every wave, same bits
    if (threadIdx.x < kG && a.head_lse) {
      float v = lse[0];
#pragma unroll
      for (int g = 1; g < kG; ++g) v = (int)threadIdx.x == g ? lse[g] : v;
      a.head_lse[(size_t)b * a.num_q_heads + (size_t)h * kG + threadIdx.x] = v;
    }
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int p = wbase + i * kWave;
      float4 l4 = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (p < n) l4 = a.ell[row * a.max_pages + p];
      phys.load(i, p, n);
      const float pi = p < n ? group_share(l4, lse) : 0.f;
      key[i] = coverage_key(pi);
      if (f.score_out && p < n) f.score_out[row * a.max_pages + p] = pi;
    }
  } else {
    const float* sc = a.scores + row * a.max_pages;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int p = wbase + i * kWave;
      key[i] = score_key(p < n ? sc[p] : 0.f);
      phys.load(i, p, n);
    }
  }
  select_row_keys<NW, KPL, COV>(f.sel, key, phys, row_shape(n, f.sel.n_sink, f.sel.n_local), row, sm);
  if (threadIdx.x == 0) f.counters[row] = 0u;
}

int launch_page_score_select(const FusedArgs& f, int head_dim, int kv_dtype, hipStream_t stream) {
  SelectGeometry g;
  if (!select_geometry(f.score.max_pages, g)) return SPD_ERR_UNSUPPORTED;
  const int per_row = f.score.blocks_per_row + tail_blocks(f.score);
  const int blocks = f.score.batch * (f.score.dyn.count * per_row + f.stream_heads.count);
  const dim3 grid((unsigned)blocks), block(g.nw * kWave);
  const bool cov = f.sel.mode == SPD_SELECT_COVERAGE;
#define SPD_FUSED_GEOM(D, KVD, NW, KPL, IT)                                                                     \
  if (g.nw == NW && g.kpl == KPL) {                                                                             \
    if (cov) hipLaunchKernelGGL((page_score_select_kernel<D, KVD, NW, IT, KPL, true>), grid, block, 0, stream, f); \
    else hipLaunchKernelGGL((page_score_select_kernel<D, KVD, NW, IT, KPL, false>), grid, block, 0, stream, f);    \
    return 0;                                                                                                   \
  }
#define SPD_FUSED_CASE(D, KVD)                 \
  if (head_dim == D && kv_dtype == KVD) {      \
    SPD_FUSED_GEOM(D, KVD, 16, 2, 2)           \
    SPD_FUSED_GEOM(D, KVD, 16, 8, 2)           \
    SPD_FUSED_GEOM(D, KVD, 16, 32, 2)          \
    SPD_FUSED_GEOM(D, KVD, 16, 64, 4)          \
    return SPD_ERR_UNSUPPORTED;                \
  }
  SPD_FUSED_CASE(64, SPD_DTYPE_F16)
  SPD_FUSED_CASE(128, SPD_DTYPE_F16)
  SPD_FUSED_CASE(128, SPD_DTYPE_FP8_E4M3FN)
  SPD_FUSED_CASE(64, SPD_DTYPE_F32)
  SPD_FUSED_CASE(128, SPD_DTYPE_F32)
#undef SPD_FUSED_CASE
#undef SPD_FUSED_GEOM
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
