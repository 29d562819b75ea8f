// Page scores from the per-page key box (LServe summary, "Hierarchical Paging", page
// importance S_j = sum_i max(q_i kmax_i, q_i kmin_i): an upper bound on q.k over every key
// of the page, two dot products per page).  The arithmetic and the work layout are in
// score_common.h.  The last page of a dynamic row is scored like the others (SPD_TAIL_NONE),
// or by one extra workgroup per row that first rebuilds its key statistics from the K pool
// (SPD_TAIL_REBUILD; LServe, "Key statistics storage and updating"), or not at all
// (SPD_TAIL_SKIP, top-K: the local window keeps it whatever its score).
//
// Top-K mode writes score_p = max_g S_{g,p}.  Coverage mode (Moira, section 3.2, Eq. 3,
// group-mean share) writes the log-mass l_{g,p} = s S_{g,p} + ln(valid_p) and per-block
// (max, sum exp) pairs; a second kernel merges the pairs of the row into the per-head
// log-sum-exp and writes pi_bar_p = (1/G) sum_g exp(l_{g,p} - lse_g).
#include "score_common.h"
#include "spd_launch.h"

namespace spd {

// A dynamic row's workgroups: blk < blocks_per_row scan pages; with SPD_TAIL_REBUILD one more,
// blk == blocks_per_row, rebuilds and scores the row's last page.  Unless the mode is
// SPD_TAIL_NONE the scan stops before that page.
struct RowRole {
  int b, h, blk;
  bool tail;
};

__device__ __forceinline__ RowRole row_role(const ScoreArgs& a) {
  const int per_row = a.blocks_per_row + tail_blocks(a);
  const int row_dyn = blockIdx.x / per_row;
  RowRole r;
  r.blk = blockIdx.x % per_row;
  r.b = row_dyn / a.dyn.count;
  r.h = a.dyn.head[row_dyn % a.dyn.count];
  r.tail = r.blk == a.blocks_per_row;
  return r;
}

template <int D, int KVD, bool COV>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_kernel(ScoreArgs a) {
  const RowRole r = row_role(a);
  const int32_t* bt_row = a.block_table + (size_t)r.b * a.max_pages;
  const int len = a.seq_lens[r.b];
  if (r.tail) {
    const int n = row_pages(len, a.max_pages);
    if (n > 0) score_tail<D, KVD, COV>(a, bt_row, n, len, r.b, r.h, (n - 1 + a.pages_per_block - 1) / a.pages_per_block);
    return;
  }
  const int p_begin = r.blk * a.pages_per_block;
  int raw[kScoreIters];
  load_block_table<D, KVD, kScoreWaves, kScoreIters>(bt_row, a.max_pages, p_begin, raw);
  const int n = row_pages(len, a.max_pages);
  const int n_scan = scan_pages(a, n);
  float* sc_row = a.scores + ((size_t)r.b * a.num_kv_heads + r.h) * a.max_pages;
  if (!COV && a.tail_mode == SPD_TAIL_SKIP && r.blk == 0 && n > 0 && threadIdx.x == 0) sc_row[n - 1] = -INFINITY;
  if (p_begin >= n_scan) return;  // uniform over the block
  if constexpr (COV) score_block_coverage<D, KVD, kScoreWaves, kScoreIters>(a, raw, n_scan, len, r.b, r.h, p_begin, r.blk);
  else score_block_topk<D, KVD, kScoreWaves, kScoreIters>(a, raw, n_scan, r.b, r.h, p_begin, sc_row);
}

// Partial slots a row's coverage pass filled: the scanning workgroups', then the tail's.
__device__ __forceinline__ int coverage_slots(const ScoreArgs& a, int n) {
  if (n == 0) return 0;
  return (scan_pages(a, n) + a.pages_per_block - 1) / a.pages_per_block + tail_blocks(a);
}

// Coverage, second pass: per-head log-sum-exp of the row, then the group-mean share.
__global__ __launch_bounds__(kScoreWaves * kWave) void coverage_share_kernel(ScoreArgs a) {
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const int p_begin = blk * a.pages_per_block;
  const int p_end = min(n, p_begin + a.pages_per_block);
  if (p_begin >= p_end && blk != 0) return;  // block 0 of an empty row still writes head_lse
  const size_t row = (size_t)b * a.num_kv_heads + h;
  float lse[kG];
  row_head_lse(a.partials + row * a.partial_stride * kG, coverage_slots(a, n), lse);  // every wave, same bits
  if (blk == 0 && threadIdx.x < kG && a.head_lse) {
    float v = lse[0];
#pragma unroll
    for (int g = 1; g < kG; ++g) v = (int)threadIdx.x == g ? lse[g] : v;
    a.head_lse[(size_t)b * a.num_q_heads + (size_t)h * kG + threadIdx.x] = v;
  }
  for (int p = p_begin + threadIdx.x; p < p_end; p += blockDim.x)
    a.scores[row * a.max_pages + p] = group_share(a.ell[row * a.max_pages + p], lse);
}

int launch_page_score(const ScoreArgs& a, int head_dim, int kv_dtype, bool coverage, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.batch * a.dyn.count);
  const dim3 grid(rows * (unsigned)(a.blocks_per_row + tail_blocks(a))), block(kScoreWaves * kWave);
  const dim3 share_grid(rows * (unsigned)a.blocks_per_row);
#define SPD_SCORE_CASE(D, KVD)                                                                  \
  if (head_dim == D && kv_dtype == KVD) {                                                       \
    if (coverage) {                                                                             \
      hipLaunchKernelGGL((page_score_kernel<D, KVD, true>), grid, block, 0, stream, a);         \
      hipLaunchKernelGGL(coverage_share_kernel, share_grid, block, 0, stream, a);               \
    } else {                                                                                    \
      hipLaunchKernelGGL((page_score_kernel<D, KVD, false>), grid, block, 0, stream, a);        \
    }                                                                                           \
    return 0;                                                                                   \
  }
  SPD_SCORE_CASE(64, SPD_DTYPE_F16)
  SPD_SCORE_CASE(128, SPD_DTYPE_F16)
  SPD_SCORE_CASE(128, SPD_DTYPE_FP8_E4M3FN)
  SPD_SCORE_CASE(64, SPD_DTYPE_F32)
  SPD_SCORE_CASE(128, SPD_DTYPE_F32)
#undef SPD_SCORE_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
