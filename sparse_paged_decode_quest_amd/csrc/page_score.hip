// Page scores from the per-page key box (LServe summary, "Hierarchical Paging", page
// importance S_j = sum_i max(q_i kmax_i, q_i kmin_i): an upper bound on q.k over every key
// of the page, two dot products per page).  The arithmetic and the work layout are in
// score_common.h.
//
// Top-K mode writes score_p = max_g S_{g,p}.  Coverage mode (Moira, section 3.2, Eq. 3,
// group-mean share) writes the log-mass l_{g,p} = s S_{g,p} + ln(valid_p) and per-block
// (max, sum exp) pairs; a second kernel merges the pairs of the row into the per-head
// log-sum-exp and writes pi_bar_p = (1/G) sum_g exp(l_{g,p} - lse_g).
#include "score_common.h"
#include "spd_launch.h"

namespace spd {

template <int D, int KVD>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_topk_kernel(ScoreArgs a) {
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  const int p_begin = blk * a.pages_per_block;
  const int len = a.seq_lens[b];
  int raw[kScoreIters];
  load_block_table<D, KVD, kScoreWaves, kScoreIters>(bt_row, a.max_pages, p_begin, raw);
  const int n = row_pages(len, a.max_pages);
  if (p_begin >= n) return;
  score_block_topk<D, KVD, kScoreWaves, kScoreIters>(a, raw, n, len, b, h, p_begin, false,
                                                     a.scores + ((size_t)b * a.num_kv_heads + h) * a.max_pages);
}

// Coverage, first pass: log-masses l_{g,p} and one (max, sum exp) pair per head and block.
template <int D, int KVD>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_coverage_kernel(ScoreArgs a) {
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  const int p_begin = blk * a.pages_per_block;
  const int len = a.seq_lens[b];
  int raw[kScoreIters];
  load_block_table<D, KVD, kScoreWaves, kScoreIters>(bt_row, a.max_pages, p_begin, raw);
  const int n = row_pages(len, a.max_pages);
  if (p_begin >= n) return;  // uniform over the block
  score_block_coverage<D, KVD, kScoreWaves, kScoreIters>(a, raw, n, len, b, h, p_begin, blk, false);
}

// Coverage, second pass: per-head log-sum-exp of the row, then the group-mean share.
__global__ __launch_bounds__(kScoreWaves * kWave) void coverage_share_kernel(ScoreArgs a) {
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const int used = (n + a.pages_per_block - 1) / a.pages_per_block;
  const int p_begin = blk * a.pages_per_block;
  const int p_end = min(n, p_begin + a.pages_per_block);
  if (p_begin >= p_end && blk != 0) return;  // block 0 of an empty row still writes head_lse
  const size_t row = (size_t)b * a.num_kv_heads + h;
  float lse[kG];
  row_head_lse(a.partials + row * a.blocks_per_row * kG, used, lse);  // every wave, same bits
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
  dim3 grid((unsigned)(a.batch * a.dyn.count * a.blocks_per_row)), block(kScoreWaves * kWave);
#define SPD_SCORE_CASE(D, KVD)                                                              \
  if (head_dim == D && kv_dtype == KVD) {                                                   \
    if (coverage) {                                                                         \
      hipLaunchKernelGGL((page_score_coverage_kernel<D, KVD>), grid, block, 0, stream, a);  \
      hipLaunchKernelGGL(coverage_share_kernel, grid, block, 0, stream, a);                 \
    } else {                                                                                \
      hipLaunchKernelGGL((page_score_topk_kernel<D, KVD>), grid, block, 0, stream, a);      \
    }                                                                                       \
    return 0;                                                                               \
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
