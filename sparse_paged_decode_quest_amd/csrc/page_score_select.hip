// Fused top-K page scoring and selection in one launch (LiteTopK, section 3.2, "Extension
// to Decoding": in decode the score write-back is small, so selection is fused into score
// computation and finished over the aggregated per-block results).
//
// Blocks of a dynamic row score their pages into the workspace, publish them with a
// device-scope release fence and take a ticket from the row's counter; the block that
// takes the last ticket acquires, selects the row's pages (select_row.h) and returns the
// counter to zero, so the workspace is ready for the next call (and for graph replay)
// without a separate clearing step.  Extra blocks write the static lists of streaming rows.
#include "score_common.h"
#include "select_row.h"

namespace spd {

static_assert(kFusedWaves * kWave == kSelThreads, "the fused block selects with kSelThreads threads");

template <int D, int QD, int MD, int KPT>
__global__ __launch_bounds__(kSelThreads) void page_score_select_kernel(FusedArgs f) {
  __shared__ SelectSmem sm;
  __shared__ int last;
  const ScoreArgs& a = f.score;
  const int dyn_blocks = a.batch * a.dyn.count * a.blocks_per_row;
  if ((int)blockIdx.x >= dyn_blocks) {
    const int k = blockIdx.x - dyn_blocks;
    const int b = k / f.stream_heads.count;
    const int h = f.stream_heads.head[k % f.stream_heads.count];
    const size_t row = (size_t)b * a.num_kv_heads + h;
    select_streaming_row(f.sel, row_pages(a.seq_lens[b], a.max_pages), row);
    return;
  }
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const int used = (n + a.pages_per_block - 1) / a.pages_per_block;
  if (n == 0) {
    if (blk == 0 && threadIdx.x == 0) f.sel.list_len[row] = 0;
    return;
  }
  if (blk >= used) return;
  const int p_begin = blk * a.pages_per_block;
  const int p_end = min(n, p_begin + a.pages_per_block);
  float* row_scores = a.scores + row * a.max_pages;
  score_block_topk<D, QD, MD, kFusedWaves, kFusedIters>(a, b, h, p_begin, p_end, row_scores);
  __threadfence();  // release this block's scores device-wide
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(&f.counters[row], 1u) == (unsigned)(used - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();  // acquire the other blocks' scores
  select_dynamic_row<KPT, false>(f.sel, row_scores, n, row, sm);
  if (threadIdx.x == 0) f.counters[row] = 0u;
}

int launch_page_score_select(const FusedArgs& f, int head_dim, int q_dtype, int meta_dtype, hipStream_t stream) {
  const int blocks = f.score.batch * (f.score.dyn.count * f.score.blocks_per_row + f.stream_heads.count);
  dim3 grid((unsigned)blocks), block(kSelThreads);
#define SPD_FUSED_CASE(D, QD, MD)                                                                  \
  if (head_dim == D && q_dtype == QD && meta_dtype == MD) {                                        \
    switch (select_kpt(f.score.max_pages)) {                                                       \
      case 8: hipLaunchKernelGGL((page_score_select_kernel<D, QD, MD, 8>), grid, block, 0, stream, f); break;     \
      case 32: hipLaunchKernelGGL((page_score_select_kernel<D, QD, MD, 32>), grid, block, 0, stream, f); break;   \
      default: hipLaunchKernelGGL((page_score_select_kernel<D, QD, MD, 0>), grid, block, 0, stream, f); break;    \
    }                                                                                              \
    return 0;                                                                                      \
  }
  SPD_FUSED_CASE(64, SPD_DTYPE_F16, SPD_DTYPE_F16)
  SPD_FUSED_CASE(128, SPD_DTYPE_F16, SPD_DTYPE_F16)
  SPD_FUSED_CASE(64, SPD_DTYPE_F32, SPD_DTYPE_F32)
  SPD_FUSED_CASE(128, SPD_DTYPE_F32, SPD_DTYPE_F32)
#undef SPD_FUSED_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
