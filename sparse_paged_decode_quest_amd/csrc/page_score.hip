// Page scores from the per-page key box (LServe summary, "Hierarchical Paging", page
// importance S_j = sum_i max(q_i kmax_i, q_i kmin_i): an upper bound on q.k over every key
// of the page, two dot products per page).  The arithmetic and the work layout are in
// score_common.h.  The last page of a dynamic row is scored like the others (SPD_TAIL_NONE),
// or by one extra workgroup per row that first rebuilds its key statistics from the K pool
// (SPD_TAIL_REBUILD; LServe, "Key statistics storage and updating"), or not at all
// (SPD_TAIL_SKIP, top-K: the local window keeps it whatever its score).
//
// Top-K mode writes score_p = max_g S_{g,p}.  Coverage mode (Moira, section 3.2, Eq. 3,
// group-mean share) writes the log-mass l_{g,p} = s S_{g,p} + ln(valid_p); a second kernel,
// one workgroup per row, takes the per-head log-sum-exp over the row's log-masses and writes
// pi_bar_p = (1/G) sum_g exp(l_{g,p} - lse_g).
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
    if (n > 0) score_tail<D, KVD, COV>(a, bt_row, n, len, r.b, r.h, -1);
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
  if constexpr (COV) score_block_ell<D, KVD, kScoreWaves, kScoreIters>(a, raw, n_scan, len, r.b, r.h, p_begin);
  else score_block_topk<D, KVD, kScoreWaves, kScoreIters>(a, raw, n_scan, r.b, r.h, p_begin, sc_row);
}

// Coverage, second pass: one workgroup per dynamic row.  Every thread folds the log-masses of
// its pages into a running (max, sum exp) per head, the workgroup combines those in a fixed
// order into lse_g, and the shares are written from a second (cached) read of the log-masses.
constexpr int kShareThreads = 1024;
constexpr int kShareBatch = 8;  // pages per thread requested together

__global__ __launch_bounds__(kShareThreads) void coverage_share_kernel(ScoreArgs a) {
  __shared__ float wm[kShareThreads / kWave][kG], ws[kShareThreads / kWave][kG];
  __shared__ float lse_s[kG];
  const int b = blockIdx.x / a.dyn.count;
  const int h = a.dyn.head[blockIdx.x % a.dyn.count];
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const size_t row = (size_t)b * a.num_kv_heads + h;
  const float4* ell = a.ell + row * a.max_pages;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  float m[kG], s[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    m[g] = -INFINITY;
    s[g] = 0.f;
  }
  for (int p0 = 0; p0 < n; p0 += kShareThreads * kShareBatch) {
    float4 v[kShareBatch];
#pragma unroll
    for (int k = 0; k < kShareBatch; ++k) {
      const int p = p0 + k * kShareThreads + (int)threadIdx.x;
      v[k] = p < n ? ell[p] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int k = 0; k < kShareBatch; ++k) {
      lse_push(m[0], s[0], v[k].x);
      lse_push(m[1], s[1], v[k].y);
      lse_push(m[2], s[2], v[k].z);
      lse_push(m[3], s[3], v[k].w);
    }
  }
  // wave: common max, then the rescaled sums; waves are folded in order by four threads
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const float M = wave_max_f(m[g]);
    const float sc = m[g] == -INFINITY ? 0.f : s[g] * expf(m[g] - M);
    const float S = wave_sum_f(sc);
    if (lane == 0) {
      wm[wave][g] = M;
      ws[wave][g] = S;
    }
  }
  __syncthreads();
  if (threadIdx.x < kG) {
    const int g = threadIdx.x;
    float M = wm[0][g], S = ws[0][g];
    for (int w = 1; w < kShareThreads / kWave; ++w) lse_combine(M, S, wm[w][g], ws[w][g]);
    const float lse = M == -INFINITY ? -INFINITY : M + logf(S);
    lse_s[g] = lse;
    if (a.head_lse) a.head_lse[(size_t)b * a.num_q_heads + (size_t)h * kG + g] = lse;
  }
  __syncthreads();
  float lse[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) lse[g] = lse_s[g];
  for (int p = threadIdx.x; p < n; p += kShareThreads) a.scores[row * a.max_pages + p] = group_share(ell[p], lse);
}

int launch_page_score(const ScoreArgs& a, int head_dim, int kv_dtype, bool coverage, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.batch * a.dyn.count);
  const dim3 grid(rows * (unsigned)(a.blocks_per_row + tail_blocks(a))), block(kScoreWaves * kWave);
  const dim3 share_grid(rows), share_block(kShareThreads);
#define SPD_SCORE_CASE(D, KVD)                                                                  \
  if (head_dim == D && kv_dtype == KVD) {                                                       \
    if (coverage) {                                                                             \
      hipLaunchKernelGGL((page_score_kernel<D, KVD, true>), grid, block, 0, stream, a);         \
      hipLaunchKernelGGL(coverage_share_kernel, share_grid, share_block, 0, stream, a);         \
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
