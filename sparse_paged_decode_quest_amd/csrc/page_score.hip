// Page scores from the per-page key box (LServe summary, "Hierarchical Paging", page
// importance S_j = sum_i max(q_i kmax_i, q_i kmin_i): an upper bound on q.k over every key
// of the page, two dot products per page).  The arithmetic and the work layout are in
// score_common.h.  The last page of a dynamic row is scored like the others (SPD_TAIL_NONE),
// or by one extra workgroup per row that first rebuilds its key statistics from the K pool
// (SPD_TAIL_REBUILD; LServe, "Key statistics storage and updating"), or not at all
// (SPD_TAIL_SKIP, top-K: the local window keeps it whatever its score).
//
// Top-K mode writes score_p = max_g S_{g,p}.  Coverage mode (Moira, section 3.2, Eq. 3,
// group-mean share) writes the log-mass l_{g,p} = s S_{g,p} + ln(valid_p); two more kernels
// take the per-head log-sum-exp over the row's log-masses and write
// pi_bar_p = (1/G) sum_g exp(l_{g,p} - lse_g).
#include "score_common.h"
#include "spd_launch.h"

namespace spd {

// The scanning workgroups take the numbered work items of score_common.h (scan_item), so a batch of
// short and long requests has no workgroups past its rows' ends among the working ones.  With
// SPD_TAIL_REBUILD the grid starts with one workgroup per (request, KV head), which rebuilds the key
// statistics of the request's last page and, for a dynamic head, scores it; being first, they run
// beside the scan instead of after it.  Unless the mode is SPD_TAIL_NONE the scan stops before that
// page.

// Pages a row's scan covers for a request of `len` tokens, in the units the workgroups step over
// (logical pages for coverage and hierarchical paging).
template <bool COV, bool HIER>
__device__ __forceinline__ int scan_limit(const ScoreArgs& a, int len) {
  if constexpr (HIER) {
    const int n_phys = row_phys_pages(len, a.max_pages, a.lgs);
    const int phys_scan = a.tail_mode == SPD_TAIL_SKIP && n_phys > 0 ? n_phys - 1 : n_phys;
    return min(row_logical_pages(len, a.max_pages, a.lgs), phys_scan << a.lgs);
  } else {
    return scan_pages(a, COV ? row_logical_pages(len, a.max_pages, a.lgs) : row_pages(len, a.max_pages));
  }
}

// HIER: top-K over physical pages of 2^lgs logical pages (hierarchical paging): the workgroups scan
// logical pages and write each physical page's largest key; SPD_TAIL_SKIP skips the row's last
// physical page (the local window keeps it).
template <int D, int KVD, bool COV, int ITERS, bool HIER>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_kernel(ScoreArgs a) {
  const int tails = a.tail_mode == SPD_TAIL_REBUILD ? a.batch * a.num_kv_heads : 0;
  if ((int)blockIdx.x < tails) {  // the last page of (request, KV head) blockIdx.x
    const int b = (int)blockIdx.x / a.num_kv_heads, h = (int)blockIdx.x % a.num_kv_heads;
    const int len = a.seq_lens[b];
    const int n = row_pages(len, a.max_pages);
    const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
    if (n > 0 && ((a.dyn.mask >> h) & 1)) score_tail<D, KVD, COV>(a, bt_row, n, len, b, h, -1);
    else if (n > 0) rebuild_tail_page<D, KVD>(a, bt_row, n, len, b, h);
    return;
  }
  constexpr int PPB = ITERS * kScoreWaves * (kWave / ScoreTraits<D, KVD>::LPP);  // = a.pages_per_block
  const int k = (int)blockIdx.x - tails;
  ScanItem it;
  const bool found = scan_item<PPB>(a, k, it, [&](int len) { return scan_limit<COV, HIER>(a, len); });
  if (found) {
    const int32_t* bt_row = a.block_table + (size_t)it.b * a.max_pages;
    const int p_begin = it.blk * PPB;
    int raw[ITERS];
    load_block_table<D, KVD, kScoreWaves, ITERS>(bt_row, a.max_pages, p_begin, raw, HIER || COV ? a.lgs : 0);
    float* sc_row = a.scores + ((size_t)it.b * a.num_kv_heads + it.h) * a.max_pages;
    if constexpr (HIER) {
      const int n_phys = row_phys_pages(it.len, a.max_pages, a.lgs);
      const int phys_scan = a.tail_mode == SPD_TAIL_SKIP && n_phys > 0 ? n_phys - 1 : n_phys;
      score_block_topk_hier<D, KVD, kScoreWaves, ITERS>(a, raw, it.n_scan, phys_scan, it.b, it.h, p_begin, sc_row);
    } else if constexpr (COV) {
      score_block_ell<D, KVD, kScoreWaves, ITERS>(a, raw, it.n_scan, it.len, it.b, it.h, p_begin);
    } else {
      score_block_topk<D, KVD, kScoreWaves, ITERS>(a, raw, it.n_scan, it.b, it.h, p_begin, sc_row);
    }
  }
  // SPD_TAIL_SKIP: workgroup r < rows writes -inf for dynamic row r's skipped last page (after its
  // own scan, so the write adds no round trip before the loads)
  const int rows = a.batch * a.dyn.count;
  if (!COV && a.tail_mode == SPD_TAIL_SKIP && k < rows) {
    const int b = k / a.dyn.count, h = a.dyn.at(k % a.dyn.count);
    const int len = a.seq_lens[b];
    const int n = HIER ? row_phys_pages(len, a.max_pages, a.lgs) : row_pages(len, a.max_pages);
    if (n > 0 && threadIdx.x == 0) a.scores[((size_t)b * a.num_kv_heads + h) * a.max_pages + n - 1] = -INFINITY;
  }
}

// Coverage, second and third passes, over blocks of kSharePages (logical) pages of a row (one page
// per thread, so the exponentials of a row are spread over many workgroups):
//  * coverage_part_kernel: each block's (max, sum exp) of the log-masses, per head;
//  * coverage_share_kernel: wave 0 folds the row's block pairs into lse_g (fixed order) while
//    every thread reads its page's log-masses; then pi_bar_p = (1/G) sum_g exp(l_{g,p} - lse_g).
constexpr int kShareThreads = 1024;
constexpr int kSharePages = kShareThreads;
constexpr int kShareWaves = kShareThreads / kWave;

__host__ __device__ inline int share_blocks_per_row(int max_pages) { return (max_pages + kSharePages - 1) / kSharePages; }
// ... of a row of logical pages (hierarchical paging: 2^lgs per block-table slot)
__host__ __device__ inline int share_blocks_per_row(const ScoreArgs& a) { return share_blocks_per_row(a.max_pages << a.lgs); }

// Workgroup max and sum over kShareThreads lanes of four values per lane (every thread receives
// them); `red` holds one entry per wave and head.
__device__ __forceinline__ float block_max_f(float v, float (&red)[kShareWaves]) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  v = wave_max_f(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float r = wave_max_f(lane < kShareWaves ? red[lane] : -INFINITY);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum_f(float v, float (&red)[kShareWaves]) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  v = wave_sum_f(v);
  if (lane == 0) red[wave] = v;
  __syncthreads();
  const float r = wave_sum_f(lane < kShareWaves ? red[lane] : 0.f);
  __syncthreads();
  return r;
}

struct ShareRole {
  int b, h, part, n;
  size_t row;
};

__device__ __forceinline__ ShareRole share_role(const ScoreArgs& a) {
  const int bpr = share_blocks_per_row(a);
  const int row_dyn = blockIdx.x / bpr;
  ShareRole r;
  r.part = blockIdx.x % bpr;
  r.b = row_dyn / a.dyn.count;
  r.h = a.dyn.at(row_dyn % a.dyn.count);
  r.n = row_logical_pages(a.seq_lens[r.b], a.max_pages, a.lgs);
  r.row = (size_t)r.b * a.num_kv_heads + r.h;
  return r;
}

__global__ __launch_bounds__(kShareThreads) void coverage_part_kernel(ScoreArgs a) {
  __shared__ float red[kG][kShareWaves];
  const ShareRole r = share_role(a);
  if (r.part * kSharePages >= r.n) return;  // uniform: the block is past the row
  const int p = r.part * kSharePages + (int)threadIdx.x;
  const float4 l4 = p < r.n ? a.ell[r.row * ell_stride(a) + p]
                            : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  const float lg[kG] = {l4.x, l4.y, l4.z, l4.w};
  float2 out[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    const float M = block_max_f(lg[g], red[g]);
    const float e = (M == -INFINITY || lg[g] == -INFINITY) ? 0.f : expf(lg[g] - M);
    out[g] = make_float2(M, block_sum_f(e, red[g]));
  }
  if (threadIdx.x < kG) {
    float2 v = out[0];
#pragma unroll
    for (int g = 1; g < kG; ++g) v = (int)threadIdx.x == g ? out[g] : v;
    a.partials[(r.row * share_blocks_per_row(a) + r.part) * kG + threadIdx.x] = v;
  }
}

__global__ __launch_bounds__(kShareThreads) void coverage_share_kernel(ScoreArgs a) {
  __shared__ float lse_s[kG];
  const ShareRole r = share_role(a);
  const int lane = threadIdx.x % kWave;
  if (r.part * kSharePages >= r.n && r.part != 0) return;  // block 0 of an empty row still writes head_lse
  const int p = r.part * kSharePages + (int)threadIdx.x;
  float4 l4 = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
  if (p < r.n) l4 = a.ell[r.row * ell_stride(a) + p];
  if (threadIdx.x < kWave) {
    // the row's block pairs, lane k holding pair k (k, k + 64, ... folded in order first)
    const int nparts = (r.n + kSharePages - 1) / kSharePages;
    const float2* pr = a.partials + r.row * share_blocks_per_row(a) * kG;
    float m[kG], s[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      m[g] = -INFINITY;
      s[g] = 0.f;
    }
    for (int k = lane; k < nparts; k += kWave) {
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        const float2 v = pr[(size_t)k * kG + g];
        lse_combine(m[g], s[g], v.x, v.y);
      }
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const float M = wave_max_f(m[g]);
      const float S = wave_sum_f(m[g] == -INFINITY ? 0.f : s[g] * expf(m[g] - M));
      const float lse = M == -INFINITY ? -INFINITY : M + logf(S);
      if (lane == g) {
        lse_s[g] = lse;
        if (r.part == 0 && a.head_lse) a.head_lse[(size_t)r.b * a.num_q_heads + (size_t)r.h * kG + g] = lse;
      }
    }
  }
  __syncthreads();
  const float lse[kG] = {lse_s[0], lse_s[1], lse_s[2], lse_s[3]};
  if (a.lgs == 0) {
    if (p < r.n) a.scores[r.row * a.max_pages + p] = group_share(l4, lse);
    return;
  }
  // hierarchical paging: a page's share is the sum of its logical pages' shares (mass is additive);
  // the 2^lgs logical pages of a page are consecutive threads of one wave
  float v = p < r.n ? group_share(l4, lse) : 0.f;
  for (int o = 1; o < (1 << a.lgs); o <<= 1) v += __shfl_xor(v, o, kWave);
  const int j = p >> a.lgs;
  if ((p & ((1 << a.lgs) - 1)) == 0 && j < row_phys_pages(a.seq_lens[r.b], a.max_pages, a.lgs))
    a.scores[r.row * a.max_pages + j] = v;
}

void launch_coverage_shares(const ScoreArgs& a, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.batch * a.dyn.count);
  const dim3 share_grid(rows * (unsigned)share_blocks_per_row(a)), share_block(kShareThreads);
  hipLaunchKernelGGL(coverage_part_kernel, share_grid, share_block, 0, stream, a);
  hipLaunchKernelGGL(coverage_share_kernel, share_grid, share_block, 0, stream, a);
}

template <int D, int KVD, bool COV, int ITERS, bool HIER>
void launch_scan(const ScoreArgs& a, hipStream_t stream) {
  const unsigned tails = a.tail_mode == SPD_TAIL_REBUILD ? (unsigned)(a.batch * a.num_kv_heads) : 0u;
  const dim3 grid(tails + (unsigned)(a.batch * a.dyn.count) * (unsigned)a.blocks_per_row), block(kScoreWaves * kWave);
  hipLaunchKernelGGL((page_score_kernel<D, KVD, COV, ITERS, HIER>), grid, block, 0, stream, a);
}

int launch_page_score(const ScoreArgs& a, int head_dim, int kv_dtype, bool coverage, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.batch * a.dyn.count);
  const bool long_scan = score_iters((long long)rows * ((long long)a.max_pages << a.lgs)) == kScoreItersLong;
#define SPD_SCORE_LAUNCH(D, KVD, COV, HIER)                                                           \
  if (long_scan) launch_scan<D, KVD, COV, kScoreItersLong, HIER>(a, stream);                          \
  else launch_scan<D, KVD, COV, kScoreItersShort, HIER>(a, stream);
#define SPD_SCORE_CASE(D, KVD)                                                                  \
  if (head_dim == D && kv_dtype == KVD) {                                                       \
    if (coverage) {                                                                             \
      SPD_SCORE_LAUNCH(D, KVD, true, false)                                                     \
      launch_coverage_shares(a, stream);                                                        \
    } else if (a.lgs > 0) {                                                                     \
      SPD_SCORE_LAUNCH(D, KVD, false, true)                                                     \
    } else {                                                                                    \
      SPD_SCORE_LAUNCH(D, KVD, false, false)                                                    \
    }                                                                                           \
    return 0;                                                                                   \
  }
  SPD_SCORE_CASE(64, SPD_DTYPE_F16)
  SPD_SCORE_CASE(128, SPD_DTYPE_F16)
  SPD_SCORE_CASE(128, SPD_DTYPE_FP8_E4M3FN)
  SPD_SCORE_CASE(64, SPD_DTYPE_F32)
  SPD_SCORE_CASE(128, SPD_DTYPE_F32)
#undef SPD_SCORE_CASE
#undef SPD_SCORE_LAUNCH
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
