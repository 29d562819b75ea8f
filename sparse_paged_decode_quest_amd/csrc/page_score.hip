// Page scores from the per-page key box (LServe summary, "Hierarchical Paging", page
// importance S_j = sum_i max(q_i kmax_i, q_i kmin_i): an upper bound on q.k over every key
// of the page, two dot products per page).
//
// Because kmax >= kmin channel-wise, max(q kmax, q kmin) is q kmax where q >= 0 and q kmin
// where q < 0, so each term is one sign-selected operand and one multiply-add.
//
// Layout: LPP lanes cover one page's [2, d] meta row with 16-byte loads (f16 d=128: 16
// lanes, 4 pages per wave instruction).  Each lane owns CW channels of the page and keeps
// the matching query channels of the G heads in registers; partial sums are reduced across
// the LPP lanes with xor shuffles.
//
// Top-K mode writes score_p = max_g S_{g,p}.  Coverage mode (Moira, section 3.2 and
// Algorithm 1, "group-mean mass") writes the log-mass l_{g,p} = s S_{g,p} + ln(valid_p)
// and per-block (max, sum exp) pairs; a second kernel merges the pairs of the row into
// the per-head log-sum-exp and writes pi_bar_p = (1/G) sum_g exp(l_{g,p} - lse_g).
#include "score_common.h"
#include "spd_launch.h"

namespace spd {

template <int D, int QD, int MD>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_topk_kernel(ScoreArgs a) {
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const int p_begin = blk * a.pages_per_block;
  const int p_end = min(n, p_begin + a.pages_per_block);
  score_block_topk<D, QD, MD, kScoreWaves, kScoreIters>(a, b, h, p_begin, p_end,
                              a.scores + ((size_t)b * a.num_kv_heads + h) * a.max_pages);
}

// Coverage, first pass: log-masses l_{g,p} and one (max, sum exp) pair per head and block.
template <int D, int QD, int MD>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_coverage_kernel(ScoreArgs a) {
  constexpr int LPP = ScoreTraits<D, QD, MD>::LPP;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int row_dyn = blockIdx.x / a.blocks_per_row;
  const int blk = blockIdx.x % a.blocks_per_row;
  const int b = row_dyn / a.dyn.count;
  const int h = a.dyn.head[row_dyn % a.dyn.count];
  const int len = a.seq_lens[b];
  const int n = row_pages(len, a.max_pages);
  const int p_begin = blk * a.pages_per_block;
  const int p_end = min(n, p_begin + a.pages_per_block);
  const size_t row = (size_t)b * a.num_kv_heads + h;
  if (p_begin >= p_end) return;  // uniform over the block

  float lm[kG], ls[kG];  // running (max, sum exp) of this lane's pages
#pragma unroll
  for (int g = 0; g < kG; ++g) { lm[g] = -INFINITY; ls[g] = 0.f; }
  score_block<D, QD, MD, kScoreWaves, kScoreIters>(a, b, h, p_begin, p_end, [&](int p, bool ok, const float (&s)[kG]) {
    if (p >= p_end) return;
    const int valid = valid_in_page(len, p);
    const float lv = valid == kPage ? 2.772588722239781f : logf((float)valid);  // ln(valid)
    float lg[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      lg[g] = ok ? fmaf(a.sm_scale, s[g], lv) : -INFINITY;
      lse_push(lm[g], ls[g], lg[g]);
    }
    *reinterpret_cast<float4*>(a.ell + (row * a.max_pages + p) * kG) = make_float4(lg[0], lg[1], lg[2], lg[3]);
  });
  // block partial: fold the lanes that own pages (sub == 0), then the four waves in order
  __shared__ float sm[kScoreWaves][kG], ss[kScoreWaves][kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    for (int o = LPP; o < kWave; o <<= 1) {
      float m2 = __shfl_xor(lm[g], o, kWave), s2 = __shfl_xor(ls[g], o, kWave);
      lse_combine(lm[g], ls[g], m2, s2);
    }
    if (lane == 0) { sm[wave][g] = lm[g]; ss[wave][g] = ls[g]; }
  }
  __syncthreads();
  if (threadIdx.x < kG) {
    const int g = threadIdx.x;
    float m = sm[0][g], s = ss[0][g];
    for (int w = 1; w < kScoreWaves; ++w) lse_combine(m, s, sm[w][g], ss[w][g]);
    a.partials[(row * a.blocks_per_row + blk) * kG + g] = make_float2(m, s);
  }
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
  __shared__ float lse_s[kG];
  if (threadIdx.x < kWave) {
    // lanes 0..63 fold the row's block partials in a fixed order, then a fixed butterfly
    const int lane = threadIdx.x;
    float m[kG], s[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) { m[g] = -INFINITY; s[g] = 0.f; }
    for (int k = lane; k < used; k += kWave)
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        float2 pr = a.partials[(row * a.blocks_per_row + k) * kG + g];
        lse_combine(m[g], s[g], pr.x, pr.y);
      }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      for (int o = 1; o < kWave; o <<= 1) {
        float m2 = __shfl_xor(m[g], o, kWave), s2 = __shfl_xor(s[g], o, kWave);
        lse_combine(m[g], s[g], m2, s2);
      }
      if (lane == 0) lse_s[g] = m[g] == -INFINITY ? -INFINITY : m[g] + logf(s[g]);
    }
  }
  __syncthreads();
  float lse[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) lse[g] = lse_s[g];
  if (blk == 0 && threadIdx.x < kG && a.head_lse)
    a.head_lse[(size_t)b * a.num_q_heads + (size_t)h * kG + threadIdx.x] = lse[threadIdx.x];
  for (int p = p_begin + threadIdx.x; p < p_end; p += blockDim.x) {
    const float4 l4 = *reinterpret_cast<const float4*>(a.ell + (row * a.max_pages + p) * kG);
    const float lg[kG] = {l4.x, l4.y, l4.z, l4.w};
    float acc = 0.f;
#pragma unroll
    for (int g = 0; g < kG; ++g)
      if (lg[g] != -INFINITY) acc += expf(lg[g] - lse[g]);
    a.scores[row * a.max_pages + p] = acc * (1.0f / kG);
  }
}

int launch_page_score(const ScoreArgs& a, int head_dim, int q_dtype, int meta_dtype, bool coverage,
                      hipStream_t stream) {
  dim3 grid((unsigned)(a.batch * a.dyn.count * a.blocks_per_row)), block(kScoreWaves * kWave);
#define SPD_SCORE_CASE(D, QD, MD)                                                              \
  if (head_dim == D && q_dtype == QD && meta_dtype == MD) {                                    \
    if (coverage) {                                                                            \
      hipLaunchKernelGGL((page_score_coverage_kernel<D, QD, MD>), grid, block, 0, stream, a);  \
      hipLaunchKernelGGL(coverage_share_kernel, grid, block, 0, stream, a);                    \
    } else {                                                                                   \
      hipLaunchKernelGGL((page_score_topk_kernel<D, QD, MD>), grid, block, 0, stream, a);      \
    }                                                                                          \
    return 0;                                                                                  \
  }
  SPD_SCORE_CASE(64, SPD_DTYPE_F16, SPD_DTYPE_F16)
  SPD_SCORE_CASE(128, SPD_DTYPE_F16, SPD_DTYPE_F16)
  SPD_SCORE_CASE(64, SPD_DTYPE_F32, SPD_DTYPE_F32)
  SPD_SCORE_CASE(128, SPD_DTYPE_F32, SPD_DTYPE_F32)
#undef SPD_SCORE_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
