// Page scores of T query tokens per request in one scan (several query tokens, top-K over 16-token
// pages).  LiteTopK, section 3.4 (LiteDSA): every draft token keeps its own candidate list, so each
// token row needs its own page scores; the tokens of a request share the cache and its key boxes,
// so the scan reads each (page, KV head) meta row once and bounds it against the T query groups
// (LServe summary, "Hierarchical Paging": S_j = sum_i max(q_i kmax_i, q_i kmin_i), then the max over
// the group).  The arithmetic per (page, token) is the single-query scorer's, so a token row's scores
// are bit for bit those of the scorer run on that row alone.
//
// Work layout: the single-query scorer's (score_common.h) over the pages of the longest token row
// (the last token, length L); lanes hold the T query groups in registers.  Token t (length
// L - T + 1 + t) gets the scores of its own pages only.  Every wave reads its query groups from L2;
// staging them through LDS once per workgroup (one copy, one barrier) measured slower.
#include "mq_score.h"
#include "score_common.h"

namespace spd {

// Pages the scan covers in a request of `len` tokens: its last token's row, less the request's last
// two pages with SPD_TAIL_SKIP.  Each token row's last page is one of those two (T <= 4 draft tokens
// lie within 16 positions), so both are in every token's local window of at least two pages or past
// the token's length; the kernel writes -inf for them where a token sees them.
__device__ __forceinline__ int mq_scan_pages(const ScoreArgs& a, int len) {
  const int n = row_pages(len, a.max_pages);
  return a.tail_mode == SPD_TAIL_SKIP ? max(n - 2, 0) : n;
}

// The pages [p_begin, p_begin + PPB) of work item `item` (score_common.h's numbering) for every token row.
template <int D, int KVD, int ITERS>
__device__ __forceinline__ void mq_score_item(const ScoreArgs& a, int num_tokens, const ScanItem& item, int p_begin) {
  using T = ScoreTraits<D, KVD>;
  constexpr int LPP = T::LPP;
  const int b = item.b, h = item.h, len = item.len, n_scan = item.n_scan;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  int raw[ITERS];
  load_block_table<D, KVD, kScoreWaves, ITERS>(bt_row, a.max_pages, p_begin, raw);

  const int lane = threadIdx.x % kWave;
  const int sub = lane % LPP;
  const int c0 = sub * T::CW;
  int pg[ITERS];
  bool ok[ITERS];
  typename T::M m[ITERS];
  // the key boxes' addresses need no block-table entry: they are requested at once, and the entries
  // only mark pages outside the pool afterwards
#pragma unroll
  for (int it = 0; it < ITERS; ++it) pg[it] = score_page<D, KVD, kScoreWaves>(p_begin, it);
  load_boxes<D, KVD, ITERS>(a, b, h, pg, c0, m);
  // the query groups after the key boxes, unconditionally (token indices clamped to the last token)
  typename T::Q qr[kMqScoreMaxTokens];
#pragma unroll
  for (int t = 0; t < kMqScoreMaxTokens; ++t) {
    const int tt = min(t, num_tokens - 1);
    T::load_q(qr[t], a.q, (((size_t)b * num_tokens + tt) * a.num_q_heads + (size_t)h * kG) * D, c0);
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) ok[it] = pg[it] < n_scan && raw[it] >= 0 && raw[it] < a.num_pool_pages;
  if constexpr (LPP == 16 && kMqScoreMaxTokens == 4) {
    // The 16 sums (token t, head g) of a page live spread over its 16 lanes.  A reduce-scatter hands
    // lane l the whole sum of k = l = 4 t + g: at each level (lane bit 1, 2, 4, 8) a lane keeps the half
    // of its partial sums whose index bit equals its lane bit and adds the partner's partials of that
    // half.  The pairs added are the butterfly's (group_sum), so the sums are bit for bit the same.
    const bool b0 = sub & 1, b1 = sub & 2, b2 = sub & 4, b3 = sub & 8;
    const int t_l = sub >> 2;
    const int n_tl = min(row_pages(len - num_tokens + 1 + t_l, a.max_pages), n_scan);
    float* sc_l = a.scores + (((size_t)b * num_tokens + min(t_l, num_tokens - 1)) * a.num_kv_heads + h) * a.max_pages;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      // a page outside the row or the pool is bounded all the same (its box is read in bounds) and its
      // sums stay within its own 16 lanes; its result is replaced by -inf below
      float v[16];
#pragma unroll
      for (int t = 0; t < kMqScoreMaxTokens; ++t) {
        float st[kG];
        T::bound(qr[t], m[it], st);
#pragma unroll
        for (int g = 0; g < kG; ++g) v[t * kG + g] = st[g];
      }
      float u[8], w[4], x[2];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float keep = b0 ? v[2 * j + 1] : v[2 * j], send = b0 ? v[2 * j] : v[2 * j + 1];
        u[j] = keep + __uint_as_float(dpp<0xb1>(__float_as_uint(send)));  // lane ^ 1
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float keep = b1 ? u[2 * j + 1] : u[2 * j], send = b1 ? u[2 * j] : u[2 * j + 1];
        w[j] = keep + __uint_as_float(dpp<0x4e>(__float_as_uint(send)));  // lane ^ 2
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float keep = b2 ? w[2 * j + 1] : w[2 * j], send = b2 ? w[2 * j] : w[2 * j + 1];
        x[j] = keep + __shfl_xor(send, 4, kWave);
      }
      const float y = (b3 ? x[1] : x[0]) + __shfl_xor(b3 ? x[0] : x[1], 8, kWave);
      // largest over the group: the four lanes of token t_l
      float mx = fmaxf(y, __uint_as_float(dpp<0xb1>(__float_as_uint(y))));
      mx = fmaxf(mx, __uint_as_float(dpp<0x4e>(__float_as_uint(mx))));
      if ((sub & 3) == 0 && t_l < num_tokens && pg[it] < n_tl) sc_l[pg[it]] = ok[it] ? mx : -INFINITY;
    }
    return;
  }
#pragma unroll
  for (int t = 0; t < kMqScoreMaxTokens; ++t) {
    if (t >= num_tokens) break;
    const int n_t = min(row_pages(len - num_tokens + 1 + t, a.max_pages), n_scan);
    float* sc_row = a.scores + (((size_t)b * num_tokens + t) * a.num_kv_heads + h) * a.max_pages;
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      float s[kG];
      if (ok[it]) T::bound(qr[t], m[it], s);
      else {
#pragma unroll
        for (int g = 0; g < kG; ++g) s[g] = 0.f;
      }
#pragma unroll
      for (int g = 0; g < kG; ++g) s[g] = group_sum<LPP>(s[g]);
      if (sub == 0 && pg[it] < n_t) sc_row[pg[it]] = ok[it] ? topk_score(s) : -INFINITY;
    }
  }
}

template <int D, int KVD, int ITERS>
__global__ __launch_bounds__(kScoreWaves * kWave) void mq_page_score_kernel(ScoreArgs a, int num_tokens) {
  constexpr int PPB = ITERS * kScoreWaves * (kWave / ScoreTraits<D, KVD>::LPP);  // = a.pages_per_block
  const int k = (int)blockIdx.x;
  ScanItem it;
  if (scan_item<PPB>(a, k, it, [&](int len) { return mq_scan_pages(a, len); }))
    mq_score_item<D, KVD, ITERS>(a, num_tokens, it, it.blk * PPB);
  // SPD_TAIL_SKIP: workgroup r < rows writes -inf for dynamic row r's skipped pages, where a token sees
  // them (after its own scan, so the writes add no round trip before the loads)
  if (a.tail_mode == SPD_TAIL_SKIP && k < a.batch * a.dyn.count && (int)threadIdx.x < 2 * num_tokens) {
    const int b = k / a.dyn.count, h = a.dyn.at(k % a.dyn.count);
    const int len = a.seq_lens[b];
    const int t = (int)threadIdx.x >> 1, p = mq_scan_pages(a, len) + ((int)threadIdx.x & 1);
    if (p < row_pages(len - num_tokens + 1 + t, a.max_pages))
      a.scores[(((size_t)b * num_tokens + t) * a.num_kv_heads + h) * a.max_pages + p] = -INFINITY;
  }
}

int launch_mq_page_score(const ScoreArgs& a, int num_tokens, int head_dim, int kv_dtype, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.batch * a.dyn.count);
  const dim3 grid(rows * (unsigned)a.blocks_per_row), block(kScoreWaves * kWave);
  const bool long_scan = score_iters((long long)rows * a.max_pages) == kScoreItersLong;
#define SPD_MQ_SCORE_CASE(D, KVD)                                                                                     \
  if (head_dim == D && kv_dtype == KVD) {                                                                             \
    if (long_scan) hipLaunchKernelGGL((mq_page_score_kernel<D, KVD, kScoreItersLong>), grid, block, 0, stream, a, num_tokens); \
    else hipLaunchKernelGGL((mq_page_score_kernel<D, KVD, kScoreItersShort>), grid, block, 0, stream, a, num_tokens);  \
    return 0;                                                                                                         \
  }
  SPD_MQ_SCORE_CASE(64, SPD_DTYPE_F16)
  SPD_MQ_SCORE_CASE(128, SPD_DTYPE_F16)
  SPD_MQ_SCORE_CASE(128, SPD_DTYPE_FP8_E4M3FN)
  SPD_MQ_SCORE_CASE(64, SPD_DTYPE_F32)
  SPD_MQ_SCORE_CASE(128, SPD_DTYPE_F32)
#undef SPD_MQ_SCORE_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
