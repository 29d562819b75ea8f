// Coverage log-masses from Moira's page summaries (section 3.1, "Page summaries and the mvar
// estimate", Eq. 2).  With mu_P and sigma^2_P the channel-wise mean and variance of the keys of
// page P (bf16, built by the stats variant of the page-meta kernel) and s the softmax scale,
//
//   l_{g,P} = s q_g . mu_P + (1/2) (s q_g)^2 . sigma^2_P + ln(tokens of P),
//
// the logarithm of the token count times the expectation of exp(s q_g . k) for keys drawn as
// independent Gaussians per channel.  The row's first page (the attention sink) and its current
// page are not estimated: one more workgroup per dynamic row computes their exact log-mass,
// log sum_{k in P} exp(s q_g . k), from the K pool, and with SPD_TAIL_REBUILD also writes the
// current page's summary.  The shares follow from the log-masses as for the key-box bound
// (Moira, section 3.2, Eq. 3).
//
// Scan layout: a page's summary is [2, d] bf16 (512 bytes at d = 128, the size of the f16 key
// box), read by LPP lanes with 16-byte loads, ITERS page groups per lane issued before any
// arithmetic (the bound scorer's layout).  Each lane keeps a_c = s q_c and b_c = a_c^2 / 2 of its
// 8 channels for the group's heads in fp32, so a page costs two fma per channel and head.
#include "meta_build.h"
#include "score_common.h"
#include "spd_launch.h"

namespace spd {

template <int D, int KVD>
struct MvarTraits {
  static constexpr int CW = 8;          // channels per lane (one 16-byte bf16 load per statistic)
  static constexpr int LPP = D / CW;    // lanes per page summary, and per key row of a page
  static constexpr int PPI = kWave / LPP;
  struct Q {
    float a[kG][CW], b[kG][CW];
  };
  struct M {
    uint4 mu, var;
  };

  // a = s q and b = (s q)^2 / 2 for channels [c0, c0 + 8) of the group's heads (q is f32 for f32
  // pools, f16 otherwise).
  __device__ static void load_q(Q& qr, const void* q, size_t base, int c0, float s) {
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float v[CW];
      if constexpr (KVD == SPD_DTYPE_F32) {
        const float* qp = reinterpret_cast<const float*>(q) + base + (size_t)g * D + c0;
        const float4 w0 = *reinterpret_cast<const float4*>(qp), w1 = *reinterpret_cast<const float4*>(qp + 4);
        v[0] = w0.x; v[1] = w0.y; v[2] = w0.z; v[3] = w0.w;
        v[4] = w1.x; v[5] = w1.y; v[6] = w1.z; v[7] = w1.w;
      } else {
        const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + base + (size_t)g * D + c0;
        const uint4 w = *reinterpret_cast<const uint4*>(qp);
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __half2 h = __builtin_bit_cast(__half2, ws[i]);
          v[2 * i] = __low2float(h);
          v[2 * i + 1] = __high2float(h);
        }
      }
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        qr.a[g][c] = s * v[c];
        qr.b[g][c] = 0.5f * qr.a[g][c] * qr.a[g][c];
      }
    }
  }

  __device__ static void load_m(M& m, const void* stats, size_t row, int c0) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(stats) + row + c0;
    m.mu = ld_stream(reinterpret_cast<const uint4*>(base));
    m.var = ld_stream(reinterpret_cast<const uint4*>(base + D));
  }

  // This lane's part of a_g . mu + b_g . sigma^2 for each head g.
  __device__ static void mass(const Q& qr, const M& m, float (&s)[kG]) {
    const uint32_t mu[4] = {m.mu.x, m.mu.y, m.mu.z, m.mu.w};
    const uint32_t var[4] = {m.var.x, m.var.y, m.var.z, m.var.w};
    float mf[CW], vf[CW];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mf[2 * i] = bf16_lo(mu[i]);
      mf[2 * i + 1] = bf16_hi(mu[i]);
      vf[2 * i] = bf16_lo(var[i]);
      vf[2 * i + 1] = bf16_hi(var[i]);
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CW; ++c) {
        acc = fmaf(qr.a[g][c], mf[c], acc);
        acc = fmaf(qr.b[g][c], vf[c], acc);
      }
      s[g] = acc;
    }
  }

  // Channels [c0, c0 + 8) of token t of a (page, KV head) of the K pool, as fp32 (exact).
  __device__ static void load_key(float (&k)[CW], const void* k_pool, const uint16_t* k_scale, size_t head_page,
                                  int t, int c0) {
    const size_t off = (head_page * kPage + t) * D + c0;
    if constexpr (KVD == SPD_DTYPE_F32) {
      const float* kp = reinterpret_cast<const float*>(k_pool) + off;
      const float4 w0 = *reinterpret_cast<const float4*>(kp), w1 = *reinterpret_cast<const float4*>(kp + 4);
      k[0] = w0.x; k[1] = w0.y; k[2] = w0.z; k[3] = w0.w;
      k[4] = w1.x; k[5] = w1.y; k[6] = w1.z; k[7] = w1.w;
    } else if constexpr (KVD == SPD_DTYPE_F16) {
      const uint4 w = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(k_pool) + off);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const __half2 h = __builtin_bit_cast(__half2, ws[i]);
        k[2 * i] = __low2float(h);
        k[2 * i + 1] = __high2float(h);
      }
    } else {  // fp8 code times the token's scale
      const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(k_pool) + off);
      const float sc = half_bits_to_float(k_scale[head_page * kPage + t]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        k[i] = fp8_to_float((w.x >> (8 * i)) & 0xffu) * sc;
        k[4 + i] = fp8_to_float((w.y >> (8 * i)) & 0xffu) * sc;
      }
    }
  }
};

__device__ __forceinline__ float ln_tokens(int valid) {
  return valid == kPage ? 2.772588722239781f : logf((float)valid);  // ln 16 for a full page
}

// Estimated log-masses of the workgroup's pages in [1, n_est) (pages 0 and n_est = n - 1 are the
// exact workgroup's).  raw holds the block-table entries of the lane's page groups.
template <int D, int KVD, int ITERS>
__device__ __forceinline__ void mvar_block_ell(const ScoreArgs& a, const int (&raw)[ITERS], int n_est, int len, int b,
                                               int h, int p_begin) {
  using T = MvarTraits<D, KVD>;
  constexpr int LPP = T::LPP;
  const int lane = threadIdx.x % kWave;
  const int wave = threadIdx.x / kWave;
  const int sub = lane % LPP;
  const int c0 = sub * T::CW;
  int pg[ITERS];
  bool ok[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    pg[it] = p_begin + (it * kScoreWaves + wave) * T::PPI + lane / LPP;
    ok[it] = pg[it] >= 1 && pg[it] < n_est && raw[it] >= 0 && raw[it] < a.num_pool_pages;
  }
  typename T::Q qr;
  T::load_q(qr, a.q, ((size_t)b * a.num_q_heads + (size_t)h * kG) * D, c0, a.sm_scale);
  // the summaries' addresses need no block-table entry, so they are requested without waiting for it
  // (a page past the row's summaries reads its last one, and its mass is discarded)
  typename T::M m[ITERS];
  const size_t base = meta_unit(b, h, 0, a.num_kv_heads, a.max_pages, a.lgs);
  const int last = (a.max_pages << a.lgs) - 1;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) T::load_m(m[it], a.meta, (base + min(pg[it], last)) * 2 * D, c0);
  const size_t row = (size_t)b * a.num_kv_heads + h;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    float s[kG];
    if (ok[it]) T::mass(qr, m[it], s);
    else {
#pragma unroll
      for (int g = 0; g < kG; ++g) s[g] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) s[g] = group_sum<LPP>(s[g]);
    if (sub == 0 && pg[it] >= 1 && pg[it] < n_est) {
      const float lv = ln_tokens(valid_in_page(len, pg[it]));
      a.ell[row * ell_stride(a) + pg[it]] =
          ok[it] ? make_float4(s[0] + lv, s[1] + lv, s[2] + lv, s[3] + lv)
                 : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);  // page outside the pool
    }
  }
}

// The exact workgroup of a dynamic row: thread (t, sub) holds channels [8 sub, 8 sub + 8) of token
// t (16 tokens x LPP lanes); the tokens' logits s q_g . k are summed over the LPP lanes, then
// log-sum-exp over the page's valid tokens, per wave and across the waves through LDS.  Pages 0
// and n - 1 (once when n = 1); a page outside the pool gets -inf.
template <int D, int KVD>
__device__ __forceinline__ void mvar_exact_pages(const ScoreArgs& a, const int32_t* bt_row, int b, int h) {
  using T = MvarTraits<D, KVD>;
  constexpr int LPT = T::LPP;
  static_assert(kPage * LPT <= kScoreWaves * kWave, "one token row per LPT threads");
  __shared__ float red_m[kScoreWaves][kG], red_s[kScoreWaves][kG];
  const int len = a.seq_lens[b];
  const int n = row_logical_pages(len, a.max_pages, a.lgs);  // 16-token pages (hierarchical paging too)
  if (n <= 0) return;  // uniform
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int t = threadIdx.x / LPT, sub = threadIdx.x % LPT;
  const int c0 = sub * T::CW;
  const size_t row = (size_t)b * a.num_kv_heads + h;
  typename T::Q qr;
  T::load_q(qr, a.q, ((size_t)b * a.num_q_heads + (size_t)h * kG) * D, c0, a.sm_scale);
  const int pages = n > 1 ? 2 : 1;
  for (int k = 0; k < pages; ++k) {
    const int p = k == 0 ? 0 : n - 1;
    const int phys = bt_row[p >> a.lgs];
    const bool tok = phys >= 0 && phys < a.num_pool_pages && t < valid_in_page(len, p);
    float x[kG];
    if (tok) {
      float kv[T::CW];
      T::load_key(kv, a.k_pool, a.k_scale, head_unit(phys, a.num_kv_heads, h, a.lgs, p & ((1 << a.lgs) - 1)), t, c0);
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < T::CW; ++c) acc = fmaf(qr.a[g][c], kv[c], acc);
        x[g] = acc;
      }
    } else {
#pragma unroll
      for (int g = 0; g < kG; ++g) x[g] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float xg = group_sum<LPT>(x[g]);  // every lane takes part; lanes without a token hold 0
      xg = tok ? xg : -INFINITY;
      const float M = wave_max_f(xg);
      const float S = wave_sum_f(sub == 0 && xg != -INFINITY ? expf(xg - M) : 0.f);
      if (lane == 0) {
        red_m[wave][g] = M;
        red_s[wave][g] = S;
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float lg[kG];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        float m = -INFINITY, s = 0.f;
        for (int w = 0; w < kScoreWaves; ++w) lse_combine(m, s, red_m[w][g], red_s[w][g]);
        lg[g] = m == -INFINITY ? -INFINITY : m + logf(s);
      }
      a.ell[row * ell_stride(a) + p] = make_float4(lg[0], lg[1], lg[2], lg[3]);
    }
    __syncthreads();
  }
  if (a.tail_mode == SPD_TAIL_REBUILD && wave == 0) {  // the current page's summary, for later steps
    MetaArgs m{};
    m.k_pool = a.k_pool;
    m.k_scale = a.k_scale;
    m.block_table = a.block_table;
    m.seq_lens = a.seq_lens;
    m.meta = a.meta_out;
    m.num_kv_heads = a.num_kv_heads;
    m.max_pages = a.max_pages;
    m.num_pool_pages = a.num_pool_pages;
    m.lgs = a.lgs;
    build_page_stats<D, KVD>(m, b, n - 1, h, len);
  }
}

// The grid starts with the exact workgroups, one per dynamic row, so their dependent reads (length,
// block table, keys) run beside the estimate instead of after it; the estimate workgroups then take the
// numbered work items of score_common.h (scan_item) over each row's pages [0, n - 1) (page 0, the
// exact sink, is left out inside).
template <int D, int KVD, int ITERS>
__global__ __launch_bounds__(kScoreWaves * kWave) void page_score_mvar_kernel(ScoreArgs a) {
  using T = MvarTraits<D, KVD>;
  constexpr int PPB = ITERS * kScoreWaves * T::PPI;  // = a.pages_per_block
  const int rows = a.batch * a.dyn.count;
  if ((int)blockIdx.x < rows) {
    const int b = (int)blockIdx.x / a.dyn.count;
    const int h = a.dyn.at((int)blockIdx.x % a.dyn.count);
    mvar_exact_pages<D, KVD>(a, a.block_table + (size_t)b * a.max_pages, b, h);
    return;
  }
  ScanItem it;
  if (!scan_item<PPB>(a, (int)blockIdx.x - rows, it,
                      [&](int len) { return max(row_logical_pages(len, a.max_pages, a.lgs) - 1, 0); }))
    return;
  const int32_t* bt_row = a.block_table + (size_t)it.b * a.max_pages;
  const int p_begin = it.blk * PPB;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  int raw[ITERS];  // block-table entries (clamped into the row)
#pragma unroll
  for (int i = 0; i < ITERS; ++i)
    raw[i] = bt_row[min((p_begin + (i * kScoreWaves + wave) * T::PPI + lane / T::LPP) >> a.lgs, a.max_pages - 1)];
  mvar_block_ell<D, KVD, ITERS>(a, raw, it.n_scan, it.len, it.b, it.h, p_begin);
}

int launch_page_score_mvar(const ScoreArgs& a, int head_dim, int kv_dtype, hipStream_t stream) {
  const unsigned rows = (unsigned)(a.batch * a.dyn.count);
  const dim3 grid(rows * (unsigned)(a.blocks_per_row + 1)), block(kScoreWaves * kWave);
  const bool long_scan = score_iters((long long)rows * ((long long)a.max_pages << a.lgs)) == kScoreItersLong;
#define SPD_MVAR_CASE(D, KVD)                                                                                        \
  if (head_dim == D && kv_dtype == KVD) {                                                                            \
    if (long_scan) hipLaunchKernelGGL((page_score_mvar_kernel<D, KVD, kScoreItersLong>), grid, block, 0, stream, a);  \
    else hipLaunchKernelGGL((page_score_mvar_kernel<D, KVD, kScoreItersShort>), grid, block, 0, stream, a);           \
    launch_coverage_shares(a, stream);                                                                               \
    return 0;                                                                                                        \
  }
  SPD_MVAR_CASE(64, SPD_DTYPE_F16)
  SPD_MVAR_CASE(128, SPD_DTYPE_F16)
  SPD_MVAR_CASE(128, SPD_DTYPE_FP8_E4M3FN)
  SPD_MVAR_CASE(64, SPD_DTYPE_F32)
  SPD_MVAR_CASE(128, SPD_DTYPE_F32)
#undef SPD_MVAR_CASE
  return SPD_ERR_UNSUPPORTED;
}

}  // namespace spd
