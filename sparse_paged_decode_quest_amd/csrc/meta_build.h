// Per-page channel-wise key min / max (LServe summary, "Hierarchical Paging": every
// logical page keeps k_min and k_max over its keys; "Key statistics storage and updating":
// the statistics of the page a new token lands in are refreshed as the token is appended).
//
// One wave per (request, logical page, KV head).  Lane l owns channels [l*CPL, (l+1)*CPL)
// of every token, so min / max over the page's valid tokens is lane-local: no cross-lane
// traffic, and the page's 16 token rows are 16 coalesced loads issued back to back.  Used by
// the meta-build kernel and by the selector's tail workgroups.
#pragma once

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

template <int D, int KVD>
struct MetaTraits;

template <int D> struct MetaTraits<D, SPD_DTYPE_F32> {
  static constexpr int CPL = D / kWave;
  using Out = float;
  __device__ static void load(const void* pool, size_t idx, float (&v)[CPL], float) {
    const float* p = reinterpret_cast<const float*>(pool) + idx;
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = p[c];
  }
  __device__ static void store(void* meta, size_t idx, const float (&lo)[CPL], const float (&hi)[CPL], int d) {
    float* m = reinterpret_cast<float*>(meta) + idx;
#pragma unroll
    for (int c = 0; c < CPL; ++c) { m[c] = lo[c]; m[d + c] = hi[c]; }
  }
};

template <int D> struct MetaTraits<D, SPD_DTYPE_F16> {
  static constexpr int CPL = D / kWave;
  __device__ static void load(const void* pool, size_t idx, float (&v)[CPL], float) {
    const __half* p = reinterpret_cast<const __half*>(pool) + idx;
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = __half2float(p[c]);
  }
  __device__ static void store(void* meta, size_t idx, const float (&lo)[CPL], const float (&hi)[CPL], int d) {
    __half* m = reinterpret_cast<__half*>(meta) + idx;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {  // exact: min / max of fp16 values
      m[c] = __float2half_rn(lo[c]);
      m[d + c] = __float2half_rn(hi[c]);
    }
  }
};

template <int D> struct MetaTraits<D, SPD_DTYPE_FP8_E4M3FN> {
  static constexpr int CPL = D / kWave;
  __device__ static void load(const void* pool, size_t idx, float (&v)[CPL], float scale) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(pool) + idx;
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = fp8_to_float(p[c]) * scale;  // exact in fp32
  }
  __device__ static void store(void* meta, size_t idx, const float (&lo)[CPL], const float (&hi)[CPL], int d) {
    uint16_t* m = reinterpret_cast<uint16_t*>(meta) + idx;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {  // outward: the stored box still contains every key
      m[c] = f32_to_f16_round_down(lo[c]);
      m[d + c] = f32_to_f16_round_up(hi[c]);
    }
  }
};

// Statistics of logical page p of request b (len tokens), KV head h, by the calling wave, read from
// the physical page that holds it (sub-page p mod 2^lgs of block-table slot p >> lgs) and stored at
// the request's logical page (meta_unit).  Pages whose block-table entry is outside the pool are
// left alone.
template <int D, int KVD>
__device__ __forceinline__ void build_page_meta(const MetaArgs& a, int b, int p, int h, int len) {
  using T = MetaTraits<D, KVD>;
  constexpr int CPL = T::CPL;
  const int lane = threadIdx.x % kWave;
  const int phys = a.block_table[(size_t)b * a.max_pages + (p >> a.lgs)];
  if (phys < 0 || phys >= a.num_pool_pages) return;
  const int valid = valid_in_page(len, p);
  const int c0 = lane * CPL;
  const size_t unit = head_unit(phys, a.num_kv_heads, h, a.lgs, p & ((1 << a.lgs) - 1));
  const size_t head_base = unit * kPage;
  // every token of the page is loaded at once (slots past `valid` are read but never used)
  float v[kPage][CPL];
#pragma unroll
  for (int t = 0; t < kPage; ++t) {
    float scale = 1.0f;
    if (KVD == SPD_DTYPE_FP8_E4M3FN) scale = half_bits_to_float(a.k_scale[head_base + t]);
    T::load(a.k_pool, (head_base + t) * D + c0, v[t], scale);
  }
  float lo[CPL], hi[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) { lo[c] = INFINITY; hi[c] = -INFINITY; }
#pragma unroll
  for (int t = 0; t < kPage; ++t) {
    const bool ok = t < valid;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      lo[c] = ok ? fminf(lo[c], v[t][c]) : lo[c];
      hi[c] = ok ? fmaxf(hi[c], v[t][c]) : hi[c];
    }
  }
  T::store(a.meta, meta_unit(b, h, p, a.num_kv_heads, a.max_pages, a.lgs) * 2 * D + c0, lo, hi, D);
}

// Moira page summary ("Page summaries and the mvar estimate"): channel-wise mean and variance of
// the page's valid keys, stored as bf16 ("Memory for page summaries").  Same work layout as the
// min / max: lane-local over the page's token rows, loaded at once.  The arithmetic is fp64 --
// the sum of up to 16 stored keys is exact there, so the mean is the correctly rounded mean, and
// the variance (mean squared deviation from it) carries only fp64 rounding -- and each value is
// rounded once, straight from fp64 to bf16: the stored summary is the exact statistic rounded to
// bf16, with no double rounding through fp32.
__device__ __forceinline__ uint16_t f64_to_bf16_rn(double x) {
  if (x != x) return 0x7fc0u;
  if (x == 0.0) return (uint16_t)(__double_as_longlong(x) >> 48);  // keeps the sign of zero
  int e;
  (void)frexp(x, &e);                         // x = m 2^e, 0.5 <= |m| < 1
  const double step = ldexp(1.0, max(e - 8, -133));  // 8 significant bits; bf16 subnormal step 2^-133
  const double r = rint(x / step) * step;     // ties to even
  if (fabs(r) > 3.3895313892515355e38) return x > 0 ? 0x7f80u : 0xff80u;  // past the largest finite bf16
  return (uint16_t)(__float_as_uint((float)r) >> 16);  // r is exact in bf16, hence in fp32
}

template <int D, int KVD>
__device__ __forceinline__ void build_page_stats(const MetaArgs& a, int b, int p, int h, int len) {
  using T = MetaTraits<D, KVD>;
  constexpr int CPL = T::CPL;
  const int lane = threadIdx.x % kWave;
  const int phys = a.block_table[(size_t)b * a.max_pages + (p >> a.lgs)];
  if (phys < 0 || phys >= a.num_pool_pages) return;
  const int valid = valid_in_page(len, p);
  if (valid <= 0) return;
  const int c0 = lane * CPL;
  const size_t unit = head_unit(phys, a.num_kv_heads, h, a.lgs, p & ((1 << a.lgs) - 1));
  const size_t head_base = unit * kPage;
  float v[kPage][CPL];
#pragma unroll
  for (int t = 0; t < kPage; ++t) {
    float scale = 1.0f;
    if (KVD == SPD_DTYPE_FP8_E4M3FN) scale = half_bits_to_float(a.k_scale[head_base + t]);
    T::load(a.k_pool, (head_base + t) * D + c0, v[t], scale);
  }
  uint16_t* m = reinterpret_cast<uint16_t*>(a.meta) + meta_unit(b, h, p, a.num_kv_heads, a.max_pages, a.lgs) * 2 * D + c0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    double sum = 0.0;
#pragma unroll
    for (int t = 0; t < kPage; ++t) sum += t < valid ? (double)v[t][c] : 0.0;
    const double mu = sum / valid;
    double sq = 0.0;
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      const double dv = (double)v[t][c] - mu;
      sq += t < valid ? dv * dv : 0.0;
    }
    m[c] = f64_to_bf16_rn(mu);
    m[D + c] = f64_to_bf16_rn(sq / valid);
  }
}

// build_page_meta for the head size and pool type given at run time (a.head_dim, a.kv_dtype).
__device__ __forceinline__ void build_page_meta_rt(const MetaArgs& a, int b, int p, int h, int len) {
#define SPD_META_RT(D, K) \
  if (a.head_dim == D && a.kv_dtype == K) return build_page_meta<D, K>(a, b, p, h, len);
  SPD_META_RT(64, SPD_DTYPE_F32)
  SPD_META_RT(128, SPD_DTYPE_F32)
  SPD_META_RT(64, SPD_DTYPE_F16)
  SPD_META_RT(128, SPD_DTYPE_F16)
  SPD_META_RT(64, SPD_DTYPE_FP8_E4M3FN)
  SPD_META_RT(128, SPD_DTYPE_FP8_E4M3FN)
#undef SPD_META_RT
}

}  // namespace spd
