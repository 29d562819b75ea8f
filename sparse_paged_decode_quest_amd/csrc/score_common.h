// Page-bound arithmetic shared by the scorer and the fused score + select kernel.
//
// LServe summary, "Hierarchical Paging": S_j = sum_i max(q_i kmax_i, q_i kmin_i).  With
// kmax >= kmin channel-wise the larger product is q kmax where q >= 0 and q kmin where
// q < 0, so each term is one sign-selected operand and one multiply-add.
//
// Work layout: LPP lanes cover one page's [2, d] meta row with 16-byte loads (f16 d = 128:
// 16 lanes, PPI = 4 pages per wave instruction).  A workgroup of NW waves owns
// ITERS * NW * PPI consecutive pages; every lane first loads the block-table entries of all
// its pages, then issues all of its meta loads, and only then computes, so each wave keeps
// ITERS * 32 bytes per lane in flight instead of walking pages one dependent load at a time.
#pragma once

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

constexpr int kG = 4;  // query heads per KV head (the compiled GQA group)
constexpr int kScoreWaves = 4, kScoreIters = 4;  // standalone scorer: 4 waves x 4 page groups
constexpr int kFusedWaves = 16, kFusedIters = 2;  // fused scorer (its last block selects)

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <int D, int QD, int MD>
struct ScoreTraits;

// f16 query, f16 meta: packed sign-select + v_dot2_f32_f16.
template <int D>
struct ScoreTraits<D, SPD_DTYPE_F16, SPD_DTYPE_F16> {
  static constexpr int CW = 8;                   // channels per 16-byte load
  static constexpr int LPP = D * 2 / 16;         // lanes per page
  struct Q {
    uint32_t h[kG][CW / 2];    // query pairs
    uint32_t pos[kG][CW / 2];  // 0xffff per half where q >= 0
  };
  struct M {
    uint4 mn, mx;
  };
  __device__ static void load_q(Q& qr, const void* q, size_t base, int c0) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + base;
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int i = 0; i < CW / 2; ++i) {
        uint16_t lo = qp[(size_t)g * D + c0 + 2 * i], hi = qp[(size_t)g * D + c0 + 2 * i + 1];
        qr.h[g][i] = (uint32_t)lo | ((uint32_t)hi << 16);
        qr.pos[g][i] = ((lo & 0x8000u) ? 0u : 0xffffu) | ((hi & 0x8000u) ? 0u : 0xffff0000u);
      }
  }
  __device__ static void load_m(M& m, const void* meta, size_t row, int c0) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(meta) + row + c0;
    m.mn = *reinterpret_cast<const uint4*>(base);
    m.mx = *reinterpret_cast<const uint4*>(base + D);
  }
  __device__ static void bound(const Q& qr, const M& m, float (&s)[kG]) {
    const uint32_t lo[4] = {m.mn.x, m.mn.y, m.mn.z, m.mn.w};
    const uint32_t hi[4] = {m.mx.x, m.mx.y, m.mx.z, m.mx.w};
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t sel = (hi[i] & qr.pos[g][i]) | (lo[i] & ~qr.pos[g][i]);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, sel), __builtin_bit_cast(h2_t, qr.h[g][i]), acc, false);
      }
      s[g] = acc;
    }
  }
};

// f32 query, f32 meta.
template <int D>
struct ScoreTraits<D, SPD_DTYPE_F32, SPD_DTYPE_F32> {
  static constexpr int CW = 4;
  static constexpr int LPP = D * 4 / 16;
  struct Q {
    float v[kG][CW];
  };
  struct M {
    float4 mn, mx;
  };
  __device__ static void load_q(Q& qr, const void* q, size_t base, int c0) {
    const float* qp = reinterpret_cast<const float*>(q) + base;
#pragma unroll
    for (int g = 0; g < kG; ++g)
#pragma unroll
      for (int c = 0; c < CW; ++c) qr.v[g][c] = qp[(size_t)g * D + c0 + c];
  }
  __device__ static void load_m(M& m, const void* meta, size_t row, int c0) {
    const float* base = reinterpret_cast<const float*>(meta) + row + c0;
    m.mn = *reinterpret_cast<const float4*>(base);
    m.mx = *reinterpret_cast<const float4*>(base + D);
  }
  __device__ static void bound(const Q& qr, const M& m, float (&s)[kG]) {
    const float lo[4] = {m.mn.x, m.mn.y, m.mn.z, m.mn.w};
    const float hi[4] = {m.mx.x, m.mx.y, m.mx.z, m.mx.w};
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < CW; ++c) acc = fmaf(qr.v[g][c], qr.v[g][c] >= 0.f ? hi[c] : lo[c], acc);
      s[g] = acc;
    }
  }
};

// Pages per workgroup of NW waves with ITERS page groups each.
__host__ __device__ constexpr int score_pages_per_block(int d, int meta_bytes, int nw, int iters) {
  return iters * nw * (kWave / (d * meta_bytes / 16));
}

__device__ __forceinline__ void lse_push(float& m, float& s, float x) {
  if (x == -INFINITY) return;
  if (x > m) {
    s = s * expf(m - x) + 1.f;
    m = x;
  } else {
    s += expf(x - m);
  }
}

__device__ __forceinline__ void lse_combine(float& m, float& s, float m2, float s2) {
  if (m2 == -INFINITY) return;
  if (m == -INFINITY) { m = m2; s = s2; return; }
  float M = fmaxf(m, m2);
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

// Bounds S_{g,p} of the pages [p_begin, p_end) owned by this workgroup.  For each of the
// kScoreIters page groups of the calling lane, `fn(p, ok, s)` is called on lanes with
// sub == 0 after the LPP-lane reduction (p may be >= p_end: then ok is false and fn must
// ignore it).  Pages whose block-table entry is outside the pool have ok = false.
template <int D, int QD, int MD, int NW, int ITERS, typename F>
__device__ __forceinline__ void score_block(const ScoreArgs& a, int b, int h, int p_begin, int p_end, F&& fn) {
  using T = ScoreTraits<D, QD, MD>;
  constexpr int LPP = T::LPP;
  constexpr int PPI = kWave / LPP;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int sub = lane % LPP;
  const int slot = lane / LPP;
  const int c0 = sub * T::CW;
  typename T::Q qr;
  T::load_q(qr, a.q, ((size_t)b * a.num_q_heads + (size_t)h * kG) * D, c0);
  int pg[ITERS], phys[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    pg[it] = p_begin + (it * NW + wave) * PPI + slot;
    phys[it] = pg[it] < p_end ? a.block_table[(size_t)b * a.max_pages + pg[it]] : -1;
  }
  typename T::M m[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    if (phys[it] >= 0 && phys[it] < a.num_pool_pages)
      T::load_m(m[it], a.meta, ((size_t)phys[it] * a.num_kv_heads + h) * 2 * D, c0);
  }
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const bool ok = phys[it] >= 0 && phys[it] < a.num_pool_pages;
    float s[kG];
    if (ok) T::bound(qr, m[it], s);
    else {
#pragma unroll
      for (int g = 0; g < kG; ++g) s[g] = 0.f;
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) s[g] = xor_sum<LPP>(s[g]);
    if (sub == 0) fn(pg[it], ok && pg[it] < p_end, s);
  }
}

// Top-K scores of pages [p_begin, p_end) of row (b, h): score_p = max_g S_{g,p} (the group
// combine keeps the score an upper bound for every query head of the group); pages whose
// block-table entry is outside the pool score -inf.
template <int D, int QD, int MD, int NW, int ITERS>
__device__ __forceinline__ void score_block_topk(const ScoreArgs& a, int b, int h, int p_begin, int p_end,
                                                 float* row_scores) {
  if (p_begin >= p_end) return;
  score_block<D, QD, MD, NW, ITERS>(a, b, h, p_begin, p_end, [&](int p, bool ok, const float (&s)[kG]) {
    if (p >= p_end) return;
    float best = s[0];
#pragma unroll
    for (int g = 1; g < kG; ++g) best = fmaxf(best, s[g]);
    row_scores[p] = ok ? best : -INFINITY;
  });
}

}  // namespace spd
