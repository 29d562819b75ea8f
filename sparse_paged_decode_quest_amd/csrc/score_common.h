// Page-bound arithmetic shared by the scorer and the fused score + select kernel.
//
// LServe summary, "Hierarchical Paging": S_j = sum_i max(q_i kmax_i, q_i kmin_i).  With
// kmax >= kmin channel-wise the larger product is q kmax where q >= 0 and q kmin where
// q < 0, so each term is one sign-selected operand and one multiply-add.
//
// Work layout: LPP lanes cover one page's [2, d] meta row with 16-byte loads (f16 d = 128:
// 16 lanes, PPI = 4 pages per wave instruction).  A workgroup of NW waves owns
// ITERS * NW * PPI consecutive pages.  The block-table entries are loaded at the same time
// as the request's length (entries past the row end are read from inside the table row and
// ignored), then every meta load of the lane is issued before any arithmetic, so a lane keeps
// ITERS * 32 bytes in flight and the whole scan is two dependent memory round trips.
//
// The last page (LServe, "Key statistics storage and updating": the statistics of the page a
// new token lands in are updated as the token is appended).  With SPD_TAIL_REBUILD each dynamic
// row gets one more workgroup, which rebuilds the min / max of the row's last page from the K
// pool, writes them to the page meta and scores the page from those registers, while the
// regular workgroups score every other page.  With SPD_TAIL_SKIP (top-K) the page is not scored
// and its meta is not read, so a separate rebuild may run concurrently with the scorer.
#pragma once

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

constexpr int kG = 4;  // query heads per KV head (the compiled GQA group)

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));

template <int D, int KVD>
struct ScoreTraits;

// f16 query, f16 meta (f16 pools, and fp8 pools whose meta is f16 rounded outward):
// packed sign-select + v_dot2_f32_f16.
template <int D, int KVD>
struct ScoreTraitsF16 {
  static constexpr int CW = 8;            // channels per 16-byte meta load
  static constexpr int LPP = D * 2 / 16;  // lanes per page
  struct Q {
    uint32_t h[kG][CW / 2];  // query pairs
  };
  struct M {
    uint4 mn, mx;
  };
  __device__ static void load_q(Q& qr, const void* q, size_t base, int c0) {
    const uint16_t* qp = reinterpret_cast<const uint16_t*>(q) + base;
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const uint4 w = *reinterpret_cast<const uint4*>(qp + (size_t)g * D + c0);
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int i = 0; i < CW / 2; ++i) qr.h[g][i] = ws[i];
    }
  }
  __device__ static void load_m(M& m, const void* meta, size_t row, int c0) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(meta) + row + c0;
    m.mn = ld_stream(reinterpret_cast<const uint4*>(base));
    m.mx = ld_stream(reinterpret_cast<const uint4*>(base + D));
  }
  __device__ static void bound(const Q& qr, const M& m, float (&s)[kG]) {
    const uint32_t lo[4] = {m.mn.x, m.mn.y, m.mn.z, m.mn.w};
    const uint32_t hi[4] = {m.mx.x, m.mx.y, m.mx.z, m.mx.w};
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // per half: 0xffff where the query's sign bit is set (a packed arithmetic shift by 15), so kmin
        // is taken there and kmax elsewhere
        uint32_t neg;
        asm("v_pk_ashrrev_i16 %0, %1, %2" : "=v"(neg) : "s"(0x000f000fu), "v"(qr.h[g][i]));
        const uint32_t sel = (lo[i] & neg) | (hi[i] & ~neg);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, sel), __builtin_bit_cast(h2_t, qr.h[g][i]), acc, false);
      }
      s[g] = acc;
    }
  }
  // this lane's CW channels of the page's keys -> min / max (valid tokens only), stored and kept
  __device__ static void rebuild(M& m, const void* k_pool, const uint16_t* k_scale, size_t head_page, int valid,
                                 int c0, void* meta, size_t row) {
    float lo[CW], hi[CW];
#pragma unroll
    for (int c = 0; c < CW; ++c) {
      lo[c] = INFINITY;
      hi[c] = -INFINITY;
    }
    if constexpr (KVD == SPD_DTYPE_F16) {
      const uint16_t* kp = reinterpret_cast<const uint16_t*>(k_pool) + head_page * kPage * D + c0;
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        const uint4 t4 = *reinterpret_cast<const uint4*>(kp + (size_t)t * D);
        const uint32_t w[4] = {t4.x, t4.y, t4.z, t4.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __half2 h = __builtin_bit_cast(__half2, w[i]);
          const float v0 = __low2float(h), v1 = __high2float(h);
          if (t < valid) {
            lo[2 * i] = fminf(lo[2 * i], v0);
            hi[2 * i] = fmaxf(hi[2 * i], v0);
            lo[2 * i + 1] = fminf(lo[2 * i + 1], v1);
            hi[2 * i + 1] = fmaxf(hi[2 * i + 1], v1);
          }
        }
      }
    } else {  // fp8 codes times the token's scale, exact in fp32
      const uint8_t* kp = reinterpret_cast<const uint8_t*>(k_pool) + head_page * kPage * D + c0;
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        const uint2 t2 = *reinterpret_cast<const uint2*>(kp + (size_t)t * D);
        const float sc = half_bits_to_float(k_scale[head_page * kPage + t]);
        const float v[CW] = {fp8_to_float(t2.x & 0xffu) * sc,         fp8_to_float((t2.x >> 8) & 0xffu) * sc,
                             fp8_to_float((t2.x >> 16) & 0xffu) * sc, fp8_to_float(t2.x >> 24) * sc,
                             fp8_to_float(t2.y & 0xffu) * sc,         fp8_to_float((t2.y >> 8) & 0xffu) * sc,
                             fp8_to_float((t2.y >> 16) & 0xffu) * sc, fp8_to_float(t2.y >> 24) * sc};
        if (t < valid) {
#pragma unroll
          for (int c = 0; c < CW; ++c) {
            lo[c] = fminf(lo[c], v[c]);
            hi[c] = fmaxf(hi[c], v[c]);
          }
        }
      }
    }
    uint32_t plo[4], phi[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint16_t l0, l1, h0, h1;
      if constexpr (KVD == SPD_DTYPE_F16) {  // exact: min / max of fp16 values
        l0 = __half_as_ushort(__float2half_rn(lo[2 * i]));
        l1 = __half_as_ushort(__float2half_rn(lo[2 * i + 1]));
        h0 = __half_as_ushort(__float2half_rn(hi[2 * i]));
        h1 = __half_as_ushort(__float2half_rn(hi[2 * i + 1]));
      } else {  // outward: the stored box still contains every key
        l0 = f32_to_f16_round_down(lo[2 * i]);
        l1 = f32_to_f16_round_down(lo[2 * i + 1]);
        h0 = f32_to_f16_round_up(hi[2 * i]);
        h1 = f32_to_f16_round_up(hi[2 * i + 1]);
      }
      plo[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      phi[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
    }
    m.mn = make_uint4(plo[0], plo[1], plo[2], plo[3]);
    m.mx = make_uint4(phi[0], phi[1], phi[2], phi[3]);
    uint16_t* mp = reinterpret_cast<uint16_t*>(meta) + row + c0;
    *reinterpret_cast<uint4*>(mp) = m.mn;
    *reinterpret_cast<uint4*>(mp + D) = m.mx;
  }
};

template <int D> struct ScoreTraits<D, SPD_DTYPE_F16> : ScoreTraitsF16<D, SPD_DTYPE_F16> {};
template <int D> struct ScoreTraits<D, SPD_DTYPE_FP8_E4M3FN> : ScoreTraitsF16<D, SPD_DTYPE_FP8_E4M3FN> {};

// f32 query, f32 meta, f32 pool.
template <int D>
struct ScoreTraits<D, SPD_DTYPE_F32> {
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
    for (int g = 0; g < kG; ++g) {
      const float4 w = *reinterpret_cast<const float4*>(qp + (size_t)g * D + c0);
      qr.v[g][0] = w.x;
      qr.v[g][1] = w.y;
      qr.v[g][2] = w.z;
      qr.v[g][3] = w.w;
    }
  }
  __device__ static void load_m(M& m, const void* meta, size_t row, int c0) {
    const float* base = reinterpret_cast<const float*>(meta) + row + c0;
    m.mn = ld_stream(reinterpret_cast<const float4*>(base));
    m.mx = ld_stream(reinterpret_cast<const float4*>(base + D));
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
  __device__ static void rebuild(M& m, const void* k_pool, const uint16_t*, size_t head_page, int valid, int c0,
                                 void* meta, size_t row) {
    const float* kp = reinterpret_cast<const float*>(k_pool) + head_page * kPage * D + c0;
    float lo[4] = {INFINITY, INFINITY, INFINITY, INFINITY}, hi[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      const float4 t4 = *reinterpret_cast<const float4*>(kp + (size_t)t * D);
      const float v[4] = {t4.x, t4.y, t4.z, t4.w};
      if (t < valid) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          lo[c] = fminf(lo[c], v[c]);
          hi[c] = fmaxf(hi[c], v[c]);
        }
      }
    }
    m.mn = make_float4(lo[0], lo[1], lo[2], lo[3]);
    m.mx = make_float4(hi[0], hi[1], hi[2], hi[3]);
    float* mp = reinterpret_cast<float*>(meta) + row + c0;
    *reinterpret_cast<float4*>(mp) = m.mn;
    *reinterpret_cast<float4*>(mp + D) = m.mx;
  }
};

// Extra workgroups per dynamic row for the tail mode, and the pages the scan covers.
__host__ __device__ __forceinline__ int tail_blocks(const ScoreArgs& a) { return a.tail_mode == SPD_TAIL_REBUILD ? 1 : 0; }
__device__ __forceinline__ int scan_pages(const ScoreArgs& a, int n) {
  return a.tail_mode != SPD_TAIL_NONE && n > 0 ? n - 1 : n;
}

// Scan work numbering shared by the scorers: the blocks of PPB pages that hold pages of a dynamic row's
// scan, numbered request-major as (request b, dynamic head, block) -- the heads of a request need the
// same number of blocks -- from the requests' lengths on the device.  `n_scan(len)` gives the pages a
// row's scan covers for a request of len tokens.  A workgroup takes one item; those past the last item
// exit, so a batch of short and long requests has its working workgroups dispatched first instead of
// scattered among the blocks past each short row's end.
struct ScanItem {
  int b, h, blk, n_scan, len;
};

// One wave's view of 64 requests: lane i holds request b0 + i's length and the inclusive count of the
// items of requests b0 .. b0 + i; `total` is the 64 requests' item count.
struct ScanChunk {
  int len, incl, total;
};

template <int PPB, typename NScan>
__device__ __forceinline__ ScanChunk scan_chunk(const ScoreArgs& a, int b0, NScan n_scan) {
  const int b = b0 + (int)threadIdx.x % kWave;
  ScanChunk c;
  c.len = b < a.batch ? a.seq_lens[b] : 0;
  const int items = b < a.batch ? (n_scan(c.len) + PPB - 1) / PPB * a.dyn.count : 0;
  c.incl = (int)wave_incl_scan((uint32_t)items);
  c.total = (int)lane_u32((uint32_t)c.incl, kWave - 1);
  return c;
}

// Item `rel` of a chunk starting at request b0 (rel < c.total).  Every result is wave-uniform.
template <int PPB, typename NScan>
__device__ __forceinline__ ScanItem chunk_item(const ScoreArgs& a, const ScanChunk& c, int b0, int rel, NScan n_scan) {
  const int i = __popcll(__ballot(c.incl <= rel));  // the first lane whose inclusive count passes rel
  ScanItem it;
  it.b = b0 + i;
  it.len = (int)lane_u32((uint32_t)c.len, i);
  it.n_scan = n_scan(it.len);
  const int nb = (it.n_scan + PPB - 1) / PPB;
  const int r = rel - ((int)lane_u32((uint32_t)c.incl, i) - nb * a.dyn.count);
  const int hi = r / nb;
  it.h = a.dyn.at(hi);
  it.blk = r - hi * nb;
  return it;
}

// Item k of the numbering; false past the last item.  A batch of up to kSmallBatch requests reads its
// lengths as scalar loads (through the constant address space, which the kernels never write, so the
// compiler issues them as such; indices clamped into the batch), all requested before the first is
// used, and finds its request by a running count on the scalar unit; larger batches read 64 lengths per
// wave with one vector load and a DPP prefix sum.  Each length is one scalar-cache request per
// workgroup: on batches of 8 with thousands of workgroups past short rows the vector load was faster
// (scorer 11.5 against 9.4 us), on full rows of 4 requests the scalar loads (35.7 against 36.7 us).
constexpr int kSmallBatch = 4;
template <int PPB, typename NScan>
__device__ __forceinline__ bool scan_item(const ScoreArgs& a, int k, ScanItem& it, NScan n_scan) {
  if (a.batch <= kSmallBatch) {
    const ConstI32Ptr lens_c = (ConstI32Ptr)a.seq_lens;
    int lens[kSmallBatch];
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i) lens[i] = lens_c[min(i, a.batch - 1)];
    // every length in a scalar register here: the loads are issued together and waited for once
    static_assert(kSmallBatch == 4, "one operand per length below");
    asm volatile("" ::"s"(lens[0]), "s"(lens[1]), "s"(lens[2]), "s"(lens[3]));
    int off = 0;
#pragma unroll
    for (int i = 0; i < kSmallBatch; ++i) {
      if (i >= a.batch) break;
      const int ns = n_scan(lens[i]);
      const int nb = (ns + PPB - 1) / PPB;
      const int cnt = nb * a.dyn.count;
      if (k - off < cnt) {
        const int hi = (k - off) / nb;
        it.b = i;
        it.len = lens[i];
        it.n_scan = ns;
        it.h = a.dyn.at(hi);
        it.blk = k - off - hi * nb;
        return true;
      }
      off += cnt;
    }
    return false;
  }
  for (int off = 0, b0 = 0; b0 < a.batch; b0 += kWave) {
    const ScanChunk c = scan_chunk<PPB>(a, b0, n_scan);
    if (k - off < c.total) {
      it = chunk_item<PPB>(a, c, b0, k - off, n_scan);
      return true;
    }
    off += c.total;
  }
  return false;
}

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
  if (m == -INFINITY) {
    m = m2;
    s = s2;
    return;
  }
  float M = fmaxf(m, m2);
  s = s * expf(m - M) + s2 * expf(m2 - M);
  m = M;
}

// Logical page of the calling lane's page group `it` in a workgroup starting at p_begin.
template <int D, int KVD, int NW>
__device__ __forceinline__ int score_page(int p_begin, int it) {
  constexpr int LPP = ScoreTraits<D, KVD>::LPP;
  constexpr int PPI = kWave / LPP;
  return p_begin + (it * NW + (int)threadIdx.x / kWave) * PPI + ((int)threadIdx.x % kWave) / LPP;
}

// Block-table entries of the calling lane's pages, read without waiting for the request's
// length: indices past the table row are clamped into it and the values discarded later.
// Pages are logical pages; with hierarchical paging (lgs > 0) the entry is that of the physical page
// holding the logical page.
template <int D, int KVD, int NW, int ITERS>
__device__ __forceinline__ void load_block_table(const int32_t* bt_row, int max_pages, int p_begin, int (&raw)[ITERS],
                                                 int lgs = 0) {
#pragma unroll
  for (int it = 0; it < ITERS; ++it) raw[it] = bt_row[min(score_page<D, KVD, NW>(p_begin, it) >> lgs, max_pages - 1)];
}

// Key boxes of the calling lane's page groups (logical pages pg) of request b, KV head h.  Their
// addresses follow from the logical pages alone, so the loads are issued at once, beside the
// block-table entries that only mark pages outside the pool; every group's box is loaded with no
// branch around the load (a page past the row's boxes reads its last box, and its bound is discarded).
template <int D, int KVD, int ITERS>
__device__ __forceinline__ void load_boxes(const ScoreArgs& a, int b, int h, const int (&pg)[ITERS], int c0,
                                           typename ScoreTraits<D, KVD>::M (&m)[ITERS]) {
  const size_t base = meta_unit(b, h, 0, a.num_kv_heads, a.max_pages, a.lgs);
  const int last = (a.max_pages << a.lgs) - 1;
#pragma unroll
  for (int it = 0; it < ITERS; ++it) ScoreTraits<D, KVD>::load_m(m[it], a.meta, (base + min(pg[it], last)) * 2 * D, c0);
}

// Bounds S_{g,p} of the pages [p_begin, p_begin + NW * ITERS * PPI) owned by this workgroup.
// Pages >= n do not count (n is the scan limit); raw holds load_block_table's entries.
// For each of the ITERS page groups of the calling lane, `fn(p, ok, s)` is called on lanes
// with sub == 0 after the LPP-lane reduction (p may be >= n: then ok is false and fn must
// ignore it).  Pages whose block-table entry is outside the pool have ok = false.
template <int D, int KVD, int NW, int ITERS, typename F>
__device__ __forceinline__ void score_block(const ScoreArgs& a, const int (&raw)[ITERS], int n, int b, int h,
                                            int p_begin, F&& fn) {
  using T = ScoreTraits<D, KVD>;
  constexpr int LPP = T::LPP;
  const int lane = threadIdx.x % kWave;
  const int sub = lane % LPP;
  const int c0 = sub * T::CW;
  int pg[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) pg[it] = score_page<D, KVD, NW>(p_begin, it);
  typename T::Q qr;
  T::load_q(qr, a.q, ((size_t)b * a.num_q_heads + (size_t)h * kG) * D, c0);
  typename T::M m[ITERS];
  load_boxes<D, KVD, ITERS>(a, b, h, pg, c0, m);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const bool ok = pg[it] < n && raw[it] >= 0 && raw[it] < a.num_pool_pages;
    float s[kG];
    T::bound(qr, m[it], s);
#pragma unroll
    for (int g = 0; g < kG; ++g) s[g] = ok ? s[g] : 0.f;
#pragma unroll
    for (int g = 0; g < kG; ++g) s[g] = group_sum<LPP>(s[g]);
    if (sub == 0) fn(pg[it], ok && pg[it] < n, s);
  }
}

// The tail workgroup of a dynamic row: lanes 0..LPP-1 of wave 0 rebuild the key statistics of
// the row's last page (n - 1) from the K pool, store them, and bound it; `fn(s)` gets the
// bounds on lane 0 (not called when the page's block-table entry is outside the pool).
template <int D, int KVD, typename F>
__device__ __forceinline__ void score_tail_page(const ScoreArgs& a, const int32_t* bt_row, int n, int len, int b,
                                                int h, F&& fn) {
  using T = ScoreTraits<D, KVD>;
  constexpr int LPP = T::LPP;
  if (threadIdx.x >= LPP) return;
  const int c0 = (int)threadIdx.x * T::CW;
  const int phys = bt_row[n - 1];
  typename T::Q qr;
  T::load_q(qr, a.q, ((size_t)b * a.num_q_heads + (size_t)h * kG) * D, c0);
  if (phys < 0 || phys >= a.num_pool_pages) return;
  const size_t head_page = (size_t)phys * a.num_kv_heads + h;
  typename T::M m;
  T::rebuild(m, a.k_pool, a.k_scale, head_page, valid_in_page(len, n - 1), c0, a.meta_out,
             meta_unit(b, h, n - 1, a.num_kv_heads, a.max_pages, 0) * 2 * D);
  float s[kG];
  T::bound(qr, m, s);
#pragma unroll
  for (int g = 0; g < kG; ++g) s[g] = group_sum<LPP>(s[g]);
  if (threadIdx.x == 0) fn(s);
}

// The last page's key statistics of a head whose row is not scored (a streaming head): lanes
// 0..LPP-1 of wave 0 rebuild them from the K pool and store them, as score_tail_page does.
template <int D, int KVD>
__device__ __forceinline__ void rebuild_tail_page(const ScoreArgs& a, const int32_t* bt_row, int n, int len, int b,
                                                  int h) {
  using T = ScoreTraits<D, KVD>;
  if (threadIdx.x >= T::LPP) return;
  const int phys = bt_row[n - 1];
  if (phys < 0 || phys >= a.num_pool_pages) return;
  typename T::M m;
  T::rebuild(m, a.k_pool, a.k_scale, (size_t)phys * a.num_kv_heads + h, valid_in_page(len, n - 1),
             (int)threadIdx.x * T::CW, a.meta_out, meta_unit(b, h, n - 1, a.num_kv_heads, a.max_pages, 0) * 2 * D);
}

// Top-K keys of the workgroup's pages: score_p = max_g S_{g,p} (the group combine keeps the
// score an upper bound for every query head of the group); pages whose block-table entry is
// outside the pool score -inf.
__device__ __forceinline__ float topk_score(const float (&s)[kG]) {
  float best = s[0];
#pragma unroll
  for (int g = 1; g < kG; ++g) best = fmaxf(best, s[g]);
  return best;
}

template <int D, int KVD, int NW, int ITERS>
__device__ __forceinline__ void score_block_topk(const ScoreArgs& a, const int (&raw)[ITERS], int n, int b, int h,
                                                 int p_begin, float* row_scores) {
  score_block<D, KVD, NW, ITERS>(a, raw, n, b, h, p_begin, [&](int p, bool ok, const float (&s)[kG]) {
    if (p >= n) return;
    row_scores[p] = ok ? topk_score(s) : -INFINITY;
  });
}

// Hierarchical paging (LServe summary, "Hierarchical Paging", physical page importance): the
// workgroup's pages are logical pages, and physical page j's score is the largest top-K key of
// its 2^lgs logical pages.  A wave instruction covers PPI consecutive logical pages (PPI a
// multiple of 2^lgs, and workgroups start on a physical page), so the logical pages of one
// physical page sit in lane groups LPP apart and one xor-shuffle per level folds them.  Logical
// pages >= n (past the request or the scan) do not count; physical pages >= n_phys are not
// written.
template <int D, int KVD, int NW, int ITERS>
__device__ __forceinline__ void score_block_topk_hier(const ScoreArgs& a, const int (&raw)[ITERS], int n, int n_phys,
                                                      int b, int h, int p_begin, float* row_scores) {
  using T = ScoreTraits<D, KVD>;
  constexpr int LPP = T::LPP;
  const int lane = threadIdx.x % kWave;
  const int sub = lane % LPP;
  const int c0 = sub * T::CW;
  const int span = LPP << a.lgs;  // lanes of one physical page
  int pg[ITERS];
#pragma unroll
  for (int it = 0; it < ITERS; ++it) pg[it] = score_page<D, KVD, NW>(p_begin, it);
  typename T::Q qr;
  T::load_q(qr, a.q, ((size_t)b * a.num_q_heads + (size_t)h * kG) * D, c0);
  typename T::M m[ITERS];
  load_boxes<D, KVD, ITERS>(a, b, h, pg, c0, m);
#pragma unroll
  for (int it = 0; it < ITERS; ++it) {
    const bool ok = pg[it] < n && raw[it] >= 0 && raw[it] < a.num_pool_pages;
    float s[kG];
    T::bound(qr, m[it], s);
#pragma unroll
    for (int g = 0; g < kG; ++g) s[g] = ok ? s[g] : 0.f;
#pragma unroll
    for (int g = 0; g < kG; ++g) s[g] = group_sum<LPP>(s[g]);  // every lane of the group holds the sums
    float v = ok ? topk_score(s) : -INFINITY;
    for (int o = LPP; o < span; o <<= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    const int j = pg[it] >> a.lgs;
    if (lane % span == 0 && j < n_phys) row_scores[j] = v;
  }
}

// Row stride of the coverage log-masses: one entry per logical page.
__host__ __device__ __forceinline__ size_t ell_stride(const ScoreArgs& a) { return (size_t)a.max_pages << a.lgs; }

// Coverage log-mass of a page: l_{g,p} = s S_{g,p} + ln(valid_p).
__device__ __forceinline__ void coverage_logmass(const ScoreArgs& a, int valid, bool ok, const float (&s)[kG],
                                                 float (&lg)[kG]) {
  const float lv = valid == kPage ? 2.772588722239781f : logf((float)valid);  // ln(valid)
#pragma unroll
  for (int g = 0; g < kG; ++g) lg[g] = ok ? fmaf(a.sm_scale, s[g], lv) : -INFINITY;
}

// Coverage log-masses of the workgroup's pages [.., n), written per page (the scorer's first
// pass; the row's per-head log-sum-exp is taken afterwards over these values).
template <int D, int KVD, int NW, int ITERS>
__device__ __forceinline__ void score_block_ell(const ScoreArgs& a, const int (&raw)[ITERS], int n, int len, int b,
                                                int h, int p_begin) {
  const size_t row = (size_t)b * a.num_kv_heads + h;
  score_block<D, KVD, NW, ITERS>(a, raw, n, b, h, p_begin, [&](int p, bool ok, const float (&s)[kG]) {
    if (p >= n) return;
    float lg[kG];
    coverage_logmass(a, valid_in_page(len, p), ok, s, lg);
    a.ell[row * ell_stride(a) + p] = make_float4(lg[0], lg[1], lg[2], lg[3]);
  });
}

// Coverage, first pass over the workgroup's pages [.., n): log-masses written per page, and one
// (max, sum exp) pair per head for the workgroup in partial slot `slot`.  Moira, section 3.2: the
// per-head softmax over pages needs the head's log-sum-exp over the whole row.
template <int D, int KVD, int NW, int ITERS>
__device__ __forceinline__ void score_block_coverage(const ScoreArgs& a, const int (&raw)[ITERS], int n, int len, int b,
                                                     int h, int p_begin, int slot) {
  constexpr int LPP = ScoreTraits<D, KVD>::LPP;
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const size_t row = (size_t)b * a.num_kv_heads + h;
  float lm[kG], ls[kG];  // running (max, sum exp) of this lane's pages
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    lm[g] = -INFINITY;
    ls[g] = 0.f;
  }
  score_block<D, KVD, NW, ITERS>(a, raw, n, b, h, p_begin, [&](int p, bool ok, const float (&s)[kG]) {
    if (p >= n) return;
    float lg[kG];
    coverage_logmass(a, valid_in_page(len, p), ok, s, lg);
#pragma unroll
    for (int g = 0; g < kG; ++g) lse_push(lm[g], ls[g], lg[g]);
    a.ell[row * ell_stride(a) + p] = make_float4(lg[0], lg[1], lg[2], lg[3]);
  });
  // fold the lanes that own pages (sub == 0), then the waves in order
  __shared__ float sm_m[NW][kG], sm_s[NW][kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    for (int o = LPP; o < kWave; o <<= 1) {
      float m2 = __shfl_xor(lm[g], o, kWave), s2 = __shfl_xor(ls[g], o, kWave);
      lse_combine(lm[g], ls[g], m2, s2);
    }
    if (lane == 0) {
      sm_m[wave][g] = lm[g];
      sm_s[wave][g] = ls[g];
    }
  }
  __syncthreads();
  if (threadIdx.x < kG) {
    const int g = threadIdx.x;
    float m = sm_m[0][g], s = sm_s[0][g];
    for (int w = 1; w < NW; ++w) lse_combine(m, s, sm_m[w][g], sm_s[w][g]);
    a.partials[(row * a.partial_stride + slot) * kG + g] = make_float2(m, s);
  }
}

// The tail workgroup's work for either rule: the last page's top-K score, or its log-masses and
// (slot >= 0, the fused kernel) the (max, 1) pair of that single page in partial slot `slot`.
template <int D, int KVD, bool COV>
__device__ __forceinline__ void score_tail(const ScoreArgs& a, const int32_t* bt_row, int n, int len, int b, int h,
                                           int slot) {
  const size_t row = (size_t)b * a.num_kv_heads + h;
  if constexpr (COV) {
    bool wrote = false;
    score_tail_page<D, KVD>(a, bt_row, n, len, b, h, [&](const float (&s)[kG]) {
      float lg[kG];
      coverage_logmass(a, valid_in_page(len, n - 1), true, s, lg);
      a.ell[row * a.max_pages + n - 1] = make_float4(lg[0], lg[1], lg[2], lg[3]);
      if (slot >= 0) {
#pragma unroll
        for (int g = 0; g < kG; ++g) a.partials[(row * a.partial_stride + slot) * kG + g] = make_float2(lg[g], 1.f);
      }
      wrote = true;
    });
    if (threadIdx.x == 0 && !wrote) {  // page outside the pool: no mass
      a.ell[row * a.max_pages + n - 1] = make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
      if (slot >= 0) {
#pragma unroll
        for (int g = 0; g < kG; ++g) a.partials[(row * a.partial_stride + slot) * kG + g] = make_float2(-INFINITY, 0.f);
      }
    }
  } else {
    bool wrote = false;
    score_tail_page<D, KVD>(a, bt_row, n, len, b, h, [&](const float (&s)[kG]) {
      a.scores[row * a.max_pages + n - 1] = topk_score(s);
      wrote = true;
    });
    if (threadIdx.x == 0 && !wrote) a.scores[row * a.max_pages + n - 1] = -INFINITY;
  }
}

// Per-head log-sum-exp of a row from its `used` workgroup partials, computed by one wave in a
// fixed order (so every caller gets the same bits): lanes fold partials lane, lane + 64, ...,
// then a fixed butterfly.  Returns lse[g] (-inf for an empty row) in every lane.
__device__ __forceinline__ void row_head_lse(const float2* partials, int used, float (&lse)[kG]) {
  const int lane = threadIdx.x % kWave;
  float m[kG], s[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    m[g] = -INFINITY;
    s[g] = 0.f;
  }
  for (int k = lane; k < used; k += kWave) {
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      const float2 pr = partials[(size_t)k * kG + g];
      lse_combine(m[g], s[g], pr.x, pr.y);
    }
  }
#pragma unroll
  for (int g = 0; g < kG; ++g) {
    for (int o = 1; o < kWave; o <<= 1) {
      float m2 = __shfl_xor(m[g], o, kWave), s2 = __shfl_xor(s[g], o, kWave);
      lse_combine(m[g], s[g], m2, s2);
    }
    lse[g] = m[g] == -INFINITY ? -INFINITY : m[g] + logf(s[g]);
  }
}

// Moira's group-mean share of one page from its G log-masses and the heads' log-sum-exps.
__device__ __forceinline__ float group_share(float4 l4, const float (&lse)[kG]) {
  const float lg[kG] = {l4.x, l4.y, l4.z, l4.w};
  float acc = 0.f;
#pragma unroll
  for (int g = 0; g < kG; ++g)
    if (lg[g] != -INFINITY) acc += expf(lg[g] - lse[g]);
  return acc * (1.0f / kG);
}

}  // namespace spd
