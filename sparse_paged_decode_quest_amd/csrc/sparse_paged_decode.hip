// Grouped-query decode attention over per-row page lists, split by a device-side plan,
// and the exact log-sum-exp merge of the split states.
//
// Sources: PersistentKV, section 3.1 (Eq. 1, decode attention; one work unit per (request,
// KV head, split) computing all query heads of the group on the same K/V tiles), section
// 3.2 (K/V read in place through the native block table; fp32 online-softmax state
// (m, l, acc)) and section 3.3 (split states, their exact merge, row-local bounds);
// Moira, section 3.3 (self-planning attention, Eq. 4 and Algorithm 2: every block reads
// the row's list length and derives its own chunk; single-chunk rows are written directly,
// others are merged); LServe summary, "Decoding Stage: Kernel Implementation with
// Two-Level Indexing" (loop over a per-head index table of pages).
//
// Block (row, j) with 4 waves: wave w takes pages j*c + w, j*c + w + 4, ... of the chunk.
// For one 16-token page a wave needs no LDS staging: lane l reads token l/4, channel
// quarter l%4 of K (16-byte loads, 64 contiguous bytes per token per instruction), and
// channels [l*d/64, (l+1)*d/64) of V for all 16 tokens (one 256-byte row per instruction).
// The G = 4 partial dot products of a lane are reduce-scattered over its quad so that lane
// l ends with the full logit of head l%4 and token l/4 -- one logit per lane.  Softmax
// max / sum run on those, the 64 probabilities go through 1 KiB of LDS so every lane can
// apply all of them to its V channels.  The waves' states are merged in LDS at the end.
#include <type_traits>

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

constexpr int kGq = 4;  // query heads per KV head

typedef _Float16 dh2_t __attribute__((ext_vector_type(2)));

template <int D, int QD, int KVD>
struct DecTraits;

// ---------------------------------------------------------------- f16 query, f16 K/V
template <int D>
struct DecTraits<D, SPD_DTYPE_F16, SPD_DTYPE_F16> {
  static constexpr int NS = D / 32;   // 16-byte K chunks per lane (8 channels each)
  static constexpr int CPL = D / 64;  // V channels per lane
  using VW = typename std::conditional<CPL == 2, uint32_t, uint16_t>::type;  // a lane's V channels of one token
  struct Q { uint32_t h[kGq][NS * 4]; };
  struct KF { uint4 k[NS]; };
  struct VF { VW v[kPage]; };
  // lane channel of K element i of chunk s: s*32 + quarter*8 + i
  __device__ static void load_q(Q& q, const void* qp, size_t base, int quarter) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(qp) + base);
#pragma unroll
    for (int g = 0; g < kGq; ++g)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) q.h[g][s * 4 + i] = p[(g * D + s * 32 + quarter * 8) / 2 + i];
  }
  __device__ static void load_k(KF& f, const void* pool, size_t tok_base, int quarter) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(pool) + tok_base;
#pragma unroll
    for (int s = 0; s < NS; ++s) f.k[s] = *reinterpret_cast<const uint4*>(p + s * 32 + quarter * 8);
  }
  __device__ static void load_v(VF& f, const void* pool, size_t page_base, int lane) {
    const VW* p = reinterpret_cast<const VW*>(reinterpret_cast<const uint16_t*>(pool) + page_base + lane * CPL);
#pragma unroll
    for (int t = 0; t < kPage; ++t) f.v[t] = p[t * (D / CPL)];
  }
  __device__ static void dots(const Q& q, const KF& f, float (&part)[kGq]) {
#pragma unroll
    for (int g = 0; g < kGq; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const uint32_t kw[4] = {f.k[s].x, f.k[s].y, f.k[s].z, f.k[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(dh2_t, kw[i]), __builtin_bit_cast(dh2_t, q.h[g][s * 4 + i]), acc, false);
      }
      part[g] = acc;
    }
  }
  __device__ static void v_values(const VF& f, int t, float (&v)[CPL]) {
    if constexpr (CPL == 2) {
      const __half2 h = __builtin_bit_cast(__half2, (uint32_t)f.v[t]);
      v[0] = __low2float(h);
      v[1] = __high2float(h);
    } else {
      v[0] = half_bits_to_float((uint16_t)f.v[t]);
    }
  }
  static constexpr bool kScaled = false;
};

// ---------------------------------------------------------------- f16 query, fp8 K/V
template <int D>
struct DecTraits<D, SPD_DTYPE_F16, SPD_DTYPE_FP8_E4M3FN> {
  static_assert(D == 128, "fp8 pools are compiled for d = 128");
  static constexpr int NS = D / 64;   // 16-byte K chunks per lane (16 channels each)
  static constexpr int CPL = D / 64;
  struct Q { uint32_t h[kGq][NS * 8]; };
  struct KF { uint4 k[NS]; };
  struct VF { uint16_t v[kPage]; };  // CPL == 2 codes per token (d = 128)
  // lane channel of K element i of chunk s: s*64 + quarter*16 + i
  __device__ static void load_q(Q& q, const void* qp, size_t base, int quarter) {
    const uint32_t* p = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint16_t*>(qp) + base);
#pragma unroll
    for (int g = 0; g < kGq; ++g)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) q.h[g][s * 8 + i] = p[(g * D + s * 64 + quarter * 16) / 2 + i];
  }
  __device__ static void load_k(KF& f, const void* pool, size_t tok_base, int quarter) {
    const uint8_t* p = reinterpret_cast<const uint8_t*>(pool) + tok_base;
#pragma unroll
    for (int s = 0; s < NS; ++s) f.k[s] = *reinterpret_cast<const uint4*>(p + s * 64 + quarter * 16);
  }
  __device__ static void load_v(VF& f, const void* pool, size_t page_base, int lane) {
    const uint16_t* p = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(pool) + page_base + lane * CPL);
#pragma unroll
    for (int t = 0; t < kPage; ++t) f.v[t] = p[t * (D / 2)];
  }
  // dot products of the codes' values times 2^-8 (the token scale and 2^8 are applied later)
  __device__ static void dots(const Q& q, const KF& f, float (&part)[kGq]) {
    uint32_t hk[NS * 8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint32_t w[4] = {f.k[s].x, f.k[s].y, f.k[s].z, f.k[s].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hk[s * 8 + 2 * i] = fp8x2_to_half2_scaled(w[i] & 0xffffu);
        hk[s * 8 + 2 * i + 1] = fp8x2_to_half2_scaled(w[i] >> 16);
      }
    }
#pragma unroll
    for (int g = 0; g < kGq; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < NS * 8; ++i)
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(dh2_t, hk[i]), __builtin_bit_cast(dh2_t, q.h[g][i]), acc, false);
      part[g] = acc;
    }
  }
  __device__ static void v_values(const VF& f, int t, float (&v)[CPL]) {
    const __half2 h = __builtin_bit_cast(__half2, fp8x2_to_half2_scaled(f.v[t]));
    v[0] = __low2float(h);
    v[1] = __high2float(h);
  }
  static constexpr bool kScaled = true;
};

// ---------------------------------------------------------------- f32 query, f32 K/V
template <int D>
struct DecTraits<D, SPD_DTYPE_F32, SPD_DTYPE_F32> {
  static constexpr int NS = D / 16;   // 16-byte K chunks per lane (4 channels each)
  static constexpr int CPL = D / 64;
  struct Q { float f[kGq][NS * 4]; };
  struct KF { float4 k[NS]; };
  struct VF { float v[kPage][CPL]; };
  // lane channel of K element i of chunk s: s*16 + quarter*4 + i
  __device__ static void load_q(Q& q, const void* qp, size_t base, int quarter) {
    const float* p = reinterpret_cast<const float*>(qp) + base;
#pragma unroll
    for (int g = 0; g < kGq; ++g)
#pragma unroll
      for (int s = 0; s < NS; ++s)
#pragma unroll
        for (int i = 0; i < 4; ++i) q.f[g][s * 4 + i] = p[g * D + s * 16 + quarter * 4 + i];
  }
  __device__ static void load_k(KF& f, const void* pool, size_t tok_base, int quarter) {
    const float* p = reinterpret_cast<const float*>(pool) + tok_base;
#pragma unroll
    for (int s = 0; s < NS; ++s) f.k[s] = *reinterpret_cast<const float4*>(p + s * 16 + quarter * 4);
  }
  __device__ static void load_v(VF& f, const void* pool, size_t page_base, int lane) {
    const float* p = reinterpret_cast<const float*>(pool) + page_base + lane * CPL;
#pragma unroll
    for (int t = 0; t < kPage; ++t)
#pragma unroll
      for (int c = 0; c < CPL; ++c) f.v[t][c] = p[t * D + c];
  }
  __device__ static void dots(const Q& q, const KF& f, float (&part)[kGq]) {
#pragma unroll
    for (int g = 0; g < kGq; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        acc = fmaf(q.f[g][s * 4 + 0], f.k[s].x, acc);
        acc = fmaf(q.f[g][s * 4 + 1], f.k[s].y, acc);
        acc = fmaf(q.f[g][s * 4 + 2], f.k[s].z, acc);
        acc = fmaf(q.f[g][s * 4 + 3], f.k[s].w, acc);
      }
      part[g] = acc;
    }
  }
  __device__ static void v_values(const VF& f, int t, float (&v)[CPL]) {
#pragma unroll
    for (int c = 0; c < CPL; ++c) v[c] = f.v[t][c];
  }
  static constexpr bool kScaled = false;
};

struct PageRef {
  int page;   // logical page, -1 when the entry is not a usable page
  int phys;
  int valid;  // valid tokens
};

// List entry i of a row: its logical page and, from the list of physical pages when the
// selector wrote one (no block-table read) or else from the block table, its physical page.
__device__ __forceinline__ PageRef resolve_page(const DecodeArgs& a, const int32_t* list, const int32_t* plist, int i,
                                                int b, int n_b, int len) {
  PageRef r{-1, 0, 0};
  const int p = list[i];
  const int pp = plist ? plist[i] : 0;
  if (p < 0 || p >= n_b) return r;
  const int phys = plist ? pp : a.block_table[(size_t)b * a.max_pages + p];
  if (phys < 0 || phys >= a.num_pool_pages) return r;
  r.page = p;
  r.phys = phys;
  r.valid = valid_in_page(len, p);
  return r;
}

template <int D, int QD, int KVD>
__global__ __launch_bounds__(256) void sparse_paged_decode_kernel(DecodeArgs a) {
  using T = DecTraits<D, QD, KVD>;
  constexpr int CPL = T::CPL;
  __shared__ float p_lds[4][kPage][kGq];
  __shared__ float alpha_lds[4][kGq];
  __shared__ float ws_m[4][kGq], ws_l[4][kGq];
  __shared__ float ws_acc[4][kGq][D];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int tok = lane >> 2;      // QK role: token of the page
  const int quarter = lane & 3;   // QK role: channel quarter, and after the reduce-scatter the head
  const int row = blockIdx.x / a.blocks_per_row;
  const int j = blockIdx.x % a.blocks_per_row;
  const int b = row / a.num_kv_heads;
  const int h = row % a.num_kv_heads;
  const size_t qrow = (size_t)b * a.num_q_heads + (size_t)h * kGq;  // first query head of the group

  int n = a.list_len[row];
  n = n < 0 ? 0 : (n > a.max_list ? a.max_list : n);
  if (n == 0) {
    if (j == 0) {
      for (int e = threadIdx.x; e < kGq * D; e += blockDim.x) a.out[qrow * D + e] = 0.f;
      if (threadIdx.x < kGq) a.out_lse[qrow + threadIdx.x] = -INFINITY;
    }
    return;
  }
  int c, m;
  plan_chunks(n, a.blocks_per_row, a.min_chunk, c, m);
  if (j >= m) return;
  const int i0 = j * c;
  const int i1 = min(n, i0 + c);
  const int len = a.seq_lens[b];
  const int n_b = row_pages(len, a.max_pages);
  const int32_t* list = a.page_list + (size_t)row * a.max_list;
  const int32_t* plist = a.page_phys ? a.page_phys + (size_t)row * a.max_list : nullptr;

  typename T::Q q;
  T::load_q(q, a.q, qrow * D, quarter);

  float m_run = -INFINITY, l_run = 0.f;
  float acc[kGq][CPL];
#pragma unroll
  for (int g = 0; g < kGq; ++g)
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) acc[g][cc] = 0.f;

  // Pages of this wave alternate between two register stages, so the next page's K / V
  // loads are in flight while the current page is computed.
  auto load = [&](const PageRef& r, typename T::KF& kd, typename T::VF& vd, float& ksd, float& vsd) {
    if (r.page < 0) return;
    const size_t head_page = (size_t)r.phys * a.num_kv_heads + h;
    T::load_k(kd, a.k_pool, (head_page * kPage + tok) * D, quarter);
    T::load_v(vd, a.v_pool, head_page * kPage * D, lane);
    if (T::kScaled) {
      ksd = half_bits_to_float(a.k_scale[head_page * kPage + tok]) * 256.f;
      vsd = half_bits_to_float(a.v_scale[head_page * kPage + tok]) * 256.f;
    }
  };
  auto process = [&](const PageRef& r, const typename T::KF& kf, const typename T::VF& vf, float ks, float vs) {
    if (r.page < 0) return;
    // logits: partial dots over this lane's channel quarter, reduce-scattered over the quad
    float part[kGq];
    T::dots(q, kf, part);
    const int b0 = quarter & 1, b1 = quarter >> 1;
    const float send0 = b0 ? part[0] : part[1];
    const float send1 = b0 ? part[2] : part[3];
    const float keep0 = b0 ? part[1] : part[0];
    const float keep1 = b0 ? part[3] : part[2];
    const float hA = keep0 + __shfl_xor(send0, 1, kWave);  // head b0
    const float hB = keep1 + __shfl_xor(send1, 1, kWave);  // head 2 + b0
    const float keep2 = b1 ? hB : hA;
    const float send2 = b1 ? hA : hB;
    const float dot = keep2 + __shfl_xor(send2, 2, kWave);  // head `quarter`, token `tok`
    float x = dot * a.sm_scale_log2 * ks;
    if (tok >= r.valid) x = -INFINITY;
    float mx = x;
#pragma unroll
    for (int o = 4; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float p = m_new == -INFINITY ? 0.f : exp2f(x - m_new);
    l_run = l_run * alpha + p;
    m_run = m_new;
    p_lds[wave][tok][quarter] = p * vs;
    if (lane < kGq) alpha_lds[wave][lane] = alpha;
    wave_fence();
    const float4 al = *reinterpret_cast<const float4*>(alpha_lds[wave]);
    const float alv[kGq] = {al.x, al.y, al.z, al.w};
#pragma unroll
    for (int g = 0; g < kGq; ++g)
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) acc[g][cc] *= alv[g];
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      if (t < r.valid) {  // invalid slots may hold NaN: never touch them
        const float4 pt = *reinterpret_cast<const float4*>(p_lds[wave][t]);
        const float pv[kGq] = {pt.x, pt.y, pt.z, pt.w};
        float v[CPL];
        T::v_values(vf, t, v);
#pragma unroll
        for (int g = 0; g < kGq; ++g)
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) acc[g][cc] = fmaf(pv[g], v[cc], acc[g][cc]);
      }
    }
    wave_fence();
  };

  const PageRef none{-1, 0, 0};
  typename T::KF ka, kb;
  typename T::VF va, vb;
  float ksa = 1.f, vsa = 1.f, ksb = 1.f, vsb = 1.f;
  int i = i0 + wave;
  PageRef ra = i < i1 ? resolve_page(a, list, plist, i, b, n_b, len) : none;
  load(ra, ka, va, ksa, vsa);
  while (i < i1) {
    const PageRef rb = i + 4 < i1 ? resolve_page(a, list, plist, i + 4, b, n_b, len) : none;
    load(rb, kb, vb, ksb, vsb);
    process(ra, ka, va, ksa, vsa);
    i += 4;
    if (i >= i1) break;
    ra = i + 4 < i1 ? resolve_page(a, list, plist, i + 4, b, n_b, len) : none;
    load(ra, ka, va, ksa, vsa);
    process(rb, kb, vb, ksb, vsb);
    i += 4;
  }

  // wave state -> LDS
#pragma unroll
  for (int o = 4; o < kWave; o <<= 1) l_run += __shfl_xor(l_run, o, kWave);
  if (lane < kGq) {
    ws_m[wave][lane] = m_run;
    ws_l[wave][lane] = l_run;
  }
#pragma unroll
  for (int g = 0; g < kGq; ++g)
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) ws_acc[wave][g][lane * CPL + cc] = acc[g][cc];
  __syncthreads();

  // merge the four wave states (fixed order) and write the chunk result
  for (int e = threadIdx.x; e < kGq * D; e += blockDim.x) {
    const int g = e / D, ch = e % D;
    float M = ws_m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, ws_m[w][g]);
    float o = 0.f, lse = -INFINITY;
    if (M != -INFINITY) {
      float L = 0.f, A = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float sc = exp2f(ws_m[w][g] - M);
        L = fmaf(ws_l[w][g], sc, L);
        A = fmaf(ws_acc[w][g][ch], sc, A);
      }
      o = A / L;
      lse = (M + log2f(L)) * kLn2;
    }
    if (m == 1) {
      a.out[(qrow + g) * D + ch] = o;
      if (ch == 0) a.out_lse[qrow + g] = lse;
    } else {
      const size_t slot = ((size_t)row * a.blocks_per_row + j) * kGq + g;
      a.part_o[slot * D + ch] = o;
      if (ch == 0) a.part_lse[slot] = lse;
    }
  }
}

// Exact merge of a row's chunk states (PersistentKV, section 3.3; states are stored
// normalised: o_j = a_j / l_j and lse_j = m_j + ln l_j).  One 1024-thread block per (row,
// query head): chunk weights exp(lse_j - lse) go through LDS, then D channels x (1024 / D)
// chunk partitions accumulate in parallel (every partial load of a thread is independent)
// and the partitions are summed in a fixed order.
constexpr int kMergeThreads = 1024;
constexpr int kMaxChunks = 1024;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(MergeArgs a) {
  constexpr int PARTS = kMergeThreads / D;
  __shared__ float w_s[kMaxChunks];
  __shared__ float red[kMergeThreads / kWave];
  __shared__ float part_s[PARTS][D];
  const int row = blockIdx.x / kGq;
  const int g = blockIdx.x % kGq;
  const int b = row / a.num_kv_heads;
  const int h = row % a.num_kv_heads;
  int n = a.list_len[row];
  n = n < 0 ? 0 : (n > a.max_list ? a.max_list : n);
  int c, m;
  plan_chunks(n, a.blocks_per_row, a.min_chunk, c, m);
  if (m <= 1) return;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const size_t slot0 = (size_t)row * a.blocks_per_row * kGq + g;  // + j * kGq

  float mx = -INFINITY;
  for (int j = threadIdx.x; j < m; j += kMergeThreads) {
    const float l = a.part_lse[slot0 + (size_t)j * kGq];
    w_s[j] = l;
    mx = fmaxf(mx, l);
  }
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o, kWave));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  float M = red[0];
  for (int w = 1; w < kMergeThreads / kWave; ++w) M = fmaxf(M, red[w]);
  __syncthreads();
  const size_t qrow = (size_t)b * a.num_q_heads + (size_t)h * kGq + g;
  if (M == -INFINITY) {
    for (int ch = threadIdx.x; ch < D; ch += kMergeThreads) a.out[qrow * D + ch] = 0.f;
    if (threadIdx.x == 0) a.out_lse[qrow] = -INFINITY;
    return;
  }
  float sum = 0.f;
  for (int j = threadIdx.x; j < m; j += kMergeThreads) {
    const float wj = expf(w_s[j] - M);
    w_s[j] = wj;
    sum += wj;
  }
  sum = xor_sum<kWave>(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  float S = 0.f;
  for (int w = 0; w < kMergeThreads / kWave; ++w) S += red[w];

  const int ch = threadIdx.x % D, part = threadIdx.x / D;
  float acc = 0.f;
#pragma unroll 8
  for (int j = part; j < m; j += PARTS) acc = fmaf(w_s[j], a.part_o[(slot0 + (size_t)j * kGq) * D + ch], acc);
  part_s[part][ch] = acc;
  __syncthreads();
  if (threadIdx.x < D) {
    float o = 0.f;
#pragma unroll
    for (int pp = 0; pp < PARTS; ++pp) o += part_s[pp][threadIdx.x];
    a.out[qrow * D + threadIdx.x] = o / S;
    if (threadIdx.x == 0) a.out_lse[qrow] = M + logf(S);
  }
}

int launch_sparse_paged_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype, hipStream_t stream) {
  dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.blocks_per_row)), block(256);
#define SPD_DEC_CASE(D, QD, KVD)                                                                 \
  if (head_dim == D && q_dtype == QD && kv_dtype == KVD) {                                       \
    hipLaunchKernelGGL((sparse_paged_decode_kernel<D, QD, KVD>), grid, block, 0, stream, a);     \
    return 0;                                                                                    \
  }
  SPD_DEC_CASE(64, SPD_DTYPE_F32, SPD_DTYPE_F32)
  SPD_DEC_CASE(128, SPD_DTYPE_F32, SPD_DTYPE_F32)
  SPD_DEC_CASE(64, SPD_DTYPE_F16, SPD_DTYPE_F16)
  SPD_DEC_CASE(128, SPD_DTYPE_F16, SPD_DTYPE_F16)
  SPD_DEC_CASE(128, SPD_DTYPE_F16, SPD_DTYPE_FP8_E4M3FN)
#undef SPD_DEC_CASE
  return SPD_ERR_UNSUPPORTED;
}

int launch_lse_merge(const MergeArgs& a, int head_dim, hipStream_t stream) {
  dim3 grid((unsigned)(a.batch * a.num_kv_heads * kGq)), block(kMergeThreads);
  if (head_dim == 64) hipLaunchKernelGGL(lse_merge_kernel<64>, grid, block, 0, stream, a);
  else if (head_dim == 128) hipLaunchKernelGGL(lse_merge_kernel<128>, grid, block, 0, stream, a);
  else return SPD_ERR_UNSUPPORTED;
  return 0;
}

}  // namespace spd
