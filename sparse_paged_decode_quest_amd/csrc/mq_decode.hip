// Several query tokens per request in one decode step (the T <= 4 draft tokens of speculative
// decoding), with the lists of the tokens shared as one scan: LiteTopK, section 3.4 (LiteDSA,
// "Candidate Union and Membership Masks", "Grouped Sparse Attention").  Each query token t has
// its own page list (selected as a single query with its causal length); the lists of a
// (request, KV head) row are merged into one ascending union with a bit mask per entry (bit t:
// the page is in token t's list), and attention reads each union page once for all T x G query
// rows, masking out the rows whose token did not select the page.
//
// Decode work layout (one 16-token page per wave, four waves per workgroup, Moira Eq. 4 split):
//  * logits: the page's 16 x 16 tile S[row = 4 t + g][token] is one chain of eight
//    v_mfma_f32_16x16x16_f16 over the 128 channels.  The channel order inside the chain is
//    permuted so that every lane's operands are contiguous: lane l holds channels
//    32 (l / 16) .. 32 (l / 16) + 31 of query row l % 16 (A) and of key l % 16 (B), and step s
//    takes channels 32 (l / 16) + 4 s .. + 3 of both.  The result puts rows 4 q .. 4 q + 3 (token
//    t = q) of key l % 16 in lane l, so each query token's rows sit in one 16-lane DPP row;
//  * masks: bit t of the page's mask, the token's causal limit (positions < len - T + 1 + t)
//    and the request's length, before the online softmax (fp32, base 2);
//  * PV on MFMA too, as O^T = V^T P^T in eight 16 x 16 x 16 tiles of channels: the wave writes
//    its page's V transposed into LDS (each lane packs its two channels' 16 keys into two 32-byte
//    rows) and P as fp16 in [row][key] order, then every lane reads four keys of one channel (A)
//    and four keys of one row (B) per tile with 8-byte LDS reads.
#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

constexpr int kMqG = 4;      // query heads per KV head
constexpr int kMqRows = 16;  // 4 query tokens x G = 4 heads
constexpr int kUnionThreads = 1024;
constexpr int kUnionRounds = 2;  // list entries per thread read up front (4 tokens x 512 entries)
constexpr int kUnionRankMinPages = 16384;  // block tables this wide merge sorted lists by rank
// Pages of a wave in flight: the next page's loads go out before the current page is computed (two
// register stages; the page's loads are scalar-addressed buffer loads and fp8 codes are decoded when
// the page is processed, so nothing waits for the next page early).
constexpr int kMqStages = 2;

__device__ __forceinline__ int mq_clamp(int n, int hi) { return n < 0 ? 0 : (n > hi ? hi : n); }

// One workgroup per (request, KV head): a byte per page of the request in LDS collects the
// tokens' bits (atomicOr on the word holding it), then an ordered compaction writes the union.
template <bool RANK>
__global__ __launch_bounds__(kUnionThreads) void page_list_union_kernel(UnionArgs a) {
  extern __shared__ uint32_t bits[];  // ceil(max_pages / 4) words
  __shared__ uint32_t wsum[kUnionThreads / kWave];
  const int row = blockIdx.x;
  const int b = row / a.num_kv_heads, h = row % a.num_kv_heads;
  // Thread k reads entry k of the tokens' lists laid end to end (token k / token_max_list) and that
  // token's length at the same time -- entries past a length are read from inside the list row and
  // dropped -- while the byte map is cleared; longer lists take further rounds.
  const int total = a.num_tokens * a.token_max_list;
  int ent[kUnionRounds], len_of[kUnionRounds];
#pragma unroll
  for (int k = 0; k < kUnionRounds; ++k) {
    const int e = (int)threadIdx.x + k * kUnionThreads;
    ent[k] = -1;
    len_of[k] = 0;
    if (e < total) {
      const size_t trow = ((size_t)b * a.num_tokens + e / a.token_max_list) * a.num_kv_heads + h;
      ent[k] = a.token_list[trow * a.token_max_list + e % a.token_max_list];
      len_of[k] = a.token_len[trow];
    }
  }
  const int n = row_pages(a.seq_lens[b], a.max_pages);
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int32_t* bt_row = a.block_table + (size_t)b * a.max_pages;
  const size_t out_row = (size_t)row * a.max_list;

  if (RANK && total <= kUnionThreads) {  // uniform over the block
    // Sorted lists (as the selector writes them) are merged by rank, with no pass over the request's
    // pages: entry e of list t goes to position sum_t' |{x in list t' : x < p}| + |{t' < t : p in list
    // t'}| of the merged sequence (ties by token), and the first of each run of equal pages collects
    // the run's token bits.  Lists that are not strictly ascending take the byte map below.  The merge
    // costs about the same at any length (7-8 us measured), the byte map grows with the request's pages
    // (5.2 us at 8192 pages, 11.9 us at 32768), so the merge is compiled in for tables of at least
    // kUnionRankMinPages pages.
    __shared__ int32_t skey[kUnionThreads];
    __shared__ int32_t merged[kUnionThreads];
    __shared__ uint8_t mtok[kUnionThreads];
    const int e = (int)threadIdx.x;
    const int cap = a.token_max_list;
    const int t = e / cap, j = e % cap;
    const bool valid = e < total && j < mq_clamp(len_of[0], cap) && ent[0] >= 0 && ent[0] < n;
    constexpr int kNone = 0x7fffffff;  // sorts after every page
    const int key = valid ? ent[0] : kNone;
    if (e < total) skey[e] = key;
    __syncthreads();
    const bool in_order = e >= total || j + 1 >= cap || skey[e + 1] == kNone || key < skey[e + 1];
    if (__syncthreads_and(in_order)) {
      const int m_total = __syncthreads_count(valid);
      if (valid) {
        int rank = 0;
        for (int u = 0; u < a.num_tokens; ++u) {
          const int32_t* lst = skey + u * cap;
          int lo = 0, hi = cap;  // first index whose key is >= key
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (lst[mid] < key) lo = mid + 1;
            else hi = mid;
          }
          rank += lo + ((u < t && lo < cap && lst[lo] == key) ? 1 : 0);
        }
        merged[rank] = key;
        mtok[rank] = (uint8_t)t;
      }
      __syncthreads();
      const int r = e;
      const bool first = r < m_total && (r == 0 || merged[r - 1] != merged[r]);
      const uint32_t f = first ? 1u : 0u;
      const uint32_t incl = wave_incl_scan(f);
      if (lane == kWave - 1) wsum[wave] = incl;
      __syncthreads();
      uint32_t base = 0;
      for (int w = 0; w < wave; ++w) base += wsum[w];
      const uint32_t pos = base + incl - f;
      if (first && pos < (uint32_t)a.max_list) {
        const int pg = merged[r];
        uint32_t mask = 0;
        for (int k = r; k < m_total && merged[k] == pg; ++k) mask |= 1u << mtok[k];
        a.page_list[out_row + pos] = pg;
        a.page_mask[out_row + pos] = mask;
        if (a.page_phys) a.page_phys[out_row + pos] = bt_row[pg];
      }
      if (threadIdx.x == kUnionThreads - 1) {
        a.list_len[row] = (int)min(base + incl, (uint32_t)a.max_list);
        if (a.path) a.path[row] = 1;
      }
      return;
    }
  }

  for (int i = threadIdx.x; i < (n + 3) / 4; i += kUnionThreads) bits[i] = 0u;
  __syncthreads();
  for (int k = 0; k < kUnionRounds; ++k) {
    const int e = (int)threadIdx.x + k * kUnionThreads;
    const int p = ent[k];
    if (e < total && e % a.token_max_list < mq_clamp(len_of[k], a.token_max_list) && p >= 0 && p < n)
      atomicOr(&bits[p >> 2], 1u << ((p & 3) * 8 + e / a.token_max_list));
  }
  for (int e = (int)threadIdx.x + kUnionRounds * kUnionThreads; e < total; e += kUnionThreads) {
    const int t = e / a.token_max_list, i = e % a.token_max_list;
    const size_t trow = ((size_t)b * a.num_tokens + t) * a.num_kv_heads + h;
    const int p = i < mq_clamp(a.token_len[trow], a.token_max_list) ? a.token_list[trow * a.token_max_list + i] : -1;
    if (p >= 0 && p < n) atomicOr(&bits[p >> 2], 1u << ((p & 3) * 8 + t));
  }
  __syncthreads();
  // thread k owns the words [k per, (k + 1) per) of the byte map (4 pages each; bytes past page n
  // are zero): count its listed pages, block scan, write them in page order
  const int words = (n + 3) / 4;
  const int per = (words + kUnionThreads - 1) / kUnionThreads;
  const int w0 = (int)threadIdx.x * per;
  uint32_t cnt = 0;
  for (int i = 0; i < per; ++i) {
    const int wi = w0 + i;
    if (wi < words) {
      uint32_t x = bits[wi];
      x |= x >> 4;
      x |= x >> 2;
      x |= x >> 1;
      cnt += __popc(x & 0x01010101u);  // bytes that hold any token's bit
    }
  }
  const uint32_t incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) wsum[wave] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wave; ++w) base += wsum[w];
  uint32_t pos = base + incl - cnt;
  for (int i = 0; i < per; ++i) {
    const int wi = w0 + i;
    if (wi >= words) break;
    const uint32_t x = bits[wi];
    if (!x) continue;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t m = (x >> (8 * k)) & 0xffu;
      if (!m) continue;
      const int p = 4 * wi + k;
      if (pos < (uint32_t)a.max_list) {
        a.page_list[out_row + pos] = p;
        a.page_mask[out_row + pos] = m;
        if (a.page_phys) a.page_phys[out_row + pos] = bt_row[p];
      }
      ++pos;
    }
  }
  if (threadIdx.x == kUnionThreads - 1) {
    a.list_len[row] = (int)min(base + incl, (uint32_t)a.max_list);
    if (a.path) a.path[row] = 0;
  }
}

typedef _Float16 mq_half4 __attribute__((ext_vector_type(4)));
typedef _Float16 mq_half8 __attribute__((ext_vector_type(8)));
typedef float mq_float4 __attribute__((ext_vector_type(4)));

struct MqPage {
  int page;  // logical page, -1 when the entry is not usable
  int phys;
  uint32_t mask;
  int valid;
};

// One page's K operand (lane: key l % 16, channels 32 (l / 16) .. + 31) and V rows (lane: channels
// 2 l, 2 l + 1 of every key), as fp16 bits; fp8 pools hold their codes' values times 2^-8 here
// (exact), with the key's scales times 256 beside them.
// One page's K and V as loaded (fp16 values, or E4M3FN codes for fp8 pools): lane l holds key l % 16's
// channels 32 (l / 16) .. + 31, and channels 2 l, 2 l + 1 of every key.  fp8 codes are decoded when the
// page is processed, not when it is loaded, so nothing waits for a page's loads before the next page's
// loads are issued.
template <int KVD> struct MqKV;
template <> struct MqKV<SPD_DTYPE_F16> {
  uint4 k[4];
  uint32_t v[kPage];
};
template <> struct MqKV<SPD_DTYPE_FP8_E4M3FN> {
  uint4 k[2];         // 32 codes
  uint32_t v[kPage];  // two codes per key (low 16 bits)
  uint32_t ks, vs;    // this lane's key (l % 16) K and V scales, fp16 bits (low 16 bits)
};

// A page's loads are issued with no branch around them: an entry that is not a usable page
// (r.page < 0) reads pool page 0 of head h instead, and its values are never used.  The page's addresses are wave-uniform:
// each load is a buffer load from a resource over the page (scalar registers) at this lane's constant
// offset, so issuing a page needs no vector registers beyond the ones it loads into.  A load under a
// branch, or vector address registers reused from a pending load's destination, made the compiler wait
// for the other page's loads first, and only one page was ever in flight.
struct MqLaneOff {
  uint32_t k, v;  // byte offsets of this lane's K channels and V channel pair in a page (key 0)
};
template <int D, int KVD>
__device__ __forceinline__ MqLaneOff mq_lane_offsets() {
  const int lane = threadIdx.x % kWave;
  constexpr uint32_t eb = KVD == SPD_DTYPE_F16 ? 2u : 1u;
  return MqLaneOff{(uint32_t)(((lane & 15) * D + 32 * (lane >> 4)) * eb), (uint32_t)(lane * 2 * eb)};
}

template <int D, int KVD>
__device__ __forceinline__ void mq_load(const MqDecodeArgs& a, const MqPage& r, int h, const MqLaneOff& off,
                                        MqKV<KVD>& kv) {
  const int lane = threadIdx.x % kWave;
  constexpr uint32_t eb = KVD == SPD_DTYPE_F16 ? 2u : 1u;
  constexpr uint32_t page_bytes = kPage * D * eb;
  const size_t head_page = (size_t)(r.page < 0 ? 0 : r.phys) * a.num_kv_heads + h;
  const __amdgpu_buffer_rsrc_t kr = make_rsrc(reinterpret_cast<const uint8_t*>(a.k_pool) + head_page * page_bytes, page_bytes);
  const __amdgpu_buffer_rsrc_t vr = make_rsrc(reinterpret_cast<const uint8_t*>(a.v_pool) + head_page * page_bytes, page_bytes);
  if constexpr (KVD == SPD_DTYPE_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) kv.k[i] = buf_load_u32x4_nt(kr, off.k + 16u * i);
#pragma unroll
    for (int t = 0; t < kPage; ++t) kv.v[t] = buf_load_u32_nt(vr, off.v + (uint32_t)t * D * eb);
  } else {  // E4M3FN codes: 32 of the key's channels, two of every key's
    kv.k[0] = buf_load_u32x4_nt(kr, off.k);
    kv.k[1] = buf_load_u32x4_nt(kr, off.k + 16u);
#pragma unroll
    for (int t = 0; t < kPage; ++t) kv.v[t] = buf_load_u16_nt(vr, off.v + (uint32_t)t * D * eb);
    const __amdgpu_buffer_rsrc_t kscr = make_rsrc(a.k_scale + head_page * kPage, kPage * 2u);
    const __amdgpu_buffer_rsrc_t vscr = make_rsrc(a.v_scale + head_page * kPage, kPage * 2u);
    kv.ks = buf_load_u16_nt(kscr, (uint32_t)(lane & 15) * 2u);
    kv.vs = buf_load_u16_nt(vscr, (uint32_t)(lane & 15) * 2u);
  }
}

// This lane's key scales times 256 (fp8 pools; 1 for fp16 pools, whose scales are not used), decoded
// when the page is processed.
template <int KVD> __device__ __forceinline__ float mq_kscale(const MqKV<KVD>& kv) {
  if constexpr (KVD == SPD_DTYPE_F16) return 1.f;
  else return half_bits_to_float((uint16_t)kv.ks) * 256.f;
}
template <int KVD> __device__ __forceinline__ float mq_vscale(const MqKV<KVD>& kv) {
  if constexpr (KVD == SPD_DTYPE_F16) return 1.f;
  else return half_bits_to_float((uint16_t)kv.vs) * 256.f;
}

// The page's K operand (fp16, 32 channels) and V values (two fp16 channels per key) of this lane: the
// loaded values, or fp8 codes decoded exactly to fp16 (value times 2^-8; the scales come later).
template <int KVD>
__device__ __forceinline__ void mq_unpack(const MqKV<KVD>& kv, uint4 (&k)[4], uint32_t (&v)[kPage]) {
  if constexpr (KVD == SPD_DTYPE_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = kv.k[i];
#pragma unroll
    for (int t = 0; t < kPage; ++t) v[t] = kv.v[t];
  } else {
    const uint32_t w[8] = {kv.k[0].x, kv.k[0].y, kv.k[0].z, kv.k[0].w, kv.k[1].x, kv.k[1].y, kv.k[1].z, kv.k[1].w};
    uint32_t hk[16];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      hk[2 * i] = fp8x2_to_half2_scaled(w[i] & 0xffffu);
      hk[2 * i + 1] = fp8x2_to_half2_scaled(w[i] >> 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) k[i] = make_uint4(hk[4 * i], hk[4 * i + 1], hk[4 * i + 2], hk[4 * i + 3]);
#pragma unroll
    for (int t = 0; t < kPage; ++t) v[t] = fp8x2_to_half2_scaled(kv.v[t] & 0xffffu);
  }
}

template <int D, int KVD>
__global__ __launch_bounds__(256) void mq_decode_kernel(MqDecodeArgs a) {
  static_assert(D == 128, "the logit tile covers 128 channels: 4 lane groups x 32");
  __shared__ _Float16 p16[4][kMqRows][kPage];  // P of the wave's page, [row][key]
  __shared__ float al_lds[4][kMqRows];           // each row's rescale of the page
  __shared__ uint4 vt[4][D][2];                  // V^T of the wave's page: channel c's 16 keys (fp16)
  __shared__ float ws_m[4][kMqRows], ws_l[4][kMqRows];
  __shared__ float ws_acc[4][kMqRows][D];
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int tok = lane & 15;  // logit role: key of the page
  const int q4 = lane >> 4;   // logit role: query token of rows 4 q4 .. 4 q4 + 3
  const int row = blockIdx.x / a.blocks_per_row;
  const int j = blockIdx.x % a.blocks_per_row;
  const int b = row / a.num_kv_heads;
  const int h = row % a.num_kv_heads;
  const int T = a.num_tokens;
  auto out_row = [&](int t, int g) { return ((size_t)b * T + t) * a.num_q_heads + (size_t)h * kMqG + g; };

  const int n = mq_clamp(a.list_len[row], a.max_list);
  if (n == 0) {
    if (j == 0) {
      for (int e = threadIdx.x; e < T * kMqG * D; e += blockDim.x)
        a.out[out_row(e / (kMqG * D), (e / D) % kMqG) * D + e % D] = 0.f;
      if ((int)threadIdx.x < T * kMqG) a.out_lse[out_row(threadIdx.x / kMqG, threadIdx.x % kMqG)] = -INFINITY;
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
  const int lim = len - T + 1 + q4;  // keys this lane's query token may see: positions < lim

  // A operand: query row l % 16 = (t_a, g_a), channels 32 q4 .. 32 q4 + 31
  const int t_a = tok >> 2, g_a = tok & 3;
  mq_half8 qa[4];
  {
    uint4 w[4] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    if (t_a < T) {
      const uint4* qp = reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(a.q) + out_row(t_a, g_a) * D +
                                                       32 * q4);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = qp[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qa[i] = __builtin_bit_cast(mq_half8, w[i]);
    }
  }

  float m_run[4], l_run[4];
  mq_float4 acc[D / 16];  // O^T tile s: lane l holds channels 16 s + 4 (l / 16) .. + 3 of row l % 16
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    m_run[jj] = -INFINITY;
    l_run[jj] = 0.f;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = mq_float4{0.f, 0.f, 0.f, 0.f};
  // fp8: acc holds the PV sums in units of 2^e_acc, e_acc being the exponent bound of the last page's
  // largest V scale (the same in every lane); f16 keeps e_acc = 0
  int e_acc = 0;

  auto process = [&](const MqPage& r, const MqKV<KVD>& kv) {
    if (r.page < 0) return;
    uint4 kk[4];
    uint32_t vv[kPage];
    mq_unpack<KVD>(kv, kk, vv);
    mq_float4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s = __builtin_amdgcn_mfma_f32_16x16x32_f16(qa[i], __builtin_bit_cast(mq_half8, kk[i]), s, 0, 0, 0);
    }
    const bool ok = q4 < T && ((r.mask >> q4) & 1u) && r.page * kPage + tok < lim && tok < r.valid;
    // fp8: key tok's K scale on its logit column; its V scale on its probabilities (P times the scale
    // is what V's fp16 values times 2^8 are weighted with).  Slots past the request's end (scales may
    // be NaN) are masked before either is used.
    const float kscale = KVD == SPD_DTYPE_F16 ? a.sm_scale_log2 : a.sm_scale_log2 * (ok ? mq_kscale<KVD>(kv) : 0.f);
    // fp8: the probabilities carry each key's V scale over 2^e_pg, the power of two just above the page's
    // largest scale (so under 1: the fp16 operand neither overflows nor loses precision to small scales);
    // the accumulator moves to units of 2^e_pg below, exactly, since every factor is a power of two
    int e_pg = 0;
    if constexpr (KVD != SPD_DTYPE_F16) {
      const float vmax = row_max(tok < r.valid ? mq_vscale<KVD>(kv) : 0.f);  // the page's 16 tokens, one per lane of the row
      e_pg = vmax > 0.f ? __builtin_amdgcn_frexp_expf(vmax) : 0;  // vmax < 2^e_pg
    }
    const float vscale = KVD == SPD_DTYPE_F16 ? 1.f : (ok ? __builtin_amdgcn_ldexpf(mq_vscale<KVD>(kv), -e_pg) : 0.f);
    float p[4], alpha[4];
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const float x = ok ? s[jj] * kscale : -INFINITY;
      const float m_new = fmaxf(m_run[jj], row_max(x));
      alpha[jj] = m_new == -INFINITY ? 1.f : exp2f(m_run[jj] - m_new);
      p[jj] = m_new == -INFINITY ? 0.f : exp2f(x - m_new);
      l_run[jj] = l_run[jj] * alpha[jj] + p[jj];
      m_run[jj] = m_new;
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) p16[wave][4 * q4 + jj][tok] = (_Float16)(p[jj] * vscale);
    if (tok == 0) *reinterpret_cast<float4*>(&al_lds[wave][4 * q4]) = make_float4(alpha[0], alpha[1], alpha[2], alpha[3]);
    // V^T: this lane's channels 2 l (low halves) and 2 l + 1 (high halves) of the 16 keys, keys past
    // the request's end zeroed (their slots may hold NaN, and 0 x NaN would reach every row)
    uint32_t v[kPage];
#pragma unroll
    for (int t = 0; t < kPage; ++t) v[t] = t < r.valid ? vv[t] : 0u;
    uint32_t lo[kPage / 2], hi[kPage / 2];
#pragma unroll
    for (int i = 0; i < kPage / 2; ++i) {
      lo[i] = __builtin_amdgcn_perm(v[2 * i + 1], v[2 * i], 0x05040100u);  // low halves of keys 2 i, 2 i + 1
      hi[i] = __builtin_amdgcn_perm(v[2 * i + 1], v[2 * i], 0x07060302u);  // high halves
    }
    vt[wave][2 * lane][0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    vt[wave][2 * lane][1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    vt[wave][2 * lane + 1][0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    vt[wave][2 * lane + 1][1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    wave_fence();
    // B = P^T: row l % 16, keys 4 q4 .. 4 q4 + 3; A = V^T tile s: channel 16 s + l % 16, the same keys
    const mq_half4 pb = *reinterpret_cast<const mq_half4*>(&p16[wave][tok][4 * q4]);
    const float al = al_lds[wave][tok];
    // fp8: in units of 2^e_pg, acc = acc al 2^(e_acc - e_pg) + V^T P'^T
    const float pre = KVD == SPD_DTYPE_F16 ? al : __builtin_amdgcn_ldexpf(al, e_acc - e_pg);
    e_acc = e_pg;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      const uint2 va = reinterpret_cast<const uint2*>(&vt[wave][16 * t + tok][0])[q4];
      acc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(mq_half4, va), pb, acc[t] * pre, 0, 0, 0);
    }
    wave_fence();
  };

  // This wave's entries are i0 + wave, i0 + wave + 4, ...; their list entries, masks and physical
  // pages are read 64 at a time (one per lane) before the K / V loads; pages alternate between two
  // register stages so the next page's loads are in flight while the current one is computed.
  const int32_t* list = a.page_list + (size_t)row * a.max_list;
  const uint32_t* mlist = a.page_mask + (size_t)row * a.max_list;
  const int32_t* plist = a.page_phys ? a.page_phys + (size_t)row * a.max_list : nullptr;
  const int my_pages = i1 - i0 > wave ? (i1 - i0 - wave + 3) / 4 : 0;
  auto page_at = [&](int lp, int lph, uint32_t lm, int u) {
    MqPage r{-1, 0, 0u, 0};
    const int p = __builtin_amdgcn_readlane(lp, u);
    const int phys = __builtin_amdgcn_readlane(lph, u);
    if (p < 0 || p >= n_b || phys < 0 || phys >= a.num_pool_pages) return r;
    r.page = p;
    r.phys = phys;
    r.mask = (uint32_t)__builtin_amdgcn_readlane((int)lm, u);
    r.valid = valid_in_page(len, p);
    return r;
  };
  MqKV<KVD> kv[kMqStages];  // ring of page buffers: page u lives in slot u mod kMqStages
  const MqLaneOff off = mq_lane_offsets<D, KVD>();
  MqPage rp[kMqStages];
  for (int bb = 0; bb < my_pages; bb += kWave) {
    const int cnt = min(kWave, my_pages - bb);
    const int idx = i0 + wave + 4 * (bb + lane);
    int lp = -1, lph = -1;
    uint32_t lm = 0u;
    if (lane < cnt) {
      lp = list[idx];
      lm = mlist[idx];
      if (plist) lph = plist[idx];
      else if (lp >= 0 && lp < n_b) lph = a.block_table[(size_t)b * a.max_pages + lp];
    }
    // Page u + 1's loads are issued before page u is processed.  Inside the loop every load is a real
    // page of the batch, so no wave reads a page it does not use; the last page (or the last two) is
    // processed after the loop with no load behind it.
    static_assert(kMqStages == 2, "the ring below alternates two slots");
    rp[0] = page_at(lp, lph, lm, 0);
    mq_load<D, KVD>(a, rp[0], h, off, kv[0]);
    int u = 0;
    for (; u + 2 < cnt; u += 2) {
      rp[1] = page_at(lp, lph, lm, u + 1);
      mq_load<D, KVD>(a, rp[1], h, off, kv[1]);
      process(rp[0], kv[0]);
      rp[0] = page_at(lp, lph, lm, u + 2);
      mq_load<D, KVD>(a, rp[0], h, off, kv[0]);
      process(rp[1], kv[1]);
    }
    if (u + 1 < cnt) {  // two pages left: the second's loads go out before the first is processed
      rp[1] = page_at(lp, lph, lm, u + 1);
      mq_load<D, KVD>(a, rp[1], h, off, kv[1]);
      process(rp[0], kv[0]);
      process(rp[1], kv[1]);
    } else {
      process(rp[0], kv[0]);
    }
  }

  // wave states -> LDS (row 4 q4 + jj is held by lane group q4; its sum spans the group's 16 lanes)
#pragma unroll
  for (int jj = 0; jj < 4; ++jj) {
    const float lt = row_sum(l_run[jj]);
    if (tok == 0) {
      ws_m[wave][4 * q4 + jj] = m_run[jj];
      ws_l[wave][4 * q4 + jj] = lt;
    }
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    mq_float4 o = acc[t];
    if constexpr (KVD != SPD_DTYPE_F16) {
#pragma unroll
      for (int c = 0; c < 4; ++c) o[c] = __builtin_amdgcn_ldexpf(o[c], e_acc);  // back from units of 2^e_acc
    }
    *reinterpret_cast<float4*>(&ws_acc[wave][tok][16 * t + 4 * q4]) = make_float4(o[0], o[1], o[2], o[3]);
  }
  __syncthreads();

  // merge the four wave states.  Each wave first takes the 64 (row, wave) weights in its own lanes --
  // lane l holds row l / 4 and wave state l % 4: the row's largest log-sum, the state's weight
  // exp2(m_w - M) / L and the row's log-sum-exp -- so the per-channel pass below is four fused
  // multiply-adds with the weights read from those lanes.
  const int fr = lane >> 2, fw = lane & 3;
  const float mw = ws_m[fw][fr];
  float M = fmaxf(mw, __uint_as_float(dpp<0xb1>(__float_as_uint(mw))));  // lane ^ 1
  M = fmaxf(M, __uint_as_float(dpp<0x4e>(__float_as_uint(M))));          // lane ^ 2
  const float sc = M == -INFINITY ? 0.f : exp2f(mw - M);
  float L = ws_l[fw][fr] * sc;
  L += __uint_as_float(dpp<0xb1>(__float_as_uint(L)));
  L += __uint_as_float(dpp<0x4e>(__float_as_uint(L)));
  const float fac = M == -INFINITY ? 0.f : sc / L;
  const int rows_out = T * kMqG;
  if (wave == 0 && fw == 0 && fr < rows_out) {
    const float lse = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
    if (m == 1) a.out_lse[out_row(fr / kMqG, fr % kMqG)] = lse;
    else a.part_lse[((size_t)row * a.blocks_per_row + j) * kMqRows + fr] = lse;
  }
  // this thread: channel threadIdx.x % D of rows 2 i + wave / 2 (uniform over the wave)
  const int ch = (int)threadIdx.x % D;
  const int half = __builtin_amdgcn_readfirstlane(wave >> 1);
  for (int rr = half; rr < rows_out; rr += 2) {
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      o = fmaf(ws_acc[w][rr][ch], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fac), 4 * rr + w)), o);
    if (m == 1) a.out[out_row(rr / kMqG, rr % kMqG) * D + ch] = o;
    else a.part_o[(((size_t)row * a.blocks_per_row + j) * kMqRows + rr) * D + ch] = o;
  }
}

int launch_page_list_union(const UnionArgs& a, hipStream_t stream) {
  const size_t lds = (size_t)((a.max_pages + 3) / 4) * sizeof(uint32_t);
  const dim3 grid((unsigned)(a.batch * a.num_kv_heads)), block(kUnionThreads);
  if (a.max_pages >= kUnionRankMinPages) hipLaunchKernelGGL(page_list_union_kernel<true>, grid, block, lds, stream, a);
  else hipLaunchKernelGGL(page_list_union_kernel<false>, grid, block, lds, stream, a);
  return 0;
}

int launch_mq_decode(const MqDecodeArgs& a, int head_dim, int kv_dtype, hipStream_t stream) {
  if (head_dim != 128) return SPD_ERR_UNSUPPORTED;
  const dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.blocks_per_row)), block(256);
  if (kv_dtype == SPD_DTYPE_F16) hipLaunchKernelGGL((mq_decode_kernel<128, SPD_DTYPE_F16>), grid, block, 0, stream, a);
  else if (kv_dtype == SPD_DTYPE_FP8_E4M3FN)
    hipLaunchKernelGGL((mq_decode_kernel<128, SPD_DTYPE_FP8_E4M3FN>), grid, block, 0, stream, a);
  else return SPD_ERR_UNSUPPORTED;
  return 0;
}

}  // namespace spd
