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
// For one 16-token page a wave needs no LDS staging: lane l = 16 q + t reads token t, channel
// quarter q of K (16-byte loads), and channels [l*d/64, (l+1)*d/64) of V for all 16 tokens
// (one 256-byte row per instruction).  The G = 4 partial dot products of a lane are
// reduce-scattered over the four lanes of its token (gfx950's permlane16 / permlane32 swaps
// exchange rows of 16 lanes in one VALU instruction) so that lane 16 h + t ends with the full
// logit of head h and token t: each 16-lane row is one head, and the softmax max / sum over
// the page's tokens are row reductions through DPP.  The 64 probabilities go through 1 KiB of
// LDS so every lane can apply all of them to its V channels; the waves' states are merged in
// LDS at the end.
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
  static constexpr uint32_t EB = 2;  // bytes per element
  // byte offsets in a 16-token page of this lane's K chunk 0 (token tok) and V channels (token 0)
  __device__ static uint32_t k_off(int tok, int quarter) { return (uint32_t)(tok * D + quarter * 8) * EB; }
  __device__ static uint32_t v_off(int lane) { return (uint32_t)(lane * CPL) * EB; }
  __device__ static void load_k(KF& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int s = 0; s < NS; ++s) f.k[s] = buf_load_u32x4_nt(r, off + (uint32_t)s * 32 * EB);
  }
  __device__ static void load_v(VF& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int t = 0; t < kPage; ++t) {
      if constexpr (CPL == 2) f.v[t] = buf_load_u32_nt(r, off + (uint32_t)t * D * EB);
      else f.v[t] = (uint16_t)buf_load_u16_nt(r, off + (uint32_t)t * D * EB);
    }
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
  static constexpr uint32_t EB = 1;
  __device__ static uint32_t k_off(int tok, int quarter) { return (uint32_t)(tok * D + quarter * 16); }
  __device__ static uint32_t v_off(int lane) { return (uint32_t)(lane * CPL); }
  __device__ static void load_k(KF& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int s = 0; s < NS; ++s) f.k[s] = buf_load_u32x4_nt(r, off + (uint32_t)s * 64);
  }
  __device__ static void load_v(VF& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int t = 0; t < kPage; ++t) f.v[t] = (uint16_t)buf_load_u16_nt(r, off + (uint32_t)t * D);
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
  static constexpr uint32_t EB = 4;
  __device__ static uint32_t k_off(int tok, int quarter) { return (uint32_t)(tok * D + quarter * 4) * EB; }
  __device__ static uint32_t v_off(int lane) { return (uint32_t)(lane * CPL) * EB; }
  __device__ static void load_k(KF& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint4 w = buf_load_u32x4_nt(r, off + (uint32_t)s * 16 * EB);
      f.k[s] = make_float4(__uint_as_float(w.x), __uint_as_float(w.y), __uint_as_float(w.z), __uint_as_float(w.w));
    }
  }
  __device__ static void load_v(VF& f, __amdgpu_buffer_rsrc_t r, uint32_t off) {
#pragma unroll
    for (int t = 0; t < kPage; ++t)
#pragma unroll
      for (int c = 0; c < CPL; ++c) f.v[t][c] = __uint_as_float(buf_load_u32_nt(r, off + (uint32_t)(t * D + c) * EB));
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

// ------------------------------------------------------------ step-wide (balanced) split
constexpr int kMaxChunks = 1024;  // chunks of one row the merge holds

__device__ __forceinline__ int clamp_len(int n, int max_list) { return n < 0 ? 0 : (n > max_list ? max_list : n); }

// Work units of a row: its list entries, 2^lgs 16-token units per entry (hierarchical paging: an
// entry is a physical page of 2^lgs logical pages, each processed like a 16-token page).
__device__ __forceinline__ int row_units(const int32_t* list_len, int r, int max_list, int lgs) {
  return clamp_len(list_len[r], max_list) << lgs;
}

// Chunk size of the balanced plan, c = max(C, ceil(T / N'), ceil(n_max / kMaxChunks)) with N' = N_T - z
// (z rows with a non-empty list) when N_T > z, else N_T, from every row's list length (computed by the
// calling wave; every lane receives it).
__device__ __forceinline__ int balanced_chunk(const int32_t* list_len, int rows, int max_list, int C, int NT, int lgs) {
  const int lane = threadIdx.x % kWave;
  unsigned long long tot = 0;
  uint32_t nmax = 0, nz = 0;
  for (int r0 = 0; r0 < rows; r0 += kWave) {
    const int r = r0 + lane;
    const int n = r < rows ? row_units(list_len, r, max_list, lgs) : 0;
    tot += (unsigned long long)n;
    nmax = max(nmax, (uint32_t)n);
    nz += n > 0 ? 1u : 0u;
  }
  tot = wave_sum(tot);
  nmax = wave_max(nmax);
  nz = (uint32_t)wave_sum((unsigned long long)nz);
  // each of the nz non-empty rows rounds its chunk count up by less than one, so with
  // c >= T / (N_T - nz) the chunks number fewer than T / c + nz <= N_T: the plan fills the N_T
  // blocks meant to be resident at once and no chunk waits for a second round
  const unsigned long long slots = (unsigned long long)NT > nz ? (unsigned long long)NT - nz : (unsigned long long)NT;
  unsigned long long c = (unsigned long long)C;
  c = max(c, (tot + slots - 1) / slots);
  c = max(c, (unsigned long long)((nmax + kMaxChunks - 1) / kMaxChunks));
  return (int)c;
}

// Chunk k of the balanced plan: its row, its index j in the row, the row's chunk count m, the
// number of the row's first chunk and the row's list length.  False when k is past the last chunk.
struct ChunkPos {
  int row, j, m, first, n;
};

__device__ __forceinline__ bool balanced_locate(const int32_t* list_len, int rows, int max_list, int c, int k,
                                                ChunkPos& cp, int lgs) {
  const int lane = threadIdx.x % kWave;
  uint32_t base = 0;
  for (int r0 = 0; r0 < rows; r0 += kWave) {
    const int r = r0 + lane;
    const int n = r < rows ? row_units(list_len, r, max_list, lgs) : 0;
    const uint32_t m = (uint32_t)((n + c - 1) / c);
    const uint32_t incl = wave_incl_scan(m) + base;
    const unsigned long long hit = __ballot(m > 0 && incl > (uint32_t)k && incl - m <= (uint32_t)k);
    if (hit) {
      const int l = __ffsll((long long)hit) - 1;
      cp.row = r0 + l;
      cp.m = (int)lane_u32(m, l);
      cp.first = (int)(lane_u32(incl, l) - (uint32_t)cp.m);
      cp.j = k - cp.first;
      cp.n = (int)lane_u32((uint32_t)n, l);
      return true;
    }
    base = lane_u32(incl, kWave - 1);
  }
  return false;
}

// First chunk number and chunk count of row `row` in the balanced plan.
__device__ __forceinline__ void balanced_row(const int32_t* list_len, int rows, int max_list, int c, int row,
                                             int& first, int& m, int lgs) {
  const int lane = threadIdx.x % kWave;
  uint32_t base = 0;
  for (int r0 = 0; r0 < rows; r0 += kWave) {
    const int r = r0 + lane;
    const int n = r < rows ? row_units(list_len, r, max_list, lgs) : 0;
    const uint32_t mm = (uint32_t)((n + c - 1) / c);
    const uint32_t incl = wave_incl_scan(mm) + base;
    if (row < r0 + kWave) {
      const int l = row - r0;
      m = (int)lane_u32(mm, l);
      first = (int)(lane_u32(incl, l) - (uint32_t)m);
      return;
    }
    base = lane_u32(incl, kWave - 1);
  }
  first = 0;
  m = 0;
}

struct PageRef {
  int page;   // logical page, -1 when the entry is not a usable page
  int phys;
  int valid;  // valid tokens
};

// Page i of this wave's batch: its logical page (lane i of `lp`), its physical page (lane i of
// `lph`) and valid token count, broadcast to the whole wave (uniform values, scalar addresses).
__device__ __forceinline__ PageRef batch_page(int lp, int lph, int i, int n_b, int len, int num_pool_pages) {
  PageRef r{-1, 0, 0};
  const int p = __builtin_amdgcn_readlane(lp, i);
  const int phys = __builtin_amdgcn_readlane(lph, i);
  if (p < 0 || p >= n_b || phys < 0 || phys >= num_pool_pages) return r;
  r.page = p;
  r.phys = phys;
  r.valid = valid_in_page(len, p);
  return r;
}

// Fused merge (the last-block variant of decode + merge): after writing its chunk state, a block
// makes it visible device-wide and takes a ticket on its row; the block that takes the last ticket
// reads every chunk state of the row, merges them exactly (PersistentKV, section 3.3) and leaves the
// ticket at zero for the next call.  No block waits for another.
template <int D>
__device__ __forceinline__ void merge_row_in_block(const DecodeArgs& a, int row, int m, size_t slot_row, size_t qrow) {
  __shared__ int last;
  __shared__ float w_s[kMaxChunks][kGq];  // chunk weights exp(lse_j - M_g); m <= kMaxChunks in both plans
  __shared__ float mg[kGq], sg[kGq];
  __threadfence();  // release this block's chunk state (agent scope)
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(&a.counters[row], 1u) == (unsigned)(m - 1);
  __syncthreads();
  if (!last) return;
  __threadfence();  // acquire the other blocks' chunk states
  // every chunk log-sum-exp at once; wave g folds head g's max and weight sum
  for (int e = threadIdx.x; e < m * kGq; e += blockDim.x) w_s[e / kGq][e % kGq] = a.part_lse[slot_row * kGq + e];
  __syncthreads();
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;  // 4 waves, one per head
  {
    float M = -INFINITY;
    for (int jj = lane; jj < m; jj += kWave) M = fmaxf(M, w_s[jj][wave]);
    M = wave_max_f(M);
    float S = 0.f;
    for (int jj = lane; jj < m; jj += kWave) {
      const float w = M == -INFINITY ? 0.f : expf(w_s[jj][wave] - M);
      w_s[jj][wave] = w;
      S += w;
    }
    S = wave_sum_f(S);
    if (lane == 0) {
      mg[wave] = M;
      sg[wave] = S;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < kGq * D; e += blockDim.x) {
    const int g = e / D, ch = e % D;
    float acc = 0.f;
#pragma unroll 8
    for (int jj = 0; jj < m; ++jj) acc = fmaf(w_s[jj][g], a.part_o[((slot_row + jj) * kGq + g) * D + ch], acc);
    const bool empty = mg[g] == -INFINITY;
    a.out[(qrow + g) * D + ch] = empty ? 0.f : acc / sg[g];
    if (ch == 0) a.out_lse[qrow + g] = empty ? -INFINITY : mg[g] + logf(sg[g]);
  }
  if (threadIdx.x == 0) a.counters[row] = 0u;
}

// MERGE: the row's chunk states are merged by the last of its blocks to finish (a ticket per row in
// a.counters), in the same launch; see merge_row_in_block.
template <int D, int QD, int KVD, bool MERGE = false>
__global__ __launch_bounds__(256) void sparse_paged_decode_kernel(DecodeArgs a) {
  using T = DecTraits<D, QD, KVD>;
  constexpr int CPL = T::CPL;
  __shared__ float p_lds[4][kPage][kGq];
  __shared__ float ws_m[4][kGq], ws_l[4][kGq];
  __shared__ float ws_acc[4][kGq][D];

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int tok = lane & (kPage - 1);  // QK role: token of the page
  const int quarter = lane >> 4;       // QK role: channel quarter, and after the reduce-scatter the head
  // Which chunk of which row this block processes: per-row plan (Moira Eq. 4, block (row, j)),
  // or the step-wide plan (block k takes chunk k of the row-by-row numbering).
  int row, j, c = 0, m = 0, n = 0;
  size_t slot_row;  // partial-state slot of chunk 0 of the row: row * J, or the row's first chunk number
  if (a.balanced) {
    const int rows = a.batch * a.num_kv_heads;
    c = balanced_chunk(a.list_len, rows, a.max_list, a.min_chunk, a.grid_target, a.lgs);
    if ((int)blockIdx.x < rows && clamp_len(a.list_len[blockIdx.x], a.max_list) == 0) {
      // row blockIdx.x has no chunk: this block writes its empty result
      const size_t q0 = (size_t)(blockIdx.x / a.num_kv_heads) * a.num_q_heads + (size_t)(blockIdx.x % a.num_kv_heads) * kGq;
      for (int e = threadIdx.x; e < kGq * D; e += blockDim.x) a.out[q0 * D + e] = 0.f;
      if (threadIdx.x < kGq) a.out_lse[q0 + threadIdx.x] = -INFINITY;
    }
    ChunkPos cp;
    if (!balanced_locate(a.list_len, rows, a.max_list, c, (int)blockIdx.x, cp, a.lgs)) return;
    row = cp.row;
    j = cp.j;
    m = cp.m;
    n = cp.n;
    slot_row = (size_t)cp.first;
  } else {
    row = blockIdx.x / a.blocks_per_row;
    j = blockIdx.x % a.blocks_per_row;
    slot_row = (size_t)row * a.blocks_per_row;
    // The argument block's pointers this prologue uses are held here, so their loads are waited for
    // once, now; the row's list length is requested right after.  (A scalar-load wait covers every
    // scalar load in flight, so an argument fetched after the length would wait for the length too,
    // and the query loads behind it.)
    asm volatile("" ::"s"(a.q), "s"(a.page_list), "s"(a.page_phys), "s"(a.seq_lens), "s"(a.list_len));
    n = ((ConstI32Ptr)a.list_len)[row];
  }
  const int b = row / a.num_kv_heads;
  const int h = row % a.num_kv_heads;
  const size_t qrow = (size_t)b * a.num_q_heads + (size_t)h * kGq;  // first query head of the group
  // the request's length, requested as soon as the row is known (per-row plan: with the list length
  // and the list entries, so no round trip of its own comes before the first K / V loads)
  const int len = ((ConstI32Ptr)a.seq_lens)[b];

  const int32_t* list = a.page_list + (size_t)row * a.max_list;
  const int32_t* plist = a.page_phys ? a.page_phys + (size_t)row * a.max_list : nullptr;
  // Per-row plan: the list entries of this wave's first 64 pages are requested together with the
  // row's list length, assuming the row's list is full (max_list entries: a top-K row holding its
  // budget), so the chunk is the plan's for that length (taken on the host) -- the minimum chunk
  // whenever max_list fits in J * min_chunk; otherwise they are read again.
  const int spec_i0 = a.balanced ? -1 : j * a.spec_chunk;
  int spec_lp = -1, spec_lph = -1;  // list entry (physical page slot when lgs > 0) and physical page of the unit
  // the row's list and physical pages through range-checked loads: entries past max_list read 0, with
  // no branch around each read
  const __amdgpu_buffer_rsrc_t list_r = make_rsrc(list, (uint32_t)a.max_list * 4u);
  const __amdgpu_buffer_rsrc_t plist_r = make_rsrc(plist, plist ? (uint32_t)a.max_list * 4u : 0u);
  // Nothing here waits for these loads: the queries and the list length are requested behind them.
  // Only lanes below the batch's page count use their entry, and those pages lie below the list
  // length, so their entries are inside the list.
  if (!a.balanced) {
    const int e = (spec_i0 + wave + 4 * lane) >> a.lgs;
    spec_lp = buf_load_i32(list_r, (uint32_t)e * 4u);
    spec_lph = buf_load_i32(plist_r, (uint32_t)e * 4u);
  }
  typename T::Q q;
  T::load_q(q, a.q, qrow * D, quarter);
  if (!a.balanced) {
    n = clamp_len(n, a.max_list) << a.lgs;  // the row's work units (row_units)
    if (n == 0) {
      if (j == 0) {
        for (int e = threadIdx.x; e < kGq * D; e += blockDim.x) a.out[qrow * D + e] = 0.f;
        if (threadIdx.x < kGq) a.out_lse[qrow + threadIdx.x] = -INFINITY;
      }
      return;
    }
    plan_chunks(n, a.blocks_per_row, a.min_chunk, c, m);
    if (j >= m) return;
  }
  const int i0 = j * c;
  const int i1 = min(n, i0 + c);
  const int n_b = row_logical_pages(len, a.max_pages, a.lgs);   // 16-token pages of the request
  const int n_phys = row_phys_pages(len, a.max_pages, a.lgs);   // list entries must be below this
  const int sub_mask = (1 << a.lgs) - 1;

  float m_run = -INFINITY, l_run = 0.f;
  float acc[kGq][CPL];
#pragma unroll
  for (int g = 0; g < kGq; ++g)
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) acc[g][cc] = 0.f;

  // Pages of this wave alternate between two register stages, so the next page's K / V
  // loads are in flight while the current page is computed.
  // A page's loads are issued with no branch around them (an entry that is not a usable page reads
  // pool unit 0 instead; its values are never used), as buffer loads from a resource over the 16-token
  // unit -- built in scalar registers from the wave-uniform page -- at this lane's constant offsets, and
  // fp8 scales stay fp16 bits until the page is processed.  A load under a branch, vector address
  // registers reused from a pending load's destination, or a decode right after the load made the
  // compiler wait for every outstanding load before the next page's, so one page was in flight.
  constexpr uint32_t unit_bytes = kPage * D * T::EB;
  const uint32_t k_lane = T::k_off(tok, quarter), v_lane = T::v_off(lane);
  auto load = [&](const PageRef& r, typename T::KF& kd, typename T::VF& vd, uint32_t& ksd, uint32_t& vsd) {
    const size_t head_page = head_unit(r.page < 0 ? 0 : r.phys, a.num_kv_heads, h, a.lgs, r.page < 0 ? 0 : r.page & sub_mask);
    T::load_k(kd, make_rsrc(reinterpret_cast<const uint8_t*>(a.k_pool) + head_page * unit_bytes, unit_bytes), k_lane);
    T::load_v(vd, make_rsrc(reinterpret_cast<const uint8_t*>(a.v_pool) + head_page * unit_bytes, unit_bytes), v_lane);
    if constexpr (T::kScaled) {
      ksd = buf_load_u16_nt(make_rsrc(a.k_scale + head_page * kPage, kPage * 2u), (uint32_t)tok * 2u);
      vsd = buf_load_u16_nt(make_rsrc(a.v_scale + head_page * kPage, kPage * 2u), (uint32_t)tok * 2u);
    }
  };
  auto process = [&](const PageRef& r, const typename T::KF& kf, const typename T::VF& vf, uint32_t ks_bits,
                     uint32_t vs_bits) {
    if (r.page < 0) return;
    const float ks = T::kScaled ? half_bits_to_float((uint16_t)ks_bits) * 256.f : 1.f;
    const float vs = T::kScaled ? half_bits_to_float((uint16_t)vs_bits) * 256.f : 1.f;
    // logits: partial dots over this lane's channel quarter, reduce-scattered over the quad
    float part[kGq];
    T::dots(q, kf, part);
    const int b0 = quarter & 1, b1 = quarter >> 1;
    const float send0 = b0 ? part[0] : part[1];
    const float send1 = b0 ? part[2] : part[3];
    const float keep0 = b0 ? part[1] : part[0];
    const float keep1 = b0 ? part[3] : part[2];
    const float hA = keep0 + xor16(send0);  // head b0
    const float hB = keep1 + xor16(send1);  // head 2 + b0
    const float keep2 = b1 ? hB : hA;
    const float send2 = b1 ? hA : hB;
    const float dot = keep2 + xor32(send2);  // head `quarter`, token `tok`
    float x = dot * a.sm_scale_log2 * ks;
    if (tok >= r.valid) x = -INFINITY;
    const float mx = row_max(x);
    const float m_new = fmaxf(m_run, mx);
    const float alpha = m_new == -INFINITY ? 1.f : exp2f(m_run - m_new);
    const float p = m_new == -INFINITY ? 0.f : exp2f(x - m_new);
    l_run = l_run * alpha + p;
    m_run = m_new;
    p_lds[wave][tok][quarter] = tok < r.valid ? p * vs : 0.f;  // invalid slots' scales may be NaN
    float alv[kGq];  // each head's rescale, read from its row
#pragma unroll
    for (int g = 0; g < kGq; ++g) alv[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), g * 16));
    wave_fence();
#pragma unroll
    for (int g = 0; g < kGq; ++g)
#pragma unroll
      for (int cc = 0; cc < CPL; ++cc) acc[g][cc] *= alv[g];
    float4 pt[kPage];  // every probability of the page, read in one batch
#pragma unroll
    for (int t = 0; t < kPage; ++t) pt[t] = *reinterpret_cast<const float4*>(p_lds[wave][t]);
    if (r.valid == kPage) {  // full page (every page but a request's last): no masking
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        const float pv[kGq] = {pt[t].x, pt[t].y, pt[t].z, pt[t].w};
        float v[CPL];
        T::v_values(vf, t, v);
#pragma unroll
        for (int g = 0; g < kGq; ++g)
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) acc[g][cc] = fmaf(pv[g], v[cc], acc[g][cc]);
      }
    } else {
#pragma unroll
      for (int t = 0; t < kPage; ++t) {
        const float pv[kGq] = {pt[t].x, pt[t].y, pt[t].z, pt[t].w};
        float v[CPL];
        T::v_values(vf, t, v);
#pragma unroll
        for (int cc = 0; cc < CPL; ++cc) v[cc] = t < r.valid ? v[cc] : 0.f;  // invalid slots may hold NaN
#pragma unroll
        for (int g = 0; g < kGq; ++g)
#pragma unroll
          for (int cc = 0; cc < CPL; ++cc) acc[g][cc] = fmaf(pv[g], v[cc], acc[g][cc]);
      }
    }
    wave_fence();
  };

  // This wave's pages are i0 + wave, i0 + wave + 4, ...  Their list entries (and physical pages)
  // are read 64 at a time, one per lane, before any K / V load is issued: a list read issued
  // behind K / V loads would have to wait for them (loads retire in order).  Pages then
  // alternate between two register stages, so the next page's K / V loads are in flight while
  // the current page is computed.
  const int my_pages = i1 - i0 > wave ? (i1 - i0 - wave + 3) / 4 : 0;
  typename T::KF ka, kb;
  typename T::VF va, vb;
  uint32_t ksa = 0, vsa = 0, ksb = 0, vsb = 0;
  for (int bb = 0; bb < my_pages; bb += kWave) {
    const int cnt = min(kWave, my_pages - bb);
    const int idx = i0 + wave + 4 * (bb + lane);
    int lp = -1, lph = -1;
    if (bb == 0 && i0 == spec_i0) {  // the speculative read covered this batch
      if (lane < cnt) {
        lp = spec_lp;
        lph = spec_lph;
      }
    } else {
      lp = buf_load_i32(list_r, (uint32_t)(idx >> a.lgs) * 4u);
      lph = buf_load_i32(plist_r, (uint32_t)(idx >> a.lgs) * 4u);
      lp = lane < cnt ? lp : -1;
    }
    // unit idx of entry lp is its logical page (lp << lgs) + (idx mod 2^lgs); entries outside the
    // request are not usable (checked before the shift, so no entry can wrap into range)
    if (lane < cnt) lp = (lp >= 0 && lp < n_phys) ? (lp << a.lgs) | (idx & sub_mask) : -1;
    if (!plist && lane < cnt && lp >= 0 && lp < n_b) lph = a.block_table[(size_t)b * a.max_pages + (lp >> a.lgs)];
    // page u + 1's loads go out before page u is processed; inside the loop every load is a page of the
    // batch, and the last page (or the last two) is processed after it with no load behind it
    PageRef ra = batch_page(lp, lph, 0, n_b, len, a.num_pool_pages), rb;
    load(ra, ka, va, ksa, vsa);
    int u = 0;
    for (; u + 2 < cnt; u += 2) {
      rb = batch_page(lp, lph, u + 1, n_b, len, a.num_pool_pages);
      load(rb, kb, vb, ksb, vsb);
      process(ra, ka, va, ksa, vsa);
      ra = batch_page(lp, lph, u + 2, n_b, len, a.num_pool_pages);
      load(ra, ka, va, ksa, vsa);
      process(rb, kb, vb, ksb, vsb);
    }
    if (u + 1 < cnt) {
      rb = batch_page(lp, lph, u + 1, n_b, len, a.num_pool_pages);
      load(rb, kb, vb, ksb, vsb);
      process(ra, ka, va, ksa, vsa);
      process(rb, kb, vb, ksb, vsb);
    } else {
      process(ra, ka, va, ksa, vsa);
    }
  }

  // wave state -> LDS
  l_run = row_sum(l_run);
  if (tok == 0) {
    ws_m[wave][quarter] = m_run;
    ws_l[wave][quarter] = l_run;
  }
#pragma unroll
  for (int g = 0; g < kGq; ++g)
#pragma unroll
    for (int cc = 0; cc < CPL; ++cc) ws_acc[wave][g][lane * CPL + cc] = acc[g][cc];
  __syncthreads();

  // merge the four wave states.  Each wave first takes the kGq x 4 (row, wave) weights in its lanes --
  // lane l holds row (l / 4) mod kGq and wave state l % 4: the row's largest log-sum, the state's
  // weight exp2(m_w - M) / L and the row's log-sum-exp -- so the per-channel pass below is four fused
  // multiply-adds with the weights read from those lanes.
  {
    const int fg = (lane >> 2) & (kGq - 1), fw = lane & 3;
    const float mw = ws_m[fw][fg];
    float M = fmaxf(mw, __uint_as_float(dpp<0xb1>(__float_as_uint(mw))));  // lane ^ 1
    M = fmaxf(M, __uint_as_float(dpp<0x4e>(__float_as_uint(M))));          // lane ^ 2
    const float sc = M == -INFINITY ? 0.f : exp2f(mw - M);
    float L = ws_l[fw][fg] * sc;
    L += __uint_as_float(dpp<0xb1>(__float_as_uint(L)));
    L += __uint_as_float(dpp<0x4e>(__float_as_uint(L)));
    const float fac = M == -INFINITY ? 0.f : sc / L;
    if (threadIdx.x < 4 * kGq && fw == 0) {
      const float lse = M == -INFINITY ? -INFINITY : (M + log2f(L)) * kLn2;
      if (m == 1) a.out_lse[qrow + fg] = lse;
      else a.part_lse[(slot_row + j) * kGq + fg] = lse;
    }
    for (int e = threadIdx.x; e < kGq * D; e += blockDim.x) {
      const int g = __builtin_amdgcn_readfirstlane(e / D), ch = e % D;  // the row is uniform over a wave
      float o = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w)
        o = fmaf(ws_acc[w][g][ch], __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fac), 4 * g + w)), o);
      if (m == 1) a.out[(qrow + g) * D + ch] = o;
      else a.part_o[((slot_row + j) * kGq + g) * D + ch] = o;
    }
  }
  if constexpr (MERGE) {
    if (m > 1) merge_row_in_block<D>(a, row, m, slot_row, qrow);
  }
}

// Exact merge of a row's chunk states (PersistentKV, section 3.3; states are stored
// normalised: o_j = a_j / l_j and lse_j = m_j + ln l_j): lse = log sum_j exp(lse_j) and
// o = sum_j exp(lse_j - lse) o_j.  One 256-thread block per (row, chunk-state row r), with no
// workgroup barrier: every wave reads all the row's chunk log-sum-exps (lane i holds chunks i,
// i + 64, ...) and takes their max and weight sum with DPP reductions -- the same bits in every
// wave -- while its lanes split the channels and the chunks: lane l of wave w owns channel
// w * D/4 + l mod (D/4) and the chunks of class l / (D/4) (chunk j belongs to class j mod CL, CL =
// 256 / D).  The classes' partial sums are combined with lane swaps.  The list length, the chunk
// log-sum-exps and the first chunk outputs are all requested at once (entries past the row's chunk
// count lie inside the partial buffers and are not used), so a row of up to 64 chunks is merged in one
// memory round trip: the first global access of a kernel costs about a microsecond, and every
// dependent one after it about half that.
constexpr int kMergeThreads = 256;

template <int D>
__global__ __launch_bounds__(kMergeThreads) void lse_merge_kernel(MergeArgs a) {
  constexpr int CL = kMergeThreads / D;   // chunk classes: 2 (d = 128) or 4 (d = 64)
  constexpr int CPW = kWave / CL;          // channels per wave
  constexpr int kSlots = kMaxChunks / kWave;
  constexpr int kPre = kWave / CL;         // chunk outputs per lane requested with the log-sum-exps: the
                                           // first 64 chunks (later ones cost one more round trip per 8)
  static_assert(CPW * (kMergeThreads / kWave) == D, "every channel has one lane per class");
  __shared__ float w_lds[kMergeThreads / kWave][kMaxChunks];  // one copy of the weights per wave
  // block (row, r): chunk-state row r of (request, KV head) row `row`; with several query tokens per
  // request r = t G + g (token t, head g of the group) and the output is [B, T, Hq, d]
  const int R = a.rows_per_head;
  const int row = blockIdx.x / R;
  const int r = blockIdx.x % R;
  const int b = row / a.num_kv_heads;
  const int h = row % a.num_kv_heads;
  if (r >= a.num_tokens * kGq) return;  // rows of absent query tokens (uniform over the block)
  const int J = a.blocks_per_row;
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int cls = lane / CPW;
  const int ch = wave * CPW + lane % CPW;
  // Balanced plan: the row's chunk count and first chunk number come from every row's list length
  // (one more dependent read before the chunk states).
  int c, m, first = 0;
  const int n = a.list_len[row];
  if (a.balanced) {
    const int rows = a.batch * a.num_kv_heads;
    c = balanced_chunk(a.list_len, rows, a.max_list, a.min_chunk, a.grid_target, a.lgs);
    balanced_row(a.list_len, rows, a.max_list, c, row, first, m, a.lgs);
  }
  const size_t slot0 = (a.balanced ? (size_t)first : (size_t)row * J) * R + r;  // + j * R
  const int J_read = a.balanced ? m : J;  // chunk slots of the row that may be read
  // range-checked loads over the row's chunk slots: chunks past J_read read as 0, with no branch
  const __amdgpu_buffer_rsrc_t lse_r = make_rsrc(a.part_lse + slot0, (uint32_t)(J_read * R) * 4u);
  const __amdgpu_buffer_rsrc_t o_r = make_rsrc(a.part_o + slot0 * D, (uint32_t)(J_read * R) * D * 4u);
  float lse_s[kSlots], pre[kPre];
#pragma unroll
  for (int k = 0; k < kSlots; ++k) lse_s[k] = buf_load_f32(lse_r, (uint32_t)((lane + k * kWave) * R) * 4u);
#pragma unroll
  for (int i = 0; i < kPre; ++i) pre[i] = buf_load_f32(o_r, ((uint32_t)((cls + CL * i) * R * D) + (uint32_t)ch) * 4u);
  if (!a.balanced) plan_chunks(clamp_len(n, a.max_list) << a.lgs, J, a.min_chunk, c, m);
  if (m <= 1) return;  // written by the decode itself

  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kSlots; ++k) M = fmaxf(M, lane + k * kWave < m ? lse_s[k] : -INFINITY);
  M = wave_max_f(M);
  const size_t qrow = ((size_t)b * a.num_tokens + r / kGq) * a.num_q_heads + (size_t)h * kGq + r % kGq;
  if (M == -INFINITY) {  // no chunk holds a key
    if (cls == 0) a.out[qrow * D + ch] = 0.f;
    if (threadIdx.x == 0) a.out_lse[qrow] = -INFINITY;
    return;
  }
  // chunk weights exp(lse_j - M), chunk j in lane j mod 64 of slot j / 64 (0 past the row's chunks)
  float w_s[kSlots];
  float S = 0.f;
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {
    w_s[k] = lane + k * kWave < m ? expf(lse_s[k] - M) : 0.f;
    S += w_s[k];
  }
  S = wave_sum_f(S);
  // the first 64 chunks: each class takes its chunk's weight from lane cls + CL i of slot 0
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < kPre; ++i) {
    float wv = 0.f;
#pragma unroll
    for (int q = 0; q < CL; ++q) {
      const float x = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w_s[0]), CL * i + q));
      wv = cls == q ? x : wv;
    }
    acc = fmaf(wv, cls + CL * i < m ? pre[i] : 0.f, acc);  // stale partials past the row may hold NaN
  }
  if (m > kWave) {  // longer rows: the remaining weights through LDS (one copy per wave)
#pragma unroll
    for (int k = 1; k < kSlots; ++k)
      if (lane + k * kWave < m) w_lds[wave][lane + k * kWave] = w_s[k];
    wave_fence();
#pragma unroll 8
    for (int jj = cls + kWave; jj < m; jj += CL)
      acc = fmaf(w_lds[wave][jj], a.part_o[(slot0 + (size_t)jj * R) * D + ch], acc);
  }
  // classes: lanes CPW apart hold the same channel
  if constexpr (CL == 4) acc += xor16(acc);
  acc += xor32(acc);
  if (cls == 0) a.out[qrow * D + ch] = acc / S;
  if (threadIdx.x == 0) a.out_lse[qrow] = M + logf(S);
}

int launch_sparse_paged_decode(const DecodeArgs& a, int head_dim, int q_dtype, int kv_dtype, hipStream_t stream) {
  // per-row plan: rows x J blocks; balanced plan: blocks_per_row holds the whole grid N_T + rows
  dim3 grid((unsigned)(a.balanced ? a.blocks_per_row : a.batch * a.num_kv_heads * a.blocks_per_row)), block(256);
#define SPD_DEC_CASE(D, QD, KVD)                                                                      \
  if (head_dim == D && q_dtype == QD && kv_dtype == KVD) {                                            \
    if (a.counters) hipLaunchKernelGGL((sparse_paged_decode_kernel<D, QD, KVD, true>), grid, block, 0, stream, a); \
    else hipLaunchKernelGGL((sparse_paged_decode_kernel<D, QD, KVD, false>), grid, block, 0, stream, a);           \
    return 0;                                                                                         \
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
  dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.rows_per_head)), block(kMergeThreads);
  if (head_dim == 64) hipLaunchKernelGGL(lse_merge_kernel<64>, grid, block, 0, stream, a);
  else if (head_dim == 128) hipLaunchKernelGGL(lse_merge_kernel<128>, grid, block, 0, stream, a);
  else return SPD_ERR_UNSUPPORTED;
  return 0;
}

}  // namespace spd
