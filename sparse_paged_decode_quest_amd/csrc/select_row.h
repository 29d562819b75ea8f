// Page selection of one (request, KV head) row by one workgroup of NT threads.
//
//  * Forced pages: sink 0..n_sink-1 and local n-n_local..n-1 (each once).  A streaming row
//    keeps exactly its forced pages -- the static index table of the LServe summary,
//    "Decoding Stage: Kernel Implementation with Two-Level Indexing".
//  * Top-K (LServe, "Token budget and physical page selection"): the forced pages plus the
//    K' = budget - |forced| best other pages by (score desc, page asc).  The K'-th largest
//    score is found exactly by a radix select over order-preserving 32-bit keys of the fp32
//    scores: each digit histograms only the keys sharing the digits chosen so far, so the
//    final selection is restricted to one bin (the bit-pattern bins of LiteTopK, section
//    3.2, "Extension to Decoding").  No sort.
//  * Coverage (Moira, section 3.2, Eq. 3): tau = the largest share value whose at-or-above
//    share mass reaches t = gamma - forced shares, found by the same radix walk with bins
//    weighted by mass.  Shares are >= 0, so their IEEE bit patterns are already ordered;
//    masses are summed as 64-bit fixed point (2^-40 units) with integer atomics, so the sums
//    -- and tau -- do not depend on thread timing.  tau is exact in fp32 order, unlike a
//    bisection that stops at a resolution.
//
// Work layout: thread t of the workgroup owns the contiguous pages [t*chunk, (t+1)*chunk)
// and keeps their keys in registers (KPT >= chunk), or re-reads them from memory (KPT == 0,
// very long rows).
// The digits start below the bits shared by the smallest and the largest free key, so the
// first histogram already spreads the (typically narrow) score range over many bins; a pass
// that finds the crossing bin needed whole ends the walk early.  Compaction is one
// workgroup-wide exclusive scan of the per-thread kept counts, which writes the list in
// ascending page order.
#pragma once

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kSelBins = 2048;  // 11-bit digits
constexpr double kMassOne = 1099511627776.0;  // 2^40

struct SelectSmem {
  union {
    uint32_t cnt[kSelBins];
    unsigned long long mass[kSelBins];
  } hist;
  unsigned long long wave_tot[kSelWaves];
  uint32_t wave_min[kSelWaves], wave_max[kSelWaves];
  unsigned long long cross_above;
  unsigned long long cross_val;
  int cross_bin;
};

__device__ __forceinline__ unsigned long long share_fx(float pi) {
  if (!(pi > 0.f)) return 0ull;
  return (unsigned long long)(pi * (float)kMassOne);
}

__device__ __forceinline__ uint32_t coverage_key(float pi) { return pi > 0.f ? __float_as_uint(pi) : 0u; }

__device__ __forceinline__ float key_to_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// Exclusive prefix (in thread order) of a 64-bit value over the workgroup; `total` = sum.
__device__ __forceinline__ unsigned long long block_excl_scan(unsigned long long v, unsigned long long& total,
                                                              SelectSmem& sm) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  unsigned long long inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    unsigned long long u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) sm.wave_tot[wave] = inc;
  __syncthreads();
  unsigned long long before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const unsigned long long t = w < (int)(blockDim.x / kWave) ? sm.wave_tot[w] : 0ull;
    before += w < wave ? t : 0ull;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + inc - v;
}

// Workgroup min and max of a 32-bit key.
__device__ __forceinline__ void block_minmax(uint32_t& mn, uint32_t& mx, SelectSmem& sm) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    mn = min(mn, (uint32_t)__shfl_xor((int)mn, o, kWave));
    mx = max(mx, (uint32_t)__shfl_xor((int)mx, o, kWave));
  }
  if (lane == 0) { sm.wave_min[wave] = mn; sm.wave_max[wave] = mx; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w)
    if (w < (int)(blockDim.x / kWave)) { mn = min(mn, sm.wave_min[w]); mx = max(mx, sm.wave_max[w]); }
  __syncthreads();
}

// One radix digit over nb bins (counts or fixed-point masses): the crossing bin is the first
// bin, walking down from the top, where (what lies above it) + bin >= need.  Returns the bin
// (or -1 when all bins together stay below `need`); `above` gets what lies strictly above
// it and `inbin` the bin's own value.
template <bool MASS>
__device__ int radix_cross(int nb, unsigned long long need, unsigned long long& above, unsigned long long& inbin,
                           SelectSmem& sm) {
  const int per = (nb + (int)blockDim.x - 1) / (int)blockDim.x;  // thread 0 owns the top bins
  const int top = nb - 1 - (int)threadIdx.x * per;
  unsigned long long local = 0;
  for (int i = 0; i < per; ++i) {
    const int bin = top - i;
    if (bin >= 0) local += MASS ? sm.hist.mass[bin] : sm.hist.cnt[bin];
  }
  if (threadIdx.x == 0) sm.cross_bin = -1;
  unsigned long long total;
  unsigned long long cum = block_excl_scan(local, total, sm);  // synchronises
  for (int i = 0; i < per; ++i) {
    const int bin = top - i;
    if (bin < 0) break;
    const unsigned long long v = MASS ? sm.hist.mass[bin] : sm.hist.cnt[bin];
    if (cum < need && cum + v >= need) {
      sm.cross_bin = bin;
      sm.cross_above = cum;
      sm.cross_val = v;
    }
    cum += v;
  }
  __syncthreads();
  const int bin = sm.cross_bin;
  above = bin >= 0 ? sm.cross_above : 0ull;
  inbin = bin >= 0 ? sm.cross_val : 0ull;
  __syncthreads();
  return bin;
}

// Keys of this thread's chunk of the row: cached in registers (KPT > 0) or re-read (KPT == 0).
template <int KPT, bool COV>
struct RowKeys {
  const float* sc;
  int base, cnt;
  uint32_t k[KPT > 0 ? KPT : 1];
  __device__ __forceinline__ void load(const float* s, int b, int c) {
    sc = s;
    base = b;
    cnt = c;
    if constexpr (KPT > 0) {
#pragma unroll
      for (int i = 0; i < KPT; ++i) {
        const float v = i < cnt ? sc[base + i] : 0.f;
        k[i] = COV ? coverage_key(v) : score_key(v);
      }
    }
  }
  __device__ __forceinline__ uint32_t operator[](int i) const {
    if constexpr (KPT > 0) return k[i];
    else return COV ? coverage_key(sc[base + i]) : score_key(sc[base + i]);
  }
  __device__ __forceinline__ int extent() const { return KPT > 0 ? KPT : cnt; }
};

// Select the pages of one dynamic row.  `sc` points at the row's scores (top-K: fp32
// scores; coverage: shares); n is the row's page count.
template <int KPT, bool COV>
__device__ void select_dynamic_row(const SelectArgs& a, const float* sc, int n, size_t row, SelectSmem& sm) {
  int32_t* out = a.page_list + row * a.max_list;
  float* out_sc = a.sel_scores ? a.sel_scores + row * a.max_list : nullptr;
  const int ns = max(0, a.n_sink), nl = max(0, a.n_local);
  const int sink_end = min(ns, n);
  const int local_begin = max(sink_end, n - nl);
  const int n_forced = sink_end + (n - local_begin);
  const int chunk = (n + (int)blockDim.x - 1) / (int)blockDim.x;
  const int base = min(n, (int)threadIdx.x * chunk);
  const int cnt = min(n, base + chunk) - base;
  RowKeys<KPT, COV> rk;
  rk.load(sc, base, cnt);
  auto is_free = [&](int i) { const int p = base + i; return i < cnt && p >= sink_end && p < local_begin; };

  // decision: 0 = forced only, 1 = all pages, 2 = threshold: take keys above `thr` (strict) or
  // at-or-above it; with `strict`, also the first need_eq keys equal to thr in page order
  int decision = 2;
  uint32_t thr = 0;
  bool strict = false;
  unsigned long long need_eq = 0;
  unsigned long long need;              // count (top-K) or mass (coverage) still to cover
  if (!COV) {
    const int kp = a.budget - n_forced;
    if (kp <= 0) decision = 0;
    else if (n - n_forced <= kp) decision = 1;
    need = kp > 0 ? (unsigned long long)kp : 0ull;
  } else {
    unsigned long long fm = 0;
#pragma unroll
    for (int i = 0; i < rk.extent(); ++i) {
      const int p = base + i;
      if (i < cnt && !(p >= sink_end && p < local_begin)) fm += share_fx(__uint_as_float(rk[i]));
    }
    unsigned long long fm_all;
    block_excl_scan(fm, fm_all, sm);
    if (fm_all >= a.gamma_fx) decision = 0;
    need = fm_all >= a.gamma_fx ? 0ull : a.gamma_fx - fm_all;
  }

  if (decision == 2) {
    // common high bits of the free keys
    uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll
    for (int i = 0; i < rk.extent(); ++i)
      if (is_free(i)) { mn = min(mn, rk[i]); mx = max(mx, rk[i]); }
    block_minmax(mn, mx, sm);
    uint32_t prefix, pmask;
    int hi;
    if (mn == mx) {  // every free key is equal: one "digit" of zero width
      prefix = mx;
      pmask = 0xffffffffu;
      hi = -1;
    } else {
      hi = 31 - __clz(mn ^ mx);
      pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
      prefix = mx & pmask;
    }
    bool exact = true;  // the walk reached bit 0 (or all keys share their bits)
    if (COV && hi < 0) {
      // all free shares are equal: they reach t together or not at all
      unsigned long long tot = 0;
#pragma unroll
      for (int i = 0; i < rk.extent(); ++i)
        if (is_free(i)) tot += share_fx(__uint_as_float(rk[i]));
      unsigned long long all;
      block_excl_scan(tot, all, sm);
      if (all < need) decision = 1;
    }
    while (hi >= 0 && decision == 2) {
      const int shift = hi > 10 ? hi - 10 : 0;
      const int nb = 1 << (hi - shift + 1);
      for (int i = threadIdx.x; i < nb; i += blockDim.x) {
        if (COV) sm.hist.mass[i] = 0ull;
        else sm.hist.cnt[i] = 0u;
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < rk.extent(); ++i) {
        const uint32_t key = rk[i];
        if (is_free(i) && (key & pmask) == prefix) {
          const int bin = (int)((key >> shift) & (uint32_t)(nb - 1));
          if (COV) atomicAdd(&sm.hist.mass[bin], share_fx(__uint_as_float(key)));
          else atomicAdd(&sm.hist.cnt[bin], 1u);
        }
      }
      __syncthreads();
      unsigned long long above, inbin;
      const int bin = radix_cross<COV>(nb, need, above, inbin, sm);
      if (bin < 0) { decision = 1; break; }  // coverage: the free pages cannot reach t: keep all
      need -= above;
      prefix |= (uint32_t)bin << shift;
      pmask |= (uint32_t)(nb - 1) << shift;
      hi = shift - 1;
      if (!COV && inbin == need && hi >= 0) {  // the whole crossing bin is taken: stop early
        exact = false;
        break;
      }
    }
    thr = prefix;
    if (!COV && exact) {  // prefix is the K'-th key: all keys above it, then ties in page order
      strict = true;
      need_eq = need;
    }
  }

  // compaction: per-thread counts, one scan each for ties (rare) and kept pages
  unsigned long long eq_before = 0;
  if (decision == 2 && strict) {
    unsigned long long e = 0, all;
#pragma unroll
    for (int i = 0; i < rk.extent(); ++i)
      if (is_free(i) && rk[i] == thr) ++e;
    eq_before = block_excl_scan(e, all, sm);
  }
  auto keep = [&](int i, unsigned long long& eq_seen) {
    if (i >= cnt) return false;
    if (!is_free(i)) return true;  // forced
    if (decision == 0) return false;
    if (decision == 1) return true;
    const uint32_t key = rk[i];
    if (strict ? key > thr : key >= thr) return true;
    if (strict && key == thr) return eq_seen++ < need_eq;
    return false;
  };
  unsigned long long mine = 0, total;
  {
    unsigned long long eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < rk.extent(); ++i) mine += keep(i, eq_seen) ? 1ull : 0ull;
  }
  unsigned long long pos = block_excl_scan(mine, total, sm);
  {
    unsigned long long eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < rk.extent(); ++i) {
      if (keep(i, eq_seen)) {
        if (pos < (unsigned long long)a.max_list) {
          out[pos] = base + i;
          if (out_sc) out_sc[pos] = COV ? __uint_as_float(rk[i]) : key_to_score(rk[i]);
        }
        ++pos;
      }
    }
  }
  if (threadIdx.x == 0) a.list_len[row] = (int)min(total, (unsigned long long)a.max_list);
}

// A streaming row keeps its static sink + local table.
__device__ __forceinline__ void select_streaming_row(const SelectArgs& a, int n, size_t row) {
  int32_t* out = a.page_list + row * a.max_list;
  const int sink_end = min(max(0, a.n_sink_stream), n);
  const int local_begin = max(sink_end, n - max(0, a.n_local_stream));
  const int n_forced = sink_end + (n - local_begin);
  for (int i = threadIdx.x; i < n_forced && i < a.max_list; i += blockDim.x)
    out[i] = i < sink_end ? i : local_begin + (i - sink_end);
  if (threadIdx.x == 0) a.list_len[row] = min(n_forced, a.max_list);
}

template <int KPT>
__device__ __forceinline__ void select_row(const SelectArgs& a, const float* sc, int n, size_t row, bool streaming,
                                           SelectSmem& sm) {
  if (streaming) select_streaming_row(a, n, row);
  else if (a.mode == SPD_SELECT_COVERAGE) select_dynamic_row<KPT, true>(a, sc, n, row, sm);
  else select_dynamic_row<KPT, false>(a, sc, n, row, sm);
}

// Keys per thread to compile for rows of up to max_pages pages with kSelThreads threads
// (0: re-read them from memory for every pass -- rows beyond 32768 pages).
__host__ __device__ constexpr int select_kpt(int max_pages) {
  return max_pages <= kSelThreads * 8 ? 8 : max_pages <= kSelThreads * 32 ? 32 : 0;
}

}  // namespace spd
