// Page selection of one (request, KV head) row by one 256-thread workgroup.
//
//  * Forced pages: sink 0..n_sink-1 and local n-n_local..n-1 (each once).  A streaming row
//    keeps exactly its forced pages -- the static index table of the LServe summary,
//    "Decoding Stage: Kernel Implementation with Two-Level Indexing".
//  * Top-K (LServe, "Token budget and physical page selection"): the forced pages plus the
//    K' = budget - |forced| best other pages by (score desc, page asc).  The K'-th largest
//    score is found exactly by a three-digit radix select over order-preserving 32-bit
//    keys of the fp32 scores (11 + 11 + 10 bits): each digit histograms only the keys that
//    share the digits chosen so far, so the final selection is restricted to one bin (the
//    bit-pattern bins of LiteTopK, section 3.2, "Extension to Decoding").  No sort.
//  * Coverage (Moira, section 3.2, Eq. 3): tau = the largest share value whose at-or-above
//    share mass reaches t = gamma - forced shares, found by the same radix walk with bins
//    weighted by mass instead of count.  Shares are >= 0, so their IEEE bit patterns are
//    already ordered; masses are summed as 64-bit fixed point (2^-40 units) with integer
//    atomics, so the sums -- and the chosen tau -- do not depend on thread timing.  tau is
//    exact in fp32 order, unlike a bisection that stops at a resolution.
//  * Compaction writes the kept pages in ascending order with ballot prefix counts.
#pragma once

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr double kMassOne = 1099511627776.0;  // 2^40

struct SelectSmem {
  union {
    uint32_t cnt[2048];
    unsigned long long mass[2048];
  } hist;
  unsigned long long wave_tot[kSelWaves];
  uint32_t ballot_tot[2][kSelWaves];
  unsigned long long forced_mass;
  unsigned long long cross_above;  // mass / count above the crossing bin within its range
  int cross_bin;
};

__device__ __forceinline__ unsigned long long share_fx(float pi) {
  if (!(pi > 0.f)) return 0ull;
  return (unsigned long long)(pi * (float)kMassOne);
}

// Exclusive prefix (in thread order) of a 64-bit value over the workgroup.
__device__ __forceinline__ unsigned long long block_excl_scan(unsigned long long v, SelectSmem& sm) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  unsigned long long inc = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    unsigned long long u = __shfl_up(inc, o, kWave);
    if (lane >= o) inc += u;
  }
  if (lane == kWave - 1) sm.wave_tot[wave] = inc;
  __syncthreads();
  unsigned long long before = 0;
  for (int w = 0; w < wave; ++w) before += sm.wave_tot[w];
  __syncthreads();
  return before + inc - v;
}

// Workgroup-wide exclusive count of `flag` in thread order; `total` gets the count of all.
__device__ __forceinline__ int block_count(bool flag, int& total, SelectSmem& sm, int& parity) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const unsigned long long m = __ballot(flag);
  const int lane_rank = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) sm.ballot_tot[parity][wave] = (uint32_t)__popcll(m);
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int c = (int)sm.ballot_tot[parity][w];
    before += w < wave ? c : 0;
    total += c;
  }
  parity ^= 1;
  return before + lane_rank;
}

// One radix digit.  Bins 0..nbins-1 hold counts (MASS = false) or fixed-point masses; the
// crossing bin is the first bin, walking down from the top, where (what lies above it) +
// bin >= need.  Returns the bin, or -1 when even all bins stay below `need`, and sets
// `above` to what lies strictly above the returned bin.
template <bool MASS>
__device__ int radix_cross(int nbins, unsigned long long need, unsigned long long& above, SelectSmem& sm) {
  const int per = nbins / kSelThreads;  // bins per thread, thread 0 owns the top bins
  const int top = nbins - 1 - threadIdx.x * per;
  unsigned long long local = 0;
  for (int i = 0; i < per; ++i) local += MASS ? sm.hist.mass[top - i] : sm.hist.cnt[top - i];
  if (threadIdx.x == 0) sm.cross_bin = -1;
  unsigned long long cum = block_excl_scan(local, sm);  // also synchronises
  for (int i = 0; i < per; ++i) {
    const unsigned long long v = MASS ? sm.hist.mass[top - i] : sm.hist.cnt[top - i];
    if (cum < need && cum + v >= need) {
      sm.cross_bin = top - i;
      sm.cross_above = cum;
    }
    cum += v;
  }
  __syncthreads();
  const int bin = sm.cross_bin;
  above = bin >= 0 ? sm.cross_above : 0ull;
  __syncthreads();
  return bin;
}

__device__ __forceinline__ uint32_t coverage_key(float pi) {
  return pi > 0.f ? __float_as_uint(pi) : 0u;
}

// Select the pages of one row.  `sc` points at the row's scores (top-K: fp32 scores;
// coverage: shares); n is the row's page count; `streaming` selects the static table.
__device__ void select_row(const SelectArgs& a, const float* sc, int n, size_t row, bool streaming,
                           SelectSmem& sm) {
  int32_t* out = a.page_list + row * a.max_list;
  float* out_sc = a.sel_scores ? a.sel_scores + row * a.max_list : nullptr;
  const int ns = max(0, streaming ? a.n_sink_stream : a.n_sink);
  const int nl = max(0, streaming ? a.n_local_stream : a.n_local);
  const int sink_end = min(ns, n);
  const int local_begin = max(sink_end, n - nl);
  const int n_forced = sink_end + (n - local_begin);

  if (streaming) {
    for (int i = threadIdx.x; i < n_forced && i < a.max_list; i += kSelThreads)
      out[i] = i < sink_end ? i : local_begin + (i - sink_end);
    if (threadIdx.x == 0) a.list_len[row] = min(n_forced, a.max_list);
    return;
  }

  // decision: 0 = forced only, 1 = all pages, 2 = top-K threshold, 3 = coverage threshold
  int decision;
  uint32_t thr = 0;            // top-K: key of the K'-th best; coverage: tau's key
  unsigned long long need_eq = 0;  // top-K: how many keys equal to thr to take
  const bool coverage = a.mode == SPD_SELECT_COVERAGE;
  const int n_free = n - n_forced;

  if (!coverage) {
    const int kp = a.budget - n_forced;
    if (kp <= 0) decision = 0;
    else if (n_free <= kp) decision = 1;
    else {
      decision = 2;
      unsigned long long k = (unsigned long long)kp;
      uint32_t prefix = 0, pmask = 0;
      const int shifts[3] = {21, 10, 0};
      const int widths[3] = {11, 11, 10};
      for (int d = 0; d < 3; ++d) {
        const int nb = 1 << widths[d];
        for (int i = threadIdx.x; i < nb; i += kSelThreads) sm.hist.cnt[i] = 0u;
        __syncthreads();
        for (int p = threadIdx.x; p < n; p += kSelThreads) {
          if (p < sink_end || p >= local_begin) continue;
          const uint32_t key = score_key(sc[p]);
          if ((key & pmask) == prefix) atomicAdd(&sm.hist.cnt[(key >> shifts[d]) & (nb - 1)], 1u);
        }
        __syncthreads();
        unsigned long long above;
        const int bin = radix_cross<false>(nb, k, above, sm);
        k -= above;  // a crossing bin always exists: the candidates outnumber k
        prefix |= (uint32_t)bin << shifts[d];
        pmask |= (uint32_t)(nb - 1) << shifts[d];
      }
      thr = prefix;
      need_eq = k;
    }
  } else {
    // forced share mass, then t = gamma - forced mass in fixed point
    if (threadIdx.x == 0) sm.forced_mass = 0ull;
    __syncthreads();
    for (int i = threadIdx.x; i < n_forced; i += kSelThreads) {
      const int p = i < sink_end ? i : local_begin + (i - sink_end);
      atomicAdd(&sm.forced_mass, share_fx(sc[p]));
    }
    __syncthreads();
    const unsigned long long fm = sm.forced_mass;
    if (fm >= a.gamma_fx) decision = 0;
    else {
      unsigned long long need = a.gamma_fx - fm;
      uint32_t prefix = 0, pmask = 0;
      const int shifts[3] = {21, 10, 0};
      const int widths[3] = {11, 11, 10};
      decision = 3;
      for (int d = 0; d < 3; ++d) {
        const int nb = 1 << widths[d];
        for (int i = threadIdx.x; i < nb; i += kSelThreads) sm.hist.mass[i] = 0ull;
        __syncthreads();
        for (int p = threadIdx.x; p < n; p += kSelThreads) {
          if (p < sink_end || p >= local_begin) continue;
          const float pi = sc[p];
          const uint32_t key = coverage_key(pi);
          if ((key & pmask) == prefix) atomicAdd(&sm.hist.mass[(key >> shifts[d]) & (nb - 1)], share_fx(pi));
        }
        __syncthreads();
        unsigned long long above;
        const int bin = radix_cross<true>(nb, need, above, sm);
        if (bin < 0) { decision = 1; break; }  // the free pages cannot reach t: keep all
        need -= above;
        prefix |= (uint32_t)bin << shifts[d];
        pmask |= (uint32_t)(nb - 1) << shifts[d];
      }
      thr = prefix;
    }
  }

  // compaction in ascending page order
  int out_pos = 0, parity = 0;
  unsigned long long eq_seen = 0;
  for (int tile = 0; tile < n; tile += kSelThreads) {
    const int p = tile + threadIdx.x;
    const bool in = p < n;
    const bool forced = in && (p < sink_end || p >= local_begin);
    const bool cand = in && !forced;
    const float s = in ? sc[p] : 0.f;
    bool take = false;
    if (decision == 1) take = cand;
    else if (decision == 3) take = cand && coverage_key(s) >= thr;
    else if (decision == 2) {
      const uint32_t key = score_key(s);
      const bool eq = cand && key == thr;
      int eq_tot;
      const int eq_rank = block_count(eq, eq_tot, sm, parity);
      take = (cand && key > thr) || (eq && eq_seen + (unsigned long long)eq_rank < need_eq);
      eq_seen += (unsigned long long)eq_tot;
    }
    const bool keep = forced || take;
    int tot;
    const int pos = out_pos + block_count(keep, tot, sm, parity);
    if (keep && pos < a.max_list) {
      out[pos] = p;
      if (out_sc) out_sc[pos] = s;
    }
    out_pos += tot;
  }
  if (threadIdx.x == 0) a.list_len[row] = min(out_pos, a.max_list);
}

}  // namespace spd
