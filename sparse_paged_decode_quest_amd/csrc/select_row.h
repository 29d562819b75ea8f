// Page selection of one (request, KV head) row by one workgroup of NW waves.
//
//  * Forced pages: sink 0..n_sink-1 and local n-n_local..n-1 (each once).  A streaming row
//    keeps exactly its forced pages -- the static index table of the LServe summary,
//    "Decoding Stage: Kernel Implementation with Two-Level Indexing".
//  * Top-K (LServe, "Token budget and physical page selection"): the forced pages plus the
//    K' = budget - |forced| best other pages by (score desc, page asc).  The K'-th largest
//    score is found exactly by a radix walk over order-preserving 32-bit keys of the fp32
//    scores: each digit histograms only the keys that share the digits chosen so far, so the
//    final choice is made inside one bin (the bit-pattern bins of LiteTopK, section 3.2,
//    "Extension to Decoding").  No sort.
//  * Coverage (Moira, section 3.2, Eq. 3): tau = the largest share whose at-or-above share
//    mass reaches t = gamma - forced shares, found by the same walk with bins weighted by
//    mass.  Shares are >= 0, so their IEEE bit patterns are already ordered; masses are
//    summed as 64-bit fixed point (2^-40 units) with integer atomics, so sums -- and tau --
//    do not depend on thread timing, and tau is exact in fp32 order.
//
// Work layout.  Wave w holds the 64 KPL consecutive pages starting at 64 KPL w; its key slot
// i holds page 64 KPL w + 64 i + lane, so every key load of a wave reads 64 consecutive scores
// and page order is (wave, slot, lane) order.  The list is compacted with one ballot per slot
// and scalar running counts inside a wave, plus one LDS exchange of the wave totals.  Each
// digit of the walk takes two workgroup barriers: after the histogram, and after wave 0 has
// found the crossing bin in it (three rotating histogram buffers let the next digit's
// histogram start at once) -- 64 lane sums over skewed addresses (no LDS bank conflicts), a
// scan, and a second scan inside the crossing lane's group of bins.  Top-K usually stops after
// one digit: when at most kCandMax keys share the crossing bin, wave 0 holds one each and counts
// the keys above and equal to its own.  Ties at the K'-th key are taken in page order.  Values every wave needs from the
// others (ranges, counts) are read one per lane and combined with DPP reductions and scans:
// one LDS read per wave instead of one per wave entry, since sixteen waves reading the same
// LDS words one by one were the bulk of the selection time.
#pragma once

#include <type_traits>

#include "spd_device.h"
#include "spd_launch.h"

namespace spd {

// Radix digits: 11 bits (2048 count bins) for top-K, 10 bits (1024 64-bit mass bins) for coverage.
template <bool COV>
struct SelectDigit {
  static constexpr int kBits = COV ? 10 : 11;
  static constexpr int kBins = 1 << kBits;
};
constexpr int kCandMax = kWave;                // crossing-bin keys ranked by one wave
constexpr int kNoLimit = 0x7fffffff;
constexpr double kMassOne = 1099511627776.0;   // 2^40

template <int NW, int KPL, bool COV>
struct SelectSmem {
  using H = typename std::conditional<COV, unsigned long long, uint32_t>::type;
  H hist[3][SelectDigit<COV>::kBins];
  unsigned long long wsum[NW];
  uint32_t wmin[NW], wmax[NW];
  alignas(16) uint32_t cand_key[kCandMax];
  uint32_t cand_count;
  uint32_t wsure[NW], weq[NW];  // per-wave counts of kept-for-sure keys and keys equal to the cut key
  struct {
    int bin;       // crossing bin of the current digit (-1: coverage target out of reach)
    H above, inbin;  // count / mass above the bin and inside it
    uint32_t kc;     // top-K cut key found by ranking the crossing bin's keys
    int need_eq;     // keys equal to kc still to take
    int gate_bin;    // top-K, first digit: the bin where 1.5 K' keys are reached, from the top (-1: fewer)
  } cross;
};

// The candidate path of the gated top-K selector (LiteTopK): the free keys at or above the gate, in page order.
struct GateSmem {
  uint32_t key[kGateCap];
  int32_t page[kGateCap];
};

__device__ __forceinline__ unsigned long long share_fx(float pi) {
  if (!(pi > 0.f)) return 0ull;
  return (unsigned long long)(pi * (float)kMassOne);
}

__device__ __forceinline__ uint32_t coverage_key(float pi) { return pi > 0.f ? __float_as_uint(pi) : 0u; }

__device__ __forceinline__ float key_to_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// The forced / free split of a row of n pages.
struct RowShape {
  int n;            // pages
  int sink_end;     // forced: [0, sink_end) and [local_begin, n)
  int local_begin;
};

__device__ __forceinline__ RowShape row_shape(int n, int n_sink, int n_local) {
  RowShape r;
  r.n = n;
  r.sink_end = min(max(0, n_sink), n);
  r.local_begin = max(r.sink_end, n - max(0, n_local));
  return r;
}

// Physical pages of a row's key slots: kept in registers for rows of up to 8 slots per lane,
// read from the block table for the listed pages only otherwise (one more dependent load, in
// exchange for KPL registers the long-row workgroups do not have).
template <int KPL>
struct SlotPhys {
  static constexpr bool kInRegs = KPL <= 8;
  int32_t v[kInRegs ? KPL : 1];
  const int32_t* bt_row;  // nullable: no list of physical pages wanted
  // slot i (page p) of a row of n block-table entries, read without a branch (past n, or with no
  // table, it reads 0)
  __device__ __forceinline__ void load(int i, int p, int n) {
    if constexpr (kInRegs) v[i] = buf_load_i32(make_rsrc(bt_row, bt_row ? (uint32_t)n * 4u : 0u), (uint32_t)p * 4u);
  }
  __device__ __forceinline__ int32_t at(int i, int p) const {
    if constexpr (kInRegs) return v[i];
    else return bt_row[p];
  }
};

// The next call's gate of row `row` (LiteTopK, section 3.3, predictive gating from the previous token's
// selection): candidates will be the free pages scoring at least the score of gate_key; with no key
// (gate_key = 0) the gate is `fallback` (-inf: every free page).  Rows that took every free page or none
// keep no gate.
__device__ __forceinline__ void gate_store(const TopkGate& g, size_t row, int dec, uint32_t gate_key, uint32_t top_key,
                                           float fallback, uint32_t path, uint32_t seen) {
  TopkGateRow v;
  v.lo = gate_key ? key_to_score(gate_key) : fallback;
  v.top = top_key ? key_to_score(top_key) : -INFINITY;
  v.valid = dec == 2 ? 1u : 0u;
  v.path = path;  // how this selection ran: 1 from the candidates, 0 over the whole row
  v.seen = seen;  // free pages at or above the gate it counted
  v.pad[0] = v.pad[1] = v.pad[2] = 0u;
  g.rows[row] = v;
}

// The cut of one row's keys: the decision dec (0: forced pages only, 1: every free page, 2: cut at key kc --
// keys above kc are taken, keys equal to kc while fewer than need_eq were taken, in page order), found by the
// radix walk described at the top of this file.  free_at / forced_at say which key slots are free or forced
// pages; n_free / n_forced count them.
// Top-K also returns top_key, the largest free key, and gate_key, the lower edge of the first digit's bin
// where 1.5 K' free keys are reached (0 when there are fewer, or no walk ran): the next call's predicted gate.
// BITS is the digit width.  With PRE (top-K only) the caller has found the range -- pre_mn at or below every
// free key, pre_mx the largest -- and has cleared the first two histogram buffers and the candidate count
// before a barrier; the cut then starts with the first digit.  Every thread of the workgroup must call this.
template <int NW, int KPL, bool COV, int BITS, bool PRE, typename SM, typename FreeAt, typename ForcedAt>
__device__ __forceinline__ void row_cut(const SelectArgs& a, const uint32_t (&key)[KPL], FreeAt free_at,
                                        ForcedAt forced_at, const int n_free, const int n_forced,
                                        SM& sm, int& dec, uint32_t& kc, int& need_eq, uint32_t& gate_key,
                                        uint32_t& top_key, uint32_t pre_mn = 0u, uint32_t pre_mx = 0u) {
  using H = typename SM::H;
  constexpr int STRIDE = NW * kWave;
  constexpr int kBits = BITS;
  constexpr int kBins = 1 << BITS;
  constexpr int PER = kBins / kWave;  // histogram bins summed by one lane
  static_assert(kBins <= SelectDigit<COV>::kBins && PER >= 1, "digit width out of range");
  static_assert(!(PRE && COV), "a given range is a top-K cut");
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  auto mass_of = [&](uint32_t k) { return share_fx(__uint_as_float(k)); };
  uint32_t mn = pre_mn, mx = pre_mx;
  unsigned long long fmass = 0;
  if constexpr (!PRE) {
    // ---- range of the free keys, forced mass (coverage); clear two histogram buffers
    mn = 0xffffffffu;
    mx = 0u;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      if (free_at(i)) {
        mn = min(mn, key[i]);
        mx = max(mx, key[i]);
      } else if (COV && forced_at(i)) {
        fmass += mass_of(key[i]);
      }
    }
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (COV) fmass = wave_sum(fmass);
    if (lane == 0) {
      sm.wmin[wave] = mn;
      sm.wmax[wave] = mx;
      sm.wsum[wave] = fmass;
    }
    for (int e = threadIdx.x; e < 2 * SelectDigit<COV>::kBins; e += STRIDE) (&sm.hist[0][0])[e] = 0;
    if (threadIdx.x == 0) sm.cand_count = 0;
    __syncthreads();
    // lane w < NW reads wave w's entries; DPP reductions give every lane the workgroup's values
    mn = wave_min(lane < NW ? sm.wmin[lane] : 0xffffffffu);
    mx = wave_max(lane < NW ? sm.wmax[lane] : 0u);
    if (COV) fmass = wave_sum(lane < NW ? sm.wsum[lane] : 0ull);
  }
  top_key = mx;
  gate_key = 0u;

  // ---- decision: 0 = forced pages only, 1 = every page, 2 = cut at key kc: keys above kc are
  // kept, keys equal to kc are kept in page order while fewer than need_eq of them were taken.
  unsigned long long need;  // count (top-K) or mass (coverage) still to cover
  if (!COV) {
    const int kp = a.budget - n_forced;
    dec = kp <= 0 ? 0 : (n_free <= kp ? 1 : 2);
    need = kp > 0 ? (unsigned long long)kp : 0ull;
  } else {
    dec = (n_free == 0 || fmass >= a.gamma_fx) ? 0 : 2;
    need = dec == 2 ? a.gamma_fx - fmass : 0ull;
  }
  kc = 0;
  need_eq = kNoLimit;
  if (dec == 2) {
    if (mn == mx) {
      // every free key is equal: top-K takes them in page order; coverage keeps them all (they
      // either reach t together, or nothing does and every page is kept)
      kc = mx;
      need_eq = COV ? kNoLimit : (int)need;
    } else {
      int hi = 31 - __clz(mn ^ mx);  // digits start below the bits every free key shares
      uint32_t pmask = hi == 31 ? 0u : ~((2u << hi) - 1u);
      uint32_t prefix = mx & pmask;
      for (int pass = 0;; ++pass) {
        const int shift = hi > kBits - 1 ? hi - (kBits - 1) : 0;
        const int nb = 1 << (hi - shift + 1);
        H* h = sm.hist[pass % 3];
#pragma unroll
        for (int i = 0; i < KPL; ++i) {
          if (free_at(i) && (key[i] & pmask) == prefix) {
            // bins are stored from the top: slot kBins - 1 - bin
            const int rbin = kBins - 1 - (int)((key[i] >> shift) & (uint32_t)(nb - 1));
            if (COV) atomicAdd(reinterpret_cast<unsigned long long*>(&h[rbin]), mass_of(key[i]));
            else atomicAdd(reinterpret_cast<uint32_t*>(&h[rbin]), 1u);
          }
        }
        __syncthreads();
        {  // the buffer of pass + 2 was last read in pass - 1, which every wave finished before the barrier
          H* hc = sm.hist[(pass + 2) % 3];
          for (int e = threadIdx.x; e < kBins; e += STRIDE) hc[e] = 0;
        }
        // Crossing bin, found by wave 0 alone (one wave's histogram reads instead of every
        // wave's): lane l sums slots [l PER, (l+1) PER) (the l-th group from the top), reading
        // them in a lane-skewed order so the reads hit distinct banks; a scan finds the group,
        // a second scan inside it the bin.  The others wait at the barrier and read the result.
        if (wave == 0) {
          H s = 0;
#pragma unroll
          for (int j = 0; j < PER; ++j) s += h[lane * PER + ((j + lane) % PER)];
          const H incl = wave_incl_scan(s);
          const H excl = incl - s;
          if constexpr (!COV) {
            // the next call's gate (LiteTopK, section 3.3): the bin where the count from the top reaches
            // 1.5 K' (the margin of a predicted filter) -- its group first, then the bin inside it
            if (pass == 0) {
              const H need2 = need + need / 2;
              const unsigned long long hit2 = __ballot(excl < need2 && incl >= need2);
              int gbin = -1;
              if (hit2) {
                const int g2 = __ffsll((long long)hit2) - 1;
                const H v2 = lane < PER ? h[g2 * PER + lane] : (H)0;
                const H incl3 = wave_incl_scan(v2) + lane_u32(excl, g2);
                const unsigned long long hit3 = __ballot(lane < PER && incl3 - v2 < need2 && incl3 >= need2);
                gbin = kBins - 1 - (g2 * PER + __ffsll((long long)hit3) - 1);
              }
              if (lane == 0) sm.cross.gate_bin = gbin;
            }
          }
          const unsigned long long hit = __ballot(excl < need && incl >= need);
          if (hit == 0ull) {  // coverage only: the free pages cannot reach t -- keep every page
            if (lane == 0) sm.cross.bin = -1;
          } else {
            const int owner = __ffsll((long long)hit) - 1;
            H owner_excl;
            if constexpr (COV) owner_excl = lane_u64(excl, owner);
            else owner_excl = lane_u32(excl, owner);
            // inside the owner's group: lane j < PER takes slot owner PER + j
            const H v = lane < PER ? h[owner * PER + lane] : (H)0;
            const H incl2 = wave_incl_scan(v) + owner_excl;
            const unsigned long long hit2 = __ballot(lane < PER && incl2 - v < need && incl2 >= need);
            const int jc = __ffsll((long long)hit2) - 1;
            if (lane == jc) {
              sm.cross.bin = kBins - 1 - (owner * PER + jc);
              sm.cross.above = incl2 - v;
              sm.cross.inbin = v;
            }
          }
        }
        __syncthreads();
        const int bin = sm.cross.bin;
        if (bin < 0) {
          dec = 1;
          break;
        }
        const H above = sm.cross.above, inbin = sm.cross.inbin;
        if (!COV && pass == 0 && sm.cross.gate_bin >= 0) gate_key = prefix | ((uint32_t)sm.cross.gate_bin << shift);
        need -= above;
        prefix |= (uint32_t)bin << shift;
        pmask |= (uint32_t)(nb - 1) << shift;
        hi = shift - 1;
        if (hi < 0) {  // every bit chosen: prefix is the cut key itself
          kc = prefix;
          need_eq = COV ? kNoLimit : (int)need;
          break;
        }
        if (!COV && inbin == need) {  // the whole crossing bin is taken
          kc = prefix;
          need_eq = kNoLimit;
          break;
        }
        if (!COV && inbin <= (H)kCandMax) {
          // few keys left in the bin: gather them (in any order); wave 0 holds one per lane, reads them all
          // back from LDS four at a time and counts the keys above and equal to its own.  The cut key is the
          // one with fewer than need keys above it and at least need at or above it; ties at the cut are
          // settled in page order by the compaction.
          uint32_t c = 0;
#pragma unroll
          for (int i = 0; i < KPL; ++i) c += (free_at(i) && (key[i] & pmask) == prefix) ? 1u : 0u;
          const uint32_t cincl = wave_incl_scan(c);
          const uint32_t wtot = lane_u32(cincl, kWave - 1);
          uint32_t base = 0;
          if (lane == 0 && wtot) base = atomicAdd(&sm.cand_count, wtot);
          uint32_t pos = lane_u32(base, 0) + cincl - c;
#pragma unroll
          for (int i = 0; i < KPL; ++i) {
            if (free_at(i) && (key[i] & pmask) == prefix) sm.cand_key[pos++] = key[i];
          }
          __syncthreads();
          if (wave == 0) {
            const int m = (int)sm.cand_count;  // == inbin
            const uint32_t ck = lane < m ? sm.cand_key[lane] : 0u;
            uint32_t above = 0, same = 0;
            for (int j = 0; j < m; j += 4) {
              const uint4 k4 = *reinterpret_cast<const uint4*>(&sm.cand_key[j]);  // past m: not counted
              const uint32_t kj[4] = {k4.x, k4.y, k4.z, k4.w};
#pragma unroll
              for (int u = 0; u < 4; ++u) {
                const bool in = j + u < m;
                above += in && kj[u] > ck ? 1u : 0u;
                same += in && kj[u] == ck ? 1u : 0u;
              }
            }
            const uint32_t nd = (uint32_t)need;
            const unsigned long long cut = __ballot(lane < m && above < nd && above + same >= nd);
            if (lane == __ffsll((long long)cut) - 1) {
              sm.cross.kc = ck;
              sm.cross.need_eq = (int)(nd - above);
            }
          }
          __syncthreads();
          kc = sm.cross.kc;
          need_eq = sm.cross.need_eq;
          break;
        }
      }
    }
  }

}

// The gated top-K path (LiteTopK, section 3.2 "Sampling" and "Top-k Selection"; section 3.3 "Predictive
// Gating").  The row's gate was predicted from its previous selection.  The free pages scoring at or above
// it are the candidates; when they number at least K' they hold the top K' free pages and every page tied
// with the K'-th, so the row's cut is the cut among the candidates.
//
// The keys arrive with every slot that is not a free page set to 0 (below every gate).  One pass over them
// finds the free keys' range and counts the candidates (one compare and a ballot per slot, summed on the
// scalar unit), beside the clearing of the histograms: one barrier.  With between K' and kGateCap
// candidates, they are gathered in page order (the slot layout is page order: wave, slot, lane) -- a slot
// with no candidate in the wave costs its compare and one uniform branch -- and cut by the radix walk over
// their bit patterns (section 3.2, "Extension to Decoding"), starting from the range the gate and the
// largest key span; each candidate's physical page is requested as soon as it is gathered, and the forced
// pages' before the first barrier.  The list is written between the sink and local pages and the next
// gate is stored.
//
// Returns 1 when the row was selected; 0 when the candidates number fewer than K' or more than kGateCap:
// nothing was written, and pre_mn / pre_mx hold the free keys' range for the whole-row cut (histograms
// cleared, past a barrier); -1 when the gate is absent or there is nothing to rank (nothing done).  `seen`
// receives the candidate count.  Every thread of the workgroup must call this.
template <int NW, int KPL>
__device__ __forceinline__ int select_row_gated(const SelectArgs& a, const uint32_t (&key)[KPL],
                                                const SlotPhys<KPL>& phys, const RowShape r, const size_t row,
                                                const TopkGateRow& gr, SelectSmem<NW, KPL, false>& sm, GateSmem& gs,
                                                uint32_t& seen, uint32_t& pre_mn, uint32_t& pre_mx) {
  constexpr int STRIDE = NW * kWave;
  constexpr int CS = kGateCap / STRIDE;  // candidate slots per lane in the cut
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int n_free = r.local_begin - r.sink_end;
  const int n_forced = r.n - n_free;
  const int kp = a.budget - n_forced;
  seen = 0u;
  if (!gr.valid || kp <= 0 || n_free <= kp) return -1;  // uniform: nothing to rank, or no prediction
  const int wbase = wave * kWave * KPL + lane;
  auto page_of = [&](int i) { return wbase + i * kWave; };
  const uint32_t gate_key = max(score_key(gr.lo), 1u);  // above 0: the cleared slots are never candidates
  const __amdgpu_buffer_rsrc_t bt_r = make_rsrc(phys.bt_row, phys.bt_row ? (uint32_t)r.n * 4u : 0u);
  // forced page threadIdx.x (sinks, then locals): its physical page, requested now, written last
  const int n_local_pages = r.n - r.local_begin;
  const int n_fixed = r.sink_end + n_local_pages;
  const int t = (int)threadIdx.x;
  const int fpg = t < r.sink_end ? t : r.local_begin + (t - r.sink_end);
  const int32_t fph = buf_load_i32(bt_r, (uint32_t)(t < n_fixed ? fpg : 0) * 4u);
  // ---- range, candidate count; clear the first two histogram buffers
  uint32_t mn = 0xffffffffu, mx = 0u, c = 0u;
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    mx = max(mx, key[i]);
    mn = min(mn, key[i] ? key[i] : 0xffffffffu);
    c += (uint32_t)__popcll(__ballot(key[i] >= gate_key));  // wave-uniform
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    sm.wmin[wave] = mn;
    sm.wmax[wave] = mx;
    sm.wsure[wave] = c;
  }
  for (int e = threadIdx.x; e < 2 * SelectDigit<false>::kBins; e += STRIDE) (&sm.hist[0][0])[e] = 0;
  if (threadIdx.x == 0) sm.cand_count = 0;
  __syncthreads();
  mn = wave_min(lane < NW ? sm.wmin[lane] : 0xffffffffu);
  mx = wave_max(lane < NW ? sm.wmax[lane] : 0u);
  const uint32_t wl = lane < NW ? sm.wsure[lane] : 0u;
  const uint32_t wincl = wave_incl_scan(wl);
  const uint32_t count = lane_u32(wincl, NW - 1);
  seen = count;
  pre_mn = mn;
  pre_mx = mx;
  if (count < (uint32_t)kp || count > (uint32_t)kGateCap) return 0;  // uniform
  // ---- gather in page order
  uint32_t pos = lane_u32(wincl - wl, wave);
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    const bool ci = key[i] >= gate_key;
    const unsigned long long m = __ballot(ci);
    if (m) {
      if (ci) {
        const uint32_t q = pos + lanes_below(m);
        gs.key[q] = key[i];
        gs.page[q] = page_of(i);
      }
      pos += (uint32_t)__popcll(m);
    }
  }
  __syncthreads();
  // the cut among the candidates: slot i of a lane holds candidate wave * 64 CS + 64 i + lane (page order)
  const int cbase = wave * kWave * CS + lane;
  uint32_t ck[CS];
  int32_t cpg[CS], cph[CS];
#pragma unroll
  for (int i = 0; i < CS; ++i) {
    const bool in = cbase + i * kWave < (int)count;
    ck[i] = in ? gs.key[cbase + i * kWave] : 0u;
    cpg[i] = in ? gs.page[cbase + i * kWave] : 0;
    cph[i] = buf_load_i32(bt_r, (uint32_t)cpg[i] * 4u);
  }
  auto order_of = [&](int i) { return cbase + i * kWave; };
  auto free_c = [&](int i) { return order_of(i) < (int)count; };
  auto forced_c = [&](int) { return false; };
  int dec;
  uint32_t kc, next_key, top_key;
  int need_eq;
  row_cut<NW, CS, false, SelectDigit<false>::kBits, true>(a, ck, free_c, forced_c, (int)count, n_forced, sm, dec, kc,
                                                         need_eq, next_key, top_key, gate_key, mx);
  if (dec == 1) {  // exactly K' candidates: all taken
    kc = 0u;
    need_eq = kNoLimit;
  }
  // compaction: the chosen candidates after the sink pages
  auto take_sure = [&](int i) { return free_c(i) && ck[i] > kc; };
  auto take_eq = [&](int i) { return free_c(i) && ck[i] == kc; };
  uint32_t sure_l = 0, eq_l = 0;
#pragma unroll
  for (int i = 0; i < CS; ++i) {
    sure_l += take_sure(i) ? 1u : 0u;
    eq_l += take_eq(i) ? 1u : 0u;
  }
  const uint32_t sure_w = wave_sum(sure_l), eq_w = wave_sum(eq_l);
  if (lane == 0) {
    sm.wsure[wave] = sure_w;
    sm.weq[wave] = eq_w;
  }
  __syncthreads();
  const uint32_t sw_l = lane < NW ? sm.wsure[lane] : 0u, ew_l = lane < NW ? sm.weq[lane] : 0u;
  const uint32_t sw_incl = wave_incl_scan(sw_l), ew_incl = wave_incl_scan(ew_l);
  const uint32_t sure_before = lane_u32(sw_incl - sw_l, wave), eq_before = lane_u32(ew_incl - ew_l, wave);
  const uint32_t ne = (uint32_t)need_eq;
  const uint32_t chosen = lane_u32(sw_incl, NW - 1) + min(lane_u32(ew_incl, NW - 1), ne);
  uint32_t q0 = (uint32_t)r.sink_end + sure_before + min(eq_before, ne);
  int eq_left = eq_before < ne ? (int)(ne - eq_before) : 0;
  int32_t* out = a.page_list + row * a.max_list;
  int32_t* out_phys = a.page_phys ? a.page_phys + row * a.max_list : nullptr;
  float* out_sc = a.sel_scores ? a.sel_scores + row * a.max_list : nullptr;
#pragma unroll
  for (int i = 0; i < CS; ++i) {
    const unsigned long long eq_mask = __ballot(take_eq(i));
    const bool take = take_sure(i) || (take_eq(i) && (int)lanes_below(eq_mask) < eq_left);
    const unsigned long long take_mask = __ballot(take);
    const uint32_t q = q0 + lanes_below(take_mask);
    if (take && q < (uint32_t)a.max_list) {
      out[q] = cpg[i];
      if (out_phys) out_phys[q] = cph[i];
      if (out_sc) out_sc[q] = key_to_score(ck[i]);
    }
    q0 += (uint32_t)__popcll(take_mask);
    eq_left -= __popcll(eq_mask);
  }
  // the forced pages: sinks first, locals last (every free page lies between them); the first round's
  // physical pages were requested at the start
  for (int i = t; i < n_fixed; i += STRIDE) {
    const bool sink = i < r.sink_end;
    const int pg = sink ? i : r.local_begin + (i - r.sink_end);
    const uint32_t q = sink ? (uint32_t)i : (uint32_t)r.sink_end + chosen + (uint32_t)(i - r.sink_end);
    if (q < (uint32_t)a.max_list) {
      out[q] = pg;
      if (out_phys) out_phys[q] = i == t ? fph : phys.bt_row[pg];
      if (out_sc) out_sc[q] = a.scores[row * a.max_pages + pg];
    }
  }
  if (threadIdx.x == 0) {
    a.list_len[row] = (int)min((uint32_t)r.sink_end + chosen + (uint32_t)n_local_pages, (uint32_t)a.max_list);
    gate_store(a.gate, row, 2, next_key, top_key, gr.lo, 1u, count);  // fewer than 1.5 K' candidates: keep the gate
  }
  return 1;
}

// Select the pages of one dynamic row from its keys (top-K: score_key of the scores;
// coverage: coverage_key of the shares).  phys gives the physical page of each slot (written
// to a.page_phys when that is set); with phys_later its registers are requested here, once the gated
// candidates have not served the row.  Top-K rows with a gate state (gr, gs) also get the next call's
// predicted gate; their keys must be 0 in every slot that is not a free page.  Every thread of the
// workgroup must call this.
template <int NW, int KPL, bool COV>
__device__ __forceinline__ void select_row_keys(const SelectArgs& a, const uint32_t (&key)[KPL],
                                                SlotPhys<KPL>& phys, const RowShape r, const size_t row,
                                                SelectSmem<NW, KPL, COV>& sm, const TopkGateRow* gr = nullptr,
                                                GateSmem* gs = nullptr, bool phys_later = false) {
  uint32_t seen = 0u;
  int gated = -1;  // 1: selected from the candidates; 0: range found, cut the whole row; -1: no gate
  uint32_t pre_mn = 0u, pre_mx = 0u;
  if constexpr (!COV && KPL <= 32) {  // (rows over 32,768 pages keep their registers for the whole-row cut)
    if (a.gate.rows && gr && gs) {
      gated = select_row_gated<NW, KPL>(a, key, phys, r, row, *gr, sm, *gs, seen, pre_mn, pre_mx);
      if (gated == 1) return;
    }
  }
  if (phys_later) {
    const int wb = (int)(threadIdx.x / kWave) * kWave * KPL + (int)(threadIdx.x % kWave);
#pragma unroll
    for (int i = 0; i < KPL; ++i) phys.load(i, wb + i * kWave, a.max_pages);
  }
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int n_free = r.local_begin - r.sink_end;
  const int n_forced = r.n - n_free;
  const int wbase = wave * kWave * KPL + lane;
  auto page_of = [&](int i) { return wbase + i * kWave; };
  auto free_at = [&](int i) { return (unsigned)(page_of(i) - r.sink_end) < (unsigned)n_free; };
  auto forced_at = [&](int i) { const int p = page_of(i); return p < r.n && !free_at(i); };
  int dec;
  uint32_t kc, gate_key, top_key;
  int need_eq;
  if (!COV && gated == 0)  // uniform: the gated attempt found the range
    row_cut<NW, KPL, false, SelectDigit<false>::kBits, true>(a, key, free_at, forced_at, n_free, n_forced, sm, dec,
                                                             kc, need_eq, gate_key, top_key, pre_mn, pre_mx);
  else
    row_cut<NW, KPL, COV, SelectDigit<COV>::kBits, false>(a, key, free_at, forced_at, n_free, n_forced, sm, dec, kc,
                                                          need_eq, gate_key, top_key);
  if (!COV && a.gate.rows && threadIdx.x == 0) gate_store(a.gate, row, dec, gate_key, top_key, -INFINITY, 0u, seen);

  // ---- compaction in ascending page order.  Decisions 0 and 1 become cuts that no free key
  // passes (every key is below 0xffffffff) or that every free key passes.
  if (dec == 0) {
    kc = 0xffffffffu;
    need_eq = 0;
  } else if (dec == 1) {
    kc = 0u;
    need_eq = kNoLimit;
  }
  auto take_sure = [&](int i) {
    const bool fr = free_at(i);
    return (page_of(i) < r.n && !fr) || (fr && key[i] > kc);
  };
  auto take_eq = [&](int i) { return free_at(i) && key[i] == kc; };
  uint32_t sure_l = 0, eq_l = 0;  // per lane, then summed over the wave
#pragma unroll
  for (int i = 0; i < KPL; ++i) {
    sure_l += take_sure(i) ? 1u : 0u;
    eq_l += take_eq(i) ? 1u : 0u;
  }
  const uint32_t sure_w = wave_sum(sure_l), eq_w = wave_sum(eq_l);
  if (lane == 0) {
    sm.wsure[wave] = sure_w;
    sm.weq[wave] = eq_w;
  }
  __syncthreads();
  // lane w < NW reads wave w's counts; inclusive scans give this wave's offsets and the totals
  const uint32_t sw_l = lane < NW ? sm.wsure[lane] : 0u, ew_l = lane < NW ? sm.weq[lane] : 0u;
  const uint32_t sw_incl = wave_incl_scan(sw_l), ew_incl = wave_incl_scan(ew_l);
  const uint32_t sure_before = lane_u32(sw_incl - sw_l, wave), eq_before = lane_u32(ew_incl - ew_l, wave);
  const uint32_t sure_total = lane_u32(sw_incl, NW - 1), eq_total = lane_u32(ew_incl, NW - 1);
  const uint32_t ne = (uint32_t)need_eq;
  uint32_t pos = sure_before + min(eq_before, ne);              // first list position of this wave
  const uint32_t total = sure_total + min(eq_total, ne);
  int eq_left = eq_before < ne ? (int)(ne - eq_before) : 0;     // equal keys this wave may take

  int32_t* out = a.page_list + row * a.max_list;
  int32_t* out_phys = a.page_phys ? a.page_phys + row * a.max_list : nullptr;
  float* out_sc = a.sel_scores ? a.sel_scores + row * a.max_list : nullptr;
  const uint32_t pos0 = pos;
  auto write = [&](int i, bool take, unsigned long long take_mask) {
    const uint32_t q = pos + lanes_below(take_mask);
    if (take && q < (uint32_t)a.max_list) {
      out[q] = page_of(i);
      if (SlotPhys<KPL>::kInRegs && out_phys) out_phys[q] = phys.at(i, page_of(i));
      // (a top-K slot with key 0 is a forced page of the separate selector: its score is read back below)
      if (out_sc && (COV || key[i] != 0u)) out_sc[q] = COV ? __uint_as_float(key[i]) : key_to_score(key[i]);
    }
    pos += (uint32_t)__popcll(take_mask);
  };
  if (eq_w <= (uint32_t)eq_left) {
    // every key of this wave equal to the cut is taken (the usual case): one ballot per slot
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const bool take = take_sure(i) || take_eq(i);
      const unsigned long long take_mask = __ballot(take);
      if (take_mask) write(i, take, take_mask);
    }
  } else {
    // the wave holds the last keys equal to the cut that are taken: rank them in page order
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const unsigned long long eq_mask = __ballot(take_eq(i));
      const bool take = take_sure(i) || (take_eq(i) && (int)lanes_below(eq_mask) < eq_left);
      write(i, take, __ballot(take));
      eq_left -= __popcll(eq_mask);
      __builtin_amdgcn_sched_barrier(0);  // one slot at a time: keeps the slot's two ballots the only live masks
    }
  }
  if constexpr (!SlotPhys<KPL>::kInRegs) {
    // Long rows keep no physical pages in registers: this wave reads back the list entries it
    // wrote, 64 at a time, and looks their physical pages up in the block table -- two reads
    // per wave, instead of a block-table read waited for in every slot that took a page.
    if (out_phys) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      const uint32_t end = min(pos, (uint32_t)a.max_list);
      for (uint32_t q = pos0 + lane; q < end; q += kWave) out_phys[q] = phys.bt_row[out[q]];
    }
  }
  if (!COV && out_sc && a.scores) {
    // the forced pages' scores, read back (sinks lead the list, locals end it)
    const int n_local_pages = r.n - r.local_begin;
    for (int i = threadIdx.x; i < r.sink_end + n_local_pages; i += NW * kWave) {
      const bool sink = i < r.sink_end;
      const int pg = sink ? i : r.local_begin + (i - r.sink_end);
      const uint32_t q = sink ? (uint32_t)i : total - (uint32_t)n_local_pages + (uint32_t)(i - r.sink_end);
      if (q < (uint32_t)a.max_list) out_sc[q] = a.scores[row * a.max_pages + pg];
    }
  }
  if (threadIdx.x == 0) a.list_len[row] = (int)min(total, (uint32_t)a.max_list);
}

// A streaming row keeps its static sink + local table.
__device__ __forceinline__ void select_streaming_row(const SelectArgs& a, int n, size_t row, const int32_t* bt_row) {
  int32_t* out = a.page_list + row * a.max_list;
  const RowShape r = row_shape(n, a.n_sink_stream, a.n_local_stream);
  const int n_forced = r.sink_end + (n - r.local_begin);
  for (int i = threadIdx.x; i < n_forced && i < a.max_list; i += blockDim.x) {
    const int p = i < r.sink_end ? i : r.local_begin + (i - r.sink_end);
    out[i] = p;
    if (a.page_phys) a.page_phys[row * a.max_list + i] = bt_row[p];
  }
  if (threadIdx.x == 0) a.list_len[row] = min(n_forced, a.max_list);
}

}  // namespace spd
