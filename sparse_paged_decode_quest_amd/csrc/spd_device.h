// Device helpers shared by the gfx950 kernels of the sparse paged decode step.
//
// Wavefronts are 64 lanes.  Every kernel here is launched with 256-thread (4-wave)
// workgroups unless its launcher says otherwise.
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spd.h"

namespace spd {

constexpr int kPage = SPD_PAGE_SIZE;  // tokens per page
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct fp8_t {
  uint8_t bits;
};

// ------------------------------------------------------------------ storage decoding

// E4M3FN code -> fp16 bits holding the code's value times 2^-8, exactly.
// The 7 magnitude bits shifted left by 7 land in fp16's exponent / mantissa fields: an
// E4M3 normal 2^(e-7)(1+m/8) becomes the fp16 normal 2^(e-15)(1+m/8) and an E4M3
// subnormal m*2^-9 the fp16 subnormal m*2^-17; both are the value times 2^-8.  NaN codes
// are not special-cased (callers never read them: they are masked slots).
__device__ __forceinline__ uint32_t fp8x2_to_half2_scaled(uint32_t two_codes_in_low16) {
  // place code0 in the high byte of half 0 and code1 in the high byte of half 1
  uint32_t y = __builtin_amdgcn_perm(0u, two_codes_in_low16, 0x010c000cu);
  return (y & 0x80008000u) | ((y >> 1) & 0x3f803f80u);
}

__device__ __forceinline__ float fp8_to_float(uint32_t code) {
  uint32_t hb = ((code & 0x80u) << 8) | ((code & 0x7fu) << 7);
  return __half2float(__ushort_as_half((unsigned short)hb)) * 256.0f;
}

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return __half2float(__ushort_as_half(b));
}

// Smallest fp16 >= x (x finite, exactly representable in fp32).
__device__ __forceinline__ uint16_t f32_to_f16_round_up(float x) {
  __half h = __float2half_rn(x);
  uint16_t bits = __half_as_ushort(h);
  if (__half2float(h) < x) {
    if (bits == 0x8000u) bits = 0x0001u;
    else if (bits & 0x8000u) bits = (uint16_t)(bits - 1u);
    else bits = (uint16_t)(bits + 1u);
  }
  return bits;
}

// Largest fp16 <= x.
__device__ __forceinline__ uint16_t f32_to_f16_round_down(float x) {
  __half h = __float2half_rn(x);
  uint16_t bits = __half_as_ushort(h);
  if (__half2float(h) > x) {
    if (bits == 0x0000u) bits = 0x8001u;
    else if (bits & 0x8000u) bits = (uint16_t)(bits + 1u);
    else bits = (uint16_t)(bits - 1u);
  }
  return bits;
}

// bfloat16 (the top 16 bits of an fp32): nearest, ties to even; NaN stays a quiet NaN and values
// past the largest finite bf16 round to infinity.
__device__ __forceinline__ uint16_t f32_to_bf16_rn(float x) {
  const uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
  return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// The two bf16 values packed in a 32-bit word, as fp32 (exact: a shift).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ------------------------------------------------------------------ streaming loads

// Loads of data read once per step (page meta in the scorer, K / V pages in decode), marked
// non-temporal: they stream past the caches instead of displacing what is reused.
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
typedef float nt_f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_stream(const uint4* p) {
  const nt_u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 ld_stream(const float4* p) {
  const nt_f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const nt_f32x4*>(p));
  return make_float4(v.x, v.y, v.z, v.w);
}
template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  return __builtin_nontemporal_load(p);
}

// ------------------------------------------------------------------ range-checked loads

// Buffer resource over [p, p + bytes), bytes < 2^31: a buffer load at a byte offset outside the
// range returns 0 and touches no memory.  Loads whose need depends on a bound (list entries past a
// list's length, chunks past a row's chunk count) are issued through it without a branch per load --
// a conditional global load compiles to an exec-masked branch around every load, which costs more
// than the load's issue.  The third descriptor word selects 32-bit raw data (gfx9 buffer format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
// (the builtin returns the 32 loaded bits as an unsigned integer: reinterpret, do not convert)
__device__ __forceinline__ float buf_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}
__device__ __forceinline__ int32_t buf_load_i32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(int32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, 0));
}
// Streamed (non-temporal, cache policy bit 1) buffer loads of 16, 4 and 2 bytes.
constexpr int kBufNt = 2;
__device__ __forceinline__ uint4 buf_load_u32x4_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kBufNt);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ uint32_t buf_load_u32_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kBufNt);
}
__device__ __forceinline__ uint32_t buf_load_u16_nt(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)byte_off, 0, kBufNt);
}

// ------------------------------------------------------------------ wave reductions

template <int WIDTH>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// An int32 array read through the constant address space: the compiler issues wave-uniform reads of it
// as scalar loads.  Only for memory the reading kernel never writes.
typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;

// Cross-lane moves through DPP (data-parallel primitives of the gfx9 vector ALU): a lane reads
// another lane's register in the same instruction, without the LDS crossbar that __shfl uses.
// Lanes whose source is out of range, or that the row / bank masks leave unwritten, get 0.
// Controls: quad_perm(1,0,3,2) = 0xb1, quad_perm(2,3,0,1) = 0x4e, row_shr:k = 0x110 + k,
// row_mirror = 0x140, row_half_mirror = 0x141, row_bcast:15 = 0x142, row_bcast:31 = 0x143.
template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

__device__ __forceinline__ unsigned long long lane_u64(unsigned long long v, int lane) {
  return (unsigned long long)lane_u32((uint32_t)v, lane) | ((unsigned long long)lane_u32((uint32_t)(v >> 32), lane) << 32);
}

// Value of the lane 16 rows away (lane ^ 16) and 32 lanes away (lane ^ 32): gfx950's row swaps.
__device__ __forceinline__ float xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
}

__device__ __forceinline__ float xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

// Max / sum over the 16 lanes of a row (every lane of the row receives it), through DPP.
__device__ __forceinline__ float row_max(float v) {
  v = fmaxf(v, __uint_as_float(dpp<0xb1>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<0x4e>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(dpp<0x141>(__float_as_uint(v))));
  return fmaxf(v, __uint_as_float(dpp<0x140>(__float_as_uint(v))));
}

__device__ __forceinline__ float row_sum(float v) {
  v += __uint_as_float(dpp<0xb1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x4e>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x141>(__float_as_uint(v)));
  return v + __uint_as_float(dpp<0x140>(__float_as_uint(v)));
}

// Max / sum over the whole wave (every lane receives it).
__device__ __forceinline__ float wave_max_f(float v) {
  v = row_max(v);
  v = fmaxf(v, xor16(v));
  return fmaxf(v, xor32(v));
}

__device__ __forceinline__ float wave_sum_f(float v) {
  v = row_sum(v);
  v += xor16(v);
  return v + xor32(v);
}

// Inclusive prefix sum over the 64 lanes: Hillis-Steele inside each row of 16 lanes, then the
// row totals are carried across rows with the two row broadcasts.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  v += dpp<0x111>(v);
  v += dpp<0x112>(v);
  v += dpp<0x114>(v);
  v += dpp<0x118>(v);
  v += dpp<0x142, 0xa>(v);
  v += dpp<0x143, 0xc>(v);
  return v;
}

// 64-bit version: the two halves move with the same control, the carry is added back.
__device__ __forceinline__ unsigned long long add_u64_halves(unsigned long long a, uint32_t lo, uint32_t hi) {
  const uint32_t alo = (uint32_t)a, ahi = (uint32_t)(a >> 32);
  const uint32_t rlo = alo + lo;
  const uint32_t rhi = ahi + hi + (rlo < alo ? 1u : 0u);
  return (unsigned long long)rlo | ((unsigned long long)rhi << 32);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ unsigned long long dpp_add_u64(unsigned long long v) {
  return add_u64_halves(v, dpp<CTRL, ROW_MASK>((uint32_t)v), dpp<CTRL, ROW_MASK>((uint32_t)(v >> 32)));
}

__device__ __forceinline__ unsigned long long wave_incl_scan(unsigned long long v) {
  v = dpp_add_u64<0x111>(v);
  v = dpp_add_u64<0x112>(v);
  v = dpp_add_u64<0x114>(v);
  v = dpp_add_u64<0x118>(v);
  v = dpp_add_u64<0x142, 0xa>(v);
  v = dpp_add_u64<0x143, 0xc>(v);
  return v;
}

// Reductions whose result every lane receives: a butterfly inside each row of 16 lanes (two quad
// permutations and two mirrors, every lane has a source), then the four row results are read as
// scalars.  OP is an associative, commutative binary functor.
template <typename OP>
__device__ __forceinline__ uint32_t wave_reduce(uint32_t v, OP op) {
  v = op(v, dpp<0xb1>(v));
  v = op(v, dpp<0x4e>(v));
  v = op(v, dpp<0x141>(v));
  v = op(v, dpp<0x140>(v));
  return op(op(lane_u32(v, 0), lane_u32(v, 16)), op(lane_u32(v, 32), lane_u32(v, 48)));
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
  return wave_reduce(v, [](uint32_t a, uint32_t b) { return a + b; });
}

__device__ __forceinline__ unsigned long long wave_sum(unsigned long long v) {
  v = add_u64_halves(v, dpp<0xb1>((uint32_t)v), dpp<0xb1>((uint32_t)(v >> 32)));
  v = add_u64_halves(v, dpp<0x4e>((uint32_t)v), dpp<0x4e>((uint32_t)(v >> 32)));
  v = add_u64_halves(v, dpp<0x141>((uint32_t)v), dpp<0x141>((uint32_t)(v >> 32)));
  v = add_u64_halves(v, dpp<0x140>((uint32_t)v), dpp<0x140>((uint32_t)(v >> 32)));
  return lane_u64(v, 0) + lane_u64(v, 16) + lane_u64(v, 32) + lane_u64(v, 48);
}

// Sum over aligned groups of WIDTH lanes (8, 16 or 32); every lane of a group receives its sum.
// Half-row / row mirrors and quad permutations stay inside the group, and gfx950's permlane16
// swap pairs the two rows of a 32-lane group.
template <int WIDTH>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(WIDTH == 8 || WIDTH == 16 || WIDTH == 32, "group of 8, 16 or 32 lanes");
  v += __uint_as_float(dpp<0xb1>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x4e>(__float_as_uint(v)));
  v += __uint_as_float(dpp<0x141>(__float_as_uint(v)));
  if constexpr (WIDTH >= 16) v += __uint_as_float(dpp<0x140>(__float_as_uint(v)));
  if constexpr (WIDTH == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v += __uint_as_float((threadIdx.x & 16) ? r[0] : r[1]);
  }
  return v;
}

// Lanes below this one whose bit is set in `mask` (a 64-lane ballot).
__device__ __forceinline__ uint32_t lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ float fmax_nan_safe(float a, float b) { return a > b ? a : b; }

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key); NaN -> 0.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (s != s) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void wave_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

// Number of pages of a request of `len` tokens, clamped to the block-table row.
__device__ __forceinline__ int row_pages(int len, int max_pages) {
  int n = len > 0 ? (len + kPage - 1) / kPage : 0;
  return n < max_pages ? n : max_pages;
}

__device__ __forceinline__ int valid_in_page(int len, int p) {
  int v = len - p * kPage;
  return v < 0 ? 0 : (v > kPage ? kPage : v);
}

// Hierarchical paging (LServe summary, "Hierarchical Paging"): a physical page of kPage << lgs
// tokens holds 2^lgs logical pages of kPage tokens.  Logical page lp of a request lives in the
// physical page of block-table slot lp >> lgs, as sub-page lp & (2^lgs - 1).  With lgs = 0 the two
// coincide.
__device__ __forceinline__ int row_logical_pages(int len, int max_pages, int lgs) {
  return row_pages(len, max_pages << lgs);
}

__device__ __forceinline__ int row_phys_pages(int len, int max_pages, int lgs) {
  static_assert(kPage == 16, "pages are 2^4 tokens");
  const int n = len > 0 ? (int)(((unsigned)len + (kPage << lgs) - 1) >> (4 + lgs)) : 0;  // shifts, no division
  return n < max_pages ? n : max_pages;
}

// Index of the kPage-token unit holding sub-page `sub` of physical page `phys`, KV head h, in the
// pools ([pages, Hkv, kPage << lgs, d]): its keys start at element unit * kPage * d and its scales
// at unit * kPage.
__device__ __forceinline__ size_t head_unit(int phys, int num_kv_heads, int h, int lgs, int sub) {
  return (((size_t)phys * num_kv_heads + h) << lgs) + (size_t)sub;
}

// Index of logical page p of request b, KV head h, in the key statistics ([B, Hkv, max_pages << lgs,
// 2, d]): its box starts at element index * 2 * d.  The statistics are kept per request in logical
// page order, head-major, so a scan over a row's pages reads one contiguous run and its addresses do
// not wait for the block table.
__device__ __forceinline__ size_t meta_unit(int b, int h, int p, int num_kv_heads, int max_pages, int lgs) {
  return ((size_t)b * num_kv_heads + h) * ((size_t)max_pages << lgs) + (size_t)p;
}

}  // namespace spd
