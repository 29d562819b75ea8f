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

// ------------------------------------------------------------------ wave reductions

template <int WIDTH>
__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int o = 1; o < WIDTH; o <<= 1) v += __shfl_xor(v, o, kWave);
  return v;
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

}  // namespace spd
