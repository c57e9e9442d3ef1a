// lowscale.h -- products below FP32's resolution in the scaled matrix
// instruction GEMMs, and their exact recomputation.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 forms the exact sum of its products, each
// scaled by 2^(cA - 127) 2^(cB - 127) (E8M0 codes cA, cB), and rounds it once
// into the FP32 accumulator, FP32 subnormals included (probed on the device
// for FP4 pairs at every code sum from 20 to 254).  The result of a K loop is
// then within its bound while every product is a multiple of 2^-149, FP32's
// subnormal spacing: sums of such values below 2^-126 are exact, and above it
// every rounding is relative.  An element of type X is an integer multiple of
// 2^-g(X), so that holds when cA + cB >= 105 + g(A) + g(B).  A tile whose
// scales could pair below that (its smallest A code plus its smallest B code)
// is computed again with its codes raised by bias codes bA, bB, so that every
// product is on the grid, and the accumulators are scaled back by
// 2^-(bA + bB) with one rounding each (v_ldexp_f32) before the epilogue.
#pragma once
#include <stdint.h>

#include "wave.h"

namespace mxk {

// Matrix-instruction element types: 0 E4M3, 1 E5M2, 2 E2M3, 3 E3M2, 4 E2M1.
// g: every value is an integer multiple of 2^-g.  m: |value| < 2^m.
__host__ __device__ constexpr int ls_grid_bits(int type) {
  return type == 0 ? 9 : type == 1 ? 16 : type == 2 ? 3 : type == 3 ? 4 : 1;
}
__host__ __device__ constexpr int ls_max_bits(int type) {
  return type == 0 ? 9 : type == 1 ? 16 : type == 2 ? 3 : type == 3 ? 5 : 3;
}
// smallest code sum whose products are all multiples of 2^-149
__host__ __device__ constexpr int ls_threshold(int ta, int tb) { return 105 + ls_grid_bits(ta) + ls_grid_bits(tb); }

typedef uint16_t ls_u16x2 __attribute__((ext_vector_type(2)));

// Running minimum (two 16-bit lanes) of the four bytes of w.
__device__ inline uint32_t ls_min_bytes(uint32_t acc, uint32_t w) {
  const ls_u16x2 lo = __builtin_bit_cast(ls_u16x2, w & 0x00FF00FFu);
  const ls_u16x2 hi = __builtin_bit_cast(ls_u16x2, (w >> 8) & 0x00FF00FFu);
  const ls_u16x2 a = __builtin_bit_cast(ls_u16x2, acc);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_elementwise_min(a, lo), hi));
}
// Running minimum of the high bytes (1 and 3) of w in the high bytes of the
// two 16-bit lanes of acc: the smallest 16-bit value has the smallest high
// byte, whatever the low bytes.  Feeding w and w << 8 covers all four bytes
// in three instructions.
__device__ inline uint32_t ls_min_hi(uint32_t acc, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(ls_u16x2, acc),
                                                                __builtin_bit_cast(ls_u16x2, w)));
}
__device__ inline uint32_t ls_fold_min_hi(uint32_t acc) {
  const uint32_t a = (acc >> 8) & 0xFFu, b = acc >> 24;
  return a < b ? a : b;
}
// the same for the maximum
__device__ inline uint32_t ls_max_bytes(uint32_t acc, uint32_t w) {
  const ls_u16x2 lo = __builtin_bit_cast(ls_u16x2, w & 0x00FF00FFu);
  const ls_u16x2 hi = __builtin_bit_cast(ls_u16x2, (w >> 8) & 0x00FF00FFu);
  const ls_u16x2 a = __builtin_bit_cast(ls_u16x2, acc);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_elementwise_max(a, lo), hi));
}
__device__ inline uint32_t ls_fold_min(uint32_t acc) {
  const uint32_t a = acc & 0xFFFFu, b = acc >> 16;
  return a < b ? a : b;
}
__device__ inline uint32_t ls_fold_max(uint32_t acc) {
  const uint32_t a = acc & 0xFFFFu, b = acc >> 16;
  return a > b ? a : b;
}

// Bias codes for a tile with code ranges [min_a, max_a] and [min_b, max_b]
// (255, NaN, propagates through the instruction unchanged and is never
// raised).  Returns false when no recomputation is needed or none is
// possible: the raised codes must stay below 255, and the largest raised sum
// of K products must stay below 2^127.
__device__ inline bool ls_bias(int ta, int tb, int64_t K, uint32_t min_a, uint32_t max_a, uint32_t min_b,
                               uint32_t max_b, uint32_t* bias_a, uint32_t* bias_b) {
  const int need = ls_threshold(ta, tb) - (int)(min_a + min_b);
  if (need <= 0) return false;
  const int room_a = max_a >= 255u ? 0 : 254 - (int)max_a;
  const int room_b = max_b >= 255u ? 0 : 254 - (int)max_b;
  if (need > room_a + room_b) return false;
  const int ba = need < room_a ? need : room_a;
  const int bb = need - ba;
  int kbits = 0;
  while (((int64_t)1 << kbits) < K) ++kbits;
  const int top_a = (int)(max_a >= 255u ? 254u : max_a) + ba, top_b = (int)(max_b >= 255u ? 254u : max_b) + bb;
  if (top_a + top_b - 254 + ls_max_bits(ta) + ls_max_bits(tb) + kbits >= 127) return false;
  *bias_a = (uint32_t)ba;
  *bias_b = (uint32_t)bb;
  return true;
}

// Shifts bias_a, bias_b that move every A code of [min_a, max_a] into
// [lo_a, hi_a] and every B code into [lo_b, hi_b] (255 aside), with every
// nonzero product of shifted values at least 2^-126, a normal FP32 value
// (element grids 2^-g_a, 2^-g_b; the BF16 instruction is not relied on for
// subnormal products), and the largest sum of K products (|values| < 2^top)
// below 2^127.  Shifts are as close to zero as the ranges allow.  False when
// none exists.
__device__ inline bool ls_shift(int min_a, int max_a, int min_b, int max_b, int lo_a, int hi_a, int lo_b,
                                int hi_b, int g_a, int g_b, int top_a, int top_b, int64_t K, int* bias_a,
                                int* bias_b) {
  if (min_a > max_a || min_b > max_b) return false;  // NaN codes only
  const int la = lo_a - min_a, ua = hi_a - max_a, lb = lo_b - min_b, ub = hi_b - max_b;
  if (la > ua || lb > ub) return false;
  int ba = la > 0 ? la : (ua < 0 ? ua : 0);
  int bb = lb > 0 ? lb : (ub < 0 ? ub : 0);
  const int need = 128 + g_a + g_b - (min_a + ba + min_b + bb);
  if (need > 0) {
    const int ra = ua - ba < need ? ua - ba : need;
    ba += ra;
    bb += need - ra;
    if (bb > ub) return false;
  }
  int kbits = 0;
  while (((int64_t)1 << kbits) < K) ++kbits;
  if (max_a + ba + max_b + bb - 254 + top_a + top_b + kbits >= 127) return false;
  *bias_a = ba;
  *bias_b = bb;
  return true;
}

// Smallest and largest codes (255 left out) of two runs of scale bytes (na,
// nb bytes from 16-byte aligned pa, pb: whole 16-byte words, then the last
// bytes one by one), over a whole workgroup of 256 threads (red: 16 words of
// LDS); the result is uniform.
__device__ inline void ls_tile_ranges(const uint8_t* pa, int64_t na, const uint8_t* pb, int64_t nb,
                                      uint32_t* red, int* min_a, int* max_a, int* min_b, int* max_b) {
  uint32_t r[4] = {255u, 0u, 255u, 0u};  // min A, max A, min B, max B
  for (int op = 0; op < 2; ++op) {
    const uint8_t* p = op ? pb : pa;
    const int64_t n = op ? nb : na;
    for (int64_t q = threadIdx.x; q < (n >> 4); q += 256) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[q];
      const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
      for (int e = 0; e < 16; ++e) {
        const uint32_t c = (w4[e >> 2] >> (8 * (e & 3))) & 0xFFu;
        if (c == 0xFFu) continue;
        r[2 * op] = c < r[2 * op] ? c : r[2 * op];
        r[2 * op + 1] = c > r[2 * op + 1] ? c : r[2 * op + 1];
      }
    }
    for (int64_t q = (n & ~(int64_t)15) + threadIdx.x; q < n; q += 256) {
      const uint32_t c = p[q];
      if (c == 0xFFu) continue;
      r[2 * op] = c < r[2 * op] ? c : r[2 * op];
      r[2 * op + 1] = c > r[2 * op + 1] ? c : r[2 * op + 1];
    }
  }
  const uint32_t lane = threadIdx.x & 63u, wid = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = lane_read(r[i], lane ^ (uint32_t)off);
      r[i] = (i & 1) ? (o > r[i] ? o : r[i]) : (o < r[i] ? o : r[i]);
    }
  __syncthreads();
  if (lane == 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[4 * wid + i] = r[i];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t x = red[4 * w + i];
      r[i] = (i & 1) ? (x > r[i] ? x : r[i]) : (x < r[i] ? x : r[i]);
    }
  *min_a = (int)r[0];
  *max_a = (int)r[1];
  *min_b = (int)r[2];
  *max_b = (int)r[3];
}

}  // namespace mxk
