// cvt.h -- round-to-nearest-even element encoders on gfx950's FP32 -> FP4 /
// FP8 conversion instructions, shared by the quantizers and the requant.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

// Round-to-nearest-even encoders on gfx950's conversion instructions (scale
// operand 1.0, i.e. no scaling).  Over every finite FP32 input they give the
// same codes as the bit-arithmetic encoders of codec.h (checked exhaustively
// on the device): E2M1 saturates to +-6 by itself; E4M3 is clamped to +-448
// first because the instruction sends values past the largest finite
// midpoint to NaN.  Element 2j goes to the low nibble (byte) of pair j.
__device__ inline uint32_t pack_e2m1_rne(const float y[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[0], y[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[2], y[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[4], y[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, y[6], y[7], 1.0f, 3);
  return w;
}

typedef short v2s __attribute__((ext_vector_type(2)));

__device__ inline void pack_e4m3_rne(const float y[8], uint32_t w[2]) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fmaxf(fminf(y[i], 448.0f), -448.0f);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v2s p = {0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, c[4 * h], c[4 * h + 1], 1.0f, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, c[4 * h + 2], c[4 * h + 3], 1.0f, true);
    w[h] = __builtin_bit_cast(uint32_t, p);
  }
}

// The same for inputs the caller has already clamped to +-448.
__device__ inline void pack_e4m3_rne_clamped(const float y[8], uint32_t w[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v2s p = {0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, y[4 * h], y[4 * h + 1], 1.0f, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(p, y[4 * h + 2], y[4 * h + 3], 1.0f, true);
    w[h] = __builtin_bit_cast(uint32_t, p);
  }
}

// E5M2: clamped to +-57344 first, as E4M3 to +-448 (checked on the device over
// every FP32 input up to +Inf and its negative, element and byte placement
// included: 0 mismatches against the software encoder of codec.h).
__device__ inline void pack_e5m2_rne(const float y[8], uint32_t w[2]) {
  float c[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = fmaxf(fminf(y[i], 57344.0f), -57344.0f);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v2s p = {0, 0};
    p = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(p, c[4 * h], c[4 * h + 1], 1.0f, false);
    p = __builtin_amdgcn_cvt_scalef32_pk_bf8_f32(p, c[4 * h + 2], c[4 * h + 3], 1.0f, true);
    w[h] = __builtin_bit_cast(uint32_t, p);
  }
}

// FP6 (E3M2 if BF6, else E2M3): gfx950 converts 32 elements per instruction
// (v_cvt_scalef32_2xpk16_{bf6,fp6}_f32): result field j (bits 6j of the six
// words) is a[j / 2] for even j and b[j / 2] for odd j (probed with distinct
// values per input).  The 8 values go in fields 0..7, zeros elsewhere, so the
// first 48 bits are their codes and the rest are zero.  Clamped to +-28 /
// +-7.5 first.  Checked on the device over every FP32 input up to +Inf and
// its negative, in every field: 0 mismatches against codec.h.
typedef float v16f_cvt __attribute__((ext_vector_type(16)));
typedef unsigned int v6u_cvt __attribute__((ext_vector_type(6)));

template <bool BF6>
__device__ inline void pack_fp6_rne(const float y[8], uint32_t w[2]) {
  constexpr float M = BF6 ? 28.0f : 7.5f;
  v16f_cvt a = {}, b = {};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = fmaxf(fminf(y[2 * i], M), -M);
    b[i] = fmaxf(fminf(y[2 * i + 1], M), -M);
  }
  v6u_cvt r;
  if constexpr (BF6) r = __builtin_amdgcn_cvt_scalef32_2xpk16_bf6_f32(a, b, 1.0f);
  else r = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(a, b, 1.0f);
  w[0] = r[0];
  w[1] = r[1];
}

// ---- stochastic rounding on the conversion instructions ---------------------
// The SR rule used throughout: with lo <= |y| < hi the neighbours, round up
// exactly when r16 < floor((|y| - lo) * 2^16 / (hi - lo)).  gfx950's scaled
// SR conversions take a 32-bit seed and round |y| up exactly when the seed's
// top 16 bits are at least 2^16 - floor((|y| - lo) * 2^16 / (hi - lo)),
// ignoring the lower fraction bits (measured on the device), so the seed
// (~r16 & 0xFFFF) << 16, lower bits zero, takes the rule's decision.
// Inputs are clamped to the largest finite value first (the rule saturates;
// the instruction would round past it).  Checked on the device against the
// software encoders of codec.h for E4M3, E5M2 and E2M1 over every FP32 input
// up to +Inf and its negative.  The FP4 pair instruction draws its first
// element from seed bits 16..31 but its second from bits 15..30, so each
// element of a pair takes a conversion of its own; for the second the seed
// is (~r16 & 0xFFFF) << 15 with every other bit zero (set bits below bit 15
// change some decisions: measured).
typedef float v2f_cvt __attribute__((ext_vector_type(2)));

__device__ inline uint32_t sr_seed(uint32_t r16) { return (~r16 & 0xFFFFu) << 16; }

#define MXK_SR8(BUILTIN, MAXV)                                                                   \
  _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                               \
    const float* c = y + 4 * h;                                                                 \
    const uint32_t* rr = r + 4 * h;                                                             \
    int a = 0;                                                                                  \
    a = BUILTIN(a, fmaxf(fminf(c[0], MAXV), -MAXV), sr_seed(rr[0]), 1.0f, 0);                   \
    a = BUILTIN(a, fmaxf(fminf(c[1], MAXV), -MAXV), sr_seed(rr[1]), 1.0f, 1);                   \
    a = BUILTIN(a, fmaxf(fminf(c[2], MAXV), -MAXV), sr_seed(rr[2]), 1.0f, 2);                   \
    a = BUILTIN(a, fmaxf(fminf(c[3], MAXV), -MAXV), sr_seed(rr[3]), 1.0f, 3);                   \
    w[h] = (uint32_t)a;                                                                         \
  }

// 8 E4M3 codes by SR (r: the 8 random 16-bit values), 4 per word
__device__ inline void pack_e4m3_sr(const float y[8], const uint32_t r[8], uint32_t w[2]) {
  MXK_SR8(__builtin_amdgcn_cvt_scalef32_sr_fp8_f32, 448.0f)
}
// the same for inputs the caller has already clamped to +-448
__device__ inline void pack_e4m3_sr_clamped(const float y[8], const uint32_t r[8], uint32_t w[2]) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const float* c = y + 4 * h;
    const uint32_t* rr = r + 4 * h;
    int a = 0;
    a = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(a, c[0], sr_seed(rr[0]), 1.0f, 0);
    a = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(a, c[1], sr_seed(rr[1]), 1.0f, 1);
    a = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(a, c[2], sr_seed(rr[2]), 1.0f, 2);
    a = __builtin_amdgcn_cvt_scalef32_sr_fp8_f32(a, c[3], sr_seed(rr[3]), 1.0f, 3);
    w[h] = (uint32_t)a;
  }
}
// 8 E5M2 codes by SR
__device__ inline void pack_e5m2_sr(const float y[8], const uint32_t r[8], uint32_t w[2]) {
  MXK_SR8(__builtin_amdgcn_cvt_scalef32_sr_bf8_f32, 57344.0f)
}
#undef MXK_SR8

// 8 E2M1 codes by SR from the four words of one Philox block (w0..w3:
// element 2k draws the low half of word k, element 2k + 1 its high half, as
// in pack_e2m1_sr), element i in nibble i.  Each pair (y[2k], y[2k+1]) is
// converted twice: seeded for element 2k (bits 16..31; its low nibble is
// kept) and for element 2k + 1 (bits 15..30; its high nibble is kept), every
// other seed bit zero.  Only
// byte 0 of each result is used: the compiler does not carry the old
// destination through this instruction, so its byte select cannot merge
// results.  A bit-field insert per pair and two byte permutes assemble the
// word.
__device__ inline uint32_t pack_e2m1_sr_words(const float y[8], uint32_t w0, uint32_t w1,
                                              uint32_t w2, uint32_t w3) {
  float c[8];  // clamped to +-6 (the inputs are not NaN: one median instruction)
#pragma unroll
  for (int i = 0; i < 8; ++i) c[i] = __builtin_amdgcn_fmed3f(y[i], -6.0f, 6.0f);
  const uint32_t n[4] = {~w0, ~w1, ~w2, ~w3};
  uint32_t x[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const v2f_cvt p = {c[2 * k], c[2 * k + 1]};
    const uint32_t lo = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, n[k] << 16, 1.0f, 0);
    const uint32_t hi = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, (n[k] >> 1) & 0x7FFF8000u, 1.0f, 0);
    x[k] = (lo & 0x0Fu) | (hi & 0xFFFFFFF0u);  // byte 0: both codes of the pair
  }
  // byte 0 of x0 and x1 into bytes 0 and 1 (selector 0x0C: a zero byte)
  const uint32_t p01 = __builtin_amdgcn_perm(x[1], x[0], 0x0C0C0400u);
  const uint32_t p23 = __builtin_amdgcn_perm(x[3], x[2], 0x0C0C0400u);
  return p01 | (p23 << 16);
}

// 8 E2M1 codes by SR, element i in nibble i
__device__ inline uint32_t pack_e2m1_sr(const float y[8], const uint32_t r[8]) {
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float c = fmaxf(fminf(y[i], 6.0f), -6.0f);
    const uint32_t t = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, v2f_cvt{c, c}, sr_seed(r[i]), 1.0f, 0);
    w |= (t & 0xFu) << (4 * i);
  }
  return w;
}

}  // namespace mxk
