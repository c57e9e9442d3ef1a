// codec.h -- element/scale encoders and decoders and the counter-based RNG
// used by the gfx950 kernels.  Everything here is __host__ __device__ and free
// of GPU builtins so the same source can be checked exhaustively on the host.
//
// Formats ("Microscaling (MX) and block-scaled 4-bit formats", sections "The
// problem", "Microscaling", "NVFP4"; "08 - FP4, MXFP4, NVFP4: The Blackwell
// Frontier", "Why 4-bit floats at all?" and the MXFP4/NVFP4 table):
//   E2M1 (S E E M): 0, 0.5, 1, 1.5, 2, 3, 4, 6 and negatives;
//   E4M3 (OCP "FN" reading: bias 7, no Inf, 0x7F/0xFF NaN, max 448);
//   E8M0: 2^(c-127), 0xFF NaN.
//
// Encoders work on the FP32 bit pattern of |y|: the kept mantissa bits are the
// top bits of the FP32 mantissa (normal range) or an integer multiple of the
// subnormal step (subnormal range).
//   RNE: round to nearest, ties to the even code; saturate at the largest
//        finite value.
//   SR:  with lo <= |y| < hi the neighbours and r a 16-bit random value,
//        round up exactly when r < floor((|y| - lo) * 2^16 / (hi - lo)); the
//        probability of rounding up is proportional to the distance from lo
//        (glossary "stochastic rounding"; "Thinking Machines ... Inkling 2
//        Small", "A precision choice for each stage").  In the normal range
//        that floor is the discarded mantissa bits shifted right.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

__host__ __device__ inline uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ inline float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// ---- E4M3 ---------------------------------------------------------------
// magnitude code of a (a >= 0, not NaN)
__host__ __device__ inline uint32_t e4m3_rne_mag(float a) {
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) return (uint32_t)rintf(a * 512.0f);  // multiples of 2^-9; 8 = 2^-6
  uint32_t b = f2u(a);
  b += 0x7FFFFu + ((b >> 20) & 1u);
  return (b >> 20) - (120u << 3);
}

__host__ __device__ inline uint32_t e4m3_sr_mag(float a, uint32_t r16) {
  if (a >= 448.0f) return 0x7Eu;
  if (a < 0.015625f) {
    float s = a * 512.0f;  // exact
    float m = floorf(s);
    uint32_t t = (uint32_t)((s - m) * 65536.0f);  // exact, floor of a positive value
    return (uint32_t)m + (r16 < t ? 1u : 0u);
  }
  uint32_t b = f2u(a);
  uint32_t t = (b & 0xFFFFFu) >> 4;
  return (b >> 20) - (120u << 3) + (r16 < t ? 1u : 0u);
}

// exact FP32 value of an E4M3 magnitude code (c in 0..0x7E)
__host__ __device__ inline float e4m3_mag_value(uint32_t c) {
  if (c < 8u) return (float)c * 0.001953125f;  // m * 2^-9
  return u2f((((c >> 3) + 120u) << 23) | ((c & 7u) << 20));
}

// ---- E2M1 ---------------------------------------------------------------
__host__ __device__ inline uint32_t e2m1_rne_mag(float a) {
  if (a >= 6.0f) return 7u;
  if (a < 1.0f) return (uint32_t)rintf(a * 2.0f);  // 0, 0.5, 1.0 -> codes 0, 1, 2
  uint32_t b = f2u(a);
  b += 0x1FFFFFu + ((b >> 22) & 1u);
  uint32_t c = (b >> 22) - 252u;
  return c > 7u ? 7u : c;
}

__host__ __device__ inline uint32_t e2m1_sr_mag(float a, uint32_t r16) {
  if (a >= 6.0f) return 7u;
  if (a < 1.0f) {
    float s = a * 2.0f;
    float m = floorf(s);
    uint32_t t = (uint32_t)((s - m) * 65536.0f);
    return (uint32_t)m + (r16 < t ? 1u : 0u);
  }
  uint32_t b = f2u(a);
  uint32_t t = (b & 0x3FFFFFu) >> 6;
  return (b >> 22) - 252u + (r16 < t ? 1u : 0u);
}

__host__ __device__ inline float e2m1_value(uint32_t c) {
  // magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6 encoded as (exponent, mantissa)
  uint32_t e = (c >> 1) & 3u, m = c & 1u;
  float mag = e == 0 ? 0.5f * (float)m : u2f(((e + 126u) << 23) | (m << 22));
  return (c & 8u) ? -mag : mag;
}

// Sign-carrying encoders for a signed FP32 y.
__host__ __device__ inline uint32_t e4m3_encode(float y, bool sr, uint32_t r16) {
  uint32_t s = (f2u(y) >> 24) & 0x80u;
  float a = __builtin_fabsf(y);
  return s | (sr ? e4m3_sr_mag(a, r16) : e4m3_rne_mag(a));
}
__host__ __device__ inline uint32_t e2m1_encode(float y, bool sr, uint32_t r16) {
  uint32_t s = (f2u(y) >> 28) & 0x8u;
  float a = __builtin_fabsf(y);
  return s | (sr ? e2m1_sr_mag(a, r16) : e2m1_rne_mag(a));
}

// ---- the other MX element types -------------------------------------------
// "Microscaling (MX) and block-scaled 4-bit formats", section "The idea", and
// "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier", section "The OCP
// Microscaling (MX) spec", name FP8 E5M2, FP6 E3M2 / E2M3 and INT8 as MX
// elements; their bits follow the OCP definitions: sign-magnitude minifloats
// with EB exponent bits, MB mantissa bits and bias BIAS (E5M2 keeps its top
// exponent for Inf/NaN, the FP6 types use every code), and INT8 two's
// complement with an implied scale 2^-6 (also the block-scaled "S2F6" combine
// format of "Thinking Machines ... Inkling 2 Small", section "Why
// communication became the next bottleneck").  Encoders saturate at the
// largest finite value; RNE and SR exactly as for E4M3 / E2M1 above.
template <int EB, int MB, int BIAS, uint32_t MAXC>
struct Minifloat {
  static constexpr int kShift = 23 - MB;
  static constexpr uint32_t kSign = 1u << (EB + MB);
  // exact FP32 value of a finite magnitude code
  static __host__ __device__ float value(uint32_t c) {
    const uint32_t e = c >> MB, m = c & ((1u << MB) - 1u);
    if (e == 0) return (float)m * u2f((uint32_t)(128 - BIAS - MB) << 23);  // m * 2^(1-BIAS-MB)
    return u2f(((e + 127u - (uint32_t)BIAS) << 23) | (m << kShift));
  }
  static __host__ __device__ float maxv() { return value(MAXC); }
  static __host__ __device__ float min_normal() { return u2f((uint32_t)(128 - BIAS) << 23); }
  static __host__ __device__ float inv_step() { return u2f((uint32_t)(126 + BIAS + MB) << 23); }
  static __host__ __device__ uint32_t rne_mag(float a) {
    if (a >= maxv()) return MAXC;
    if (a < min_normal()) return (uint32_t)rintf(a * inv_step());
    uint32_t b = f2u(a);
    b += (1u << (kShift - 1)) - 1u + ((b >> kShift) & 1u);
    const uint32_t c = (b >> kShift) - ((127u - (uint32_t)BIAS) << MB);
    return c > MAXC ? MAXC : c;
  }
  static __host__ __device__ uint32_t sr_mag(float a, uint32_t r16) {
    if (a >= maxv()) return MAXC;
    if (a < min_normal()) {
      const float sc = a * inv_step();  // exact
      const float m = floorf(sc);
      const uint32_t t = (uint32_t)((sc - m) * 65536.0f);
      return (uint32_t)m + (r16 < t ? 1u : 0u);
    }
    const uint32_t b = f2u(a);
    const uint32_t t = (b & ((1u << kShift) - 1u)) >> (kShift - 16);
    return (b >> kShift) - ((127u - (uint32_t)BIAS) << MB) + (r16 < t ? 1u : 0u);
  }
  static __host__ __device__ uint32_t encode(float y, bool sr, uint32_t r16) {
    const uint32_t s = (f2u(y) >> 31) ? kSign : 0u;
    const float a = __builtin_fabsf(y);
    return s | (sr ? sr_mag(a, r16) : rne_mag(a));
  }
};
typedef Minifloat<5, 2, 15, 0x7Bu> E5M2;  // largest finite 57344
typedef Minifloat<3, 2, 3, 0x1Fu> E3M2;   // largest 28
typedef Minifloat<2, 3, 1, 0x1Fu> E2M3;   // largest 7.5

// signed value of an E5M2 code (Inf and NaN in the top exponent)
__host__ __device__ inline float e5m2_value(uint32_t c) {
  const uint32_t mag = c & 0x7Fu;
  float v = mag >= 0x7Du ? __builtin_nanf("") : (mag == 0x7Cu ? __builtin_inff() : E5M2::value(mag));
  return (c & 0x80u) ? -v : v;
}
template <class F>
__host__ __device__ inline float fp6_value(uint32_t c) {
  const float v = F::value(c & 0x1Fu);
  return (c & 0x20u) ? -v : v;
}

// INT8 with 6 fraction bits: y * 64 rounded (RNE, or SR on the signed value:
// up toward +inf), saturated to [-128, 127]; the code is the two's
// complement byte.
// The SR threshold floor((s - floor(s)) * 2^16) is formed as
// floor(s * 2^16) - floor(s) * 2^16: for a small negative s, s - floor(s) =
// 1 - |s| would round in FP32, while both terms here are integers below 2^24
// once s is clamped to [-129, 128] (which keeps the saturation).
__host__ __device__ inline uint32_t int8_encode(float y, bool sr, uint32_t r16) {
  const float s = fminf(fmaxf(y * 64.0f, -129.0f), 128.0f);  // y * 64 is exact
  float v;
  if (!sr) {
    v = rintf(s);
  } else {
    const float m = floorf(s);
    const uint32_t t = (uint32_t)(floorf(s * 65536.0f) - m * 65536.0f);
    v = m + (r16 < t ? 1.0f : 0.0f);
  }
  v = fminf(fmaxf(v, -128.0f), 127.0f);
  return (uint32_t)(uint8_t)(int8_t)(int)v;
}
__host__ __device__ inline float int8_value(uint32_t c) { return (float)(int8_t)(uint8_t)c * 0.015625f; }

// ---- E8M0 shared scale of an MX block ------------------------------------
// From the FP32 bits of the block's max |x| (sign cleared): the exponent of
// the largest power of two <= amax, minus the element's emax, clamped so the
// code stays in [0, 254]; 0xFF when the block holds NaN or Inf.
__host__ __device__ inline uint32_t e8m0_from_amax_bits(uint32_t amax_bits, uint32_t emax) {
  if (amax_bits >= 0x7F800000u) return 0xFFu;
  uint32_t e = amax_bits >> 23;  // biased exponent; 0 for zero and subnormals
  return e > emax ? e - emax : 0u;
}
// The same block under the ceil (no-saturation) rule: the smallest scale with
// amax <= gmax * X.  That is the floor code, plus one when amax's significand
// exceeds gmax's (gmax_mant: the element maximum's FP32 mantissa field, E4M3
// 448 = 1.75 * 2^8 -> 0x600000, E2M1 6 = 1.5 * 2^2 -> 0x400000).  Below
// 2^emax * 2^-127 the floor code is clamped to 0 and nothing saturates.
__host__ __device__ inline uint32_t e8m0_ceil_from_amax_bits(uint32_t amax_bits, uint32_t emax,
                                                             uint32_t gmax_mant) {
  if (amax_bits >= 0x7F800000u) return 0xFFu;
  uint32_t e = amax_bits >> 23;
  if (e < emax) return 0u;
  const uint32_t c = e - emax + ((amax_bits & 0x7FFFFFu) > gmax_mant ? 1u : 0u);
  return c > 254u ? 254u : c;  // e clamped to 127 (INT8, emax 0, near the FP32 maximum)
}
// 1 / 2^(code-127) as an exact FP32 (code in 0..253)
__host__ __device__ inline float e8m0_inverse(uint32_t code) { return u2f((254u - code) << 23); }
// v / 2^(code-127) exactly, code in 0..254 (254 would need the FP32
// subnormal 2^-127: two exact steps instead)
__host__ __device__ inline float e8m0_unscale(float v, uint32_t code) {
  return code <= 253u ? v * e8m0_inverse(code) : (v * 0x1p-64f) * 0x1p-63f;
}

// ---- bf16 ---------------------------------------------------------------
__host__ __device__ inline float bf16_to_f32(uint16_t h) { return u2f((uint32_t)h << 16); }
// round to nearest even (inputs here are finite)
__host__ __device__ inline uint16_t f32_to_bf16(float f) {
  uint32_t b = f2u(f);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)(b >> 16);
}

// ---- Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ------------------
struct u32x4 {
  uint32_t x, y, z, w;
};
// a ^ b ^ c: one v_bitop3_b32 on the device (truth table 0x96), which the
// compiler does not always form from two xors by itself
__host__ __device__ inline uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
#if __HIP_DEVICE_COMPILE__
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
#else
  return a ^ b ^ c;
#endif
}

__host__ __device__ inline u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    uint32_t n0 = xor3((uint32_t)(p1 >> 32), c1, k0);
    uint32_t n2 = xor3((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// The Philox block of output elements 8q .. 8q+7 of a stream: element
// 8q + 2k draws the low 16 bits of word k, element 8q + 2k + 1 the high 16.
__host__ __device__ inline u32x4 rand_words(uint64_t seed, uint64_t counter, uint64_t q) {
  const uint64_t c = counter + q;
  return philox4x32_10((uint32_t)c, (uint32_t)(c >> 32), 0u, 0u, (uint32_t)seed,
                       (uint32_t)(seed >> 32));
}

// Eight 16-bit random values for output elements 8q .. 8q+7 of a stream.
__host__ __device__ inline void rand16x8(uint64_t seed, uint64_t counter, uint64_t q,
                                         uint32_t out[8]) {
  const u32x4 w = rand_words(seed, counter, q);
  out[0] = w.x & 0xFFFFu; out[1] = w.x >> 16;
  out[2] = w.y & 0xFFFFu; out[3] = w.y >> 16;
  out[4] = w.z & 0xFFFFu; out[5] = w.z >> 16;
  out[6] = w.w & 0xFFFFu; out[7] = w.w >> 16;
}

// ---- 16-point Hadamard butterflies on 8 in-lane values ---------------------
// Strides 1, 2, 4 inside a half-group of 8 (the stride-8 stage pairs two
// lanes and is done by the caller).
__host__ __device__ inline void hadamard8_stages(float v[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

}  // namespace mxk
