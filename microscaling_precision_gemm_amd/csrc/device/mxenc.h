// mxenc.h -- the MX block encoder shared by the quantizers and the GEMM
// epilogue that writes its output quantized: a lane holds 8 consecutive
// elements of a row and a lane quad one 32-element block ("Microscaling (MX)
// and block-scaled 4-bit formats", sections "Microscaling" and "The idea":
// one shared power-of-two scale per block; "08 - FP4, MXFP4, NVFP4: The
// Blackwell Frontier", section "The two Blackwell formats: MXFP4 vs NVFP4",
// for the ceil rule's waste-or-saturate choice).
#pragma once
#include <stdint.h>

#include "../launch.h"
#include "codec.h"
#include "cvt.h"
#include "wave.h"

namespace mxk {

__device__ inline uint32_t max_abs_bits(const float v[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t b = f2u(v[i]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  return m;
}

// Encoder parameters: the scale rule and the random stream of SR (element n
// of the quantized tensor draws from counter + n / 8).
struct MxEnc {
  bool ceil;
  uint64_t seed, counter;
};

// Per MX format: emax (exponent of the element's largest power of two), the
// FP32 mantissa field of the largest element value (for the ceil rule) and
// bits per element.
template <int FMT>
struct MxFmt;
template <>
struct MxFmt<FMT_MXFP8> { static constexpr uint32_t emax = 8, gmant = 0x600000, bits = 8; };       // 448
template <>
struct MxFmt<FMT_MXFP4> { static constexpr uint32_t emax = 2, gmant = 0x400000, bits = 4; };       // 6
template <>
struct MxFmt<FMT_NVFP4> { static constexpr uint32_t emax = 2, gmant = 0x400000, bits = 4; };       // codes only
template <>
struct MxFmt<FMT_MXINT8> { static constexpr uint32_t emax = 0, gmant = 0x7E0000, bits = 8; };      // 127/64
template <>
struct MxFmt<FMT_MXFP8_E5M2> { static constexpr uint32_t emax = 15, gmant = 0x600000, bits = 8; }; // 57344
template <>
struct MxFmt<FMT_MXFP6_E3M2> { static constexpr uint32_t emax = 4, gmant = 0x600000, bits = 6; };  // 28
template <>
struct MxFmt<FMT_MXFP6_E2M3> { static constexpr uint32_t emax = 2, gmant = 0x700000, bits = 6; };  // 7.5

// One element code of an MX format (RNE, or SR with the 16-bit value r).
template <int FMT>
__device__ inline uint32_t mx_elem_encode(float y, bool sr, uint32_t r) {
  if constexpr (FMT == FMT_MXFP8) return e4m3_encode(y, sr, r);
  else if constexpr (FMT == FMT_MXFP4) return e2m1_encode(y, sr, r);
  else if constexpr (FMT == FMT_MXINT8) return int8_encode(y, sr, r);
  else if constexpr (FMT == FMT_MXFP8_E5M2) return E5M2::encode(y, sr, r);
  else if constexpr (FMT == FMT_MXFP6_E3M2) return E3M2::encode(y, sr, r);
  else return E2M3::encode(y, sr, r);
}

// Encoded chunk: 8 codes packed (8-bit elements: two words, FP4: one, FP6:
// 48 bits in w[0] and the low half of w[1], element i at bits 6i) and the
// block's scale byte.  q is the chunk's linear index (element index / 8).
template <int FMT>
struct Enc {
  uint32_t w[MxFmt<FMT>::bits == 4 ? 1 : 2];
  uint32_t sc;
};

template <int FMT, bool SR>
__device__ inline void encode_mx(const MxEnc& a, int64_t q, const float v[8], Enc<FMT>& e) {
  constexpr uint32_t emax = MxFmt<FMT>::emax;
  uint32_t m = max_abs_bits(v);
  uint32_t o = dpp_xor1(m);
  m = o > m ? o : m;
  o = dpp_xor2(m);
  m = o > m ? o : m;
  constexpr uint32_t gmax_mant = MxFmt<FMT>::gmant;
  const uint32_t sc = a.ceil ? e8m0_ceil_from_amax_bits(m, emax, gmax_mant) : e8m0_from_amax_bits(m, emax);
  float y[8];
  if constexpr (MxFmt<FMT>::emax == 0) {  // INT8: the code can reach 254
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = e8m0_unscale(v[i], sc);  // exact
  } else {
    const float inv = e8m0_inverse(sc);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * inv;  // exact scaling by a power of two
  }
  if constexpr (FMT == FMT_MXFP8_E5M2) {  // RNE and SR on the conversion instructions
    if constexpr (SR) {
      uint32_t r[8];
      rand16x8(a.seed, a.counter, (uint64_t)q, r);
      pack_e5m2_sr(y, r, e.w);
    } else {
      pack_e5m2_rne(y, e.w);
    }
  } else if constexpr ((FMT == FMT_MXFP6_E3M2 || FMT == FMT_MXFP6_E2M3) && !SR) {  // RNE on the conversion
    pack_fp6_rne<FMT == FMT_MXFP6_E3M2>(y, e.w);
  } else if constexpr (FMT != FMT_MXFP8 && FMT != FMT_MXFP4) {
    uint32_t r[8] = {0u, 0u, 0u, 0u, 0u, 0u, 0u, 0u};
    if constexpr (SR) rand16x8(a.seed, a.counter, (uint64_t)q, r);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = mx_elem_encode<FMT>(y[i], SR, r[i]);
    if constexpr (MxFmt<FMT>::bits == 8) {
      e.w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      e.w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    } else {
      e.w[0] = c[0] | (c[1] << 6) | (c[2] << 12) | (c[3] << 18) | (c[4] << 24) | (c[5] << 30);
      e.w[1] = (c[5] >> 2) | (c[6] << 4) | (c[7] << 10);
    }
  } else if constexpr (!SR) {
    if constexpr (FMT == FMT_MXFP8) {
      pack_e4m3_rne(y, e.w);
    } else {
      e.w[0] = pack_e2m1_rne(y);
    }
  } else if constexpr (FMT == FMT_MXFP8) {  // SR on the conversion instructions (cvt.h)
    uint32_t r[8];
    rand16x8(a.seed, a.counter, (uint64_t)q, r);
    pack_e4m3_sr(y, r, e.w);
  } else {
    const u32x4 w = rand_words(a.seed, a.counter, (uint64_t)q);
    e.w[0] = pack_e2m1_sr_words(y, w.x, w.y, w.z, w.w);
  }
  if (sc == 0xFFu) {  // NaN / Inf in the block
#pragma unroll
    for (int i = 0; i < (MxFmt<FMT>::bits == 4 ? 1 : 2); ++i) e.w[i] = 0u;
  }
  e.sc = sc;
}

}  // namespace mxk
