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

// Encoded chunk: 8 codes packed (FP8: two words, FP4: one) and the block's
// scale byte.  q is the chunk's linear index (element index / 8).
template <int FMT>
struct Enc {
  uint32_t w[FMT == FMT_MXFP8 ? 2 : 1];
  uint32_t sc;
};

template <int FMT, bool SR>
__device__ inline void encode_mx(const MxEnc& a, int64_t q, const float v[8], Enc<FMT>& e) {
  constexpr uint32_t emax = FMT == FMT_MXFP8 ? 8u : 2u;
  uint32_t m = max_abs_bits(v);
  uint32_t o = dpp_xor1(m);
  m = o > m ? o : m;
  o = dpp_xor2(m);
  m = o > m ? o : m;
  constexpr uint32_t gmax_mant = FMT == FMT_MXFP8 ? 0x600000u : 0x400000u;
  const uint32_t sc = a.ceil ? e8m0_ceil_from_amax_bits(m, emax, gmax_mant) : e8m0_from_amax_bits(m, emax);
  const float inv = e8m0_inverse(sc);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = v[i] * inv;  // exact scaling by a power of two
  if constexpr (!SR) {
    if constexpr (FMT == FMT_MXFP8) {
      pack_e4m3_rne(y, e.w);
    } else {
      e.w[0] = pack_e2m1_rne(y);
    }
  } else {
    uint32_t r[8];
    rand16x8(a.seed, a.counter, (uint64_t)q, r);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      c[i] = FMT == FMT_MXFP8 ? e4m3_encode(y[i], true, r[i]) : e2m1_encode(y[i], true, r[i]);
    if constexpr (FMT == FMT_MXFP8) {
      e.w[0] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
      e.w[1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
    } else {
      uint32_t p = 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) p |= c[i] << (4 * i);
      e.w[0] = p;
    }
  }
  if (sc == 0xFFu) {  // NaN / Inf in the block
#pragma unroll
    for (int i = 0; i < (FMT == FMT_MXFP8 ? 2 : 1); ++i) e.w[i] = 0u;
  }
  e.sc = sc;
}

}  // namespace mxk
