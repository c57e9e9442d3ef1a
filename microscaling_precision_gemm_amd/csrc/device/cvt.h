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

}  // namespace mxk
