// gemm_common.h -- pieces shared by the MX GEMM kernels: operand vector
// types, the XCD-aware workgroup -> output tile mapping and the LDS-staged
// epilogue of a wave's 128x128 accumulator tile.
#pragma once
#include <stdint.h>

#include "../launch.h"
#include "codec.h"
#include "wave.h"

namespace mxk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));  // plain vector: stays in registers

// Map a linear workgroup id to a (tile_m, tile_n) so that the ids that land
// on one XCD (id mod 8) form compact groups of tiles.
__device__ inline void tile_of(uint32_t id, uint32_t tm, uint32_t tn, uint32_t* m, uint32_t* n) {
  const uint32_t total = tm * tn;
  uint32_t lin = id;
  if ((total & 7u) == 0) {
    const uint32_t per = total >> 3;
    lin = (id & 7u) * per + (id >> 3);
  }
  const uint32_t G = 4;  // groups of G tile-rows, column-major inside a group
  const uint32_t group = lin / (G * tn);
  const uint32_t first_m = group * G;
  const uint32_t gsize = (tm - first_m) < G ? (tm - first_m) : G;
  const uint32_t in = lin - group * G * tn;
  *m = first_m + in % gsize;
  *n = in / gsize;
}

// Nonzero when some byte of w lies outside [lo, hi], for 1 <= lo <= 128 and
// 127 <= hi <= 254: a byte below lo borrows into its bit 7 when lo is
// subtracted from every byte while its own bit 7 is clear (exact as a test of
// the whole word), and a byte above hi is one whose complement is below
// 255 - hi.
__device__ inline uint32_t bytes_outside(uint32_t w, uint32_t lo, uint32_t hi) {
  const uint32_t below = (w - lo * 0x01010101u) & ~w & 0x80808080u;
  const uint32_t nw = ~w;
  const uint32_t above = (nw - (255u - hi) * 0x01010101u) & ~nw & 0x80808080u;
  return below | above;
}

// Epilogue through LDS: each wave writes its 128x128 accumulator tile into
// LDS in 64-row halves and stores it back row-contiguous, 16 bytes per lane.
template <int CDT>
__device__ inline void store_tile(uint8_t* __restrict__ smem, const v16f (&acc)[4][4], void* C,
                                  int64_t ldc, int64_t M, int64_t N, int64_t r0, int64_t c0,
                                  bool vec, uint32_t wid, uint32_t lane) {
  constexpr int EB = CDT == DT_F32 ? 4 : 2;   // bytes per element
  constexpr int PITCH = 128 * EB + 16;        // LDS row pitch (bank spread)
  uint8_t* W = smem + wid * (64 * PITCH);
  const uint32_t lr = lane & 31u, lg = lane >> 5;
#pragma unroll
  for (int h = 0; h < 2; ++h) {           // row halves 0..63, 64..127 of the wave tile
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {      // instruction-tile rows inside the half
      const int i = 2 * h + i2;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t row = i2 * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
          const uint32_t col = j * 32 + lr;
          if constexpr (CDT == DT_F32) *reinterpret_cast<float*>(W + row * PITCH + col * 4) = acc[i][j][v];
          else *reinterpret_cast<uint16_t*>(W + row * PITCH + col * 2) = f32_to_bf16(acc[i][j][v]);
        }
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // own LDS writes done
    asm volatile("" ::: "memory");
    // 64 rows x (128 * EB) bytes; each lane moves 16 bytes per step
    constexpr int LPR = 128 * EB / 16;  // lanes per row
    constexpr int RPI = 64 / LPR;       // rows per instruction
#pragma unroll
    for (int k = 0; k < 64 / RPI; ++k) {
      const uint32_t row = k * RPI + lane / LPR;
      const uint32_t cb = (lane % LPR) * 16;
      const u4 val = *reinterpret_cast<const u4*>(W + row * PITCH + cb);
      const int64_t grow = r0 + h * 64 + row;
      const int64_t gcol = c0 + cb / EB;
      if (grow < M) {
        if (vec && gcol + 16 / EB <= N) {
          store_nt(static_cast<uint8_t*>(C) + (grow * ldc + gcol) * EB, val[0], val[1], val[2], val[3]);
        } else {
          for (int e = 0; e < 16 / EB; ++e)
            if (gcol + e < N) {
              if constexpr (CDT == DT_F32) static_cast<uint32_t*>(C)[grow * ldc + gcol + e] = val[e];
              else static_cast<uint16_t*>(C)[grow * ldc + gcol + e] = (uint16_t)(val[e / 2] >> (16 * (e & 1)));
            }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // reads done before reuse
    asm volatile("" ::: "memory");
  }
}

}  // namespace mxk
