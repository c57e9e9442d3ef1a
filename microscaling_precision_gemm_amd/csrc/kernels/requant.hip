// requant.hip -- backward-pass requantization: dequantize (NVFP4 or BF16
// source), transpose in FP32 through LDS, and re-quantize to MXFP8 E4M3 with
// 32-element blocks along the former row axis, round-to-nearest-even or
// stochastic ("Thinking Machines ... Inkling 2 Small", section "A precision
// choice for each stage": saved values are de-quantized, transposed at higher
// precision, then stochastically re-quantized to MXFP8).
//
// One workgroup (256 lanes) owns a tile of 64 source rows x 256 source
// columns.  Phase 1: each lane decodes one 16-element source block of one
// row into FP32 and writes it down a column of the LDS tile (a lane per row,
// so the 64 lanes of a wave write 64 consecutive words).  Phase 2: each lane
// reads 8 consecutive source rows of one output row, the 4 lanes of a quad
// form one 32-element MXFP8 block (E8M0 scale via DPP max), encode and store
// 8 codes with one 64-bit store.
#include "../device/codec.h"
#include "../device/wave.h"
#include "../launch.h"

namespace mxk {

namespace {

constexpr int kTR = 64;    // source rows per tile (two MXFP8 blocks)
constexpr int kTC = 256;   // source columns per tile
constexpr int kPitch = 68; // LDS row pitch in floats (16-byte multiple)

template <bool NV, bool SR>
__global__ __launch_bounds__(256) void k_requant_t(const uint8_t* __restrict__ src_codes,
                                                   const uint8_t* __restrict__ src_scales,
                                                   const float* __restrict__ src_ts,
                                                   const uint16_t* __restrict__ xb, int64_t ld_x,
                                                   int64_t rows, int64_t cols,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, uint64_t seed,
                                                   uint64_t counter) {
  __shared__ float tile[kTC * kPitch];
  const int64_t r0 = (int64_t)blockIdx.y * kTR;
  const int64_t c0 = (int64_t)blockIdx.x * kTC;
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u;
  const int rows_here = (int)((rows - r0) < kTR ? (rows - r0) : kTR);   // 32 or 64
  const int cols_here = (int)((cols - c0) < kTC ? (cols - c0) : kTC);   // multiple of 16
  float S = 1.0f;
  if constexpr (NV) S = *src_ts;

  // phase 1: decode source blocks into tile[col][row]
  for (int u = (int)t; u < (kTC / 16) * kTR; u += 256) {
    const int blk = u >> 6;  // 16-column block within the tile
    const int r = u & 63;
    float v[16];
    if (r < rows_here && blk * 16 < cols_here) {
      const int64_t gr = r0 + r, gc = c0 + blk * 16;
      if constexpr (NV) {
        const uint2 p = *reinterpret_cast<const uint2*>(src_codes + gr * (cols >> 1) + (gc >> 1));
        const float sbv = e4m3_mag_value(src_scales[gr * (cols >> 4) + (gc >> 4)]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[i] = (e2m1_value((p.x >> (4 * i)) & 0xFu) * sbv) * S;
          v[8 + i] = (e2m1_value((p.y >> (4 * i)) & 0xFu) * sbv) * S;
        }
      } else {
        const uint4* p = reinterpret_cast<const uint4*>(xb + gr * ld_x + gc);
        const uint4 a = p[0], b = p[1];
        const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          v[2 * i] = u2f(wv[i] << 16);
          v[2 * i + 1] = u2f(wv[i] & 0xFFFF0000u);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) tile[(blk * 16 + i) * kPitch + r] = v[i];
  }
  __syncthreads();

  // phase 2: output row c (a source column) covers source rows r0 .. r0+63
  for (int u = (int)t; u < kTC * (kTR / 8); u += 256) {
    const int c = u >> 3;   // output row within the tile
    const int r8 = u & 7;   // 8-row chunk within the output row
    const float4* src = reinterpret_cast<const float4*>(&tile[c * kPitch + r8 * 8]);
    const float4 a = src[0], b = src[1];
    float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bb = f2u(v[i]) & 0x7FFFFFFFu;
      m = bb > m ? bb : m;
    }
    uint32_t o = dpp_xor1(m);
    m = o > m ? o : m;
    o = dpp_xor2(m);
    m = o > m ? o : m;
    const uint32_t sc = e8m0_from_amax_bits(m, 8u);
    const float inv = e8m0_inverse(sc);
    const bool valid = c < cols_here && r8 * 8 < rows_here;
    const int64_t oc = c0 + c;                 // output row
    const int64_t orow = r0 + r8 * 8;          // first output column of this lane
    const int64_t n = oc * rows + orow;        // output linear index (multiple of 8)
    uint32_t rnd[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (SR) rand16x8(seed, counter, (uint64_t)(n >> 3), rnd);
    uint32_t cc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      cc[i] = e4m3_encode(v[i] * inv, SR, rnd[i]);
      if (sc == 0xFFu) cc[i] = 0u;
    }
    if (valid) {
      uint2 p;
      p.x = cc[0] | (cc[1] << 8) | (cc[2] << 16) | (cc[3] << 24);
      p.y = cc[4] | (cc[5] << 8) | (cc[6] << 16) | (cc[7] << 24);
      *reinterpret_cast<uint2*>(codes + n) = p;
      if ((lane & 3u) == 0) scales[oc * (rows >> 5) + (orow >> 5)] = (uint8_t)sc;
    }
  }
}

}  // namespace

hipError_t launch_requant_transpose(const uint8_t* src_codes, const uint8_t* src_scales,
                                    const float* src_tensor_scale, const uint16_t* x_bf16,
                                    int64_t ld_x, int64_t rows, int64_t cols, uint8_t* codes,
                                    uint8_t* scales, bool sr, uint64_t seed, uint64_t counter,
                                    hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  dim3 grid((unsigned)((cols + kTC - 1) / kTC), (unsigned)((rows + kTR - 1) / kTR));
  const bool nv = src_codes != nullptr;
#define MXK_RQ(NV, SR)                                                                          \
  hipLaunchKernelGGL((k_requant_t<NV, SR>), grid, dim3(256), 0, s, src_codes, src_scales,        \
                     src_tensor_scale, x_bf16, ld_x, rows, cols, codes, scales, seed, counter)
  if (nv) {
    if (sr) MXK_RQ(true, true);
    else MXK_RQ(true, false);
  } else {
    if (sr) MXK_RQ(false, true);
    else MXK_RQ(false, false);
  }
#undef MXK_RQ
  return hipGetLastError();
}

}  // namespace mxk
