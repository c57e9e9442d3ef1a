// requant.hip -- backward-pass requantization: dequantize (NVFP4 or BF16
// source), transpose through LDS (as exact 16-bit values; NVFP4's per-tensor
// scale is applied in FP32 after the transpose), and re-quantize to MXFP8 E4M3 with
// 32-element blocks along the former row axis, round-to-nearest-even or
// stochastic ("Thinking Machines ... Inkling 2 Small", section "A precision
// choice for each stage": saved values are de-quantized, transposed at higher
// precision, then stochastically re-quantized to MXFP8).
//
// One workgroup (256 lanes) owns a tile of 128 source rows x 64 source
// columns; the output is the 64 x 128 transpose, four MXFP8 blocks per output
// row.
//
// Phase 1 (load, decode): lane task (m, k) takes source rows 2m and 2m+1,
// columns 8k .. 8k+7.  A BF16 row chunk is one 16-byte load, so one load
// instruction reads 8 rows x 128 contiguous bytes; an NVFP4 chunk is 4 code
// bytes and one E4M3 scale byte, decoded to the exact product e2m1 * e4m3
// (at most 6 significant bits, between 2^-10 and 2688: exact in BF16).  For
// each column the two rows are packed into one 32-bit LDS word (row 2m low),
// so the LDS tile holds 16-bit values, column-major: 64 columns x 64 row
// pairs, 16 KB.
//
// Phase 2 (encode, store): lane task (c, j) takes output row c and source
// rows 8j .. 8j+7 (one 16-byte LDS read); a lane quad is one 32-row MXFP8
// block (E8M0 scale from the DPP max), the NVFP4 tensor scale is applied in
// FP32 after the read (the same rounding as decoding in FP32 directly), and
// the 16 lanes of an output row store 128 contiguous code bytes.
#include "../device/codec.h"
#include "../device/cvt.h"
#include "../device/wave.h"
#include "../launch.h"

namespace mxk {

namespace {

constexpr int kTR = 128;        // source rows per tile (four MXFP8 blocks)
constexpr uint32_t kGroup = 8;  // row-tiles per group of the workgroup order

// Source columns per tile and per phase-1 task (8: one 16-byte BF16 load,
// or 4 NVFP4 code bytes and a scale byte, per row).  Wider NVFP4 tasks (32
// columns in 128-column tiles) measured slower, with stochastic rounding
// most of all.
constexpr int kTC = 64;
constexpr int kCH = 8;
constexpr int kChunks = kTC / kCH;          // tasks per row pair
constexpr int kTasks = 64 * kChunks / 256;  // phase-1 tasks per lane

// LDS word of (column c, row pair m).  The row-pair index is XOR-swizzled
// with bits 3..5 of the column, so that the 64 lanes of one phase-1 write
// (8 row pairs x 8 chunks of 8 columns) land in 64 distinct banks, while a
// 16-byte group of 4 row pairs stays contiguous for the phase-2 reads.
__device__ inline uint32_t lds_word(uint32_t c, uint32_t m) { return c * 64u + (m ^ (((c >> 3) & 7u) << 3)); }

// 8 NVFP4 elements (4 code bytes, element 2d in the low nibble of byte d)
// times their E4M3 block scale, as 4 words of exact BF16 pairs.
__device__ inline void decode_nv8(uint32_t p, float sbv, uint32_t* h) {
  // E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as BF16: high bytes
  // 00 3F 3F 3F 40 40 40 40, low bytes 00 00 80 C0 00 40 80 C0.  v_perm
  // looks up four codes at once (selector byte m picks table byte m; the
  // first operand holds entries 4..7).  Even elements are the low nibbles.
  const uint32_t me = p & 0x07070707u, mo = (p >> 4) & 0x07070707u;
  const uint32_t hi_e = __builtin_amdgcn_perm(0x40404040u, 0x3F3F3F00u, me) | ((p << 4) & 0x80808080u);
  const uint32_t lo_e = __builtin_amdgcn_perm(0xC0804000u, 0xC0800000u, me);
  const uint32_t hi_o = __builtin_amdgcn_perm(0x40404040u, 0x3F3F3F00u, mo) | (p & 0x80808080u);
  const uint32_t lo_o = __builtin_amdgcn_perm(0xC0804000u, 0xC0800000u, mo);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // FP32 bits of element 2d (2d+1): byte 3 from the high table, byte 2
    // from the low one, bytes 1, 0 zero (selector 0x0C)
    const uint32_t sel = ((4u + d) << 24) | ((uint32_t)d << 16) | 0x0C0Cu;
    const float a = u2f(__builtin_amdgcn_perm(hi_e, lo_e, sel)) * sbv;  // exact
    const float b = u2f(__builtin_amdgcn_perm(hi_o, lo_o, sel)) * sbv;
    h[d] = (f2u(a) >> 16) | (f2u(b) & 0xFFFF0000u);                     // exact BF16 pair
  }
}

// One phase-1 task's 8 elements of source row gr, columns gc .. gc + 7, as
// BF16 bit patterns, two per word (even column low).
template <bool NV>
__device__ inline void load_task_row(const uint8_t* __restrict__ src_codes,
                                     const uint8_t* __restrict__ src_scales,
                                     const uint16_t* __restrict__ xb, int64_t ld_x, int64_t cols,
                                     int64_t gr, int64_t gc, uint32_t (&h)[4]) {
  if constexpr (NV) {
    const uint32_t p = *reinterpret_cast<const uint32_t*>(src_codes + gr * (cols >> 1) + (gc >> 1));
    decode_nv8(p, e4m3_mag_value(src_scales[gr * (cols >> 4) + (gc >> 4)]), h);
  } else {
    const uint4 v = *reinterpret_cast<const uint4*>(xb + gr * ld_x + gc);
    h[0] = v.x; h[1] = v.y; h[2] = v.z; h[3] = v.w;
  }
}

template <bool NV, bool SR>
__global__ __launch_bounds__(256) void k_requant_t(const uint8_t* __restrict__ src_codes,
                                                   const uint8_t* __restrict__ src_scales,
                                                   const float* __restrict__ src_ts,
                                                   const uint16_t* __restrict__ xb, int64_t ld_x,
                                                   int64_t rows, int64_t cols,
                                                   uint8_t* __restrict__ codes,
                                                   uint8_t* __restrict__ scales, uint64_t seed,
                                                   uint64_t counter, uint32_t tiles_x,
                                                   uint32_t tiles_y) {
  __shared__ uint32_t tile[kTC * (kTR / 2)];
  // Workgroup -> tile: groups of kGroup row-tiles, row-tile fastest inside a
  // group.  The workgroups that run together then cover kGroup x (many)
  // tiles: every source row is read in long runs, and every output row gets
  // kGroup x 128 contiguous bytes (output rows are strided by `rows` bytes).
  uint32_t tx, ty;
  {
    const uint32_t id = blockIdx.x;
    const uint32_t group = id / (kGroup * tiles_x);
    const uint32_t first = group * kGroup;
    const uint32_t gsize = tiles_y - first < kGroup ? tiles_y - first : kGroup;
    const uint32_t in = id - group * kGroup * tiles_x;
    ty = first + in % gsize;
    tx = in / gsize;
  }
  const int64_t r0 = (int64_t)ty * kTR;
  const int64_t c0 = (int64_t)tx * kTC;
  const uint32_t t = threadIdx.x;
  const int rows_here = (int)((rows - r0) < kTR ? (rows - r0) : kTR);  // multiple of 32
  const int cols_here = (int)((cols - c0) < kTC ? (cols - c0) : kTC);  // multiple of 16

  // phase 1: 64 row pairs x kChunks column chunks; all loads first
  uint32_t ha[kTasks][kCH / 2], hb[kTasks][kCH / 2];
#pragma unroll
  for (int u = 0; u < kTasks; ++u) {
    const uint32_t id = (uint32_t)u * 256u + t;
    const uint32_t m = id / kChunks, k = id % kChunks;
    if ((int)(2 * m) < rows_here && (int)(kCH * k) < cols_here) {  // whole chunks: cols % 16 == 0
      const int64_t gr = r0 + 2 * m, gc = c0 + kCH * k;
      load_task_row<NV>(src_codes, src_scales, xb, ld_x, cols, gr, gc, ha[u]);
      load_task_row<NV>(src_codes, src_scales, xb, ld_x, cols, gr + 1, gc, hb[u]);
    }
  }
#pragma unroll
  for (int u = 0; u < kTasks; ++u) {
    const uint32_t id = (uint32_t)u * 256u + t;
    const uint32_t m = id / kChunks, k = id % kChunks;
    if ((int)(2 * m) < rows_here && (int)(kCH * k) < cols_here) {
#pragma unroll
      for (int d = 0; d < kCH / 2; ++d) {
        // columns kCH k + 2d (low halves) and kCH k + 2d + 1 (high halves)
        tile[lds_word(kCH * k + 2 * d, m)] = (ha[u][d] & 0xFFFFu) | (hb[u][d] << 16);
        tile[lds_word(kCH * k + 2 * d + 1, m)] = (ha[u][d] >> 16) | (hb[u][d] & 0xFFFF0000u);
      }
    }
  }
  __syncthreads();

  // phase 2: kTC output rows x 16 eight-row chunks, kTC / 16 tasks per lane
  float S = 1.0f;
  if constexpr (NV) S = *src_ts;
  const uint32_t lane = t & 63u;
#pragma unroll
  for (int u = 0; u < kTC / 16; ++u) {
    const uint32_t id = (uint32_t)u * 256u + t;
    const uint32_t c = id >> 4, j = id & 15u;
    const uint4 w = *reinterpret_cast<const uint4*>(&tile[lds_word(c, 4 * j)]);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float v[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = u2f(ww[d] << 16);
      v[2 * d + 1] = u2f(ww[d] & 0xFFFF0000u);
    }
    if constexpr (NV) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] *= S;
    }
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bb = f2u(v[i]) & 0x7FFFFFFFu;
      mx = bb > mx ? bb : mx;
    }
    uint32_t o = dpp_xor1(mx);
    mx = o > mx ? o : mx;
    o = dpp_xor2(mx);
    mx = o > mx ? o : mx;
    const uint32_t sc = e8m0_from_amax_bits(mx, 8u);
    const float inv = e8m0_inverse(sc);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * inv;  // exact scaling by a power of two
    const int64_t oc = c0 + c;         // output row
    const int64_t orow = r0 + 8 * j;   // first output column of this lane
    const int64_t n = oc * rows + orow;
    uint32_t p[2];
    if constexpr (SR) {
      uint32_t rnd[8];
      rand16x8(seed, counter, (uint64_t)(n >> 3), rnd);
      pack_e4m3_sr(y, rnd, p);  // SR on the conversion instruction
    } else {
      pack_e4m3_rne(y, p);
    }
    if (sc == 0xFFu) p[0] = p[1] = 0u;  // NaN / Inf in the block
    if ((int)c < cols_here && (int)(8 * j) < rows_here) {
      *reinterpret_cast<uint2*>(codes + n) = make_uint2(p[0], p[1]);
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
  const bool nv = src_codes != nullptr;
  const uint32_t tiles_x = (uint32_t)((cols + kTC - 1) / kTC), tiles_y = (uint32_t)((rows + kTR - 1) / kTR);
  if ((uint64_t)tiles_x * tiles_y > 0x7FFFFFFFull) return hipErrorInvalidValue;
  const dim3 grid(tiles_x * tiles_y);
#define MXK_RQ(NV, SR)                                                                          \
  hipLaunchKernelGGL((k_requant_t<NV, SR>), grid, dim3(256), 0, s, src_codes, src_scales,        \
                     src_tensor_scale, x_bf16, ld_x, rows, cols, codes, scales, seed, counter,   \
                     tiles_x, tiles_y)
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
