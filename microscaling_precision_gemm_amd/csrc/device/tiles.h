// tiles.h -- byte offsets of the matrix-instruction tile layout of MX code
// and scale arrays (the layout is specified with mx_layout in include/mx.h).
//
// codes: tiles of 32 rows x 128 code bytes, 4096 bytes each, row-tile major;
//        chunk c (16 bytes) of tile row r at (c/2)*1024 + ((c%2)*32 + r)*16.
// scales: tiles of 32 rows x 32 blocks, 1024 bytes each, row-tile major;
//        block b of tile row r at ((b%2)*32 + r)*16 + b/2.
#pragma once
#include <stdint.h>

namespace mxk {

// Offset of code byte `kb` (within its row) of row `row`; row_bytes is the
// code bytes per row (a multiple of 512).
__host__ __device__ inline int64_t tiled_code_off(int64_t row, int64_t kb, int64_t row_bytes) {
  const int64_t tile = (row >> 5) * (row_bytes >> 7) + (kb >> 7);
  const uint32_t c = (uint32_t)(kb >> 4) & 7u, r = (uint32_t)row & 31u;
  return tile * 4096 + (c >> 1) * 1024 + ((c & 1u) * 32u + r) * 16u + (uint32_t)(kb & 15);
}

// Offset of the scale of block `blk` (within its row) of row `row`; cols is
// the element count per row (a multiple of 1024).
__host__ __device__ inline int64_t tiled_scale_off(int64_t row, int64_t blk, int64_t cols) {
  const int64_t tile = (row >> 5) * (cols >> 10) + (blk >> 5);
  const uint32_t b = (uint32_t)blk & 31u, r = (uint32_t)row & 31u;
  return tile * 1024 + ((b & 1u) * 32u + r) * 16u + (b >> 1);
}

}  // namespace mxk
