// wave.h -- cross-lane helpers for 64-wide CDNA wavefronts (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

// DPP quad permutations: lane i of each quad reads lane perm[i].
// [1,0,3,2] -> 0xB1 (exchange with lane ^ 1); [2,3,0,1] -> 0x4E (lane ^ 2).
__device__ inline uint32_t dpp_xor1(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);
}
__device__ inline uint32_t dpp_xor2(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);
}
__device__ inline float dpp_xor1f(float v) { return __builtin_bit_cast(float, dpp_xor1(__builtin_bit_cast(uint32_t, v))); }

__device__ inline uint32_t lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// value of `v` held by lane `src` (any lane of the wave)
__device__ inline uint32_t lane_read(uint32_t v, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src << 2), (int)v);
}

// max over the 64 lanes
__device__ inline uint32_t wave_max_u32(uint32_t v) {
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = lane_read(v, lane_id() ^ (uint32_t)off);
    v = v > o ? v : o;
  }
  return v;
}

// Streaming stores (the nt bit) for outputs that no kernel of this library
// reads back at once: GEMM results, decoded tensors, transposed
// re-quantizations larger than the L2s.  Their lines leave the XCD's L2 early
// instead of waiting for the write-back at the end of the kernel.  Quantizer
// outputs, which the GEMM reads next, keep ordinary stores (streamed, the
// quantize + GEMM step measured slower), and so does the FP32 decode, whose
// store instructions each cover every other 16 bytes (streamed, 1.7 times
// slower).  p must be aligned to the store size.
typedef uint32_t st_u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t st_u32x4 __attribute__((ext_vector_type(4)));
__device__ inline void store_nt(void* p, uint32_t a) { __builtin_nontemporal_store(a, static_cast<uint32_t*>(p)); }
__device__ inline void store_nt(void* p, uint32_t a, uint32_t b) {
  __builtin_nontemporal_store(st_u32x2{a, b}, static_cast<st_u32x2*>(p));
}
__device__ inline void store_nt(void* p, uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  __builtin_nontemporal_store(st_u32x4{a, b, c, d}, static_cast<st_u32x4*>(p));
}

}  // namespace mxk
