// pipe.h -- shared pieces of the DMA-pipelined 256x256 GEMM kernels on
// row-layout operands: stage layout in LDS, the global-to-LDS copy
// assignment, scale staging, the swizzled chunk addressing, waits, barriers
// and instruction-interleave helpers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

constexpr int kTile = 256;                  // BM = BN
constexpr int kRowsAll = 2 * kTile;         // A rows then B rows in a stage
constexpr int kSeg = 128;                   // code bytes per row per K step
constexpr int kCodeBytes = kRowsAll * kSeg; // 64 KB
constexpr int kStageBytes = kCodeBytes;
constexpr int kStages = 2;
// Scales are staged per period of steps: 16 bytes of every row (two FP4
// steps or four FP8 steps), in three rotating 8 KB buffers after the code
// stages, loaded two periods ahead.
constexpr int kScaleRow = 16;
constexpr int kScaleBuf = kRowsAll * kScaleRow;
constexpr int kScaleBufs = 3;
constexpr int kScaleBase = kStages * kStageBytes;
constexpr int kSmemBytes = kScaleBase + kScaleBufs * kScaleBuf;  // 152 KB

// Workgroup barrier for the DMA pipeline: this wave's LDS reads are complete
// (lgkmcnt 0) and the compiler may not move memory accesses across it, but
// DMAs still in flight are not waited for (a memory fence would drain them).
__device__ inline void dma_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Scheduling barrier: no instruction moves across it.
__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// sched_group_barrier masks
constexpr int kSgMfma = 0x008, kSgVmem = 0x010, kSgDsRead = 0x100;

// Order a region as N rounds of (1 MFMA, V vector-memory ops, D LDS reads),
// then the remaining MFMAs of the region's 16.
template <int N, int V, int D>
__device__ inline void interleave() {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    if constexpr (V > 0) __builtin_amdgcn_sched_group_barrier(kSgVmem, V, 0);
    if constexpr (D > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, D, 0);
  }
  if constexpr (N < 16) __builtin_amdgcn_sched_group_barrier(kSgMfma, 16 - N, 0);
}

// s_waitcnt limiting only the vector-memory counter (gfx9 encoding: vmcnt in
// bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef const __attribute__((address_space(1))) void* gbl_ptr_t;

// Copy assignment of one thread: wave-uniform operand bases (waves 0-1 copy
// A rows, waves 2-3 B rows) and 32-bit per-lane byte offsets.  Code
// instruction i of wave w fills LDS rows 8*(16w+i) .. +7 (8 lanes per
// 128-byte row).  Scale instruction of wave w fills 16 bytes of rows
// 64w + lane of operand A (even steps) or B (odd steps).
struct PipeCtx {
  const uint8_t* cbase;
  const uint8_t* sA;
  const uint8_t* sB;
  uint32_t coff[16];
  uint32_t soffA, soffB;
  uint32_t wid;
  uint32_t nper;  // scale periods in K
};

__device__ inline void issue_stage(const PipeCtx& x, uint32_t step, uint8_t* __restrict__ stage) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(x.cbase + (x.coff[i] + step * (uint32_t)kSeg)),
                                     (lds_ptr_t)(stage + (8u * (16u * x.wid + i)) * kSeg), 16, 0, 0);
}

// One scale DMA: period `per` (clamped to the last one; a clamped copy lands
// in a buffer nobody reads) of operand `op`'s rows 64w .. 64w+63 into scale
// buffer `buf`.
__device__ inline void issue_scales(const PipeCtx& x, uint8_t* __restrict__ smem, uint32_t per,
                                    uint32_t buf, uint32_t op) {
  per = per < x.nper ? per : x.nper - 1;
  const uint8_t* base = op ? x.sB : x.sA;
  const uint32_t off = (op ? x.soffB : x.soffA) + per * (uint32_t)kScaleRow;
  __builtin_amdgcn_global_load_lds((gbl_ptr_t)(base + off),
                                   (lds_ptr_t)(smem + kScaleBase + buf * kScaleBuf + op * (kTile * kScaleRow) +
                                               x.wid * (64 * kScaleRow)),
                                   16, 0, 0);
}

// LDS byte offset of logical 16-byte chunk c of stage row r.  The LDS banks
// span 256 bytes (two rows) and a 16-byte read is served 16 lanes at a time,
// so the chunks of a row are XOR-swizzled by (row >> 1) & 7: 16 consecutive
// rows reading the same logical chunk land on 16 distinct 16-byte slots.
__device__ inline uint32_t swz(uint32_t r) { return (r >> 1) & 7u; }
__device__ inline uint32_t chunk_off(uint32_t r, uint32_t c) { return r * kSeg + 16u * (c ^ swz(r)); }

constexpr int kSgValu = 0x002;

// Order a region as 16 matrix instructions with V VALU, D LDS-read and M
// vector-memory instructions spread between them.
template <int V, int D, int M, int I = 0>
__device__ inline void spread_x() {
  if constexpr (I < 16) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    constexpr int v = ((I + 1) * V + 15) / 16 - (I * V + 15) / 16;
    constexpr int d = ((I + 1) * D + 15) / 16 - (I * D + 15) / 16;
    constexpr int m = ((I + 1) * M + 15) / 16 - (I * M + 15) / 16;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(kSgValu, v, 0);
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, d, 0);
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(kSgVmem, m, 0);
    spread_x<V, D, M, I + 1>();
  }
}

// As spread_x, with the D LDS reads issued within the first 8 matrix
// instructions, so that they have landed when the next region's VALU work
// (which consumes them) starts.
template <int V, int D, int M, int I = 0>
__device__ inline void spread_front() {
  if constexpr (I < 16) {
    __builtin_amdgcn_sched_group_barrier(kSgMfma, 1, 0);
    constexpr int v = ((I + 1) * V + 15) / 16 - (I * V + 15) / 16;
    constexpr int d = I < 8 ? ((I + 1) * D + 7) / 8 - (I * D + 7) / 8 : 0;
    constexpr int m = ((I + 1) * M + 15) / 16 - (I * M + 15) / 16;
    if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(kSgDsRead, d, 0);
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(kSgValu, v, 0);
    if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(kSgVmem, m, 0);
    spread_front<V, D, M, I + 1>();
  }
}

}  // namespace mxk
