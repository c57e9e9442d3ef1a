// gemm_tiled.hip -- block-scaled GEMM C = A * B^T for MX operands stored in
// the matrix-instruction tile layout (mx_layout MX_LAYOUT_TILED, specified in
// include/mx.h), on gfx950's scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4 ("Microscaling (MX) and block-scaled 4-bit
// formats", section "Hardware and kernels": the block scales are applied
// inside the matrix instruction).
//
// In the tile layout, the operand fragment of one 32-row x 64-element
// matrix instruction is 1024 contiguous bytes (FP4; FP8 two such runs), with
// lane l's 16 bytes at offset 16 l, and the scales a lane applies over 1024
// elements of K are one 16-byte word.  So every wave loads its fragments
// straight from global memory into registers with fully coalesced 16-byte
// loads, and the main loop uses no LDS at all.  (Measured on gfx950 with
// realistic operands: a variant that shares fragments between the waves
// through a global-to-LDS DMA ring moves fewer bytes per CU, but runs the
// matrix instructions at a lower, power-limited clock and ends up slower
// over the whole quantize + GEMM step.)
//
// Workgroup: 4 waves (2 x 2) over a 256x256 C tile, each wave 128x128 (4x4
// instruction tiles, 256 accumulator registers), one wave per SIMD.  Per K
// step (128 code bytes per row: 256 FP4 or 128 FP8 elements) a wave loads 8
// row tiles (4 of A, 4 of B) x 4 KB.  Fragments are kept one step ahead:
// after the matrix instructions of slice q of step s, the registers of slice
// q receive the loads of step s+1.  Scales are loaded one 1024-element group
// ahead.  The epilogue stages each wave's tile through LDS for row-contiguous
// 16-byte stores.
#include <atomic>

#include "../device/codec.h"
#include "../device/gemm_common.h"
#include "../device/lowscale.h"
#include "../device/mxenc.h"
#include "../device/wave.h"
#include "../launch.h"

namespace mxk {

namespace {

// global-address-space pointers (plain pointers rebuilt from integers would
// compile to flat accesses, which also count against the LDS counter)
typedef const __attribute__((address_space(1))) uint8_t* gptr;
typedef const __attribute__((address_space(1))) u4* gptr4;

template <int FMT>
struct TCfg {
  static constexpr int kSlices = FMT == FMT_MXFP8 ? 2 : 4;        // instructions per step along K
  static constexpr int kParts = FMT == FMT_MXFP8 ? 2 : 1;         // 1 KB loads per tile and slice
  static constexpr int kStepsPerGroup = FMT == FMT_MXFP8 ? 8 : 4; // steps per 1024-element group
};

// Fragments of one slice: 8 row tiles (A 0..3, B 4..7) x parts.
template <int FMT>
struct TSlice {
  u4 f[8][TCfg<FMT>::kParts];
};

template <int FMT>
__device__ inline void load_slice_t(const gptr (&base)[8], uint32_t step, uint32_t q,
                                    uint32_t lane16, TSlice<FMT>& s) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int p = 0; p < TCfg<FMT>::kParts; ++p)
      s.f[t][p] = *reinterpret_cast<gptr4>(
          base[t] + (uint32_t)(step * 4096u + (q * TCfg<FMT>::kParts + p) * 1024u + lane16));
}

__device__ inline v8i widen4(u4 lo) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
}
__device__ inline v8i widen(u4 lo, u4 hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Matrix-instruction element types (cbsz / blgp): FP8 E4M3 0, FP8 E5M2 1,
// FP4 E2M1 4.  A and B may differ within a width class (8-bit or FP4).
template <int FMT>
constexpr int kDefaultType = FMT == FMT_MXFP8 ? 0 : 4;

// 16 instructions of slice Q of step S (within the scale group).  The
// lane's scale byte: FP4 byte Q of dword S; FP8 byte 2 (S % 2) + Q of dword
// S / 2 (opsel selects the byte).
template <int FMT, int S, int Q, int TA, int TB>
__device__ inline void mfma_slice_t(const TSlice<FMT>& f, const u4 (&sc)[8], v16f (&acc)[4][4]) {
  constexpr int D = FMT == FMT_MXFP8 ? S / 2 : S;
  constexpr int OPSEL = FMT == FMT_MXFP8 ? 2 * (S % 2) + Q : Q;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FMT == FMT_MXFP8)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            widen(f.f[i][0], f.f[i][1]), widen(f.f[4 + j][0], f.f[4 + j][1]), acc[i][j], TA, TB, OPSEL,
            (int)sc[i][D], OPSEL, (int)sc[4 + j][D]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            widen4(f.f[i][0]), widen4(f.f[4 + j][0]), acc[i][j], TA, TB, OPSEL, (int)sc[i][D], OPSEL,
            (int)sc[4 + j][D]);
    }
}

__device__ inline void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// A wave-uniform 64-bit value moved to scalar registers.  readfirstlane
// returns a signed int: each half goes through uint32_t so that the low half
// is not sign-extended into the high one.
__device__ inline uint64_t uniform_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return ((uint64_t)hi << 32) | lo;
}

// Steps S .. kStepsPerGroup-1 of group g: after slice q's instructions, slice
// q of the next step (clamped to the last step, a harmless reload) is loaded
// into the same registers.  CHECK: between the group's first instructions and
// the reload of their fragment registers (free registers there), every scale
// code of the group is tested against the quick bound of tiled_wave, and
// lanes that fail set their bit in `low` (wave-uniform, scalar registers).
template <int FMT, int S, int Q, int TA, int TB, bool CHECK>
__device__ inline void run_group(const gptr (&base)[8], uint32_t g, uint32_t steps,
                                 uint32_t lane16, TSlice<FMT> (&fr)[TCfg<FMT>::kSlices],
                                 const u4 (&sc)[8], v16f (&acc)[4][4], uint64_t& low) {
  constexpr int SPG = TCfg<FMT>::kStepsPerGroup, KS = TCfg<FMT>::kSlices;
  if constexpr (S < SPG) {
    if constexpr (Q < KS) {
      const uint32_t st = g * SPG + S;
      const uint32_t nst = st + 1 < steps ? st + 1 : st;
      mfma_slice_t<FMT, S, Q, TA, TB>(fr[Q], sc, acc);
      if constexpr (CHECK && S == 0 && Q == 0) {
        // bit 7 of every byte stays set while every code is at least 64
        // (bit 6 or 7 set), or 96 (bit 7, or bits 6 and 5)
        uint32_t ok = 0x80808080u;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t w = sc[t][d];
            ok &= ls_threshold(TA, TB) <= 128 ? (w << 1) | w : w | ((w << 1) & (w << 2));
          }
        low |= __builtin_amdgcn_ballot_w64((ok & 0x80808080u) != 0x80808080u);
      }
      load_slice_t<FMT>(base, nst, Q, lane16, fr[Q]);
      sched_fence();
      run_group<FMT, S, Q + 1, TA, TB, CHECK>(base, g, steps, lane16, fr, sc, acc, low);
    } else {
      run_group<FMT, S + 1, 0, TA, TB, CHECK>(base, g, steps, lane16, fr, sc, acc, low);
    }
  }
}

// The main loop: the accumulators of this wave's 128x128 part of the C tile
// at (m0, n0).  `low` gets the bits of lanes that saw a scale code below the
// quick bound of tiled_wave.
template <int FMT, int TA, int TB>
__device__ inline void tiled_mainloop(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                      int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                      uint32_t wm, uint32_t wn, uint32_t lane, v16f (&acc)[4][4],
                                      uint64_t& low) {
  using TC = TCfg<FMT>;
  const uint32_t steps = (uint32_t)((FMT == FMT_MXFP8 ? K : K / 2) / 128);  // code tiles per row tile
  const uint32_t groups = (uint32_t)(K / 1024);
  const uint32_t lane16 = lane * 16u;

  // Row tiles of this wave (tiles past M / N repeat the last one; their
  // results are not stored).  Bases are wave-uniform.
  gptr cb[8];
  gptr sb[8];
  const int64_t last_a = M / 32 - 1, last_b = N / 32 - 1;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    int64_t rt = t < 4 ? m0 / 32 + wm * 4 + t : n0 / 32 + wn * 4 + (t - 4);
    const int64_t last = t < 4 ? last_a : last_b;
    rt = rt < last ? rt : last;
    // wave-uniform: keep the bases in scalar registers
    const uint64_t c = reinterpret_cast<uint64_t>((t < 4 ? A : B) + rt * (int64_t)steps * 4096);
    const uint64_t d = reinterpret_cast<uint64_t>((t < 4 ? SA : SB) + rt * (int64_t)groups * 1024);
    cb[t] = (gptr)uniform_u64(c);
    sb[t] = (gptr)uniform_u64(d);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  u4 sc[8], scn[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) sc[t] = *reinterpret_cast<gptr4>(sb[t] + (uint32_t)lane16);
  TSlice<FMT> fr[TC::kSlices];
#pragma unroll
  for (int q = 0; q < TC::kSlices; ++q) load_slice_t<FMT>(cb, 0, q, lane16, fr[q]);

  for (uint32_t g = 0; g < groups; ++g) {
    // next group's scales (the last group reloads its own)
    const uint32_t ng = g + 1 < groups ? g + 1 : g;
#pragma unroll
    for (int t = 0; t < 8; ++t) scn[t] = *reinterpret_cast<gptr4>(sb[t] + (uint32_t)(ng * 1024u + lane16));
    sched_fence();
    run_group<FMT, 0, 0, TA, TB, true>(cb, g, steps, lane16, fr, sc, acc, low);
#pragma unroll
    for (int t = 0; t < 8; ++t) sc[t] = scn[t];
  }

  // the clamped reloads of the last step are still in flight: let them land
  __builtin_amdgcn_s_waitcnt((0 & 15) | (0 << 14) | (7 << 4) | (15 << 8));  // vmcnt(0)
}

// Smallest and largest scale codes over the row tiles this wave reads (A:
// its 4 row tiles of the tile at m0, B: its 4 at n0; clamped at M and N as in
// the main loop), read again from memory: only waves whose quick test fails
// come here.  A scale row tile (32 rows) is K / 1024 tiles of 1 KB,
// contiguous.
__device__ inline void wave_scale_range(const uint8_t* __restrict__ SA, const uint8_t* __restrict__ SB, int64_t M,
                                        int64_t N, int64_t K, int64_t m0, int64_t n0, uint32_t wm, uint32_t wn,
                                        uint32_t lane, uint32_t* min_a, uint32_t* max_a, uint32_t* min_b,
                                        uint32_t* max_b) {
  uint32_t r[4] = {0x00FF00FFu, 0u, 0x00FF00FFu, 0u};  // min A, max A, min B, max B
  for (int t = 0; t < 8; ++t) {
    int64_t rt = t < 4 ? m0 / 32 + wm * 4 + t : n0 / 32 + wn * 4 + (t - 4);
    const int64_t last = (t < 4 ? M : N) / 32 - 1;
    rt = rt < last ? rt : last;
    const uint8_t* p = (t < 4 ? SA : SB) + rt * K;
    const int o = t < 4 ? 0 : 2;
    for (int64_t q = 16 * (int64_t)lane; q < K; q += 16 * 64) {
      const u4 v = *reinterpret_cast<const u4*>(p + q);
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        r[o] = ls_min_bytes(r[o], v[d]);
        r[o + 1] = ls_max_bytes(r[o + 1], v[d]);
      }
    }
  }
  uint32_t f[4] = {ls_fold_min(r[0]), ls_fold_max(r[1]), ls_fold_min(r[2]), ls_fold_max(r[3])};
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t o = lane_read(f[i], lane ^ (uint32_t)off);
      f[i] = (i & 1) ? (o > f[i] ? o : f[i]) : (o < f[i] ? o : f[i]);
    }
  *min_a = (uint32_t)__builtin_amdgcn_readfirstlane(f[0]);
  *max_a = (uint32_t)__builtin_amdgcn_readfirstlane(f[1]);
  *min_b = (uint32_t)__builtin_amdgcn_readfirstlane(f[2]);
  *max_b = (uint32_t)__builtin_amdgcn_readfirstlane(f[3]);
}

// The wave's 128x128 accumulators computed again with every A scale code
// raised by bias_a and every B code by bias_b (no code reaches 255), then
// scaled back by 2^-(bias_a + bias_b) with one rounding each.  A plain loop,
// one 32x32 instruction tile at a time (it reloads fragments, and only waves
// that need it run it), so that it adds few registers to the kernel.
template <int FMT, int TA, int TB>
__device__ inline void tiled_recompute_raised(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                              const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                              int64_t M, int64_t N, int64_t K, int64_t m0, int64_t n0,
                                              uint32_t wm, uint32_t wn, uint32_t lane, uint32_t bias_a,
                                              uint32_t bias_b, v16f (&acc)[4][4]) {
  using TC = TCfg<FMT>;
  const int64_t steps = (FMT == FMT_MXFP8 ? K : K / 2) / 128;
  const uint32_t lane16 = lane * 16u;
  const int sh = -(int)(bias_a + bias_b);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // unrolled: acc stays in registers
      int64_t ra = m0 / 32 + wm * 4 + i, rb = n0 / 32 + wn * 4 + j;
      ra = ra < M / 32 - 1 ? ra : M / 32 - 1;
      rb = rb < N / 32 - 1 ? rb : N / 32 - 1;
      const uint8_t* ca = A + ra * steps * 4096 + lane16;
      const uint8_t* cb = B + rb * steps * 4096 + lane16;
      const uint8_t* sa = SA + ra * K + lane16;  // K / 1024 scale tiles of 1 KB per row tile
      const uint8_t* sb = SB + rb * K + lane16;
      v16f c;
#pragma unroll
      for (int v = 0; v < 16; ++v) c[v] = 0.0f;
      for (int64_t st = 0; st < steps; ++st) {
        const int64_t g = st / TC::kStepsPerGroup;
        const uint32_t S = (uint32_t)(st % TC::kStepsPerGroup);
        const u4 wa = *reinterpret_cast<const u4*>(sa + g * 1024);
        const u4 wb = *reinterpret_cast<const u4*>(sb + g * 1024);
#pragma unroll
        for (int q = 0; q < TC::kSlices; ++q) {
          // the scale byte of slice q of step S (see mfma_slice_t), raised
          const uint32_t byte = (FMT == FMT_MXFP8 ? 2 * S : 4 * S) + (uint32_t)q;
          const uint32_t xa = ((wa[byte >> 2] >> (8 * (byte & 3))) & 0xFFu) + bias_a;
          const uint32_t xb = ((wb[byte >> 2] >> (8 * (byte & 3))) & 0xFFu) + bias_b;
          const uint8_t* pa = ca + st * 4096 + q * TC::kParts * 1024;
          const uint8_t* pb = cb + st * 4096 + q * TC::kParts * 1024;
          if constexpr (FMT == FMT_MXFP8)
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                widen(*reinterpret_cast<const u4*>(pa), *reinterpret_cast<const u4*>(pa + 1024)),
                widen(*reinterpret_cast<const u4*>(pb), *reinterpret_cast<const u4*>(pb + 1024)), c, TA, TB, 0,
                (int)xa, 0, (int)xb);
          else
            c = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen4(*reinterpret_cast<const u4*>(pa)),
                                                                 widen4(*reinterpret_cast<const u4*>(pb)), c, TA,
                                                                 TB, 0, (int)xa, 0, (int)xb);
        }
      }
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = __builtin_amdgcn_ldexpf(c[v], sh);
    }
}

// One wave's part of a tile with the exactness check of lowscale.h: the
// main loop, then -- when the smallest scale codes of the wave's A rows and B
// rows could pair below the threshold of the element types -- the
// accumulators again with raised codes, scaled back, then the epilogue
// `epi(acc)`.  The loop tests every code against a quick bound in two
// instructions per scale dword: at least 64 (96 for pairs whose threshold
// exceeds 128) on both sides settles it, as the sum of the two smallest codes
// then reaches the threshold.  A wave that saw a smaller code (all-zero blocks
// have code 0) reads its exact code ranges.  Waves decide alone: the loop,
// the check and the epilogue are wave-local.
template <int FMT, int TA, int TB, class Epi>
__device__ inline void tiled_wave(const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA,
                                  const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB, int64_t M,
                                  int64_t N, int64_t K, int64_t m0, int64_t n0, uint32_t wm, uint32_t wn,
                                  uint32_t lane, Epi epi) {
  constexpr int kThr = ls_threshold(TA, TB);
  static_assert(kThr <= 192, "threshold above 192");
  v16f acc[4][4];
  uint64_t low = 0;
  tiled_mainloop<FMT, TA, TB>(A, SA, B, SB, M, N, K, m0, n0, wm, wn, lane, acc, low);
  if (low != 0) {  // wave-uniform, rare
    uint32_t a, b, max_a, max_b, ba, bb;
    wave_scale_range(SA, SB, M, N, K, m0, n0, wm, wn, lane, &a, &max_a, &b, &max_b);
    if ((int)(a + b) < kThr && ls_bias(TA, TB, K, a, max_a, b, max_b, &ba, &bb))
      tiled_recompute_raised<FMT, TA, TB>(A, SA, B, SB, M, N, K, m0, n0, wm, wn, lane, ba, bb, acc);
  }
  epi(acc);
}

template <int FMT, int CDT, int TA = kDefaultType<FMT>, int TB = kDefaultType<FMT>>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx_tiled(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t vec) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * 256, n0 = (int64_t)tni * 256;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  tiled_wave<FMT, TA, TB>(A, SA, B, SB, M, N, K, m0, n0, wm, wn, lane, [=](const v16f(&acc)[4][4]) {
    store_tile<CDT>(smem, acc, C, ldc, M, N, m0 + wm * 128, n0 + wn * 128, vec != 0, wid, lane);
  });
}

// ---- GEMM with its output quantized (fused quantize-and-GEMM) --------------
// "Microscaling (MX) and block-scaled 4-bit formats", section "Open points":
// fused quantize-and-GEMM kernels, because computing block scales is memory
// traffic of its own.  The output C = A * B^T is not written in 16 or 32 bits:
// each wave stages its FP32 accumulators through LDS (as the FP32 epilogue
// does), reads 8 consecutive columns of a row per lane -- a lane quad is one
// 32-column block -- and runs the quantizer's block encoder on them, so the
// result is what the MX quantizer makes of the FP32 product matrix, and the
// codes and scales go straight to their layout (row-major, or the
// matrix-instruction tile layout, ready to be the next product's operand).
// The random stream of SR is indexed by the element's row-major position in
// C, as for a quantizer call on C.
template <int OFMT, bool SR, bool OTILED>
__device__ inline void store_tile_quant(uint8_t* __restrict__ smem, const v16f (&acc)[4][4],
                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                        int64_t M, int64_t N, int64_t r0, int64_t c0, uint32_t wid,
                                        uint32_t lane, const MxEnc& enc) {
  constexpr int PITCH = 128 * 4 + 16;  // FP32 rows, as the FP32 epilogue
  constexpr bool kO8 = MxFmt<OFMT>::bits == 8;  // E4M3 or E5M2 codes (else E2M1)
  uint8_t* W = smem + wid * (64 * PITCH);
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  const uint32_t ch = lane & 15u;  // 8-column chunk of the wave tile's row
  const int64_t row_bytes = kO8 ? N : N >> 1;
  const int64_t spr = N >> 5;  // scale bytes per row
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const int i = 2 * h + i2;
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const uint32_t row = i2 * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
          *reinterpret_cast<float*>(W + row * PITCH + (j * 32 + lr) * 4) = acc[i][j][v];
        }
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // own LDS writes done
    asm volatile("" ::: "memory");
#pragma unroll 4
    for (int k = 0; k < 16; ++k) {
      const uint32_t row = 4 * k + (lane >> 4);
      const u4 lo = *reinterpret_cast<const u4*>(W + row * PITCH + ch * 32);
      const u4 hi = *reinterpret_cast<const u4*>(W + row * PITCH + ch * 32 + 16);
      float v[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[e] = u2f(lo[e]);
        v[4 + e] = u2f(hi[e]);
      }
      const int64_t grow = r0 + h * 64 + row;
      const int64_t gcol = c0 + 8 * ch;
      Enc<OFMT> e;
      encode_mx<OFMT, SR>(enc, (grow * N + gcol) >> 3, v, e);
      // the scale bytes of the row's 4 blocks, gathered in its first lane
      const uint32_t s1 = lane_read(e.sc, lane + 4u), s2 = lane_read(e.sc, lane + 8u),
                     s3 = lane_read(e.sc, lane + 12u);
      if (grow < M && gcol < N) {  // N % 32 == 0: a block is all in or all out
        if constexpr (!OTILED) {
          if constexpr (kO8)
            *reinterpret_cast<uint2*>(codes + grow * row_bytes + gcol) = make_uint2(e.w[0], e.w[1]);
          else
            *reinterpret_cast<uint32_t*>(codes + grow * row_bytes + (gcol >> 1)) = e.w[0];
          // one 32-bit store of the row's 4 blocks when they are all in range
          // and 4-byte aligned, else one byte per block
          const bool wide = (spr & 3) == 0 && c0 + 128 <= N;
          if (wide ? ch == 0 : (ch & 3u) == 0) {
            uint8_t* sp = scales + grow * spr + (gcol >> 5);
            if (wide) *reinterpret_cast<uint32_t*>(sp) = e.sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
            else *sp = (uint8_t)e.sc;
          }
        } else {
          // tile layout (M % 32 == 0, N % 1024 == 0): code byte b of the row
          // is byte b % 16 of chunk (b % 128) / 16 of code tile b / 128
          const int64_t T = grow >> 5;
          const uint32_t r = (uint32_t)grow & 31u;
          const int64_t b = kO8 ? gcol : gcol >> 1;
          const uint32_t c = (uint32_t)(b & 127) >> 4;
          uint8_t* cp = codes + (T * (row_bytes >> 7) + (b >> 7)) * 4096 + (c >> 1) * 1024u +
                        ((c & 1u) * 32u + r) * 16u + (uint32_t)(b & 15);
          if constexpr (kO8)
            *reinterpret_cast<uint2*>(cp) = make_uint2(e.w[0], e.w[1]);
          else
            *reinterpret_cast<uint32_t*>(cp) = e.w[0];
          // block bi of the row: byte bi / 2 % 16 of the word ((bi % 2) * 32 + r)
          // in scale tile bi / 32
          if ((ch & 3u) == 0) {
            const int64_t bi = gcol >> 5;
            const uint32_t bb = (uint32_t)(bi & 31);
            scales[(T * (N >> 10) + (bi >> 5)) * 1024 + ((bb & 1u) * 32u + r) * 16u + (bb >> 1)] =
                (uint8_t)e.sc;
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (0 << 8));  // reads done before reuse
    asm volatile("" ::: "memory");
  }
}

template <int FMT, int OFMT, bool SR, bool OTILED>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx_tiled_q(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, MxEnc enc, uint32_t tiles_m, uint32_t tiles_n) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * 256, n0 = (int64_t)tni * 256;
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  tiled_wave<FMT, kDefaultType<FMT>, kDefaultType<FMT>>(
      A, SA, B, SB, M, N, K, m0, n0, wm, wn, lane, [=](const v16f(&acc)[4][4]) {
        store_tile_quant<OFMT, SR, OTILED>(smem, acc, codes, scales, M, N, m0 + wm * 128, n0 + wn * 128, wid,
                                           lane, enc);
      });
}

// Raise a kernel's dynamic LDS limit once per device, so later launches (also
// inside HIP graphs) make no call beyond the launch itself.
inline hipError_t ensure_smem(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    done.fetch_or(bit, std::memory_order_acq_rel);
  }
  return hipSuccess;
}

template <int FMT, int OFMT, bool SR, bool OTILED>
hipError_t launch_q(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
                    int64_t N, int64_t K, uint8_t* codes, uint8_t* scales, const MxEnc& enc,
                    hipStream_t s) {
  const uint32_t tm = (uint32_t)((M + 255) / 256), tn = (uint32_t)((N + 255) / 256);
  constexpr int kEpiBytes = 4 * 64 * (128 * 4 + 16);
  auto kern = k_gemm_mx_tiled_q<FMT, OFMT, SR, OTILED>;
  static std::atomic<uint64_t> attr_done{0};
  const hipError_t e = ensure_smem((const void*)kern, kEpiBytes, attr_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(256), kEpiBytes, s, a, sa, b, sb, M, N, K, codes, scales, enc,
                     tm, tn);
  return hipGetLastError();
}

template <int FMT, int OFMT>
hipError_t launch_q_d(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
                      int64_t N, int64_t K, uint8_t* codes, uint8_t* scales, const MxEnc& enc, bool sr,
                      bool otiled, hipStream_t s) {
  if (sr)
    return otiled ? launch_q<FMT, OFMT, true, true>(a, sa, b, sb, M, N, K, codes, scales, enc, s)
                  : launch_q<FMT, OFMT, true, false>(a, sa, b, sb, M, N, K, codes, scales, enc, s);
  return otiled ? launch_q<FMT, OFMT, false, true>(a, sa, b, sb, M, N, K, codes, scales, enc, s)
                : launch_q<FMT, OFMT, false, false>(a, sa, b, sb, M, N, K, codes, scales, enc, s);
}

template <int FMT, int CDT, int TA = kDefaultType<FMT>, int TB = kDefaultType<FMT>>
hipError_t launch_t(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                    int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const uint32_t tm = (uint32_t)((M + 255) / 256), tn = (uint32_t)((N + 255) / 256);
  constexpr int kEpiBytes = 4 * 64 * (128 * (CDT == DT_F32 ? 4 : 2) + 16);  // store_tile staging
  auto kern = k_gemm_mx_tiled<FMT, CDT, TA, TB>;
  // raised once per device, so later launches (also inside HIP graphs) make
  // no call beyond the launch itself
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kEpiBytes);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int64_t eb = CDT == DT_F32 ? 4 : 2;
  const uint32_t vec = ((reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * eb) % 16 == 0) ? 1u : 0u;
  hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(256), kEpiBytes, s, a, sa, b, sb, M, N, K, C, ldc, tm, tn, vec);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mx_tiled_quant(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                      const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                      int64_t N, int64_t K, int ofmt, bool otiled, uint8_t* codes,
                                      uint8_t* scales, bool sr, uint64_t seed, uint64_t counter,
                                      bool ceil, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  const MxEnc enc{ceil, seed, counter};
#define MXK_Q(F, O) \
  launch_q_d<F, O>(a_codes, a_scales, b_codes, b_scales, M, N, K, codes, scales, enc, sr, otiled, s)
  if (fmt == FMT_MXFP8)
    return ofmt == FMT_MXFP8 ? MXK_Q(FMT_MXFP8, FMT_MXFP8)
           : ofmt == FMT_MXFP8_E5M2 ? MXK_Q(FMT_MXFP8, FMT_MXFP8_E5M2) : MXK_Q(FMT_MXFP8, FMT_MXFP4);
  return ofmt == FMT_MXFP8 ? MXK_Q(FMT_MXFP4, FMT_MXFP8)
         : ofmt == FMT_MXFP8_E5M2 ? MXK_Q(FMT_MXFP4, FMT_MXFP8_E5M2) : MXK_Q(FMT_MXFP4, FMT_MXFP4);
#undef MXK_Q
}

hipError_t launch_gemm_mx_tiled(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                int64_t N, int64_t K, void* C, int cdt, int64_t ldc,
                                hipStream_t s, int fmt_b) {
  if (M == 0 || N == 0) return hipSuccess;
  // FP8 pairs with E5M2 on either side
  if (fmt == FMT_MXFP8_E5M2 || fmt_b == FMT_MXFP8_E5M2) {
#define MXK_T8(TA, TB) \
  (cdt == DT_F32 ? launch_t<FMT_MXFP8, DT_F32, TA, TB>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s) \
                 : launch_t<FMT_MXFP8, DT_BF16, TA, TB>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s))
    if (fmt == FMT_MXFP8_E5M2 && fmt_b == FMT_MXFP8_E5M2) return MXK_T8(1, 1);
    if (fmt == FMT_MXFP8_E5M2) return MXK_T8(1, 0);
    return MXK_T8(0, 1);
#undef MXK_T8
  }
  if (fmt == FMT_MXFP8)
    return cdt == DT_F32 ? launch_t<FMT_MXFP8, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                         : launch_t<FMT_MXFP8, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
  return cdt == DT_F32 ? launch_t<FMT_MXFP4, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                       : launch_t<FMT_MXFP4, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
}

}  // namespace mxk
