// gemm_mx.hip -- block-scaled GEMM C = A * B^T for MX operands (E8M0 scale
// per 32 elements of K) on gfx950's scaled matrix instruction
// v_mfma_scale_f32_32x32x64_f8f6f4, which applies one E8M0 scale per lane and
// K-block inside the instruction ("Microscaling (MX) and block-scaled 4-bit
// formats", section "Hardware and kernels": the scale factors are applied
// inside the matrix instruction).
//
// Operand register layout of the 32x32x64 instruction (measured on gfx950):
//   lane l holds row (l mod 32) of its operand; the E8M0 scale passed by lane
//   l (byte selected by opsel) covers K-block (l / 32) of that row.
//   FP4: lane l holds the 32 elements of its K-block in 16 bytes, element k
//        in nibble k (low nibble first) -- the packed bytes verbatim.
//   FP8: lane l holds 32 bytes: bytes 0..15 are elements 16*(l/32) .. +15 of
//        K-block 0 and bytes 16..31 the same positions of K-block 1.
//
// MXFP4 is exact on this instruction (FP32 accumulation of exact products).
// The FP8 variant is offered as the hardware-native MXFP8 path: gfx950 sums
// the FP8 products of each 8-element group in a narrow aligned window (about
// 14 bits below the group's largest product) before FP32 accumulation, so it
// does not meet a 1e-5 relative bound in general.  The exact MXFP8 GEMM is the
// BF16-staged kernel in gemm_staged.hip.
//
// Kernel structure: 256 threads (4 waves in 2x2), a BM x BN C tile per
// workgroup, (BM/2) x (BN/2) per wave as 32x32 instruction tiles.  Each K
// step moves 64 code bytes per row (FP4: 128 elements, two instructions;
// FP8: 64 elements, one instruction) plus the row's scale bytes for that step
// into a double-buffered LDS tile whose row pitch (80 bytes) keeps the
// 16-byte fragment reads of 8 consecutive rows on distinct banks.  The scale
// dword sits in the row's padding.  Workgroup -> tile mapping keeps the
// tiles of one XCD (workgroups are dealt round-robin over the 8 XCDs)
// adjacent in M and N for L2 reuse.
#include "../device/codec.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kPitch = 80;     // LDS bytes per row: 64 code bytes, 4 scale bytes, pad
constexpr int kRowBytes = 64;  // code bytes per row per K step

template <int FMT>
struct StepCfg {
  static constexpr int kKElems = FMT == FMT_MXFP8 ? 64 : 128;  // K elements per step
  static constexpr int kInstr = FMT == FMT_MXFP8 ? 1 : 2;      // instructions per step
  static constexpr int kBlocks = kKElems / 32;                 // scale bytes per row per step
};

// Map a linear workgroup id to a (tile_m, tile_n) so that the ids that land
// on one XCD (id mod 8) form compact groups of tiles.
__device__ inline void tile_of(uint32_t id, uint32_t tm, uint32_t tn, uint32_t* m, uint32_t* n) {
  const uint32_t total = tm * tn;
  uint32_t lin = id;
  if ((total & 7u) == 0) {
    const uint32_t per = total >> 3;
    lin = (id & 7u) * per + (id >> 3);
  }
  // grouped order: groups of G tile-rows, column-major inside a group
  const uint32_t G = 4;
  const uint32_t group = lin / (G * tn);
  const uint32_t first_m = group * G;
  const uint32_t gsize = (tm - first_m) < G ? (tm - first_m) : G;
  const uint32_t in = lin - group * G * tn;
  *m = first_m + in % gsize;
  *n = in / gsize;
}

template <int FMT, int CDT, int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_mx(const uint8_t* __restrict__ A,
                                                 const uint8_t* __restrict__ SA,
                                                 const uint8_t* __restrict__ B,
                                                 const uint8_t* __restrict__ SB, int64_t M,
                                                 int64_t N, int64_t K, void* __restrict__ C,
                                                 int64_t ldc, uint32_t tiles_m, uint32_t tiles_n) {
  using SC = StepCfg<FMT>;
  constexpr int kRows = BM + BN;
  constexpr int kPieces = kRows * (kRowBytes / 16) / 256;  // 16-byte code pieces per thread
  constexpr int kScaleLoads = (kRows + 255) / 256;         // scale dwords per thread
  constexpr int FM = BM / 2 / 32, FN = BN / 2 / 32;        // instruction tiles per wave
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kRows * kPitch];

  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t rowbytes = FMT == FMT_MXFP8 ? K : K / 2;
  const int64_t kblocks = K / 32;
  const int64_t steps = (K + SC::kKElems - 1) / SC::kKElems;

  // global source rows of this thread's pieces (fixed over the K loop)
  const uint8_t* src[kPieces];
  uint32_t piece_off[kPieces];
#pragma unroll
  for (int j = 0; j < kPieces; ++j) {
    const uint32_t p = t + 256u * j;
    const uint32_t r = p >> 2;
    piece_off[j] = r * kPitch + (p & 3u) * 16;
    const bool isA = r < (uint32_t)BM;
    const int64_t grow = isA ? m0 + r : n0 + (r - BM);
    const int64_t lim = isA ? M : N;
    src[j] = (grow < lim) ? (isA ? A : B) + grow * rowbytes + (p & 3u) * 16 : nullptr;
  }
  const uint8_t* ssrc[kScaleLoads];
#pragma unroll
  for (int j = 0; j < kScaleLoads; ++j) {
    const uint32_t r = t + 256u * j;
    ssrc[j] = nullptr;
    if (r < (uint32_t)kRows) {
      const bool isA = r < (uint32_t)BM;
      const int64_t grow = isA ? m0 + r : n0 + (r - BM);
      const int64_t lim = isA ? M : N;
      if (grow < lim) ssrc[j] = (isA ? SA : SB) + grow * kblocks;
    }
  }

  uint4 reg[kPieces];
  uint32_t sreg[kScaleLoads];
  auto load_step = [&](int64_t step) {
    const int64_t kb = step * kRowBytes;
#pragma unroll
    for (int j = 0; j < kPieces; ++j) {
      const int64_t off = kb + (int64_t)((t + 256u * j) & 3u) * 16;
      reg[j] = (src[j] != nullptr && off < rowbytes)
                   ? *reinterpret_cast<const uint4*>(src[j] + kb)
                   : make_uint4(0, 0, 0, 0);
    }
    const int64_t b0 = step * SC::kBlocks;
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j) {
      uint32_t w = 0;
      if (ssrc[j] != nullptr) {
        if (b0 + SC::kBlocks <= kblocks) {
          if constexpr (SC::kBlocks == 4) w = *reinterpret_cast<const uint32_t*>(ssrc[j] + b0);
          else w = *reinterpret_cast<const uint16_t*>(ssrc[j] + b0);
        } else {
          for (int i = 0; i < SC::kBlocks; ++i)
            if (b0 + i < kblocks) w |= (uint32_t)ssrc[j][b0 + i] << (8 * i);
        }
      }
      sreg[j] = w;
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kPieces; ++j)
      *reinterpret_cast<uint4*>(&lds[buf][piece_off[j]]) = reg[j];
#pragma unroll
    for (int j = 0; j < kScaleLoads; ++j) {
      const uint32_t r = t + 256u * j;
      if (r < (uint32_t)kRows) *reinterpret_cast<uint32_t*>(&lds[buf][r * kPitch + kRowBytes]) = sreg[j];
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // alignment of the per-row scale words: K % 128 == 0 (FP4) / K % 64 == 0
  // (FP8) keeps every step's scale bytes inside the row; otherwise the byte
  // loop above handles the tail.
  load_step(0);
  store_step(0);
  __syncthreads();

  const uint32_t lr = lane & 31u, lg = lane >> 5;
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < steps) load_step(st + 1);
    const uint8_t* L = lds[buf];
    // scale words of this lane's rows, shifted so byte 0 is this lane's block
    uint32_t sa[FM], sb[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa[i] = *reinterpret_cast<const uint32_t*>(L + (wm * (BM / 2) + i * 32 + lr) * kPitch + kRowBytes) >> (8 * lg);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      sb[j] = *reinterpret_cast<const uint32_t*>(L + (BM + wn * (BN / 2) + j * 32 + lr) * kPitch + kRowBytes) >> (8 * lg);
#pragma unroll
    for (int ins = 0; ins < SC::kInstr; ++ins) {
      v8i af[FM], bf[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint8_t* row = L + (wm * (BM / 2) + i * 32 + lr) * kPitch;
        if constexpr (FMT == FMT_MXFP8) {
          const uint4 a0 = *reinterpret_cast<const uint4*>(row + 16 * lg);
          const uint4 a1 = *reinterpret_cast<const uint4*>(row + 32 + 16 * lg);
          af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        } else {
          const uint4 a0 = *reinterpret_cast<const uint4*>(row + ins * 32 + 16 * lg);
          af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const uint8_t* row = L + (BM + wn * (BN / 2) + j * 32 + lr) * kPitch;
        if constexpr (FMT == FMT_MXFP8) {
          const uint4 b0 = *reinterpret_cast<const uint4*>(row + 16 * lg);
          const uint4 b1 = *reinterpret_cast<const uint4*>(row + 32 + 16 * lg);
          bf[j] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        } else {
          const uint4 b0 = *reinterpret_cast<const uint4*>(row + ins * 32 + 16 * lg);
          bf[j] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          if constexpr (FMT == FMT_MXFP8)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, (int)sa[i], 0, (int)sb[j]);
          else if (ins == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, (int)sa[i], 0, (int)sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 2, (int)sa[i], 2, (int)sb[j]);
        }
    }
    if (st + 1 < steps) store_step(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds C[row][col], col = lane % 32,
  // row = 8*(v/4) + 4*(lane/32) + v%4 inside each 32x32 instruction tile
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * (BN / 2) + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
        if (row < M && col < N) {
          if constexpr (CDT == DT_F32)
            static_cast<float*>(C)[row * ldc + col] = acc[i][j][v];
          else
            static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
}

template <int FMT, int CDT, int BM, int BN>
hipError_t run(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
               int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const uint32_t tm = (uint32_t)((M + BM - 1) / BM), tn = (uint32_t)((N + BN - 1) / BN);
  hipLaunchKernelGGL((k_gemm_mx<FMT, CDT, BM, BN>), dim3(tm * tn), dim3(256), 0, s, a, sa, b, sb,
                     M, N, K, C, ldc, tm, tn);
  return hipGetLastError();
}

template <int FMT, int CDT>
hipError_t run_sized(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                     int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  // large problems: 256x256 tiles (one tile per CU at 4096^2); small ones
  // keep more workgroups in flight with 128x128
  if (M * N >= (int64_t)256 * 256 * 192) return run<FMT, CDT, 256, 256>(a, sa, b, sb, M, N, K, C, ldc, s);
  return run<FMT, CDT, 128, 128>(a, sa, b, sb, M, N, K, C, ldc, s);
}

}  // namespace

hipError_t launch_gemm_mx(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                          int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fmt == FMT_MXFP8) {
    return cdt == DT_F32 ? run_sized<FMT_MXFP8, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                         : run_sized<FMT_MXFP8, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
  }
  return cdt == DT_F32 ? run_sized<FMT_MXFP4, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                       : run_sized<FMT_MXFP4, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
}

}  // namespace mxk
