// gemm_mx.hip -- block-scaled GEMM C = A * B^T for MX operands (E8M0 scale
// per 32 elements of K) on gfx950's scaled matrix instructions
// v_mfma_scale_f32_32x32x64_f8f6f4, which apply one E8M0 scale per lane and
// K-block inside the instruction ("Microscaling (MX) and block-scaled 4-bit
// formats", section "Hardware and kernels": scales applied inside the matrix
// instruction).
//
// Operand register layout of the 32x32x64 instruction (measured on gfx950):
//   lane l holds row (l mod 32) of the 32-row operand; the E8M0 scale passed by
//   lane l covers K-block (l / 32) of that row (K = 64 = two blocks of 32).
//   FP4: lane l holds the 32 elements of its block in 16 bytes, element k in
//        nibble k (low nibble first), i.e. the block's packed bytes verbatim.
//   FP8: lane l holds 32 bytes: bytes 0..15 are elements 16*(l/32) .. +15 of
//        block 0 and bytes 16..31 the same positions of block 1; the two
//        lanes l and l+32 together hold both blocks.
//
// Kernel structure: a 256-thread workgroup computes a 128x128 C tile, each
// wave a 64x64 sub-tile (2x2 instructions).  A and B tiles for one K step of
// 128 (FP4) / 64 (FP8) are staged through LDS (double-buffered), scales are
// read per lane from global memory (L2-resident, 1 byte per lane per step).
#include "../device/codec.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kBM = 128, kBN = 128;

// bytes of K per step held in LDS per row: FP8 64 (one 32x32x64 instruction),
// FP4 64 (two instructions of K = 64, 128 elements)
template <int FMT>
struct Cfg {
  static constexpr int kKElems = FMT == FMT_MXFP8 ? 64 : 128;  // K elements per step
  static constexpr int kRowBytes = 64;                         // code bytes per row per step
  static constexpr int kInstr = FMT == FMT_MXFP8 ? 1 : 2;      // MFMAs (K=64) per step
  static constexpr int kPitch = kRowBytes + 16;                // LDS row pitch (bank spread)
};

template <int FMT, int CDT>
__global__ __launch_bounds__(256) void k_gemm_mx(const uint8_t* __restrict__ A,
                                                 const uint8_t* __restrict__ SA,
                                                 const uint8_t* __restrict__ B,
                                                 const uint8_t* __restrict__ SB, int64_t M,
                                                 int64_t N, int64_t K, void* __restrict__ C,
                                                 int64_t ldc) {
  using CF = Cfg<FMT>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(kBM + kBN) * CF::kPitch];
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;  // wave position in the 2x2 wave grid
  const int64_t m0 = (int64_t)blockIdx.y * kBM, n0 = (int64_t)blockIdx.x * kBN;
  const int64_t rowbytes = FMT == FMT_MXFP8 ? K : K / 2;  // code bytes per operand row
  const int64_t kblocks = K / 32;
  const int64_t steps = (K + CF::kKElems - 1) / CF::kKElems;

  // global -> LDS copy assignment: 256 rows (128 A + 128 B) x 64 bytes = 4 x 16 B per row;
  // thread t copies 16-byte pieces p = t + 256*j, j = 0..3: row p / 4, piece p % 4
  auto load_tile = [&](int64_t step, uint4 (&reg)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p = t + 256u * j;
      const uint32_t r = p >> 2, piece = p & 3u;
      const bool isA = r < kBM;
      const int64_t grow = isA ? m0 + r : n0 + (r - kBM);
      const int64_t lim = isA ? M : N;
      const int64_t kb = step * CF::kRowBytes + piece * 16;  // byte offset in the row
      uint4 v = make_uint4(0, 0, 0, 0);
      if (grow < lim && kb < rowbytes) {
        const uint8_t* base = isA ? A : B;
        v = *reinterpret_cast<const uint4*>(base + grow * rowbytes + kb);
      }
      reg[j] = v;
    }
  };
  auto store_tile = [&](int buf, const uint4 (&reg)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p = t + 256u * j;
      const uint32_t r = p >> 2, piece = p & 3u;
      *reinterpret_cast<uint4*>(&lds[buf][r * CF::kPitch + piece * 16]) = reg[j];
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 reg[4];
  load_tile(0, reg);
  store_tile(0, reg);
  __syncthreads();

  const uint32_t lr = lane & 31u, lg = lane >> 5;
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < steps) load_tile(st + 1, reg);
#pragma unroll
    for (int ins = 0; ins < CF::kInstr; ++ins) {
      // K-block of this lane for this instruction
      const int64_t kblk = (st * CF::kKElems + ins * 64) / 32 + lg;
      v8i af[2], bf[2];
      int sa[2], sb[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t ra = wm * 64 + i * 32 + lr;           // A row in tile
        const uint32_t rb = kBM + wn * 64 + i * 32 + lr;      // B row in tile (LDS)
        if constexpr (FMT == FMT_MXFP8) {
          const uint4 a0 = *reinterpret_cast<const uint4*>(&lds[buf][ra * CF::kPitch + 16 * lg]);
          const uint4 a1 = *reinterpret_cast<const uint4*>(&lds[buf][ra * CF::kPitch + 32 + 16 * lg]);
          const uint4 b0 = *reinterpret_cast<const uint4*>(&lds[buf][rb * CF::kPitch + 16 * lg]);
          const uint4 b1 = *reinterpret_cast<const uint4*>(&lds[buf][rb * CF::kPitch + 32 + 16 * lg]);
          af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          bf[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        } else {
          const uint32_t off = ins * 32 + 16 * lg;
          const uint4 a0 = *reinterpret_cast<const uint4*>(&lds[buf][ra * CF::kPitch + off]);
          const uint4 b0 = *reinterpret_cast<const uint4*>(&lds[buf][rb * CF::kPitch + off]);
          af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
          bf[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
        }
        int64_t gra = m0 + wm * 64 + i * 32 + lr;
        int64_t grb = n0 + wn * 64 + i * 32 + lr;
        gra = gra < M ? gra : M - 1;
        grb = grb < N ? grb : N - 1;
        sa[i] = kblk < kblocks ? (int)SA[gra * kblocks + kblk] : 127;
        sb[i] = kblk < kblocks ? (int)SB[grb * kblocks + kblk] : 127;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (FMT == FMT_MXFP8)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 0, 0, 0, sa[i], 0, sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
        }
    }
    if (st + 1 < steps) {
      store_tile(buf ^ 1, reg);
    }
    __syncthreads();
  }

  // epilogue: lane holds C[row][col] with col = lane % 32 and
  // row = 8*(v/4) + 4*(lane/32) + v%4 inside each 32x32 instruction tile
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
        if (row < M && col < N) {
          if constexpr (CDT == DT_F32)
            static_cast<float*>(C)[row * ldc + col] = acc[i][j][v];
          else
            static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm_mx(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                          int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
#define MXK_G(F, D) \
  hipLaunchKernelGGL((k_gemm_mx<F, D>), grid, dim3(256), 0, s, a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc)
  if (fmt == FMT_MXFP8) {
    if (cdt == DT_F32) MXK_G(FMT_MXFP8, DT_F32);
    else MXK_G(FMT_MXFP8, DT_BF16);
  } else {
    if (cdt == DT_F32) MXK_G(FMT_MXFP4, DT_F32);
    else MXK_G(FMT_MXFP4, DT_BF16);
  }
#undef MXK_G
  return hipGetLastError();
}

}  // namespace mxk
