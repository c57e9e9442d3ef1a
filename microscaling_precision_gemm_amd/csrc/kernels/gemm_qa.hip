// gemm_qa.hip -- block-scaled GEMM C = Q(A) * B^T whose A operand arrives
// unquantized (BF16) and is quantized to an MX format inside the GEMM's
// prologue ("Microscaling (MX) and block-scaled 4-bit formats", section
// "Open points": efficient fused quantize-and-GEMM kernels, since computing
// block scales is memory traffic of its own).  The epilogue half of that
// point (the product written quantized) lives in gemm_tiled.hip.
//
// Each 32-element block of an A row is encoded exactly as the quantizer
// encodes it (E8M0 floor rule, RNE or SR with the quantizer's random stream
// indexed by the element's row-major position in A), optionally written out
// (by the workgroups of the first column tile only, so every block once) for
// later use, and decoded to exact BF16 in LDS.  B (MXFP8 E4M3 or MXFP4, row
// layout) is decoded the same way, and the staged BF16 contraction of
// gemm_staged.hip follows: v_mfma_f32_32x32x16_bf16 on exact products, FP32
// accumulation.
//
// Workgroup: 256 threads (2x2 waves), BM x BN tile, K step 64 elements,
// double-buffered BF16 tiles in LDS (144-byte row pitch).  Thread unit
// u = t + 256 j covers row u / 2 (A rows first, then B rows) and the K half
// u % 2 of each step: 32 elements, one MX block.
//
// Exactness: MXFP4 values times 2^(c-127) are BF16 values for every code;
// E4M3 values for codes 3 .. 246 (a block maximum at least 2^-116 in
// magnitude).  Codes 0 and 255 are decoded through FP32.
#include "../device/codec.h"
#include "../device/cvt.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef float v16f_q __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf_q __attribute__((ext_vector_type(8)));
typedef float v2f_q __attribute__((ext_vector_type(2)));

constexpr int kQBK = 64;                // K elements per step
constexpr int kQPitch = kQBK * 2 + 16;  // LDS bytes per row

template <int F>
struct QCodes {
  static constexpr int kWords = F == FMT_MXFP8 ? 8 : 4;  // code dwords of a 32-element block
  static constexpr uint32_t kEmax = F == FMT_MXFP8 ? 8u : 2u;
};

// 32 codes of format F (element 2d of an FP4 word in the low nibble of byte d)
// scaled by 2^(sc-127), as 16 exact BF16 pairs stored at dst.
template <int F>
__device__ inline void decode_store(const uint32_t (&w)[QCodes<F>::kWords], uint32_t sc, uint8_t* dst) {
  uint32_t out[16];
  if constexpr (F == FMT_MXFP8) {
    if (sc >= 1u && sc != 0xFFu) {
      const float X = u2f(sc << 23);
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        out[2 * wd] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[wd], X, false));
        out[2 * wd + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[wd], X, true));
      }
    } else {  // 2^-127 is an FP32 subnormal the converter does not take; 0xFF is NaN
      const float X = sc == 0u ? u2f(0x00400000u) : __builtin_nanf("");
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const v2f_q lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[wd], 1.0f, false);
        const v2f_q hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w[wd], 1.0f, true);
        out[2 * wd] = (f2u(lo[0] * X) >> 16) | (f2u(lo[1] * X) & 0xFFFF0000u);
        out[2 * wd + 1] = (f2u(hi[0] * X) >> 16) | (f2u(hi[1] * X) & 0xFFFF0000u);
      }
    }
  } else {
    // e2m1 * 2^(c-127): at most 2 significant bits and at least 2^-128, so
    // the FP32 product is a BF16 value for every code (NaN for 0xFF)
    const float X = sc == 0xFFu ? __builtin_nanf("") : (sc == 0u ? u2f(0x00400000u) : u2f(sc << 23));
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      const v2f_q f[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[wd], 1.0f, 0),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[wd], 1.0f, 1),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[wd], 1.0f, 2),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[wd], 1.0f, 3)};
#pragma unroll
      for (int b = 0; b < 4; ++b) out[4 * wd + b] = (f2u(f[b][0] * X) >> 16) | (f2u(f[b][1] * X) & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
}

// One 32-element block of BF16 values (16 words, element 2i low) encoded in
// format F as the quantizer encodes it: E8M0 floor rule, RNE or SR (chunk q0
// of the random stream for the first 8 elements).
template <int F, bool SR>
__device__ inline void encode_block(const uint32_t (&x)[16], uint64_t seed, uint64_t counter, uint64_t q0,
                                    uint32_t (&w)[QCodes<F>::kWords], uint32_t& sc) {
  float v[32];
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    v[2 * i] = u2f(x[i] << 16);
    v[2 * i + 1] = u2f(x[i] & 0xFFFF0000u);
    const uint32_t a = (x[i] << 16) & 0x7FFFFFFFu, b = x[i] & 0x7FFF0000u;
    m = a > m ? a : m;
    m = b > m ? b : m;
  }
  sc = e8m0_from_amax_bits(m, QCodes<F>::kEmax);
  const float inv = e8m0_inverse(sc);
  float y[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) y[i] = v[i] * inv;  // exact scaling by a power of two
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    if constexpr (SR && F == FMT_MXFP8) {
      uint32_t r[8];
      rand16x8(seed, counter, q0 + (uint64_t)c, r);
      pack_e4m3_sr(y + 8 * c, r, w + 2 * c);
    } else if constexpr (SR) {
      const u32x4 rw = rand_words(seed, counter, q0 + (uint64_t)c);
      w[c] = pack_e2m1_sr_words(y + 8 * c, rw.x, rw.y, rw.z, rw.w);
    } else {
      if constexpr (F == FMT_MXFP8) pack_e4m3_rne(y + 8 * c, w + 2 * c);
      else w[c] = pack_e2m1_rne(y + 8 * c);
    }
  }
  if (sc == 0xFFu) {  // NaN / Inf in the block
#pragma unroll
    for (int i = 0; i < QCodes<F>::kWords; ++i) w[i] = 0u;
  }
}

template <int AF, int BF, int CDT, bool SR, int BM, int BN>
__global__ __launch_bounds__(256) void k_gemm_qa(const uint16_t* __restrict__ A, int64_t lda,
                                                 const uint8_t* __restrict__ B, const uint8_t* __restrict__ SB,
                                                 int64_t M, int64_t N, int64_t K, void* __restrict__ C,
                                                 int64_t ldc, uint8_t* __restrict__ a_codes,
                                                 uint8_t* __restrict__ a_scales, uint64_t seed, uint64_t counter,
                                                 uint32_t tiles_m, uint32_t tiles_n) {
  constexpr int kAU = BM / 128, kBU = BN / 128;  // A / B units per thread
  constexpr int FM = BM / 2 / 32, FN = BN / 2 / 32;
  constexpr int kRows = BM + BN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kRows * kQPitch];

  // workgroup -> (m tile, n tile): consecutive ids share the m tile, and ids
  // on one XCD (id mod 8) are adjacent
  uint32_t id = blockIdx.x;
  const uint32_t total = tiles_m * tiles_n;
  if ((total & 7u) == 0) id = (id & 7u) * (total >> 3) + (id >> 3);
  const int64_t m0 = (int64_t)(id / tiles_n) * BM, n0 = (int64_t)(id % tiles_n) * BN;
  const bool emit = a_codes != nullptr && n0 == 0;

  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t a_rowbytes = AF == FMT_MXFP8 ? K : K / 2, b_rowbytes = BF == FMT_MXFP8 ? K : K / 2;
  const int64_t kb = K / 32;
  const int64_t steps = (K + kQBK - 1) / kQBK;
  const uint32_t h = t & 1u;  // K half of every unit of this thread

  int64_t arow[kAU];
  const uint8_t* bsrc[kBU];
  const uint8_t* bssrc[kBU];
#pragma unroll
  for (int j = 0; j < kAU; ++j) {
    const int64_t r = m0 + (int64_t)((t + 256u * j) >> 1);
    arow[j] = r < M ? r : -1;
  }
#pragma unroll
  for (int j = 0; j < kBU; ++j) {
    const int64_t r = n0 + (int64_t)((t + 256u * (kAU + j)) >> 1) - BM;
    bsrc[j] = r < N ? B + r * b_rowbytes + h * (BF == FMT_MXFP8 ? 32 : 16) : nullptr;
    bssrc[j] = r < N ? SB + r * kb + h : nullptr;
  }

  uint32_t xa[kAU][16];
  uint32_t wb[kBU][QCodes<BF>::kWords];
  uint32_t sb[kBU];
  auto load_step = [&](int64_t step) {
    const int64_t k0 = step * kQBK + 32 * h;  // first K element of this thread's units
    const bool kin = k0 < K;                  // K % 32 == 0: a unit is all in or out
#pragma unroll
    for (int j = 0; j < kAU; ++j) {
      uint4 v[4] = {};
      if (arow[j] >= 0 && kin) {
        const uint4* p = reinterpret_cast<const uint4*>(A + arow[j] * lda + k0);
        v[0] = p[0]; v[1] = p[1]; v[2] = p[2]; v[3] = p[3];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        xa[j][4 * q] = v[q].x; xa[j][4 * q + 1] = v[q].y; xa[j][4 * q + 2] = v[q].z; xa[j][4 * q + 3] = v[q].w;
      }
    }
#pragma unroll
    for (int j = 0; j < kBU; ++j) {
      uint4 v0 = {}, v1 = {};
      uint32_t s = 127u;
      if (bsrc[j] && kin) {
        const uint4* p = reinterpret_cast<const uint4*>(bsrc[j] + step * (BF == FMT_MXFP8 ? kQBK : kQBK / 2));
        v0 = p[0];
        if constexpr (BF == FMT_MXFP8) v1 = p[1];
        s = bssrc[j][step * 2];
      }
      wb[j][0] = v0.x; wb[j][1] = v0.y; wb[j][2] = v0.z; wb[j][3] = v0.w;
      if constexpr (BF == FMT_MXFP8) {
        wb[j][4] = v1.x; wb[j][5] = v1.y; wb[j][6] = v1.z; wb[j][7] = v1.w;
      }
      sb[j] = s;
    }
  };
  auto store_step = [&](int64_t step, int buf) {
    const int64_t k0 = step * kQBK + 32 * h;
#pragma unroll
    for (int j = 0; j < kAU; ++j) {
      uint32_t w[QCodes<AF>::kWords], sc;
      const int64_t row = arow[j] >= 0 ? arow[j] : 0;
      encode_block<AF, SR>(xa[j], seed, counter, (uint64_t)((row * K + k0) >> 3), w, sc);
      if (emit && arow[j] >= 0 && k0 < K) {
        uint4* dst = reinterpret_cast<uint4*>(a_codes + row * a_rowbytes + (AF == FMT_MXFP8 ? k0 : k0 / 2));
        dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
        if constexpr (AF == FMT_MXFP8) dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
        a_scales[row * kb + k0 / 32] = (uint8_t)sc;
      }
      decode_store<AF>(w, sc, &lds[buf][((t + 256u * j) >> 1) * kQPitch + h * 64]);
    }
#pragma unroll
    for (int j = 0; j < kBU; ++j)
      decode_store<BF>(wb[j], sb[j], &lds[buf][((t + 256u * (kAU + j)) >> 1) * kQPitch + h * 64]);
  };

  v16f_q acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_step(0);
  store_step(0, 0);
  __syncthreads();
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < steps) load_step(st + 1);
    const uint8_t* L = lds[buf];
#pragma unroll
    for (int kk = 0; kk < kQBK / 16; ++kk) {
      const uint32_t off = (kk * 16 + lg * 8) * 2;
      v8bf_q af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(v8bf_q, *reinterpret_cast<const uint4*>(L + (wm * (BM / 2) + i * 32 + lr) * kQPitch + off));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(v8bf_q, *reinterpret_cast<const uint4*>(L + (BM + wn * (BN / 2) + j * 32 + lr) * kQPitch + off));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < steps) store_step(st + 1, buf ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * (BN / 2) + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
        if (row < M && col < N) {
          if constexpr (CDT == DT_F32) static_cast<float*>(C)[row * ldc + col] = acc[i][j][v];
          else static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(acc[i][j][v]);
        }
      }
    }
}

template <int AF, int BF, int CDT, bool SR>
hipError_t launch_qa_t(const uint16_t* a, int64_t lda, const uint8_t* b, const uint8_t* sb, int64_t M, int64_t N,
                       int64_t K, void* C, int64_t ldc, uint8_t* a_codes, uint8_t* a_scales, uint64_t seed,
                       uint64_t counter, hipStream_t s) {
  if (M * N >= (int64_t)256 * 256 * 128) {
    constexpr int BM = 256, BN = 256;
    const uint32_t tm = (uint32_t)((M + BM - 1) / BM), tn = (uint32_t)((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_qa<AF, BF, CDT, SR, BM, BN>), dim3(tm * tn), dim3(256), 0, s, a, lda, b, sb, M, N,
                       K, C, ldc, a_codes, a_scales, seed, counter, tm, tn);
  } else {
    constexpr int BM = 128, BN = 128;
    const uint32_t tm = (uint32_t)((M + BM - 1) / BM), tn = (uint32_t)((N + BN - 1) / BN);
    hipLaunchKernelGGL((k_gemm_qa<AF, BF, CDT, SR, BM, BN>), dim3(tm * tn), dim3(256), 0, s, a, lda, b, sb, M, N,
                       K, C, ldc, a_codes, a_scales, seed, counter, tm, tn);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_quantize_a(int afmt, const uint16_t* a, int64_t lda, const uint8_t* b_codes,
                                  const uint8_t* b_scales, int bfmt, int64_t M, int64_t N, int64_t K, void* C,
                                  int cdt, int64_t ldc, uint8_t* a_codes, uint8_t* a_scales, bool sr,
                                  uint64_t seed, uint64_t counter, hipStream_t s) {
  if (M == 0 || N == 0) return hipSuccess;
  if ((uint64_t)((M + 127) / 128) * (uint64_t)((N + 127) / 128) > 0x7FFFFFFFull) return hipErrorInvalidValue;
#define MXK_QA(AF, BF, D, SR) \
  return launch_qa_t<AF, BF, D, SR>(a, lda, b_codes, b_scales, M, N, K, C, ldc, a_codes, a_scales, seed, counter, s)
#define MXK_QA_SR(AF, BF, D) \
  do {                       \
    if (sr) MXK_QA(AF, BF, D, true); \
    MXK_QA(AF, BF, D, false);        \
  } while (0)
#define MXK_QA_D(AF, BF)                                   \
  do {                                                     \
    if (cdt == DT_F32) MXK_QA_SR(AF, BF, DT_F32);          \
    MXK_QA_SR(AF, BF, DT_BF16);                            \
  } while (0)
  if (afmt == FMT_MXFP8) {
    if (bfmt == FMT_MXFP8) MXK_QA_D(FMT_MXFP8, FMT_MXFP8);
    MXK_QA_D(FMT_MXFP8, FMT_MXFP4);
  }
  if (bfmt == FMT_MXFP8) MXK_QA_D(FMT_MXFP4, FMT_MXFP8);
  MXK_QA_D(FMT_MXFP4, FMT_MXFP4);
#undef MXK_QA_D
#undef MXK_QA_SR
#undef MXK_QA
}

}  // namespace mxk
