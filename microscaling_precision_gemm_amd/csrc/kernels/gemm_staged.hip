// gemm_staged.hip -- block-scaled GEMMs whose block scales are applied
// explicitly while the operands are staged into LDS as exact BF16 values, then
// contracted on v_mfma_f32_32x32x16_bf16 (exact products, FP32 accumulation).
//
//  * NVFP4 ("Microscaling (MX) and block-scaled 4-bit formats", section
//    "NVFP4"): E2M1 elements, an E4M3 scale per 16 and an FP32 scale per
//    tensor.  The E4M3 block scale has no counterpart in the matrix
//    instructions (their block scale is an E8M0 power of two per 32), so each
//    element is multiplied by it here; e2m1 * e4m3 has at most 2 + 4
//    significant bits and is exact in BF16.  The per-tensor scales multiply
//    the FP32 accumulator in the epilogue.  Plain and grouped (mixture-of-
//    experts forward: "Thinking Machines ... Inkling 2 Small", section "A
//    precision choice for each stage") variants, with an optional row gather
//    of A.
//  * MXFP8, exact: E4M3 * 2^(c-127) is exact in BF16 for scale codes c in
//    [3, 246].  (gfx950's FP8 matrix instruction truncates products inside
//    8-element groups, see gemm_mx.hip, so the exact MXFP8 product is formed
//    on the BF16 instruction.)
//
// Conversion: gfx950's v_cvt_scalef32_pk_* instructions scale by the
// exponent of their FP32 scale operand only (measured), which is exactly the
// E8M0 scale of MXFP8.  NVFP4 elements are converted with scale 1 and
// multiplied by the E4M3 scale in FP32 (exact), then truncated to BF16
// (exact).
//
// Workgroup: 256 threads (2x2 waves), BM x BN tile, K step 64 elements,
// double-buffered BF16 tiles in LDS with a 144-byte row pitch (8 consecutive
// rows hit distinct banks for the 16-byte fragment reads).  Grouped launch:
// the workgroup index enumerates (n tile, group, m tile); the grid is sized
// with an upper bound of ceil(R/BM) + groups m tiles and surplus workgroups
// exit.
#include "../device/codec.h"
#include "../device/gemm_common.h"
#include "../device/lowscale.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int kBK = 64;                // K elements per step
constexpr int kPitch = kBK * 2 + 16;   // LDS bytes per row

// staged unit: 32 consecutive K elements of one row
template <int SRC>
struct Unit {
  static constexpr int kCodeWords = SRC == FMT_NVFP4 ? 4 : 8;  // dwords of codes
  uint32_t w[kCodeWords];
  uint32_t s;  // NVFP4: two E4M3 bytes; MXFP8: one E8M0 byte
};

// F: the element type of MXFP8 units -- FMT_MXFP8 (E4M3), FMT_MXFP8_E5M2 or
// FMT_MXINT8 (two's complement times 2^-6, decoded in software: the exact
// FP32 product k * 2^(c-133), truncated to BF16).
// bias: added to an MXFP8 unit's scale code (not to 255, NaN) -- the fix-up
// pass's shift of a tile's codes into the exact range (see k_gemm_staged).
template <int SRC, int F = FMT_MXFP8>
__device__ inline void convert_store(const Unit<SRC>& u, uint8_t* dst, int bias = 0) {
  constexpr bool BF8 = F == FMT_MXFP8_E5M2;
  uint32_t out[16];
  if constexpr (SRC == FMT_NVFP4) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      const float sbv = e4m3_mag_value((u.s >> (8 * blk)) & 0xFFu);
#pragma unroll
      for (int wd = 0; wd < 2; ++wd) {
        const uint32_t word = u.w[blk * 2 + wd];
        const v2f f[4] = {__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 0),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 1),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 2),
                          __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, 3)};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float lo = f[b][0] * sbv, hi = f[b][1] * sbv;  // exact products
          out[blk * 8 + wd * 4 + b] = (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
        }
      }
    }
  } else if constexpr (F == FMT_MXINT8) {
    const uint32_t c0 = u.s & 0xFFu;
    const uint32_t c = c0 == 0xFFu ? c0 : (uint32_t)((int)c0 + bias);
    // 2^(c-127): c = 0 is the FP32 subnormal 2^-127, 0xFF is NaN
    const float X = c == 0xFFu ? __builtin_nanf("") : (c == 0u ? u2f(0x00400000u) : u2f(c << 23));
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      // k 2^-6 first (exact), then the scale: k X alone overflows at code 254
      const float v0 = (float)(int8_t)(u.w[wd] & 0xFFu) * 0.015625f * X;
      const float v1 = (float)(int8_t)((u.w[wd] >> 8) & 0xFFu) * 0.015625f * X;
      const float v2 = (float)(int8_t)((u.w[wd] >> 16) & 0xFFu) * 0.015625f * X;
      const float v3 = (float)(int8_t)(u.w[wd] >> 24) * 0.015625f * X;
      out[2 * wd] = (f2u(v0) >> 16) | (f2u(v1) & 0xFFFF0000u);
      out[2 * wd + 1] = (f2u(v2) >> 16) | (f2u(v3) & 0xFFFF0000u);
    }
  } else {
    const uint32_t c0 = u.s & 0xFFu;
    const uint32_t c = c0 == 0xFFu ? c0 : (uint32_t)((int)c0 + bias);
    if (c >= 1u && c != 0xFFu) {
      const float X = u2f(c << 23);  // 2^(c-127), a normal FP32
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        if constexpr (BF8) {
          out[2 * wd] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(u.w[wd], X, false));
          out[2 * wd + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(u.w[wd], X, true));
        } else {
          out[2 * wd] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.w[wd], X, false));
          out[2 * wd + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.w[wd], X, true));
        }
      }
    } else {
      // scale code 0 (2^-127 is an FP32 subnormal, which the converter does
      // not take as a scale) or 0xFF (NaN): convert at scale 1, multiply in FP32
      const float X = c == 0u ? u2f(0x00400000u) : __builtin_nanf("");
#pragma unroll
      for (int wd = 0; wd < 8; ++wd) {
        const v2f lo = BF8 ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(u.w[wd], 1.0f, false)
                           : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u.w[wd], 1.0f, false);
        const v2f hi = BF8 ? __builtin_amdgcn_cvt_scalef32_pk_f32_bf8(u.w[wd], 1.0f, true)
                           : __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(u.w[wd], 1.0f, true);
        out[2 * wd] = (f2u(lo[0] * X) >> 16) | (f2u(lo[1] * X) & 0xFFFF0000u);
        out[2 * wd + 1] = (f2u(hi[0] * X) >> 16) | (f2u(hi[1] * X) & 0xFFFF0000u);
      }
    }
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
}

// Scale codes for which the pipelined exact 8-bit kernel converts every
// element exactly to BF16 (the scaled value is a BF16 value): E4M3 3..246,
// E5M2 17..239, INT8 7..254.
template <int F>
constexpr uint32_t kExactLo = F == FMT_MXFP8_E5M2 ? 17u : F == FMT_MXINT8 ? 7u : 3u;
template <int F>
constexpr uint32_t kExactHi = F == FMT_MXFP8_E5M2 ? 239u : F == FMT_MXINT8 ? 254u : 246u;

// Every value of element type F is an integer multiple of 2^-kGrid<F>, below
// 2^kTop<F> in magnitude.
template <int F>
constexpr int kGrid = F == FMT_MXFP8_E5M2 ? 16 : F == FMT_MXINT8 ? 6 : 9;
template <int F>
constexpr int kTop = F == FMT_MXFP8_E5M2 ? 16 : F == FMT_MXINT8 ? 1 : 9;

// Lowest scale code of an F operand (against a G operand) whose tiles the
// pipelined kernel computes exactly: inside the conversion range, and at
// least half of 128 + g_F + g_G (rounded up), so that every nonzero product
// of two such codes is a normal FP32 value (the BF16 instruction is not
// relied on for subnormal products).
template <int F, int G>
constexpr uint32_t kScanLo = kExactLo<F> > (128u + kGrid<F> + kGrid<G> + 1u) / 2u
                                 ? kExactLo<F>
                                 : (128u + kGrid<F> + kGrid<G> + 1u) / 2u;

// FIXUP (MXFP8, K % 512 == 0): the workgroup first scans the scale rows of
// its tile and computes the tile only if one holds a code outside the range
// the pipelined exact 8-bit kernel computes exactly (kScanLo .. kExactHi of
// the operand's element type; 255, NaN, always); the output of that kernel
// for such tiles is overwritten.  BA / BB: the element types of A and B for
// MXFP8 units (FMT_MXFP8, FMT_MXFP8_E5M2 or FMT_MXINT8).
template <int SRC, int CDT, int BM, int BN, bool GATHER, bool FIXUP = false, int BA = FMT_MXFP8,
          int BB = FMT_MXFP8>
__global__ __launch_bounds__(256) void k_gemm_staged(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const float* __restrict__ a_ts,
    const int32_t* __restrict__ row_index, int64_t a_rows, int64_t R, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ b_ts, int32_t groups,
    const int64_t* __restrict__ offsets, int64_t N, int64_t K, void* __restrict__ C, int64_t ldc,
    uint32_t tiles_n, uint32_t tiles_m_bound) {
  constexpr int kRows = BM + BN;
  constexpr int kUnits = kRows * 2 / 256;  // 32-element units per thread per step
  constexpr int FM = BM / 2 / 32, FN = BN / 2 / 32;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kRows * kPitch];

  // workgroup -> (n tile, m tile over all groups); consecutive ids share the
  // m tile (A rows) and walk n, and ids on one XCD (id mod 8) are adjacent
  uint32_t id = blockIdx.x;
  const uint32_t total = tiles_n * tiles_m_bound;
  if ((total & 7u) == 0) id = (id & 7u) * (total >> 3) + (id >> 3);
  const int64_t tile = id / tiles_n;
  const int64_t n0 = (int64_t)(id % tiles_n) * BN;

  int64_t g = -1, g_lo = 0, g_hi = 0;
  if (offsets == nullptr) {
    if (tile * BM < R) {
      g = 0;
      g_lo = tile * BM;
      g_hi = R;
    }
  } else {
    int64_t acc = 0;
    for (int32_t e = 0; e < groups; ++e) {
      // clamped into [0, R]: offsets that break their contract (decreasing,
      // past R) cannot move a write outside C
      int64_t lo = offsets[e], hi = offsets[e + 1];
      lo = lo < 0 ? 0 : (lo > R ? R : lo);
      hi = hi < lo ? lo : (hi > R ? R : hi);
      const int64_t nt = (hi - lo + BM - 1) / BM;
      if (tile < acc + nt) {
        g = e;
        g_lo = lo + (tile - acc) * BM;
        g_hi = hi;
        break;
      }
      acc += nt;
    }
  }
  if (g < 0) return;  // surplus workgroup (uniform across the block)

  const uint32_t t = threadIdx.x;
  int bias_a = 0, bias_b = 0;  // the fix-up pass's code shifts
  if constexpr (FIXUP) {
    static_assert(SRC == FMT_MXFP8 && BM == 256 && BN == 256, "fix-up pass of the exact MXFP8 GEMM");
    __shared__ uint32_t found[4];
    const int64_t kb = K / 32;  // scale bytes per row, a multiple of 16
    uint32_t sp = 0;
    // The tile's A scale rows (and its B scale rows) are one contiguous run
    // of rows * kb bytes: consecutive lanes read consecutive 16-byte words.
    const int64_t ca = (g_hi - g_lo < BM ? g_hi - g_lo : BM) * kb / 16;
    const int64_t cb = (N - n0 < BN ? N - n0 : BN) * kb / 16;
    const u4* pa = reinterpret_cast<const u4*>(SA + g_lo * kb);
    const u4* pb = reinterpret_cast<const u4*>(SB + n0 * kb);
    const int64_t cmax = ca > cb ? ca : cb;
    for (int64_t q0 = t; q0 < cmax; q0 += 256 * 8) {  // 16 loads in flight per lane
      u4 v[16];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t q = q0 + 256 * u;
        // past the run: code 127 (2^0) in every byte, which is not special
        v[u] = q < ca ? pa[q] : u4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
        v[8 + u] = q < cb ? pb[q] : u4{0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu, 0x7F7F7F7Fu};
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          sp |= bytes_outside(v[u][e], kScanLo<BA, BB>, kExactHi<BA>) |
                bytes_outside(v[8 + u][e], kScanLo<BB, BA>, kExactHi<BB>);
    }
    const bool wave_found = __builtin_amdgcn_ballot_w64(sp != 0u) != 0;
    if ((t & 63u) == 0) found[t >> 6] = wave_found ? 1u : 0u;
    __syncthreads();
    if ((found[0] | found[1] | found[2] | found[3]) == 0u) return;  // uniform
    // The tile is recomputed.  Its codes are shifted, A's by bias_a and B's by
    // bias_b, into the exact range when one shift per operand fits them all
    // there with every product on FP32's 2^-149 grid and no sum beyond 2^127;
    // the result is scaled back with one rounding.  Else (codes spanning more
    // than the range) they are decoded as they are.
    __shared__ uint32_t red[16];
    int mna, mxa, mnb, mxb;
    ls_tile_ranges(reinterpret_cast<const uint8_t*>(pa), 16 * ca, reinterpret_cast<const uint8_t*>(pb), 16 * cb,
                   red, &mna, &mxa, &mnb, &mxb);
    if (!ls_shift(mna, mxa, mnb, mxb, (int)kExactLo<BA>, (int)kExactHi<BA>, (int)kExactLo<BB>, (int)kExactHi<BB>,
                  kGrid<BA>, kGrid<BB>, kTop<BA>, kTop<BB>, K, &bias_a, &bias_b))
      bias_a = bias_b = 0;
  }
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t m0 = g_lo;
  const int64_t rowbytes = SRC == FMT_NVFP4 ? K / 2 : K;
  const int64_t sblocks = SRC == FMT_NVFP4 ? K / 16 : K / 32;
  const int64_t steps = (K + kBK - 1) / kBK;
  const uint8_t* Bg = B + g * N * rowbytes;
  const uint8_t* SBg = SB + g * N * sblocks;

  // per-unit sources (fixed over the K loop): unit u = t + 256 j covers row
  // u / 2, K half u % 2 of each step
  const uint8_t* csrc[kUnits];
  const uint8_t* ssrc[kUnits];
  uint32_t dst_off[kUnits];
#pragma unroll
  for (int j = 0; j < kUnits; ++j) {
    const uint32_t u = t + 256u * j;
    const uint32_t r = u >> 1, h = u & 1u;
    dst_off[j] = r * kPitch + h * 64;
    csrc[j] = nullptr;
    ssrc[j] = nullptr;
    if (r < (uint32_t)BM) {
      const int64_t rr = m0 + r;
      if (rr < g_hi) {
        int64_t src_row = rr;
        if constexpr (GATHER) {  // entries outside [0, a_rows) clamped
          src_row = row_index[rr];
          src_row = src_row < 0 ? 0 : (src_row < a_rows ? src_row : a_rows - 1);
        }
        csrc[j] = A + src_row * rowbytes + h * (SRC == FMT_NVFP4 ? 16 : 32);
        ssrc[j] = SA + src_row * sblocks + h * (SRC == FMT_NVFP4 ? 2 : 1);
      }
    } else {
      const int64_t rr = n0 + (r - BM);
      if (rr < N) {
        csrc[j] = Bg + rr * rowbytes + h * (SRC == FMT_NVFP4 ? 16 : 32);
        ssrc[j] = SBg + rr * sblocks + h * (SRC == FMT_NVFP4 ? 2 : 1);
      }
    }
  }

  Unit<SRC> reg[kUnits];
  auto load_step = [&](int64_t step) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      const uint32_t h = (t + 256u * j) & 1u;
      const int64_t k0 = step * kBK + h * 32;  // first K element of the unit
      const bool ok = csrc[j] != nullptr && k0 < K;  // K % 32 == 0: a unit is all in or out
      if constexpr (SRC == FMT_NVFP4) {
        uint4 v = make_uint4(0, 0, 0, 0);
        uint32_t s = 0;
        if (ok) {
          v = *reinterpret_cast<const uint4*>(csrc[j] + step * (kBK / 2));
          s = *reinterpret_cast<const uint16_t*>(ssrc[j] + step * (kBK / 16));
        }
        reg[j].w[0] = v.x; reg[j].w[1] = v.y; reg[j].w[2] = v.z; reg[j].w[3] = v.w;
        reg[j].s = s;
      } else {
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
        uint32_t s = 127u;
        if (ok) {
          const uint4* p = reinterpret_cast<const uint4*>(csrc[j] + step * kBK);
          v0 = p[0];
          v1 = p[1];
          s = ssrc[j][step * (kBK / 32)];
        }
        reg[j].w[0] = v0.x; reg[j].w[1] = v0.y; reg[j].w[2] = v0.z; reg[j].w[3] = v0.w;
        reg[j].w[4] = v1.x; reg[j].w[5] = v1.y; reg[j].w[6] = v1.z; reg[j].w[7] = v1.w;
        reg[j].s = s;
      }
    }
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kUnits; ++j) {
      if (j < BM / 128) convert_store<SRC, BA>(reg[j], &lds[buf][dst_off[j]], bias_a);  // A rows
      else convert_store<SRC, BB>(reg[j], &lds[buf][dst_off[j]], bias_b);
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  load_step(0);
  store_step(0);
  __syncthreads();
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < steps) load_step(st + 1);
    const uint8_t* L = lds[buf];
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      const uint32_t off = (kk * 16 + lg * 8) * 2;
      v8bf af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(L + (wm * (BM / 2) + i * 32 + lr) * kPitch + off));
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(L + (BM + wn * (BN / 2) + j * 32 + lr) * kPitch + off));
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < steps) store_step(buf ^ 1);
    __syncthreads();
  }

  float sab = 1.0f;
  if constexpr (SRC == FMT_NVFP4) sab = *a_ts * b_ts[g];
  const int unshift = -(bias_a + bias_b);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * (BN / 2) + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * (BM / 2) + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
        if (row < g_hi && col < N) {
          const float val = SRC == FMT_NVFP4 ? acc[i][j][v] * sab
                                             : (FIXUP ? __builtin_amdgcn_ldexpf(acc[i][j][v], unshift) : acc[i][j][v]);
          if constexpr (CDT == DT_F32) static_cast<float*>(C)[row * ldc + col] = val;
          else static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(val);
        }
      }
    }
}

template <int SRC, int CDT, int BM, int BN, bool GATHER, bool FIXUP = false, int BA = FMT_MXFP8,
          int BB = FMT_MXFP8>
hipError_t run(const uint8_t* a, const uint8_t* sa, const float* ats, const int32_t* ri, int64_t a_rows, int64_t R,
               const uint8_t* b, const uint8_t* sb, const float* bts, int32_t groups,
               const int64_t* off, int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const uint32_t tn = (uint32_t)((N + BN - 1) / BN);
  const uint32_t tmb = (uint32_t)((R + BM - 1) / BM + (off ? groups : 0));
  hipLaunchKernelGGL((k_gemm_staged<SRC, CDT, BM, BN, GATHER, FIXUP, BA, BB>), dim3(tn * tmb), dim3(256), 0, s,
                     a, sa, ats, ri, a_rows, R, b, sb, bts, groups, off, N, K, C, ldc, tn, tmb);
  return hipGetLastError();
}

template <int SRC, int CDT, bool GATHER>
hipError_t run_sized(const uint8_t* a, const uint8_t* sa, const float* ats, const int32_t* ri,
                     int64_t a_rows, int64_t R, const uint8_t* b, const uint8_t* sb, const float* bts,
                     int32_t groups, const int64_t* off, int64_t N, int64_t K, void* C,
                     int64_t ldc, hipStream_t s) {
  if (R * N >= (int64_t)256 * 256 * 192)
    return run<SRC, CDT, 256, 256, GATHER>(a, sa, ats, ri, a_rows, R, b, sb, bts, groups, off, N, K, C, ldc, s);
  return run<SRC, CDT, 128, 128, GATHER>(a, sa, ats, ri, a_rows, R, b, sb, bts, groups, off, N, K, C, ldc, s);
}

}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                             const int32_t* row_index, int64_t a_rows, int64_t routed_rows,
                             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                             int32_t groups, const int64_t* offsets, int64_t N, int64_t K,
                             void* C, int cdt, int64_t ldc, hipStream_t s) {
  if (routed_rows == 0 || N == 0) return hipSuccess;
  // large shapes: FP4 stages through LDS, converted after the fragment
  // reads (gemm_nvpipe.hip)
  if (gemm_nvfp4_pipe_fits(a_rows, routed_rows, N, K))
    return launch_gemm_nvfp4_pipe(a_codes, a_scales, a_ts, row_index, a_rows, routed_rows, b_codes, b_scales,
                                  b_ts, groups, offsets, N, K, C, cdt, ldc, s);
#define MXK_NV(D, G) \
  run_sized<FMT_NVFP4, D, G>(a_codes, a_scales, a_ts, row_index, a_rows, routed_rows, b_codes, b_scales, b_ts, groups, offsets, N, K, C, ldc, s)
  if (row_index) return cdt == DT_F32 ? MXK_NV(DT_F32, true) : MXK_NV(DT_BF16, true);
  return cdt == DT_F32 ? MXK_NV(DT_F32, false) : MXK_NV(DT_BF16, false);
#undef MXK_NV
}

namespace {
// the exact pipelined kernel, then the fix-up pass, for element types BA / BB
template <int CDT, int BA, int BB>
hipError_t exact_pipe_and_fixup(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* b_codes,
                                const uint8_t* b_scales, int64_t M, int64_t N, int64_t K, void* C, int64_t ldc,
                                hipStream_t s) {
  const hipError_t e =
      launch_gemm_mxfp8_exact_pipe(a_codes, a_scales, b_codes, b_scales, M, N, K, C, CDT, ldc, s, BA, BB);
  if (e != hipSuccess) return e;
  // tiles whose operands hold scale codes 0 or 255, recomputed here
  return run<FMT_MXFP8, CDT, 256, 256, false, true, BA, BB>(a_codes, a_scales, nullptr, nullptr, M, M, b_codes,
                                                             b_scales, nullptr, 1, nullptr, N, K, C, ldc, s);
}
}  // namespace

hipError_t launch_gemm_mxfp8_exact(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                   int64_t N, int64_t K, void* C, int cdt, int64_t ldc,
                                   hipStream_t s, int fa, int fb) {
  if (M == 0 || N == 0) return hipSuccess;
  // large shapes: raw 8-bit stages through LDS, converted after the fragment
  // reads (gemm_mx.hip)
  if (gemm_mxfp8_exact_pipe_fits(M, N, K)) {
#define MXK_EX(A_, B_)                                                                                    \
  if (fa == A_ && fb == B_)                                                                               \
    return cdt == DT_F32                                                                                  \
               ? exact_pipe_and_fixup<DT_F32, A_, B_>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s) \
               : exact_pipe_and_fixup<DT_BF16, A_, B_>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
    MXK_EX(FMT_MXFP8, FMT_MXFP8)
    MXK_EX(FMT_MXFP8_E5M2, FMT_MXFP8)
    MXK_EX(FMT_MXFP8, FMT_MXFP8_E5M2)
    MXK_EX(FMT_MXFP8_E5M2, FMT_MXFP8_E5M2)
    MXK_EX(FMT_MXINT8, FMT_MXINT8)
    MXK_EX(FMT_MXINT8, FMT_MXFP8)
    MXK_EX(FMT_MXFP8, FMT_MXINT8)
    MXK_EX(FMT_MXINT8, FMT_MXFP8_E5M2)
    MXK_EX(FMT_MXFP8_E5M2, FMT_MXINT8)
#undef MXK_EX
    return hipErrorInvalidValue;
  }
  // pairs other than E4M3 x E4M3 take this path only where the pipeline fits
  if (fa != FMT_MXFP8 || fb != FMT_MXFP8) return hipErrorInvalidValue;
  const hipError_t e =
      cdt == DT_F32
          ? run_sized<FMT_MXFP8, DT_F32, false>(a_codes, a_scales, nullptr, nullptr, M, M, b_codes, b_scales, nullptr, 1, nullptr, N, K, C, ldc, s)
          : run_sized<FMT_MXFP8, DT_BF16, false>(a_codes, a_scales, nullptr, nullptr, M, M, b_codes, b_scales, nullptr, 1, nullptr, N, K, C, ldc, s);
  if (e != hipSuccess) return e;
  // tiles with a code below kScanLo (products that could be subnormal FP32
  // values) or above the generic kernel's exact range, recomputed there
  return launch_gemm_mx_any(FMT_MXFP8, a_codes, a_scales, FMT_MXFP8, b_codes, b_scales, M, N, K, C, cdt, ldc, s,
                            kScanLo<FMT_MXFP8, FMT_MXFP8>, 239u);
}

}  // namespace mxk
