// gemm_any.hip -- block-scaled GEMM C = A * B^T for any pair of MX formats
// (E8M0 scales per 32 along K): the MX element types MXFP8 E4M3 / E5M2,
// MXFP6 E3M2 / E2M3, MXFP4 and MXINT8, the same or different for A and B
// ("Microscaling (MX) and block-scaled 4-bit formats", section "The idea";
// "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier", section "The OCP
// Microscaling (MX) spec").
//
// Every element of these types times its power-of-two scale has at most 8
// significant bits (INT8: 7), so it is exact in BF16 whenever the product is
// a normal BF16 value; the operands are decoded into LDS as BF16 and
// contracted on v_mfma_f32_32x32x16_bf16 (exact products, FP32
// accumulation), as the staged kernel does for MXFP8 and NVFP4.  The formats
// are kernel arguments: a uniform switch picks the decoder of each 32-element
// unit, so one kernel serves all 36 pairs.
//
// Decoding: gfx950's scaled conversions to BF16 (v_cvt_scalef32_pk_bf16_fp8 /
// _bf8 / _fp4 and the 32-wide v_cvt_scalef32_pk32_bf16_fp6 / _bf6) multiply
// by 2^(exponent of their FP32 scale) -- exactly the E8M0 scale -- and round
// once, so they are exact while the scaled values are normal BF16 values:
// scale codes 17 .. 239 cover every element type (checked on the device
// against the software decoders; the FP6 one reads element i at bits 6 i of
// its six words, the packing used here).  Other scale codes, and INT8, take
// the software decoders (exact FP32 products, truncated to BF16).
//
// Workgroup: 256 threads (2 x 2 waves), 128 x 128 C tile, K step 64,
// double-buffered BF16 tiles in LDS, two workgroups per CU.
#include "../device/codec.h"
#include "../device/gemm_common.h"
#include "../device/lowscale.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kStepK = 64;
constexpr int kPitch = kStepK * 2 + 16;  // LDS bytes per row (bank spread)

__device__ inline int code_bits(int fmt) {
  return fmt == FMT_MXFP4 ? 4 : (fmt == FMT_MXFP6_E3M2 || fmt == FMT_MXFP6_E2M3) ? 6 : 8;
}

// 32 elements of one row: up to 32 code bytes, and the block's scale code.
struct Unit {
  uint32_t w[8];
  uint32_t s;
};

// Element i of the unit as an exact FP32 value (before the block scale).
template <int FMT>
__device__ __attribute__((always_inline)) inline float unit_elem(const Unit& u, int i) {
  if constexpr (FMT == FMT_MXFP4) {
    const uint32_t c = (u.w[i >> 3] >> (4 * (i & 7))) & 0xFu;
    return e2m1_value(c);
  } else if constexpr (FMT == FMT_MXFP6_E3M2 || FMT == FMT_MXFP6_E2M3) {
    const int bit = 6 * i;  // element i at bits 6 i of the unit's 24 bytes
    const uint64_t two = (uint64_t)u.w[bit >> 5] | ((uint64_t)u.w[(bit >> 5) + 1 < 6 ? (bit >> 5) + 1 : 5] << 32);
    const uint32_t c = (uint32_t)(two >> (bit & 31)) & 0x3Fu;
    return FMT == FMT_MXFP6_E3M2 ? fp6_value<E3M2>(c) : fp6_value<E2M3>(c);
  } else {
    const uint32_t c = (u.w[i >> 2] >> (8 * (i & 3))) & 0xFFu;
    if constexpr (FMT == FMT_MXFP8) {
      const uint32_t mag = c & 0x7Fu;
      const float e = mag == 0x7Fu ? __builtin_nanf("") : e4m3_mag_value(mag);
      return (c & 0x80u) ? -e : e;
    } else if constexpr (FMT == FMT_MXFP8_E5M2) {
      return e5m2_value(c);
    } else {
      return int8_value(c);
    }
  }
}

typedef unsigned int v6u __attribute__((ext_vector_type(6)));
typedef __bf16 v32bf __attribute__((ext_vector_type(32)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Hardware path (scale code c in 17 .. 239, FMT not INT8): whole vectors are
// stored, never single elements of them.
template <int FMT>
__device__ __attribute__((always_inline)) inline void decode_store_hw(const Unit& u, float X, uint8_t* dst) {
  if constexpr (FMT == FMT_MXFP6_E3M2 || FMT == FMT_MXFP6_E2M3) {
    const v6u a = {u.w[0], u.w[1], u.w[2], u.w[3], u.w[4], u.w[5]};
    v32bf r;
    if constexpr (FMT == FMT_MXFP6_E2M3) r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_fp6(a, X);
    else r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(a, X);
    *reinterpret_cast<v32bf*>(dst) = r;
  } else if constexpr (FMT == FMT_MXFP4) {
    v2bf r[16];
#pragma unroll
    for (int wd = 0; wd < 4; ++wd) {
      r[4 * wd + 0] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u.w[wd], X, 0);
      r[4 * wd + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u.w[wd], X, 1);
      r[4 * wd + 2] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u.w[wd], X, 2);
      r[4 * wd + 3] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(u.w[wd], X, 3);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<v2bf*>(dst + 4 * i) = r[i];
  } else {
    v2bf r[16];
#pragma unroll
    for (int wd = 0; wd < 8; ++wd) {
      if constexpr (FMT == FMT_MXFP8) {
        r[2 * wd] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.w[wd], X, false);
        r[2 * wd + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(u.w[wd], X, true);
      } else {
        r[2 * wd] = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(u.w[wd], X, false);
        r[2 * wd + 1] = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(u.w[wd], X, true);
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) *reinterpret_cast<v2bf*>(dst + 4 * i) = r[i];
  }
}

// Decode a unit to 32 BF16 values and store them as 64 contiguous bytes;
// shift: added to the scale code (not to 255, NaN) by the fix-up mode.
template <int FMT>
__device__ __attribute__((always_inline)) inline void decode_store(const Unit& u, uint8_t* dst, int shift) {
  const uint32_t c0 = u.s & 0xFFu;
  const uint32_t c = c0 == 0xFFu ? c0 : (uint32_t)((int)c0 + shift);
  if constexpr (FMT != FMT_MXINT8) {
    if (c >= 17u && c <= 239u) {
      decode_store_hw<FMT>(u, u2f(c << 23), dst);
      return;
    }
  }
  // 2^(c-127): c = 0 is the FP32 subnormal 2^-127, 0xFF is NaN
  const float X = c == 0xFFu ? __builtin_nanf("") : (c == 0u ? u2f(0x00400000u) : u2f(c << 23));
  uint32_t out[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    const float lo = unit_elem<FMT>(u, 2 * p) * X, hi = unit_elem<FMT>(u, 2 * p + 1) * X;
    out[p] = (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<uint4*>(dst + 16 * q) = make_uint4(out[4 * q], out[4 * q + 1], out[4 * q + 2], out[4 * q + 3]);
}

__device__ __attribute__((always_inline)) inline void decode_store_any(int fmt, const Unit& u, uint8_t* dst,
                                                                     int shift) {
  switch (fmt) {
    case FMT_MXFP8: decode_store<FMT_MXFP8>(u, dst, shift); break;
    case FMT_MXFP4: decode_store<FMT_MXFP4>(u, dst, shift); break;
    case FMT_MXINT8: decode_store<FMT_MXINT8>(u, dst, shift); break;
    case FMT_MXFP8_E5M2: decode_store<FMT_MXFP8_E5M2>(u, dst, shift); break;
    case FMT_MXFP6_E3M2: decode_store<FMT_MXFP6_E3M2>(u, dst, shift); break;
    default: decode_store<FMT_MXFP6_E2M3>(u, dst, shift); break;
  }
}

// Element grids (values are multiples of 2^-g) and magnitudes (below 2^top).
__device__ inline int fmt_grid(int fmt) {
  return fmt == FMT_MXFP8 ? 9 : fmt == FMT_MXFP8_E5M2 ? 16 : fmt == FMT_MXINT8 ? 6 : fmt == FMT_MXFP6_E3M2 ? 4
         : fmt == FMT_MXFP6_E2M3 ? 3 : 1;
}
__device__ inline int fmt_top(int fmt) {
  return fmt == FMT_MXFP8 ? 9 : fmt == FMT_MXFP8_E5M2 ? 16 : fmt == FMT_MXINT8 ? 1 : fmt == FMT_MXFP6_E3M2 ? 5 : 3;
}

// Load the unit of K elements k0 .. k0+31 of a row (codes at `row`, scales
// at `srow`); a unit past the row (k0 >= K) or of a missing row is zero.
__device__ __attribute__((always_inline)) inline void load_unit(int bits, const uint8_t* row, const uint8_t* srow, int64_t k0, bool ok, Unit& u) {
#pragma unroll
  for (int i = 0; i < 8; ++i) u.w[i] = 0u;
  u.s = 127u;
  if (!ok) return;
  const uint8_t* p = row + k0 * bits / 8;  // 16-byte aligned for 8-bit and FP4, 8-byte for FP6
  if (bits == 8) {
    const uint4 a = reinterpret_cast<const uint4*>(p)[0], b = reinterpret_cast<const uint4*>(p)[1];
    u.w[0] = a.x; u.w[1] = a.y; u.w[2] = a.z; u.w[3] = a.w;
    u.w[4] = b.x; u.w[5] = b.y; u.w[6] = b.z; u.w[7] = b.w;
  } else if (bits == 6) {
    const uint2* q = reinterpret_cast<const uint2*>(p);
    const uint2 a = q[0], b = q[1], c = q[2];
    u.w[0] = a.x; u.w[1] = a.y; u.w[2] = b.x; u.w[3] = b.y; u.w[4] = c.x; u.w[5] = c.y;
  } else {
    const uint4 a = *reinterpret_cast<const uint4*>(p);
    u.w[0] = a.x; u.w[1] = a.y; u.w[2] = a.z; u.w[3] = a.w;
  }
  u.s = srow[k0 >> 5];
}

// Thread t stages, per step, the units t + 256 j: row (t + 256 j) / 2 of the
// stacked [A tile; B tile] rows, K half t % 2 -- j < U/2 are A rows.
// fix_lo > 0: the workgroup first scans the scale rows of its tile (fix-up
// mode: of its 2 x 2 tiles) for a code outside [fix_lo, fix_hi]; if there is
// one it computes them with shifted codes (below), else it computes them as
// they are when `every`, or leaves them -- the fix-up pass behind a kernel
// that is exact only for codes in that range.
template <int CDT, int T>
__global__ __launch_bounds__(256) void k_gemm_mx_any(int fa, int fb, const uint8_t* __restrict__ A,
                                                     const uint8_t* __restrict__ SA,
                                                     const uint8_t* __restrict__ B,
                                                     const uint8_t* __restrict__ SB, int64_t M, int64_t N,
                                                     int64_t K, void* __restrict__ C, int64_t ldc,
                                                     uint32_t tiles_n, uint32_t fix_lo, uint32_t fix_hi,
                                                     bool every) {
  constexpr int U = 2 * T * 2 / 256;  // units per thread and step (2 or 4)
  constexpr int F = T / 64;           // 32 x 32 instruction tiles per wave and dimension
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2 * T * kPitch];
  // Fix-up mode (fix_lo > 0, not every): one workgroup per region of 2 x 2
  // tiles, whose scale rows it scans once; otherwise one per tile.
  const int span = (fix_lo > 0 && !every) ? 2 : 1;
  const int64_t r0 = (int64_t)(blockIdx.x / tiles_n) * T * span, c0 = (int64_t)(blockIdx.x % tiles_n) * T * span;
  const uint32_t t = threadIdx.x, lane = t & 63u, wid = t >> 6;
  int shift_a = 0, shift_b = 0;  // the fix-up mode's code shifts
  if (fix_lo > 0) {
    __shared__ uint32_t found;
    if (t == 0) found = 0u;
    __syncthreads();
    // The scale rows of the region's A rows (and of its B rows) are one
    // contiguous run of rows * K/32 bytes, 16-byte aligned (the scale arrays
    // are, and 128 rows of K/32 bytes are a multiple of 16): read as
    // consecutive 16-byte words by consecutive lanes, then the last bytes
    // one by one.
    const int64_t kbytes = K / 32, R = (int64_t)span * T;
    const int64_t na = (M - r0 < R ? M - r0 : R) * kbytes, nb = (N - c0 < R ? N - c0 : R) * kbytes;
    const uint8_t* pa = SA + r0 * kbytes;
    const uint8_t* pb = SB + c0 * kbytes;
    uint32_t sp = 0u;
    const uint32_t pad = fix_lo * 0x01010101u;  // a word of codes inside the range
    for (int op = 0; op < 2; ++op) {
      const uint8_t* p = op ? pb : pa;
      const int64_t n = op ? nb : na;
      // 8 loads in flight per lane
      for (int64_t q0 = 16 * (int64_t)t; q0 + 16 <= n; q0 += 16 * 256 * 8) {
        uint4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int64_t q = q0 + 16 * 256 * u;
          v[u] = q + 16 <= n ? *reinterpret_cast<const uint4*>(p + q) : make_uint4(pad, pad, pad, pad);
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          sp |= bytes_outside(v[u].x, fix_lo, fix_hi) | bytes_outside(v[u].y, fix_lo, fix_hi) |
                bytes_outside(v[u].z, fix_lo, fix_hi) | bytes_outside(v[u].w, fix_lo, fix_hi);
      }
      // a lone byte, padded with codes inside the range in the other bytes
      for (int64_t q = (n & ~(int64_t)15) + t; q < n; q += 256)
        sp |= bytes_outside((pad & 0xFFFFFF00u) | p[q], fix_lo, fix_hi);
    }
    if (sp) atomicOr(&found, 1u);
    __syncthreads();
    if (found == 0u) {  // uniform
      if (!every) return;
    } else {
      // The tile is computed with its codes shifted, A's by shift_a and B's
      // by shift_b, into the range the hardware conversions take exactly (17
      // .. 239; INT8's software decode 7 .. 254) when one shift per operand
      // fits them all there with every product a normal FP32 value and no
      // sum beyond 2^127; the result is scaled back with one rounding.  Else
      // the codes are decoded as they are.
      __shared__ uint32_t red[16];
      int mna, mxa, mnb, mxb;
      ls_tile_ranges(pa, na, pb, nb, red, &mna, &mxa, &mnb, &mxb);
      const int la = fa == FMT_MXINT8 ? 7 : 17, ha = fa == FMT_MXINT8 ? 254 : 239;
      const int lb = fb == FMT_MXINT8 ? 7 : 17, hb = fb == FMT_MXINT8 ? 254 : 239;
      if (!ls_shift(mna, mxa, mnb, mxb, la, ha, lb, hb, fmt_grid(fa), fmt_grid(fb), fmt_top(fa), fmt_top(fb), K,
                    &shift_a, &shift_b))
        shift_a = shift_b = 0;
    }
  }
  // the region's tiles (one outside the fix-up mode); the barrier that ends
  // a tile's last step also ends every LDS read before the next tile's stores
  for (int sub = 0; sub < span * span; ++sub) {
    const int64_t m0 = r0 + (int64_t)(sub / span) * T, n0 = c0 + (int64_t)(sub % span) * T;
    if (m0 >= M || n0 >= N) continue;  // uniform
    const uint32_t wm = wid >> 1, wn = wid & 1u;
    const int ba = code_bits(fa), bb = code_bits(fb);
    const int64_t rba = K * ba / 8, rbb = K * bb / 8, kb = K / 32;
    const uint32_t h = t & 1u;
    const uint8_t* crow[U];
    const uint8_t* srow[U];
    bool ok[U];
    uint32_t dst[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const uint32_t r = (t + 256u * j) >> 1;  // stacked row: A rows 0 .. T-1, then B rows
      dst[j] = r * kPitch + h * 64;
      if (j < U / 2) {
        const int64_t ra = m0 + r;
        ok[j] = ra < M;
        crow[j] = A + (ok[j] ? ra : 0) * rba;
        srow[j] = SA + (ok[j] ? ra : 0) * kb;
      } else {
        const int64_t rb = n0 + (r - T);
        ok[j] = rb < N;
        crow[j] = B + (ok[j] ? rb : 0) * rbb;
        srow[j] = SB + (ok[j] ? rb : 0) * kb;
      }
    }
    const int64_t steps = (K + kStepK - 1) / kStepK;

    Unit un[U];
    auto load = [&](int64_t st) {
      const int64_t k0 = st * kStepK + h * 32;  // K % 32 == 0: a unit is all in or out
#pragma unroll
      for (int j = 0; j < U; ++j) load_unit(j < U / 2 ? ba : bb, crow[j], srow[j], k0, ok[j] && k0 < K, un[j]);
    };
    auto store = [&](int buf) {
#pragma unroll
      for (int j = 0; j < U; ++j)
        decode_store_any(j < U / 2 ? fa : fb, un[j], &lds[buf][dst[j]], j < U / 2 ? shift_a : shift_b);
    };

    v16f acc[F][F];
#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

    load(0);
    store(0);
    __syncthreads();
    const uint32_t lr = lane & 31u, lg = lane >> 5;
    for (int64_t st = 0; st < steps; ++st) {
      const int buf = (int)(st & 1);
      if (st + 1 < steps) load(st + 1);
      const uint8_t* L = lds[buf];
#pragma unroll
      for (int kk = 0; kk < kStepK / 16; ++kk) {
        const uint32_t off = (kk * 16 + lg * 8) * 2;
        v8bf af[F], bfr[F];
#pragma unroll
        for (int i = 0; i < F; ++i)
          af[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(L + (wm * (T / 2) + i * 32 + lr) * kPitch + off));
#pragma unroll
        for (int j = 0; j < F; ++j)
          bfr[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const uint4*>(L + (T + wn * (T / 2) + j * 32 + lr) * kPitch + off));
#pragma unroll
        for (int i = 0; i < F; ++i)
#pragma unroll
          for (int j = 0; j < F; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      }
      if (st + 1 < steps) store(buf ^ 1);
      __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < F; ++i)
#pragma unroll
      for (int j = 0; j < F; ++j) {
        const int64_t col = n0 + wn * (T / 2) + j * 32 + lr;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int64_t row = m0 + wm * (T / 2) + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
          if (row < M && col < N) {
            const float val = __builtin_amdgcn_ldexpf(acc[i][j][v], -(shift_a + shift_b));  // exact at shift 0
            if constexpr (CDT == DT_F32) static_cast<float*>(C)[row * ldc + col] = val;
            else static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(val);
          }
        }
      }
  }
}

}  // namespace

hipError_t launch_gemm_mx_any(int fa, const uint8_t* a_codes, const uint8_t* a_scales, int fb,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                              int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s, uint32_t fix_lo,
                              uint32_t fix_hi, bool every) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fix_lo > 0 && (fix_lo > 128 || fix_hi < 127 || fix_hi > 254)) return hipErrorInvalidValue;
  // 128 x 128 tiles, two workgroups per CU: with 256 x 256 tiles the six
  // inlined decoders of four units per thread spill registers
  constexpr int64_t T = 128;
  const int64_t R = (fix_lo > 0 && !every) ? 2 * T : T;  // the kernel's span
  const uint32_t tm = (uint32_t)((M + R - 1) / R), tn = (uint32_t)((N + R - 1) / R);
  if ((uint64_t)tm * tn > 0x7FFFFFFFull) return hipErrorInvalidValue;
#define MXK_ANY(D, TT)                                                                                    \
  hipLaunchKernelGGL((k_gemm_mx_any<D, TT>), dim3(tm * tn), dim3(256), 0, s, fa, fb, a_codes, a_scales, b_codes, \
                     b_scales, M, N, K, C, ldc, tn, fix_lo, fix_hi, every)
  if (cdt == DT_F32) MXK_ANY(DT_F32, 128);
  else MXK_ANY(DT_BF16, 128);
#undef MXK_ANY
  return hipGetLastError();
}

}  // namespace mxk
