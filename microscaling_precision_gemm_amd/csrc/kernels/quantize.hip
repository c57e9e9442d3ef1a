// quantize.hip -- block-scaled quantizers, per-tensor amax, decoder and the
// standalone 16-point Hadamard transform for gfx950.
//
// All kernels here are HBM-bound streaming kernels.  Work unit: a "chunk" of
// 8 consecutive elements of a row, held by one lane (one 128-bit BF16 load).
// A 64-lane wave covers a slab of 64 consecutive chunks, so an MX block of 32
// elements is one lane quad and an NVFP4 block of 16 (or a Hadamard group of
// 16) is one lane pair; block maxima and the stride-8 butterfly use DPP quad
// permutes.  Each wave owns kU consecutive slabs and issues all their loads
// before any arithmetic, so every lane keeps kU 128-bit loads in flight.
// Codes are stored with one 64-bit (MXFP8) or 32-bit (FP4) store per lane and
// the scale bytes of 4 blocks are gathered into one 32-bit store.
//
// Chunk q of a [rows, cols] matrix is chunk q % (cols/8) of row q / (cols/8);
// blocks never straddle rows (cols is a multiple of the block), so block,
// scale and random-number indices are all linear in q and only the input
// address needs the row (a division, skipped when rows are dense).
//
// Method sources: "Microscaling (MX) and block-scaled 4-bit formats"
// (sections "Microscaling", "The idea", "NVFP4", glossary "scale factor",
// "stochastic rounding"); "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier"
// (MXFP4/NVFP4 table and the paragraph on two-level scaling).
#include "../device/codec.h"
#include "../device/cvt.h"
#include "../device/mxenc.h"
#include "../device/tiles.h"
#include "../device/wave.h"
#include "../launch.h"

namespace mxk {

namespace {

constexpr int kThreads = 256;

constexpr int kU = 4;  // slabs (64 chunks each) per wave

typedef uint32_t u4 __attribute__((ext_vector_type(4)));

// Element offset of chunk q in a [rows, cols] matrix with row pitch ld
// (cpr = cols / 8 chunks per row).
__device__ inline int64_t chunk_offset(int64_t q, int64_t cpr, int64_t ld, bool dense) {
  if (dense) return 8 * q;
  int64_t row;
  if (q < ((int64_t)1 << 32) && cpr < ((int64_t)1 << 32))
    row = (int64_t)((uint32_t)q / (uint32_t)cpr);
  else
    row = q / cpr;
  return row * ld + 8 * (q - row * cpr);
}

// The raw bits of one chunk: 16 bytes (BF16) or 32 bytes (FP32).
template <int XDT>
struct Raw {
  u4 w[XDT == DT_BF16 ? 1 : 2];
};

template <int XDT>
__device__ inline void load_raw(const void* base, int64_t off, Raw<XDT>& r) {
  if constexpr (XDT == DT_BF16) {
    r.w[0] = *reinterpret_cast<const u4*>(static_cast<const uint16_t*>(base) + off);
  } else {
    const u4* p = reinterpret_cast<const u4*>(static_cast<const float*>(base) + off);
    r.w[0] = p[0];
    r.w[1] = p[1];
  }
}

// Issue the loads of the kU slabs starting at chunk q0 (this lane's chunk of
// the first slab).  Chunks past the end (q >= Q, Q >= 1) load chunk Q - 1
// instead, so every load is unconditional; their values are never stored.
template <int XDT>
__device__ inline void load_slabs(const void* x, int64_t q0, int64_t Q, int64_t cpr, int64_t ld,
                                  bool dense, Raw<XDT> (&raw)[kU]) {
  int64_t off[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    int64_t q = q0 + 64 * u;
    q = q < Q ? q : Q - 1;
    off[u] = chunk_offset(q, cpr, ld, dense);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) load_raw<XDT>(x, off[u], raw[u]);
}

template <int XDT>
__device__ inline void widen(const Raw<XDT>& r, float v[8]) {
  if constexpr (XDT == DT_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = u2f(r.w[0][i] << 16);
      v[2 * i + 1] = u2f(r.w[0][i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = u2f(r.w[0][i]);
      v[4 + i] = u2f(r.w[1][i]);
    }
  }
}

template <int YDT>
__device__ inline void store8(void* base, int64_t off, const float v[8]) {
  if constexpr (YDT == DT_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    store_nt(static_cast<uint16_t*>(base) + off, w[0], w[1], w[2], w[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// The random signs D of the forward transform as XOR masks on the raw bits
// of a chunk (bit i of the lane's byte of the mask negates element i): one
// XOR per word instead of a select per element.  The masks depend only on
// the lane's half, so a wave computes them once.
template <int XDT>
struct SignBits {
  u4 w[XDT == DT_BF16 ? 1 : 2];
};

template <int XDT>
__device__ inline SignBits<XDT> rht_sign_bits(uint32_t mask, uint32_t half) {
  const uint32_t m = (mask >> (8 * half)) & 0xFFu;
  SignBits<XDT> s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (XDT == DT_BF16) {  // word i: elements 2i (bits 0..15) and 2i + 1
      s.w[0][i] = (((m >> (2 * i)) & 1u) << 15) | (((m >> (2 * i + 1)) & 1u) << 31);
    } else {
      s.w[0][i] = ((m >> i) & 1u) << 31;
      s.w[1][i] = ((m >> (4 + i)) & 1u) << 31;
    }
  }
  return s;
}

template <int XDT>
__device__ inline void apply_signs(Raw<XDT>& r, const SignBits<XDT>& s) {
#pragma unroll
  for (int h = 0; h < (XDT == DT_BF16 ? 1 : 2); ++h) r.w[h] ^= s.w[h];
}

// Forward 16-point transform of a group split over a lane pair, for values
// whose signs D are already applied (apply_signs): this lane holds elements
// 8*half .. 8*half+7.  y = (1/4) H16 D x, stages 1, 2, 4 in the lane, stage 8
// across the pair (the lower lane keeps a + b, the upper lane a - b, with a
// the lower lane's value).
__device__ inline void rht_forward_signed(float v[8], uint32_t half) {
  hadamard8_stages(v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float p = dpp_xor1f(v[i]);
    v[i] = half ? (p - v[i]) : (v[i] + p);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) v[i] = 0.25f * v[i];
}

__device__ inline void rht_inverse(float v[8], uint32_t mask, uint32_t half) {
  hadamard8_stages(v);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float p = dpp_xor1f(v[i]);
    v[i] = half ? (p - v[i]) : (v[i] + p);
  }
  uint32_t m = (mask >> (8 * half)) & 0xFFu;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float u = 0.25f * v[i];
    v[i] = ((m >> i) & 1u) ? -u : u;
  }
}

// Gather the scale byte of `group` consecutive lane groups (group = 4 lanes
// per MX block, 2 per NVFP4 block) into lane 4*group*k and store 4 bytes at a
// time; `blocks_left` is the number of valid blocks from this lane's block on.
__device__ inline void store_scales(uint8_t* scales, int64_t block, uint32_t sc, uint32_t lane,
                                    uint32_t group, int64_t blocks_left) {
  uint32_t s1 = lane_read(sc, lane + group);
  uint32_t s2 = lane_read(sc, lane + 2 * group);
  uint32_t s3 = lane_read(sc, lane + 3 * group);
  if ((lane & (4 * group - 1)) != 0 || blocks_left <= 0) return;
  if (blocks_left >= 4) {
    *reinterpret_cast<uint32_t*>(scales + block) = sc | (s1 << 8) | (s2 << 16) | (s3 << 24);
  } else {
    uint32_t s[4] = {sc, s1, s2, s3};
    for (int64_t i = 0; i < blocks_left; ++i) scales[block + i] = (uint8_t)s[i];
  }
}

// ---- MX (E8M0 per 32) quantizer -------------------------------------------
template <int FMT, bool SR>
__device__ inline void encode_mx(const QuantArgs& a, int64_t q, const float v[8], Enc<FMT>& e) {
  encode_mx<FMT, SR>(MxEnc{a.ceil, a.seed, a.counter}, q, v, e);
}

template <int FMT>
__device__ inline void store_enc(const QuantArgs& a, int64_t q, int64_t Q, uint32_t lane,
                                 uint32_t lanes_per_block, const Enc<FMT>& e) {
  if (q < Q) {
    if constexpr (MxFmt<FMT>::bits == 8) {
      *reinterpret_cast<uint2*>(a.codes + q * 8) = make_uint2(e.w[0], e.w[1]);
    } else if constexpr (MxFmt<FMT>::bits == 6) {  // 6 bytes at 6 q: 2-byte aligned
      uint16_t* p = reinterpret_cast<uint16_t*>(a.codes + q * 6);
      p[0] = (uint16_t)e.w[0];
      p[1] = (uint16_t)(e.w[0] >> 16);
      p[2] = (uint16_t)e.w[1];
    } else {
      *reinterpret_cast<uint32_t*>(a.codes + q * 4) = e.w[0];
    }
  }
  const uint32_t sh = lanes_per_block == 4 ? 2 : 1;
  store_scales(a.scales, q >> sh, e.sc, lane, lanes_per_block, (Q - q) >> sh);
}

// Each wave: load kU slabs, encode them all, then store them all (so the
// waits for the loads are not held up by stores).
template <int XDT, int FMT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_mx(QuantArgs a, int64_t Q) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t cpr = a.cols >> 3;
  const bool dense = a.ld_x == a.cols;
  const int64_t q0 = wave * (64 * kU) + lane;
  Raw<XDT> raw[kU];
  load_slabs<XDT>(a.x, q0, Q, cpr, a.ld_x, dense, raw);
  // q0 is even: the lane's half of its Hadamard group is lane & 1 in every slab
  SignBits<XDT> sg;
  if constexpr (RHT) sg = rht_sign_bits<XDT>(a.sign_mask, lane & 1u);
  Enc<FMT> enc[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t q = q0 + 64 * u;
    float v[8];
    if constexpr (RHT) apply_signs<XDT>(raw[u], sg);
    widen<XDT>(raw[u], v);
    if constexpr (RHT) rht_forward_signed(v, lane & 1u);
    encode_mx<FMT, SR>(a, q, v, enc[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) store_enc<FMT>(a, q0 + 64 * u, Q, lane, 4u, enc[u]);
}

// ---- MX quantizer writing the matrix-instruction tile layout --------------
// One wave per 8 rows x 64 NT columns (NT = 4 load instructions, a quarter
// of a 1024-column scale group).  Load instruction t of the wave covers
// columns 64 t .. 64 t + 63 of its 8 rows (t counted from the start of the
// scale group): lane 8 i + k holds chunk k (8 elements) of row i, so an MX
// block is a lane quad and a Hadamard group a lane pair, exactly as in the
// row layout, and the element arithmetic is encode_mx's (random stream
// indexed by the chunk's row-major position).  Each load instruction reads
// 8 rows x 128 contiguous bytes, and the codes of one instruction fill whole
// 128-byte runs of the code tile (two for FP4, four for FP8).  The first
// lane of a quad sees blocks of one parity of its row, which are
// consecutive bytes of its row's 16-byte word of the scale tile: the NT = 4
// bytes go out in one 32-bit store.
// Load instructions per wave: 4 (a quarter of a scale group) measured faster
// than 8 or 16 for both roundings -- more waves in flight, which SR's
// branchy encoders need most.
constexpr int kTiledNT = 4;

// One wave of the tile-layout quantizer (wave index within its tensor).
template <int XDT, int FMT, bool SR, bool RHT>
__device__ __attribute__((always_inline)) inline void quant_tiled_wave(const QuantArgs& a, int64_t wave) {
  constexpr int NT = kTiledNT;
  constexpr int kParts = 16 / NT;  // waves per scale group and row octet
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t gpr = a.cols >> 10;  // scale groups per row
  const int64_t wpr = gpr * kParts;  // waves per row octet
  const int64_t R8 = wave / wpr, rem = wave - R8 * wpr;
  const int64_t G = rem / kParts;
  const int t0 = (int)(rem - G * kParts) * NT;  // first instruction index in the group
  const uint32_t i = lane >> 3, k = lane & 7u;
  const int64_t row = 8 * R8 + i;
  const int64_t col0 = G * 1024 + 64 * t0 + 8 * k;  // the lane's element in the wave's instruction 0
  Raw<XDT> raw[NT];
  {
    const int64_t xoff = row * a.ld_x + col0;
#pragma unroll
    for (int t = 0; t < NT; ++t) load_raw<XDT>(a.x, xoff + 64 * t, raw[t]);
  }
  const int64_t q0 = (row * a.cols + col0) >> 3;
  SignBits<XDT> sg;
  if constexpr (RHT) sg = rht_sign_bits<XDT>(a.sign_mask, k & 1u);
  Enc<FMT> enc[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    float v[8];
    if constexpr (RHT) apply_signs<XDT>(raw[t], sg);
    widen<XDT>(raw[t], v);
    if constexpr (RHT) rht_forward_signed(v, k & 1u);
    encode_mx<FMT, SR>(a, q0 + 8 * t, v, enc[t]);
  }
  // Codes: instruction index T = t0 + t in the group.  FP4: code byte
  // 512 G + 32 T + 4 k of the row, i.e. code tile 4 G + T/4, chunk
  // 2 (T%4) + k/4, byte 4 (k%4).  FP8: code byte 1024 G + 64 T + 8 k, i.e.
  // code tile 8 G + T/2, chunk 4 (T%2) + k/2, byte 8 (k%2).
  const uint32_t r = (uint32_t)row & 31u;
  constexpr bool k8 = MxFmt<FMT>::bits == 8;  // E4M3 or E5M2 (else E2M1)
  const int64_t row_bytes = k8 ? a.cols : a.cols >> 1;
  uint8_t* cbase = a.codes + ((row >> 5) * (row_bytes >> 7) + G * (k8 ? 8 : 4)) * 4096;
  if constexpr (k8) {
    cbase += (k >> 2) * 1024u + (((k >> 1) & 1u) * 32u + r) * 16u + 8u * (k & 1u) + (t0 >> 1) * 4096;
#pragma unroll
    for (int t = 0; t < NT; ++t)  // t0 is even
      *reinterpret_cast<uint2*>(cbase + (t >> 1) * 4096 + (t & 1) * 2048) = make_uint2(enc[t].w[0], enc[t].w[1]);
  } else {
    cbase += ((k >> 2) * 32u + r) * 16u + 4u * (k & 3u) + (t0 >> 2) * 4096;
#pragma unroll
    for (int t = 0; t < NT; ++t)  // t0 is a multiple of 4
      *reinterpret_cast<uint32_t*>(cbase + (t >> 2) * 4096 + (t & 3) * 1024) = enc[t].w[0];
  }
  // Scales: block 32 G + 2 T + k/4 of the row is byte T of the word at
  // ((k/4) * 32 + r) * 16 in scale tile G of the row tile.  (Restaging the
  // 4 waves' parts through LDS into whole 16-byte words measured slower: the
  // workgroup barrier costs more than the 4-byte stores.)
  if ((k & 3u) == 0) {
    uint32_t w[NT / 4];
#pragma unroll
    for (int d = 0; d < NT / 4; ++d)
      w[d] = enc[4 * d].sc | (enc[4 * d + 1].sc << 8) | (enc[4 * d + 2].sc << 16) | (enc[4 * d + 3].sc << 24);
    static_assert(NT == 4, "one 32-bit scale store per quad");
    *reinterpret_cast<uint32_t*>(a.scales + ((row >> 5) * gpr + G) * 1024 + ((k >> 2) * 32u + r) * 16u + t0) = w[0];
  }
}

template <int XDT, int FMT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_mx_tiled(QuantArgs a, int64_t nwaves) {
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  if (wave >= nwaves) return;  // whole waves
  quant_tiled_wave<XDT, FMT, SR, RHT>(a, wave);
}

// Several tensors in one launch (same format, input dtype, rounding and
// transform): the waves of job j are [first[j], first[j+1]).  Every job has
// a multiple of 4 waves, so a workgroup never spans two jobs.
// The job is chosen from the workgroup's first wave, so the choice is
// uniform and its arguments come in through scalar loads.
template <int XDT, int FMT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_mx_tiled_batch(QuantBatch b) {
  const int64_t wave0 = (int64_t)blockIdx.x * (kThreads / 64);
  int j = 0;
#pragma unroll
  for (int k = 1; k < kMaxBatch; ++k) j += (k < b.n && wave0 >= b.first[k]) ? 1 : 0;
  const int64_t wave = wave0 + (threadIdx.x >> 6);
  if (wave >= b.first[b.n]) return;
  quant_tiled_wave<XDT, FMT, SR, RHT>(b.job[j], wave - b.first[j]);
}

template <int XDT, int FMT, bool SR, bool RHT>
hipError_t quant_mx_tiled_t(const QuantArgs& a, hipStream_t s) {
  const int64_t nwaves = (a.rows / 8) * (a.cols / (64 * kTiledNT));
  const int64_t blocks = (nwaves + 3) / 4;
  hipLaunchKernelGGL((k_quant_mx_tiled<XDT, FMT, SR, RHT>), dim3((uint32_t)blocks), dim3(kThreads), 0, s, a, nwaves);
  return hipGetLastError();
}
template <int XDT, int FMT, bool SR, bool RHT>
hipError_t quant_mx_tiled_batch_t(const QuantBatch& b, hipStream_t s) {
  const int64_t blocks = (b.first[b.n] + 3) / 4;
  hipLaunchKernelGGL((k_quant_mx_tiled_batch<XDT, FMT, SR, RHT>), dim3((uint32_t)blocks), dim3(kThreads), 0, s, b);
  return hipGetLastError();
}
template <int XDT, int FMT>
hipError_t quant_mx_tiled_batch_d(const QuantBatch& b, hipStream_t s) {
  const QuantArgs& a = b.job[0];
  if (a.sr) return a.rht ? quant_mx_tiled_batch_t<XDT, FMT, true, true>(b, s) : quant_mx_tiled_batch_t<XDT, FMT, true, false>(b, s);
  return a.rht ? quant_mx_tiled_batch_t<XDT, FMT, false, true>(b, s) : quant_mx_tiled_batch_t<XDT, FMT, false, false>(b, s);
}

template <int XDT, int FMT>
hipError_t quant_mx_tiled_d(const QuantArgs& a, hipStream_t s) {
  if (a.sr) return a.rht ? quant_mx_tiled_t<XDT, FMT, true, true>(a, s) : quant_mx_tiled_t<XDT, FMT, true, false>(a, s);
  return a.rht ? quant_mx_tiled_t<XDT, FMT, false, true>(a, s) : quant_mx_tiled_t<XDT, FMT, false, false>(a, s);
}

// ---- NVFP4 (E4M3 per 16 + FP32 per tensor) quantizer ----------------------
// Per 16-block: q = fl(a_b / d) (d = 6 S, or 4 S for the second Four Over Six
// candidate), sb = E4M3 RNE of q, rcp = 1 / fl(dec(sb) S).  Both FP32
// divisions are replaced by exact equivalents:
//  * rcp comes from a per-workgroup table of the reciprocals for the 127
//    finite E4M3 magnitudes, filled with the same FP32 operations (code 0, and
//    a product that overflows to +Inf, give 0);
//  * q is the product a_b fl(1/d) corrected once by its residual
//    a_b - q0 d, which a fused multiply-add forms exactly (Markstein's
//    correction step: the rounded result is the correctly rounded quotient
//    when fl(1/d) is the rounded reciprocal and no step under- or
//    overflows).  For 2^-80 <= d <= 2^80 the residual of every quotient that
//    can round to a nonzero E4M3 code (q >= 2^-11) is exact, smaller quotients
//    (code 0 either way) stay below 2^-10, and a product past the FP32 range
//    keeps its +Inf.  Other divisors take the division.
struct NvDiv {
  float d, rd;
  bool exact;
};

__device__ inline NvDiv nv_div(float d) {
#pragma clang fp contract(off)
  NvDiv k;
  k.d = d;
  k.rd = 1.0f / d;
  k.exact = d >= 0x1p-80f && d <= 0x1p80f;
  return k;
}

__device__ inline float nv_quot(float m, const NvDiv& k) {
#pragma clang fp contract(off)
  if (!k.exact) return m / k.d;
  const float q0 = m * k.rd;
  const float r = __builtin_fmaf(-q0, k.d, m);
  const float q1 = __builtin_fmaf(r, k.rd, q0);
  return q1 == q1 ? q1 : q0;  // NaN: the product overflowed (or m is not finite)
}

// The reciprocal table of one tensor scale S, filled by the first 128
// threads of the workgroup (all of its threads call this).
constexpr int kNvRcp = 128;

__device__ inline void nv_fill_recips(float* tab, float S) {
#pragma clang fp contract(off)
  const uint32_t c = threadIdx.x;
  if (c < (uint32_t)kNvRcp) {
    float r = 0.0f;
    if (c < 0x7Fu) {
      const float dsb = e4m3_mag_value(c);
      if (dsb != 0.0f) {
        const float p = dsb * S;
        r = 1.0f / p;
      }
    }
    tab[c] = r;
  }
  __syncthreads();
}

// Codes of finite quotients are at most 0x7E; the mask keeps the read in the
// table for any input.
__device__ inline float nv_recip(const float* tab, uint32_t sb) { return tab[sb & 0x7Fu]; }

// For S < 2^-100 a reciprocal 1 / fl(dec(sb) S) can overflow to +Inf, and a
// zero element's product 0 * Inf is NaN: zero elements keep their +-0, the
// code every finite reciprocal gives them.  Infinite products need nothing:
// the conversions saturate +-Inf to +-6.  (`tiny` is kernel-wide, so this is
// a scalar branch.)
constexpr float kNvTinyS = 0x1p-100f;

__device__ inline void nv_keep_zeros(bool tiny, const float v[8], float y[8]) {
  if (tiny) {
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] == 0.0f ? v[i] : y[i];
  }
}

template <bool SR>
__device__ inline void encode_nv(const QuantArgs& a, const float* rtab, const NvDiv& dk, bool tiny,
                                 int64_t q, const float v[8], Enc<FMT_NVFP4>& e) {
#pragma clang fp contract(off)
  uint32_t m = max_abs_bits(v);
  uint32_t o = dpp_xor1(m);
  m = o > m ? o : m;
  const uint32_t sb = e4m3_rne_mag(nv_quot(u2f(m), dk));
  // rcp = 0 (a zero block scale) gives y = +-0 and so the codes +-0
  const float rcp = nv_recip(rtab, sb);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = v[i] * rcp;
  nv_keep_zeros(tiny, v, y);
  if constexpr (!SR) {
    e.w[0] = pack_e2m1_rne(y);
  } else {
    const u32x4 w = rand_words(a.seed, a.counter, (uint64_t)q);
    e.w[0] = pack_e2m1_sr_words(y, w.x, w.y, w.z, w.w);  // SR on the conversion instruction
  }
  e.sc = sb;
}

// Four Over Six ("Thinking Machines ... Inkling 2 Small", section "A
// precision choice for each stage": a choice between block scales that
// lowers the quantization error).  The block is encoded with its maximum
// mapped to 6 (d6 = 6 S, the format's rule) and to 4 (d4 = 4 S); the one
// whose decoded values fp32(e2m1 * e4m3 * S) have the smaller squared error
// -- the exact sum, with no rounding -- is kept, 6 on a tie.  Round-to-nearest
// only.
//
// Each lane of the pair first sums the squares of its 8 differences in FP32
// (fused multiply-adds) and the pair adds the halves.  Each sum is then
// within 11 * 2^-24 of the exact one (relative), plus at most 2^-120 from
// underflow, so when the two sums differ by more than 2^-18 of their total
// plus 2^-100, their order is the exact order.  Otherwise (and whenever a sum
// is not finite) the pair compares the exact errors with integers
// (nv46_exact_four), which near ties make rare.
// The 8 codes are decoded by the hardware conversion (scale 1: exact), two
// per instruction, byte b giving elements 2b (low nibble) and 2b + 1.
__device__ inline void nv_decode8(uint32_t w, float dsb, float S, float xh[8]) {
#pragma clang fp contract(off)
  typedef float v2f __attribute__((ext_vector_type(2)));
  v2f q[4];
  q[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  q[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  q[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  q[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) xh[i] = (q[i >> 1][i & 1] * dsb) * S;  // first product exact
}

__device__ inline float nv_sq_err(const float v[8], uint32_t w, float dsb, float S) {
#pragma clang fp contract(off)
  float xh[8];
  nv_decode8(w, dsb, S, xh);
  float acc = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float d = v[i] - xh[i];
    acc = __builtin_fmaf(d, d, acc);
  }
  return acc;
}

// Exact comparison: true when error(4) < error(6).  error(6) - error(4) is the
// sum over the block of (xh4 - xh6) (2 x - xh6 - xh4), since
// (x - a)^2 - (x - b)^2 = (b - a)(2 x - a - b); an element with xh6 == xh4
// adds nothing.  Any other element has a nonzero code under one candidate, so
// |x| > ab / 36 (a nonzero code needs |x| r > 1/4, and the decoded block
// scale is at least 2/3 of its target ab / (k S), k <= 6), and its decoded
// values lie below 3 ab.  With E = floor(log2 ab), every value involved is
// then a multiple of u = max(2^(E - 29), 2^-149) below 2^32 u, so both
// factors divided by u are integers below 2^34, formed exactly in FP64; their
// product is below 2^68 and the block's sum below 2^72: exact in 128 bits.
__device__ inline bool nv46_exact_four(const float v[8], uint32_t w6, float dsb6, uint32_t w4,
                                       float dsb4, float S, float ab) {
  float x6[8], x4[8];
  nv_decode8(w6, dsb6, S, x6);
  nv_decode8(w4, dsb4, S, x4);
  const int eb = (int)((__builtin_bit_cast(uint32_t, ab) >> 23) & 0xFFu);
  const int eu = eb == 0 ? -149 : (eb - 127 - 29 > -149 ? eb - 127 - 29 : -149);
  __int128 sum = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double a = (double)x4[i] - (double)x6[i];
    const double b = (2.0 * (double)v[i] - (double)x6[i]) - (double)x4[i];
    const int64_t ia = (int64_t)__builtin_ldexp(a, -eu);
    const int64_t ib = (int64_t)__builtin_ldexp(b, -eu);
    sum += (__int128)ia * (__int128)ib;
  }
  // add the other lane's sum (addition commutes: both lanes get the same)
  const unsigned __int128 us = (unsigned __int128)sum;
  const uint32_t p0 = dpp_xor1((uint32_t)us), p1 = dpp_xor1((uint32_t)(us >> 32)),
                 p2 = dpp_xor1((uint32_t)(us >> 64)), p3 = dpp_xor1((uint32_t)(us >> 96));
  const unsigned __int128 other = ((unsigned __int128)p3 << 96) | ((unsigned __int128)p2 << 64) |
                                  ((unsigned __int128)p1 << 32) | (unsigned __int128)p0;
  return (__int128)(us + other) > 0;
}

__device__ inline void encode_nv46(float S, const float* rtab, const NvDiv& d6, const NvDiv& d4,
                                   bool tiny, const float v[8], Enc<FMT_NVFP4>& e) {
#pragma clang fp contract(off)
  uint32_t m = max_abs_bits(v);
  uint32_t o = dpp_xor1(m);
  m = o > m ? o : m;
  const float ab = u2f(m);
  uint32_t sb[2], w[2];
  float err[2], dsbk[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    sb[k] = e4m3_rne_mag(nv_quot(ab, k == 0 ? d6 : d4));
    const float dsb = e4m3_mag_value(sb[k]);
    dsbk[k] = dsb;
    const float rcp = nv_recip(rtab, sb[k]);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * rcp;
    nv_keep_zeros(tiny, v, y);
    w[k] = pack_e2m1_rne(y);
    const float part = nv_sq_err(v, w[k], dsb, S);
    err[k] = part + dpp_xor1f(part);  // addition commutes: both lanes get the same sum
  }
  bool four = err[1] < err[0];
  // both lanes of the pair hold the same sums, so they take this branch together
  const float gap = __builtin_fabsf(err[0] - err[1]);
  if (!(gap > (err[0] + err[1]) * 0x1p-18f + 0x1p-100f))
    four = nv46_exact_four(v, w[0], dsbk[0], w[1], dsbk[1], S, ab);
  e.w[0] = four ? w[1] : w[0];
  e.sc = four ? sb[1] : sb[0];
}

// One wave of the 1-D NVFP4 quantizer (wave index within its tensor; wave 0
// publishes the tensor scale).
template <int XDT, bool SR, bool RHT, bool F46>
__device__ __attribute__((always_inline)) inline void nv1d_wave(const QuantArgs& a, int64_t Q, int64_t wave) {
#pragma clang fp contract(off)
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t cpr = a.cols >> 3;
  const bool dense = a.ld_x == a.cols;
  const int64_t q0 = wave * (64 * kU) + lane;
  Raw<XDT> raw[kU];
  load_slabs<XDT>(a.x, q0, Q, cpr, a.ld_x, dense, raw);
  const float T = *a.amax;
  const float S = (T == 0.0f) ? 1.0f : T / 2688.0f;
  if (wave == 0 && lane == 0) *a.tensor_scale = S;
  __shared__ float rtab[kNvRcp];
  nv_fill_recips(rtab, S);
  const NvDiv d6 = nv_div(6.0f * S);
  NvDiv d4 = d6;
  if constexpr (F46) d4 = nv_div(4.0f * S);
  const bool tiny = S < kNvTinyS;
  // q0 is even, so the lane's half of its Hadamard group is lane & 1 in every slab
  SignBits<XDT> sg;
  if constexpr (RHT) sg = rht_sign_bits<XDT>(a.sign_mask, lane & 1u);
  Enc<FMT_NVFP4> enc[kU];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t q = q0 + 64 * u;
    float v[8];
    if constexpr (RHT) apply_signs<XDT>(raw[u], sg);
    widen<XDT>(raw[u], v);
    if constexpr (RHT) rht_forward_signed(v, lane & 1u);
    if constexpr (F46) encode_nv46(S, rtab, d6, d4, tiny, v, enc[u]);
    else encode_nv<SR>(a, rtab, d6, tiny, q, v, enc[u]);
  }
#pragma unroll
  for (int u = 0; u < kU; ++u) store_enc<FMT_NVFP4>(a, q0 + 64 * u, Q, lane, 2u, enc[u]);
}

template <int XDT, bool SR, bool RHT, bool F46>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4(QuantArgs a, int64_t Q) {
  nv1d_wave<XDT, SR, RHT, F46>(a, Q, ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6);
}

// Empty tensor: only the tensor scale is published.
__global__ void k_nv_scale_only(const float* amax, float* tensor_scale) {
#pragma clang fp contract(off)
  const float T = *amax;
  *tensor_scale = (T == 0.0f) ? 1.0f : T / 2688.0f;
}

// ---- NVFP4 with 2-D blocks --------------------------------------------------
// "Microscaling (MX) and block-scaled 4-bit formats", section "NVFP4":
// two-dimensional weight quantisation, so that the forward and the backward
// (transposed) use see the same values.  One E4M3 block scale per tile of
// 16 rows x 16 columns, from the tile's max |x| (the last band of rows may be
// shorter), stored in each of the tile's rows so the tensor keeps the
// ordinary row layout; elements are encoded as in the 1-D quantizer.
// One wave per band of 16 rows x 64 k2dGroups columns: lane 8 i + k holds
// chunk k (8 elements) of rows i and i + 8 of each 64-column group, so each
// load instruction reads 8 rows x 128 contiguous bytes (BF16) and a wave
// writes 32 k2dGroups contiguous code bytes per row.  A tile is the 16 lanes
// with the same k >> 1 over both row halves: the in-lane max over the
// halves, then lane exchanges at distance 1, 8, 16 and 32.
constexpr int k2dGroups = 4;  // measured: 2 groups (64-byte code runs) ran at the same speed
constexpr int k2dCols = 64 * k2dGroups;
constexpr int k2dLoads = 2 * k2dGroups;

// One wave of the 2-D quantizer (wave index within its tensor).
template <int XDT, bool SR, bool RHT>
__device__ __attribute__((always_inline)) inline void nv2d_wave(const QuantArgs& a, int64_t nwaves,
                                                                int64_t groups_per_band, int64_t wave) {
#pragma clang fp contract(off)
  const uint32_t lane = threadIdx.x & 63u;
  const float T = *a.amax;
  const float S = (T == 0.0f) ? 1.0f : T / 2688.0f;
  __shared__ float rtab[kNvRcp];
  nv_fill_recips(rtab, S);  // before any wave of the workgroup leaves
  if (wave >= nwaves) return;
  const int64_t band = wave / groups_per_band;
  const int64_t G = wave - band * groups_per_band;
  const uint32_t i = lane >> 3, k = lane & 7u;
  const int64_t rows = a.rows, cols = a.cols;
  // load u: row half h = u & 1, column group c = u >> 1
  int64_t row[k2dLoads], col[k2dLoads];
  bool ok[k2dLoads];
  Raw<XDT> raw[k2dLoads];
#pragma unroll
  for (int u = 0; u < k2dLoads; ++u) {
    row[u] = band * 16 + 8 * (u & 1) + i;
    col[u] = G * k2dCols + 64 * (u >> 1) + 8 * k;
    ok[u] = row[u] < rows && col[u] < cols;
    const int64_t r = row[u] < rows ? row[u] : rows - 1;
    const int64_t c = col[u] < cols ? col[u] : cols - 8;
    load_raw<XDT>(a.x, r * a.ld_x + c, raw[u]);
  }
  if (wave == 0 && lane == 0) *a.tensor_scale = S;
  const NvDiv d6 = nv_div(6.0f * S);
  const bool tiny = S < kNvTinyS;
  float v[k2dLoads][8];
  uint32_t m[k2dGroups];
#pragma unroll
  for (int c = 0; c < k2dGroups; ++c) m[c] = 0u;
  SignBits<XDT> sg;
  if constexpr (RHT) sg = rht_sign_bits<XDT>(a.sign_mask, k & 1u);
#pragma unroll
  for (int u = 0; u < k2dLoads; ++u) {
    if constexpr (RHT) apply_signs<XDT>(raw[u], sg);
    widen<XDT>(raw[u], v[u]);
    if constexpr (RHT) rht_forward_signed(v[u], k & 1u);
    const uint32_t b = ok[u] ? max_abs_bits(v[u]) : 0u;
    m[u >> 1] = b > m[u >> 1] ? b : m[u >> 1];
  }
#pragma unroll
  for (int c = 0; c < k2dGroups; ++c) {
    uint32_t t = m[c];
    uint32_t o = dpp_xor1(t);
    t = o > t ? o : t;
    o = lane_read(t, lane ^ 8u);
    t = o > t ? o : t;
    o = lane_read(t, lane ^ 16u);
    t = o > t ? o : t;
    o = lane_read(t, lane ^ 32u);
    m[c] = o > t ? o : t;
  }
  const int64_t spr = cols >> 4;  // scale bytes per row
  // Full groups (cols a multiple of 64 k2dGroups): every chunk of the wave
  // is in range column-wise and the wave's code bytes of a row are one
  // 32 k2dGroups-byte run, its scale bytes one 4 k2dGroups-byte run.
  const bool full = (cols % k2dCols) == 0;
  uint32_t w[k2dLoads], sw[k2dLoads];
#pragma unroll
  for (int u = 0; u < k2dLoads; ++u) {
    const uint32_t sb = e4m3_rne_mag(nv_quot(u2f(m[u >> 1]), d6));
    const float rcp = nv_recip(rtab, sb);
    float y[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) y[j] = v[u][j] * rcp;
    nv_keep_zeros(tiny, v[u], y);
    if constexpr (!SR) {
      w[u] = pack_e2m1_rne(y);
    } else {
      const u32x4 rw = rand_words(a.seed, a.counter, (uint64_t)((row[u] * cols + col[u]) >> 3));
      w[u] = pack_e2m1_sr_words(y, rw.x, rw.y, rw.z, rw.w);  // SR on the conversion instruction
    }
    // lane 8 i + 2 p holds block p of its row's 64-column group: gather the
    // group's 4 scale bytes into lane 8 i
    const uint32_t s1 = lane_read(sb, lane + 2u), s2 = lane_read(sb, lane + 4u),
                   s3 = lane_read(sb, lane + 6u);
    sw[u] = sb | (s1 << 8) | (s2 << 16) | (s3 << 24);
    if (!full && ok[u]) {
      *reinterpret_cast<uint32_t*>(a.codes + row[u] * (cols >> 1) + (col[u] >> 1)) = w[u];
      uint8_t* sp = a.scales + row[u] * spr + (col[u] >> 4);
      if ((spr & 3) == 0) {
        if (k == 0u) *reinterpret_cast<uint32_t*>(sp) = sw[u];
      } else if ((k & 1u) == 0u) {
        *sp = (uint8_t)sb;
      }
    }
  }
  if (!full) return;
  // Full groups: the codes are restaged through LDS so that every store
  // instruction writes 8 rows x 128 contiguous bytes, and lane 8 i stores its
  // row's scale run with one 16-byte store.  Each wave uses its own 2 KB of
  // LDS; LDS operations of one wave complete in order.
  static_assert(k2dGroups == 4, "the restaging assumes 128 code bytes per row");
  __shared__ uint32_t stage[kThreads / 64][16][32];
  uint32_t (*st)[32] = stage[threadIdx.x >> 6];
#pragma unroll
  for (int u = 0; u < k2dLoads; ++u) st[8 * (u & 1) + i][8 * (u >> 1) + k] = w[u];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t r = band * 16 + 8 * h + i;
    const uint4 q = *reinterpret_cast<const uint4*>(&st[8 * h + i][4 * k]);
    if (r < rows) {
      *reinterpret_cast<uint4*>(a.codes + r * (cols >> 1) + G * (k2dCols / 2) + 16 * k) = q;
      if (k == 0u)
        *reinterpret_cast<uint4*>(a.scales + r * spr + G * (k2dCols / 16)) =
            make_uint4(sw[h], sw[2 + h], sw[4 + h], sw[6 + h]);
    }
  }
}

template <int XDT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4_2d(QuantArgs a, int64_t nwaves,
                                                             int64_t groups_per_band) {
  nv2d_wave<XDT, SR, RHT>(a, nwaves, groups_per_band, ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6);
}

// ---- per-tensor amax ------------------------------------------------------
__global__ void k_zero_f32(float* p) { *p = 0.0f; }

// Grid-stride over groups of kU slabs with 1024-lane workgroups and a grid
// of at most one workgroup per CU: every workgroup ends with one atomic max
// on the same word, and those serialize, so the count is kept at 256.
constexpr int kAmaxThreads = 1024;

// Max |x| bits over the chunks of waves wave, wave + nwaves, ... of a tensor,
// reduced over the workgroup into one atomic max on *amax.
template <int XDT, bool RHT>
__device__ __attribute__((always_inline)) inline void amax_part(const void* x, int64_t cols, int64_t ld_x,
                                                                int64_t Q, uint32_t sign_mask, float* amax,
                                                                int64_t wave, int64_t nwaves) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t cpr = cols >> 3;
  const bool dense = ld_x == cols;
  uint32_t m = 0;
  // every q0 - lane is a multiple of 64: the lane's half of its group is lane & 1
  SignBits<XDT> sg;
  if constexpr (RHT) sg = rht_sign_bits<XDT>(sign_mask, lane & 1u);
  for (int64_t q0 = wave * (64 * kU) + lane; q0 - lane < Q; q0 += nwaves * (64 * kU)) {
    Raw<XDT> raw[kU];
    load_slabs<XDT>(x, q0, Q, cpr, ld_x, dense, raw);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      float v[8];
      if constexpr (RHT) apply_signs<XDT>(raw[u], sg);
      widen<XDT>(raw[u], v);
      if constexpr (RHT) rht_forward_signed(v, lane & 1u);
      // Chunks past the end reload chunk Q - 1 and are left out: after the
      // Hadamard transform a pair of them is not a group of the input.
      const uint32_t b = q0 + 64 * u < Q ? max_abs_bits(v) : 0u;
      m = b > m ? b : m;
    }
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[kAmaxThreads / 64];
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = red[0];
    for (int i = 1; i < kAmaxThreads / 64; ++i) t = red[i] > t ? red[i] : t;
    // non-negative floats order like their bit patterns
    atomicMax(reinterpret_cast<unsigned int*>(amax), t);
  }
}

template <int XDT, bool RHT>
__global__ __launch_bounds__(kAmaxThreads) void k_amax(const void* x, int64_t cols, int64_t ld_x,
                                                       int64_t Q, uint32_t sign_mask, float* amax) {
  amax_part<XDT, RHT>(x, cols, ld_x, Q, sign_mask, amax, ((int64_t)blockIdx.x * kAmaxThreads + threadIdx.x) >> 6,
                      ((int64_t)gridDim.x * kAmaxThreads) >> 6);
}

// ---- several NVFP4 tensors per launch --------------------------------------
// Jobs with the same input dtype, rounding, transform and variant share one
// launch per pass: zero the amax slots, the per-tensor amax (each job its own
// slot), then the encode.  first[j] counts workgroups; a workgroup picks its
// job from its index (a uniform choice, so the job's arguments come in
// through scalar loads) and never spans two jobs.
__global__ void k_zero_amax_batch(NvBatch b) {
  if (threadIdx.x < (uint32_t)b.n) *b.job[threadIdx.x].amax = 0.0f;
}

__device__ inline int batch_job(const NvBatch& b, int64_t wg) {
  int j = 0;
#pragma unroll
  for (int k = 1; k < kMaxNvBatch; ++k) j += (k < b.n && wg >= b.first[k]) ? 1 : 0;
  return j;
}

template <int XDT, bool RHT>
__global__ __launch_bounds__(kAmaxThreads) void k_amax_batch(NvBatch b) {
  const int j = batch_job(b, blockIdx.x);
  const QuantArgs& a = b.job[j];
  const int64_t wgs = b.first[j + 1] - b.first[j];
  amax_part<XDT, RHT>(a.x, a.cols, a.ld_x, a.rows * (a.cols >> 3), a.sign_mask, a.amax,
                      ((blockIdx.x - b.first[j]) * kAmaxThreads + threadIdx.x) >> 6, (wgs * kAmaxThreads) >> 6);
}

template <int XDT, bool SR, bool RHT, bool F46>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4_batch(NvBatch b) {
  const int j = batch_job(b, blockIdx.x);
  const QuantArgs& a = b.job[j];
  // surplus waves of the job's last workgroup find no chunk (q >= Q) and
  // store nothing
  nv1d_wave<XDT, SR, RHT, F46>(a, a.rows * (a.cols >> 3),
                               ((blockIdx.x - b.first[j]) * kThreads + threadIdx.x) >> 6);
}

template <int XDT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4_2d_batch(NvBatch b) {
  const int j = batch_job(b, blockIdx.x);
  const QuantArgs& a = b.job[j];
  const int64_t gpb = (a.cols + k2dCols - 1) / k2dCols;
  nv2d_wave<XDT, SR, RHT>(a, (a.rows + 15) / 16 * gpb, gpb,
                          ((blockIdx.x - b.first[j]) * kThreads + threadIdx.x) >> 6);
}

// ---- decoder ----------------------------------------------------------------
template <int FMT, int YDT, bool RHT>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* codes, const uint8_t* scales,
                                                      const float* tensor_scale, int64_t cols,
                                                      void* y, int64_t ld_y, int64_t Q,
                                                      uint32_t sign_mask, bool tiled) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const float S = FMT == FMT_NVFP4 ? *tensor_scale : 1.0f;
  const int64_t cpr = cols >> 3;
  const bool dense = ld_y == cols;
  const int64_t q0 = wave * (64 * kU) + lane;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t q = q0 + 64 * u;
    const bool valid = q < Q;
    float v[8];
    if (valid) {
      uint32_t cw[8];
      // tiled layout (MX only): code and scale offsets of this chunk
      constexpr int kBits = FMT == FMT_NVFP4 ? 4 : (int)MxFmt<FMT>::bits;
      int64_t coff = q * kBits, soff = q >> 2;
      if constexpr (FMT == FMT_MXFP8 || FMT == FMT_MXFP4 || FMT == FMT_MXFP8_E5M2) {
        if (tiled) {
          const int64_t row = q / cpr, c8 = q - row * cpr;
          coff = tiled_code_off(row, c8 * kBits, cpr * kBits);
          soff = tiled_scale_off(row, c8 >> 2, cols);
        }
      }
      if constexpr (kBits == 8) {
        uint2 p = *reinterpret_cast<const uint2*>(codes + coff);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cw[i] = (p.x >> (8 * i)) & 0xFFu;
          cw[4 + i] = (p.y >> (8 * i)) & 0xFFu;
        }
      } else if constexpr (kBits == 6) {  // element i at bits 6 i of the chunk's 6 bytes
        const uint16_t* p = reinterpret_cast<const uint16_t*>(codes + coff);
        const uint64_t b = (uint64_t)p[0] | ((uint64_t)p[1] << 16) | ((uint64_t)p[2] << 32);
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[i] = (uint32_t)(b >> (6 * i)) & 0x3Fu;
      } else {
        uint32_t p = *reinterpret_cast<const uint32_t*>(codes + coff);
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[i] = (p >> (4 * i)) & 0xFu;
      }
      if constexpr (FMT == FMT_NVFP4) {
        const float sbv = e4m3_mag_value(scales[q >> 1]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (e2m1_value(cw[i]) * sbv) * S;  // first product exact
      } else {
        const uint32_t sc = scales[soff];
        // 2^(sc-127) as FP32 (sc = 0 is the subnormal 2^-127); 0xFF is NaN
        const float X = sc == 0xFFu ? __builtin_nanf("") : (sc == 0u ? u2f(0x00400000u) : u2f(sc << 23));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float e;
          if constexpr (FMT == FMT_MXFP8) {
            const uint32_t mag = cw[i] & 0x7Fu;
            e = mag == 0x7Fu ? __builtin_nanf("") : e4m3_mag_value(mag);
            if (cw[i] & 0x80u) e = -e;
          } else if constexpr (FMT == FMT_MXFP4) {
            e = e2m1_value(cw[i]);
          } else if constexpr (FMT == FMT_MXINT8) {
            e = int8_value(cw[i]);
          } else if constexpr (FMT == FMT_MXFP8_E5M2) {
            e = e5m2_value(cw[i]);
          } else if constexpr (FMT == FMT_MXFP6_E3M2) {
            e = fp6_value<E3M2>(cw[i]);
          } else {
            e = fp6_value<E2M3>(cw[i]);
          }
          v[i] = e * X;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    if constexpr (RHT) rht_inverse(v, sign_mask, (uint32_t)(q & 1));
    if (valid) store8<YDT>(y, chunk_offset(q, cpr, ld_y, dense), v);
  }
}

// ---- standalone Hadamard ----------------------------------------------------
template <int XDT, int YDT, bool INV>
__global__ __launch_bounds__(kThreads) void k_hadamard(const void* x, void* y, int64_t cols,
                                                       int64_t Q, uint32_t sign_mask) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t q0 = wave * (64 * kU) + lane;
  Raw<XDT> raw[kU];
  load_slabs<XDT>(x, q0, Q, cols >> 3, cols, true, raw);
  SignBits<XDT> sg;  // q0 is even: the lane's half is lane & 1
  if constexpr (!INV) sg = rht_sign_bits<XDT>(sign_mask, lane & 1u);
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int64_t q = q0 + 64 * u;
    float v[8];
    if constexpr (!INV) apply_signs<XDT>(raw[u], sg);
    widen<XDT>(raw[u], v);
    if constexpr (INV) rht_inverse(v, sign_mask, lane & 1u);
    else rht_forward_signed(v, lane & 1u);
    if (q < Q) store8<YDT>(y, q * 8, v);
  }
}

// one wave per kU slabs, 4 waves per workgroup
int grid_for(int64_t Q) {
  const int64_t waves = (Q + 64 * kU - 1) / (64 * kU);
  const int64_t blocks = (waves + 3) / 4;
  return (int)(blocks < 1 ? 1 : blocks);
}

// grid of the grid-stride amax: at most 256 workgroups of 1024 lanes
int grid_for_amax(int64_t Q) {
  const int64_t waves = (Q + 64 * kU - 1) / (64 * kU);
  const int64_t b = (waves + kAmaxThreads / 64 - 1) / (kAmaxThreads / 64);
  return (int)(b > 256 ? 256 : (b < 1 ? 1 : b));
}

template <int XDT, int FMT, bool SR, bool RHT>
hipError_t quant_mx_t(const QuantArgs& a, int64_t Q, hipStream_t s) {
  hipLaunchKernelGGL((k_quant_mx<XDT, FMT, SR, RHT>), dim3(grid_for(Q)), dim3(kThreads), 0, s, a, Q);
  return hipGetLastError();
}
template <int XDT, bool SR, bool RHT>
hipError_t quant_nv_t(const QuantArgs& a, int64_t Q, hipStream_t s) {
  if (a.block2d) {
    const int64_t gpb = (a.cols + k2dCols - 1) / k2dCols;
    const int64_t nwaves = (a.rows + 15) / 16 * gpb;
    const int64_t blocks = (nwaves + kThreads / 64 - 1) / (kThreads / 64);
    hipLaunchKernelGGL((k_quant_nvfp4_2d<XDT, SR, RHT>), dim3((unsigned)blocks), dim3(kThreads), 0, s,
                       a, nwaves, gpb);
  } else if (a.four6) {
    if constexpr (SR) return hipErrorInvalidValue;  // rejected before launch
    hipLaunchKernelGGL((k_quant_nvfp4<XDT, false, RHT, true>), dim3(grid_for(Q)), dim3(kThreads), 0, s, a, Q);
  } else {
    hipLaunchKernelGGL((k_quant_nvfp4<XDT, SR, RHT, false>), dim3(grid_for(Q)), dim3(kThreads), 0, s, a, Q);
  }
  return hipGetLastError();
}
template <int XDT, int FMT>
hipError_t quant_mx_d(const QuantArgs& a, int64_t Q, hipStream_t s) {
  if (a.sr) return a.rht ? quant_mx_t<XDT, FMT, true, true>(a, Q, s) : quant_mx_t<XDT, FMT, true, false>(a, Q, s);
  return a.rht ? quant_mx_t<XDT, FMT, false, true>(a, Q, s) : quant_mx_t<XDT, FMT, false, false>(a, Q, s);
}
template <int XDT>
hipError_t quant_nv_d(const QuantArgs& a, int64_t Q, hipStream_t s) {
  if (a.sr) return a.rht ? quant_nv_t<XDT, true, true>(a, Q, s) : quant_nv_t<XDT, true, false>(a, Q, s);
  return a.rht ? quant_nv_t<XDT, false, true>(a, Q, s) : quant_nv_t<XDT, false, false>(a, Q, s);
}

}  // namespace

hipError_t launch_amax(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ld_x, bool rht,
                       uint32_t sign_mask, float* amax, hipStream_t s) {
  hipLaunchKernelGGL(k_zero_f32, dim3(1), dim3(1), 0, s, amax);
  const int64_t Q = rows * (cols / 8);
  if (Q == 0) return hipGetLastError();
  const int g = grid_for_amax(Q);
  if (xdt == DT_BF16) {
    if (rht) hipLaunchKernelGGL((k_amax<DT_BF16, true>), dim3(g), dim3(kAmaxThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
    else hipLaunchKernelGGL((k_amax<DT_BF16, false>), dim3(g), dim3(kAmaxThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
  } else {
    if (rht) hipLaunchKernelGGL((k_amax<DT_F32, true>), dim3(g), dim3(kAmaxThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
    else hipLaunchKernelGGL((k_amax<DT_F32, false>), dim3(g), dim3(kAmaxThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s) {
  const int64_t Q = a.rows * (a.cols / 8);
  if (a.fmt == FMT_NVFP4) {
    if (!a.amax_given) {
      hipError_t e = launch_amax(a.x, a.xdt, a.rows, a.cols, a.ld_x, a.rht, a.sign_mask, a.amax, s);
      if (e != hipSuccess) return e;
    }
    if (Q == 0) {
      // still publish S for an empty tensor
      hipLaunchKernelGGL(k_nv_scale_only, dim3(1), dim3(1), 0, s, a.amax, a.tensor_scale);
      return hipGetLastError();
    }
    return a.xdt == DT_BF16 ? quant_nv_d<DT_BF16>(a, Q, s) : quant_nv_d<DT_F32>(a, Q, s);
  }
  if (Q == 0) return hipSuccess;
  if (a.tiled) {
    if (a.fmt == FMT_MXFP8)
      return a.xdt == DT_BF16 ? quant_mx_tiled_d<DT_BF16, FMT_MXFP8>(a, s) : quant_mx_tiled_d<DT_F32, FMT_MXFP8>(a, s);
    if (a.fmt == FMT_MXFP8_E5M2)
      return a.xdt == DT_BF16 ? quant_mx_tiled_d<DT_BF16, FMT_MXFP8_E5M2>(a, s)
                              : quant_mx_tiled_d<DT_F32, FMT_MXFP8_E5M2>(a, s);
    return a.xdt == DT_BF16 ? quant_mx_tiled_d<DT_BF16, FMT_MXFP4>(a, s) : quant_mx_tiled_d<DT_F32, FMT_MXFP4>(a, s);
  }
#define MXK_QD(F) \
  return a.xdt == DT_BF16 ? quant_mx_d<DT_BF16, F>(a, Q, s) : quant_mx_d<DT_F32, F>(a, Q, s)
  switch (a.fmt) {
    case FMT_MXFP8: MXK_QD(FMT_MXFP8);
    case FMT_MXFP4: MXK_QD(FMT_MXFP4);
    case FMT_MXINT8: MXK_QD(FMT_MXINT8);
    case FMT_MXFP8_E5M2: MXK_QD(FMT_MXFP8_E5M2);
    case FMT_MXFP6_E3M2: MXK_QD(FMT_MXFP6_E3M2);
    default: MXK_QD(FMT_MXFP6_E2M3);
  }
#undef MXK_QD
}

namespace {
// jobs that can share one tile-layout launch
bool batchable(const QuantArgs& a) {
  return a.tiled && (a.fmt == FMT_MXFP8 || a.fmt == FMT_MXFP4 || a.fmt == FMT_MXFP8_E5M2) &&
         a.rows * a.cols > 0;
}
bool same_kernel(const QuantArgs& a, const QuantArgs& b) {
  return a.fmt == b.fmt && a.xdt == b.xdt && a.sr == b.sr && a.rht == b.rht;
}
// NVFP4 jobs that can share the launches of one NvBatch
bool nv_batchable(const QuantArgs& a) { return a.fmt == FMT_NVFP4 && a.rows * a.cols > 0; }
bool nv_same(const QuantArgs& a, const QuantArgs& b) {
  return a.xdt == b.xdt && a.sr == b.sr && a.rht == b.rht && a.sign_mask == b.sign_mask &&
         a.four6 == b.four6 && a.block2d == b.block2d && a.amax_given == b.amax_given;
}

// a[m] may join the group a[0 .. m-1]: no two jobs share an amax or tensor
// scale slot (sequential calls would keep them apart; a shared amax slot
// given as input is only read, and may be shared)
bool nv_disjoint(const QuantArgs* a, int m) {
  for (int k = 0; k < m; ++k) {
    if (a[k].tensor_scale == a[m].tensor_scale || a[k].tensor_scale == a[m].amax ||
        a[k].amax == a[m].tensor_scale)
      return false;
    if (!a[m].amax_given && a[k].amax == a[m].amax) return false;
  }
  return true;
}

template <int XDT, bool SR, bool RHT>
hipError_t nv_encode_batch_t(const NvBatch& b, bool four6, bool block2d, hipStream_t s) {
  const dim3 g((unsigned)b.first[b.n]), t(kThreads);
  if (block2d) {
    hipLaunchKernelGGL((k_quant_nvfp4_2d_batch<XDT, SR, RHT>), g, t, 0, s, b);
  } else if (four6) {
    if constexpr (SR) return hipErrorInvalidValue;  // rejected before launch
    hipLaunchKernelGGL((k_quant_nvfp4_batch<XDT, false, RHT, true>), g, t, 0, s, b);
  } else {
    hipLaunchKernelGGL((k_quant_nvfp4_batch<XDT, SR, RHT, false>), g, t, 0, s, b);
  }
  return hipGetLastError();
}
template <int XDT>
hipError_t nv_batch_d(NvBatch& b, hipStream_t s) {
  const QuantArgs& a0 = b.job[0];
  if (!a0.amax_given) {
    hipLaunchKernelGGL(k_zero_amax_batch, dim3(1), dim3(64), 0, s, b);
    // amax workgroups per job: about 512 in all, at most what the job fills
    const int64_t per = 512 / b.n > 1 ? 512 / b.n : 1;
    b.first[0] = 0;
    for (int k = 0; k < b.n; ++k) {
      const int64_t g = grid_for_amax(b.job[k].rows * (b.job[k].cols >> 3));
      b.first[k + 1] = b.first[k] + (g < per ? g : per);
    }
    if (a0.rht) hipLaunchKernelGGL((k_amax_batch<XDT, true>), dim3((unsigned)b.first[b.n]), dim3(kAmaxThreads), 0, s, b);
    else hipLaunchKernelGGL((k_amax_batch<XDT, false>), dim3((unsigned)b.first[b.n]), dim3(kAmaxThreads), 0, s, b);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  b.first[0] = 0;
  for (int k = 0; k < b.n; ++k) {
    const QuantArgs& a = b.job[k];
    int64_t g;
    if (a.block2d) {
      const int64_t nwaves = (a.rows + 15) / 16 * ((a.cols + k2dCols - 1) / k2dCols);
      g = (nwaves + kThreads / 64 - 1) / (kThreads / 64);
    } else {
      g = grid_for(a.rows * (a.cols >> 3));
    }
    b.first[k + 1] = b.first[k] + g;
  }
  if (a0.sr) return a0.rht ? nv_encode_batch_t<XDT, true, true>(b, a0.four6, a0.block2d, s)
                           : nv_encode_batch_t<XDT, true, false>(b, a0.four6, a0.block2d, s);
  return a0.rht ? nv_encode_batch_t<XDT, false, true>(b, a0.four6, a0.block2d, s)
                : nv_encode_batch_t<XDT, false, false>(b, a0.four6, a0.block2d, s);
}
}  // namespace

hipError_t launch_quantize_batch(const QuantArgs* a, int n, hipStream_t s) {
  static_assert(sizeof(NvBatch) <= 3072, "kernel argument size");
  int i = 0;
  while (i < n) {
    if (nv_batchable(a[i])) {
      int m = 1;
      while (m < kMaxNvBatch && i + m < n && nv_batchable(a[i + m]) && nv_same(a[i], a[i + m]) &&
             nv_disjoint(a + i, m))
        ++m;
      if (m > 1) {
        NvBatch b{};
        b.n = m;
        for (int k = 0; k < m; ++k) b.job[k] = a[i + k];
        const hipError_t e = a[i].xdt == DT_BF16 ? nv_batch_d<DT_BF16>(b, s) : nv_batch_d<DT_F32>(b, s);
        if (e != hipSuccess) return e;
        i += m;
        continue;
      }
    }
    int m = 1;
    if (batchable(a[i]))
      while (m < kMaxBatch && i + m < n && batchable(a[i + m]) && same_kernel(a[i], a[i + m])) ++m;
    hipError_t e;
    if (m == 1) {
      e = launch_quantize(a[i], s);
    } else {
      QuantBatch b{};
      b.n = m;
      b.first[0] = 0;
      for (int k = 0; k < m; ++k) {
        b.job[k] = a[i + k];
        b.first[k + 1] = b.first[k] + (a[i + k].rows / 8) * (a[i + k].cols / (64 * kTiledNT));
      }
      if (a[i].fmt == FMT_MXFP8)
        e = a[i].xdt == DT_BF16 ? quant_mx_tiled_batch_d<DT_BF16, FMT_MXFP8>(b, s) : quant_mx_tiled_batch_d<DT_F32, FMT_MXFP8>(b, s);
      else if (a[i].fmt == FMT_MXFP8_E5M2)
        e = a[i].xdt == DT_BF16 ? quant_mx_tiled_batch_d<DT_BF16, FMT_MXFP8_E5M2>(b, s)
                                : quant_mx_tiled_batch_d<DT_F32, FMT_MXFP8_E5M2>(b, s);
      else
        e = a[i].xdt == DT_BF16 ? quant_mx_tiled_batch_d<DT_BF16, FMT_MXFP4>(b, s) : quant_mx_tiled_batch_d<DT_F32, FMT_MXFP4>(b, s);
    }
    if (e != hipSuccess) return e;
    i += m;
  }
  return hipSuccess;
}

hipError_t launch_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales,
                             const float* tensor_scale, int64_t rows, int64_t cols, void* y,
                             int ydt, int64_t ld_y, bool rht, uint32_t sign_mask, bool tiled,
                             hipStream_t s) {
  const int64_t Q = rows * (cols / 8);
  if (Q == 0) return hipSuccess;
  const int g = grid_for(Q);
#define MXK_DQ(F, Y, R)                                                                       \
  hipLaunchKernelGGL((k_dequant<F, Y, R>), dim3(g), dim3(kThreads), 0, s, codes, scales,       \
                     tensor_scale, cols, y, ld_y, Q, sign_mask, tiled)
#define MXK_DQ_Y(F, R)                 \
  if (ydt == DT_BF16) MXK_DQ(F, DT_BF16, R); \
  else MXK_DQ(F, DT_F32, R);
#define MXK_DQ_R(F)                    \
  if (rht) { MXK_DQ_Y(F, true) }       \
  else { MXK_DQ_Y(F, false) }
  if (fmt == FMT_MXFP8) { MXK_DQ_R(FMT_MXFP8) }
  else if (fmt == FMT_MXFP4) { MXK_DQ_R(FMT_MXFP4) }
  else if (fmt == FMT_MXINT8) { MXK_DQ_R(FMT_MXINT8) }
  else if (fmt == FMT_MXFP8_E5M2) { MXK_DQ_R(FMT_MXFP8_E5M2) }
  else if (fmt == FMT_MXFP6_E3M2) { MXK_DQ_R(FMT_MXFP6_E3M2) }
  else if (fmt == FMT_MXFP6_E2M3) { MXK_DQ_R(FMT_MXFP6_E2M3) }
  else { MXK_DQ_R(FMT_NVFP4) }
#undef MXK_DQ_R
#undef MXK_DQ_Y
#undef MXK_DQ
  return hipGetLastError();
}

hipError_t launch_hadamard16(const void* x, int xdt, void* y, int ydt, int64_t rows, int64_t cols,
                             uint32_t sign_mask, bool inverse, hipStream_t s) {
  const int64_t Q = rows * (cols / 8);
  if (Q == 0) return hipSuccess;
  const int g = grid_for(Q);
#define MXK_H(X, Y, I) \
  hipLaunchKernelGGL((k_hadamard<X, Y, I>), dim3(g), dim3(kThreads), 0, s, x, y, cols, Q, sign_mask)
#define MXK_H_I(X, Y)             \
  if (inverse) MXK_H(X, Y, true); \
  else MXK_H(X, Y, false);
  if (xdt == DT_BF16) {
    if (ydt == DT_BF16) { MXK_H_I(DT_BF16, DT_BF16) } else { MXK_H_I(DT_BF16, DT_F32) }
  } else {
    if (ydt == DT_BF16) { MXK_H_I(DT_F32, DT_BF16) } else { MXK_H_I(DT_F32, DT_F32) }
  }
#undef MXK_H_I
#undef MXK_H
  return hipGetLastError();
}

}  // namespace mxk
