// quantize.hip -- block-scaled quantizers, per-tensor amax, decoder and the
// standalone 16-point Hadamard transform for gfx950.
//
// All kernels here are HBM-bound streaming kernels.  Work unit: a "chunk" of
// 8 consecutive elements of a row, held by one lane (one 128-bit BF16 load).
// A 64-lane wave covers 64 consecutive chunks, so an MX block of 32 elements
// is one lane quad and an NVFP4 block of 16 (or a Hadamard group of 16) is one
// lane pair; block maxima and the stride-8 butterfly use DPP quad permutes.
// Codes are stored with one 64-bit (MXFP8) or 32-bit (FP4) store per lane and
// the scale bytes of 4 blocks are gathered into one 32-bit store.
//
// Method sources: "Microscaling (MX) and block-scaled 4-bit formats"
// (sections "Microscaling", "The idea", "NVFP4", glossary "scale factor",
// "stochastic rounding"); "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier"
// (MXFP4/NVFP4 table and the paragraph on two-level scaling).
#include "../device/codec.h"
#include "../device/wave.h"
#include "../launch.h"

namespace mxk {

namespace {

constexpr int kThreads = 256;

// Walks chunk indices q = q0 + lane with a wave-uniform q0, tracking
// (row, chunk-in-row) incrementally so the loop needs no integer division.
struct ChunkWalk {
  int64_t q0, row, c8;  // position of lane 0 of this wave
  int64_t step, step_rows, step_rem, cpr;
  __device__ void init(int64_t start, int64_t stride, int64_t cpr_) {
    cpr = cpr_;
    q0 = start;
    row = start / cpr;
    c8 = start - row * cpr;
    step = stride;
    step_rows = stride / cpr;
    step_rem = stride - step_rows * cpr;
  }
  __device__ void advance() {
    q0 += step;
    row += step_rows;
    c8 += step_rem;
    if (c8 >= cpr) {
      c8 -= cpr;
      row += 1;
    }
  }
  // (row, chunk-in-row) of this lane's chunk
  __device__ void lane_pos(uint32_t lane, int64_t* r, int64_t* c) const {
    int64_t cc = c8 + lane, rr = row;
    while (cc >= cpr) {  // at most 64 / cpr + 1 steps; cpr >= 2
      cc -= cpr;
      rr += 1;
    }
    *r = rr;
    *c = cc;
  }
};

template <int XDT>
__device__ inline void load8(const void* base, int64_t off, bool valid, float v[8]) {
  if (!valid) {
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    return;
  }
  if constexpr (XDT == DT_BF16) {
    uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + off);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = u2f(w[i] << 16);
      v[2 * i + 1] = u2f(w[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(base) + off);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

template <int YDT>
__device__ inline void store8(void* base, int64_t off, const float v[8]) {
  if constexpr (YDT == DT_BF16) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)f32_to_bf16(v[2 * i]) | ((uint32_t)f32_to_bf16(v[2 * i + 1]) << 16);
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(base) + off) = make_uint4(w[0], w[1], w[2], w[3]);
  } else {
    float4* p = reinterpret_cast<float4*>(static_cast<float*>(base) + off);
    p[0] = make_float4(v[0], v[1], v[2], v[3]);
    p[1] = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// Forward 16-point transform of a group split over a lane pair: this lane
// holds elements 8*half .. 8*half+7.  y = (1/4) H16 D x, stages 1, 2, 4 in
// the lane, stage 8 across the pair (the lower lane keeps a + b, the upper
// lane a - b, with a the lower lane's value).
__device__ inline void rht_forward(float v[8], uint32_t mask, uint32_t half) {
  uint32_t m = (mask >> (8 * half)) & 0xFFu;
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((m >> i) & 1u) v[i] = -v[i];
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

__device__ inline uint32_t max_abs_bits(const float v[8]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    uint32_t b = f2u(v[i]) & 0x7FFFFFFFu;
    m = b > m ? b : m;
  }
  return m;
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
template <int XDT, int FMT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_mx(QuantArgs a, int64_t Q) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t cpr = a.cols >> 3;
  constexpr uint32_t emax = FMT == FMT_MXFP8 ? 8u : 2u;
  ChunkWalk w;
  w.init(wave * 64, nwaves * 64, cpr);
  for (; w.q0 < Q; w.advance()) {
    const int64_t q = w.q0 + lane;
    const bool valid = q < Q;
    int64_t row, c8;
    w.lane_pos(lane, &row, &c8);
    float v[8];
    load8<XDT>(a.x, row * a.ld_x + 8 * c8, valid, v);
    if constexpr (RHT) rht_forward(v, a.sign_mask, (uint32_t)(c8 & 1));
    uint32_t m = max_abs_bits(v);
    uint32_t o = dpp_xor1(m);
    m = o > m ? o : m;
    o = dpp_xor2(m);
    m = o > m ? o : m;
    const uint32_t sc = e8m0_from_amax_bits(m, emax);
    const float inv = e8m0_inverse(sc);
    uint32_t r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (SR) rand16x8(a.seed, a.counter, (uint64_t)q, r);
    uint32_t c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float y = v[i] * inv;  // exact scaling by a power of two
      c[i] = FMT == FMT_MXFP8 ? e4m3_encode(y, SR, r[i]) : e2m1_encode(y, SR, r[i]);
      if (sc == 0xFFu) c[i] = 0u;
    }
    if (valid) {
      if constexpr (FMT == FMT_MXFP8) {
        uint2 p;
        p.x = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
        p.y = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
        *reinterpret_cast<uint2*>(a.codes + q * 8) = p;
      } else {
        uint32_t p = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) p |= c[i] << (4 * i);
        *reinterpret_cast<uint32_t*>(a.codes + q * 4) = p;
      }
    }
    store_scales(a.scales, q >> 2, sc, lane, 4u, (Q - q) >> 2);
  }
}

// ---- NVFP4 (E4M3 per 16 + FP32 per tensor) quantizer ----------------------
template <int XDT, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void k_quant_nvfp4(QuantArgs a, int64_t Q) {
#pragma clang fp contract(off)
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const int64_t cpr = a.cols >> 3;
  const float T = *a.amax;
  const float S = (T == 0.0f) ? 1.0f : T / 2688.0f;
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.tensor_scale = S;
  const float d = 6.0f * S;
  ChunkWalk w;
  w.init(wave * 64, nwaves * 64, cpr);
  for (; w.q0 < Q; w.advance()) {
    const int64_t q = w.q0 + lane;
    const bool valid = q < Q;
    int64_t row, c8;
    w.lane_pos(lane, &row, &c8);
    float v[8];
    load8<XDT>(a.x, row * a.ld_x + 8 * c8, valid, v);
    if constexpr (RHT) rht_forward(v, a.sign_mask, (uint32_t)(c8 & 1));
    uint32_t m = max_abs_bits(v);
    uint32_t o = dpp_xor1(m);
    m = o > m ? o : m;
    const float qb = u2f(m) / d;
    const uint32_t sb = e4m3_rne_mag(qb);
    const float dsb = e4m3_mag_value(sb);
    float rcp = 0.0f;
    if (dsb != 0.0f) {
      const float p = dsb * S;
      rcp = 1.0f / p;
    }
    uint32_t r[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (SR) rand16x8(a.seed, a.counter, (uint64_t)q, r);
    uint32_t packed = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t c;
      if (rcp == 0.0f) {
        c = (f2u(v[i]) >> 28) & 0x8u;
      } else {
        const float y = v[i] * rcp;
        c = e2m1_encode(y, SR, r[i]);
      }
      packed |= c << (4 * i);
    }
    if (valid) *reinterpret_cast<uint32_t*>(a.codes + q * 4) = packed;
    store_scales(a.scales, q >> 1, sb, lane, 2u, (Q - q) >> 1);
  }
}

// ---- per-tensor amax ------------------------------------------------------
__global__ void k_zero_f32(float* p) { *p = 0.0f; }

template <int XDT, bool RHT>
__global__ __launch_bounds__(kThreads) void k_amax(const void* x, int64_t cols, int64_t ld_x,
                                                   int64_t Q, uint32_t sign_mask, float* amax) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  ChunkWalk w;
  w.init(wave * 64, nwaves * 64, cols >> 3);
  uint32_t m = 0;
  for (; w.q0 < Q; w.advance()) {
    const int64_t q = w.q0 + lane;
    int64_t row, c8;
    w.lane_pos(lane, &row, &c8);
    float v[8];
    load8<XDT>(x, row * ld_x + 8 * c8, q < Q, v);
    if constexpr (RHT) rht_forward(v, sign_mask, (uint32_t)(c8 & 1));
    uint32_t b = max_abs_bits(v);
    m = b > m ? b : m;
  }
  m = wave_max_u32(m);
  __shared__ uint32_t red[kThreads / 64];
  if (lane == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = red[0];
    for (int i = 1; i < kThreads / 64; ++i) t = red[i] > t ? red[i] : t;
    // non-negative floats order like their bit patterns
    atomicMax(reinterpret_cast<unsigned int*>(amax), t);
  }
}

// ---- decoder ----------------------------------------------------------------
template <int FMT, int YDT, bool RHT>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* codes, const uint8_t* scales,
                                                      const float* tensor_scale, int64_t cols,
                                                      void* y, int64_t ld_y, int64_t Q,
                                                      uint32_t sign_mask) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  const float S = FMT == FMT_NVFP4 ? *tensor_scale : 1.0f;
  ChunkWalk w;
  w.init(wave * 64, nwaves * 64, cols >> 3);
  for (; w.q0 < Q; w.advance()) {
    const int64_t q = w.q0 + lane;
    const bool valid = q < Q;
    int64_t row, c8;
    w.lane_pos(lane, &row, &c8);
    float v[8];
    if (valid) {
      uint32_t cw[8];
      if constexpr (FMT == FMT_MXFP8) {
        uint2 p = *reinterpret_cast<const uint2*>(codes + q * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          cw[i] = (p.x >> (8 * i)) & 0xFFu;
          cw[4 + i] = (p.y >> (8 * i)) & 0xFFu;
        }
      } else {
        uint32_t p = *reinterpret_cast<const uint32_t*>(codes + q * 4);
#pragma unroll
        for (int i = 0; i < 8; ++i) cw[i] = (p >> (4 * i)) & 0xFu;
      }
      if constexpr (FMT == FMT_NVFP4) {
        const float sbv = e4m3_mag_value(scales[q >> 1]);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (e2m1_value(cw[i]) * sbv) * S;  // first product exact
      } else {
        const uint32_t sc = scales[q >> 2];
        // 2^(sc-127) as FP32 (sc = 0 is the subnormal 2^-127); 0xFF is NaN
        const float X = sc == 0xFFu ? __builtin_nanf("") : (sc == 0u ? u2f(0x00400000u) : u2f(sc << 23));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float e;
          if constexpr (FMT == FMT_MXFP8) {
            const uint32_t mag = cw[i] & 0x7Fu;
            e = mag == 0x7Fu ? __builtin_nanf("") : e4m3_mag_value(mag);
            if (cw[i] & 0x80u) e = -e;
          } else {
            e = e2m1_value(cw[i]);
          }
          v[i] = e * X;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.0f;
    }
    if constexpr (RHT) rht_inverse(v, sign_mask, (uint32_t)(c8 & 1));
    if (valid) store8<YDT>(y, row * ld_y + 8 * c8, v);
  }
}

// ---- standalone Hadamard ----------------------------------------------------
template <int XDT, int YDT, bool INV>
__global__ __launch_bounds__(kThreads) void k_hadamard(const void* x, void* y, int64_t cols,
                                                       int64_t Q, uint32_t sign_mask) {
  const uint32_t lane = threadIdx.x & 63u;
  const int64_t wave = ((int64_t)blockIdx.x * kThreads + threadIdx.x) >> 6;
  const int64_t nwaves = ((int64_t)gridDim.x * kThreads) >> 6;
  for (int64_t q0 = wave * 64; q0 < Q; q0 += nwaves * 64) {
    const int64_t q = q0 + lane;
    const bool valid = q < Q;
    float v[8];
    load8<XDT>(x, q * 8, valid, v);
    if constexpr (INV) rht_inverse(v, sign_mask, (uint32_t)(q & 1));
    else rht_forward(v, sign_mask, (uint32_t)(q & 1));
    if (valid) store8<YDT>(y, q * 8, v);
  }
}

int grid_for(int64_t Q) {
  int64_t waves = (Q + 63) / 64;
  int64_t blocks = (waves + 3) / 4;
  const int64_t cap = 256 * 16;
  if (blocks > cap) blocks = cap;
  return (int)(blocks < 1 ? 1 : blocks);
}

template <int XDT, int FMT, bool SR, bool RHT>
hipError_t quant_mx_t(const QuantArgs& a, int64_t Q, hipStream_t s) {
  hipLaunchKernelGGL((k_quant_mx<XDT, FMT, SR, RHT>), dim3(grid_for(Q)), dim3(kThreads), 0, s, a, Q);
  return hipGetLastError();
}
template <int XDT, bool SR, bool RHT>
hipError_t quant_nv_t(const QuantArgs& a, int64_t Q, hipStream_t s) {
  hipLaunchKernelGGL((k_quant_nvfp4<XDT, SR, RHT>), dim3(grid_for(Q)), dim3(kThreads), 0, s, a, Q);
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
  const int g = grid_for(Q);
  if (xdt == DT_BF16) {
    if (rht) hipLaunchKernelGGL((k_amax<DT_BF16, true>), dim3(g), dim3(kThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
    else hipLaunchKernelGGL((k_amax<DT_BF16, false>), dim3(g), dim3(kThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
  } else {
    if (rht) hipLaunchKernelGGL((k_amax<DT_F32, true>), dim3(g), dim3(kThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
    else hipLaunchKernelGGL((k_amax<DT_F32, false>), dim3(g), dim3(kThreads), 0, s, x, cols, ld_x, Q, sign_mask, amax);
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
      hipLaunchKernelGGL((k_quant_nvfp4<DT_BF16, false, false>), dim3(1), dim3(kThreads), 0, s, a, (int64_t)0);
      return hipGetLastError();
    }
    return a.xdt == DT_BF16 ? quant_nv_d<DT_BF16>(a, Q, s) : quant_nv_d<DT_F32>(a, Q, s);
  }
  if (Q == 0) return hipSuccess;
  if (a.fmt == FMT_MXFP8)
    return a.xdt == DT_BF16 ? quant_mx_d<DT_BF16, FMT_MXFP8>(a, Q, s) : quant_mx_d<DT_F32, FMT_MXFP8>(a, Q, s);
  return a.xdt == DT_BF16 ? quant_mx_d<DT_BF16, FMT_MXFP4>(a, Q, s) : quant_mx_d<DT_F32, FMT_MXFP4>(a, Q, s);
}

hipError_t launch_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales,
                             const float* tensor_scale, int64_t rows, int64_t cols, void* y,
                             int ydt, int64_t ld_y, bool rht, uint32_t sign_mask, hipStream_t s) {
  const int64_t Q = rows * (cols / 8);
  if (Q == 0) return hipSuccess;
  const int g = grid_for(Q);
#define MXK_DQ(F, Y, R)                                                                       \
  hipLaunchKernelGGL((k_dequant<F, Y, R>), dim3(g), dim3(kThreads), 0, s, codes, scales,       \
                     tensor_scale, cols, y, ld_y, Q, sign_mask)
#define MXK_DQ_Y(F, R)                 \
  if (ydt == DT_BF16) MXK_DQ(F, DT_BF16, R); \
  else MXK_DQ(F, DT_F32, R);
#define MXK_DQ_R(F)                    \
  if (rht) { MXK_DQ_Y(F, true) }       \
  else { MXK_DQ_Y(F, false) }
  if (fmt == FMT_MXFP8) { MXK_DQ_R(FMT_MXFP8) }
  else if (fmt == FMT_MXFP4) { MXK_DQ_R(FMT_MXFP4) }
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
