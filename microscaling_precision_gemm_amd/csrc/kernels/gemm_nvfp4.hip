// gemm_nvfp4.hip -- NVFP4 GEMM with explicit per-16 E4M3 block scales, plain
// and grouped over experts (mixture-of-experts forward), on gfx950.
//
// The E4M3 block scale of NVFP4 has no counterpart in the matrix
// instructions (their block scale is E8M0 per 32 elements), so each E2M1
// element is multiplied by its block scale while it is staged into LDS.  The
// product has at most 2 + 4 significant bits, so it is exact in BF16, and the
// contraction runs on v_mfma_f32_32x32x16_bf16 with FP32 accumulation.  The
// per-tensor FP32 scales multiply the accumulator in the epilogue
// ("Microscaling (MX) and block-scaled 4-bit formats", section "NVFP4":
// FP4 elements, an E4M3 scale per 16, a second-level FP32 scale per tensor;
// "Thinking Machines ... Inkling 2 Small", section "A precision choice for
// each stage": NVFP4 forward passes in the expert layers).
//
// Workgroup: 256 threads, 128x128 C tile, K step 64 (4 instructions of K=16),
// double-buffered LDS holding BF16.  Grouped launch: blockIdx.y enumerates
// (expert, 128-row tile) pairs; the grid has an upper bound of
// ceil(R/128) + groups rows of tiles and surplus workgroups exit.
#include "../device/codec.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kPitchB = kBK * 2 + 16;  // bytes per LDS row (BF16 values + pad)

__device__ inline uint32_t pack_bf16x2_exact(float lo, float hi) {
  // exact: the values carry at most 6 significant bits
  return (f2u(lo) >> 16) | (f2u(hi) & 0xFFFF0000u);
}

template <int CDT, bool GATHER>
__global__ __launch_bounds__(256) void k_gemm_nvfp4(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const float* __restrict__ a_ts,
    const int32_t* __restrict__ row_index, int64_t R, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ b_ts, int32_t groups,
    const int64_t* __restrict__ offsets, int64_t N, int64_t K, void* __restrict__ C, int64_t ldc) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(kBM + kBN) * kPitchB];
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t n0 = (int64_t)blockIdx.x * kBN;

  // find this workgroup's (group, row range)
  int64_t tile = blockIdx.y, g = -1, g_lo = 0, g_hi = 0;
  if (offsets == nullptr) {  // plain GEMM: one group of R rows
    if (tile * kBM < R) {
      g = 0;
      g_lo = tile * kBM;
      g_hi = R;
    }
  } else {
    int64_t acc = 0;
    for (int32_t e = 0; e < groups; ++e) {
      const int64_t lo = offsets[e], hi = offsets[e + 1];
      const int64_t nt = (hi - lo + kBM - 1) / kBM;
      if (tile < acc + nt) {
        g = e;
        g_lo = lo + (tile - acc) * kBM;
        g_hi = hi;
        break;
      }
      acc += nt;
    }
  }
  if (g < 0) return;  // surplus workgroup (uniform across the block)
  const int64_t m0 = g_lo;
  const int64_t rowbytes = K / 2, sblocks = K / 16;
  const int64_t steps = (K + kBK - 1) / kBK;
  const uint8_t* Bg = B + g * N * rowbytes;
  const uint8_t* SBg = SB + g * N * sblocks;

  // staging: thread t converts 32 elements (half a K step) of one A row and of
  // one B row: row r = t / 2, half h = t % 2 -> 16 code bytes + 2 scale bytes
  const uint32_t sr = t >> 1, sh = t & 1u;
  int64_t a_src = -1;
  {
    const int64_t rr = m0 + sr;
    if (rr < g_hi) a_src = GATHER ? (int64_t)row_index[rr] : rr;
  }
  const int64_t b_src = (n0 + sr < N) ? n0 + sr : -1;

  auto load_stage = [&](int64_t step, uint4& ca, uint32_t& sca, uint4& cb, uint32_t& scb) {
    const int64_t kb = step * (kBK / 2) + sh * 16;  // code byte offset in row
    const int64_t ks = step * (kBK / 16) + sh * 2;  // scale index in row
    ca = make_uint4(0, 0, 0, 0);
    cb = make_uint4(0, 0, 0, 0);
    sca = 0;
    scb = 0;
    if (kb < rowbytes) {  // rowbytes is a multiple of 8: a 16-byte piece is all in or half in
      const bool full = kb + 16 <= rowbytes;
      if (a_src >= 0) {
        const uint8_t* p = A + a_src * rowbytes + kb;
        if (full) ca = *reinterpret_cast<const uint4*>(p);
        else { uint2 h = *reinterpret_cast<const uint2*>(p); ca = make_uint4(h.x, h.y, 0, 0); }
        sca = SA[a_src * sblocks + ks] | (full ? (uint32_t)SA[a_src * sblocks + ks + 1] << 8 : 0u);
      }
      if (b_src >= 0) {
        const uint8_t* p = Bg + b_src * rowbytes + kb;
        if (full) cb = *reinterpret_cast<const uint4*>(p);
        else { uint2 h = *reinterpret_cast<const uint2*>(p); cb = make_uint4(h.x, h.y, 0, 0); }
        scb = SBg[b_src * sblocks + ks] | (full ? (uint32_t)SBg[b_src * sblocks + ks + 1] << 8 : 0u);
      }
    }
  };
  auto store_stage = [&](int buf, const uint4& ca, uint32_t sca, const uint4& cb, uint32_t scb) {
    const uint32_t cw[2][4] = {{ca.x, ca.y, ca.z, ca.w}, {cb.x, cb.y, cb.z, cb.w}};
    const uint32_t sw[2] = {sca, scb};
#pragma unroll
    for (int op = 0; op < 2; ++op) {
      const uint32_t r = op == 0 ? sr : kBM + sr;
      uint8_t* dst = &lds[buf][r * kPitchB + sh * 64];
#pragma unroll
      for (int blk = 0; blk < 2; ++blk) {
        const float s = e4m3_mag_value((sw[op] >> (8 * blk)) & 0xFFu);
        uint32_t out[8];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const uint32_t word = cw[op][blk * 2 + w];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float lo = e2m1_value((word >> (8 * i)) & 0xFu) * s;
            const float hi = e2m1_value((word >> (8 * i + 4)) & 0xFu) * s;
            out[w * 4 + i] = pack_bf16x2_exact(lo, hi);
          }
        }
        *reinterpret_cast<uint4*>(dst + blk * 32) = make_uint4(out[0], out[1], out[2], out[3]);
        *reinterpret_cast<uint4*>(dst + blk * 32 + 16) = make_uint4(out[4], out[5], out[6], out[7]);
      }
    }
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  uint4 ca, cb;
  uint32_t sca, scb;
  load_stage(0, ca, sca, cb, scb);
  store_stage(0, ca, sca, cb, scb);
  __syncthreads();
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  for (int64_t st = 0; st < steps; ++st) {
    const int buf = (int)(st & 1);
    if (st + 1 < steps) load_stage(st + 1, ca, sca, cb, scb);
#pragma unroll
    for (int kk = 0; kk < kBK / 16; ++kk) {
      v8bf af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint32_t ra = wm * 64 + i * 32 + lr;
        const uint32_t rb = kBM + wn * 64 + i * 32 + lr;
        const uint32_t off = (kk * 16 + lg * 8) * 2;
        const uint4 a = *reinterpret_cast<const uint4*>(&lds[buf][ra * kPitchB + off]);
        const uint4 b = *reinterpret_cast<const uint4*>(&lds[buf][rb * kPitchB + off]);
        af[i] = __builtin_bit_cast(v8bf, a);
        bfr[i] = __builtin_bit_cast(v8bf, b);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (st + 1 < steps) store_stage(buf ^ 1, ca, sca, cb, scb);
    __syncthreads();
  }

  const float sab = *a_ts * b_ts[g];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
        if (row < g_hi && col < N) {
          const float val = acc[i][j][v] * sab;
          if constexpr (CDT == DT_F32) static_cast<float*>(C)[row * ldc + col] = val;
          else static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(val);
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                             const int32_t* row_index, int64_t routed_rows,
                             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                             int32_t groups, const int64_t* offsets, int64_t N, int64_t K,
                             void* C, int cdt, int64_t ldc, hipStream_t s) {
  if (routed_rows == 0 || N == 0) return hipSuccess;
  const int64_t ytiles = (routed_rows + kBM - 1) / kBM + groups;
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)ytiles);
#define MXK_NV(D, G)                                                                           \
  hipLaunchKernelGGL((k_gemm_nvfp4<D, G>), grid, dim3(256), 0, s, a_codes, a_scales, a_ts,     \
                     row_index, routed_rows, b_codes, b_scales, b_ts, groups, offsets, N, K, C, ldc)
  if (row_index) {
    if (cdt == DT_F32) MXK_NV(DT_F32, true);
    else MXK_NV(DT_BF16, true);
  } else {
    if (cdt == DT_F32) MXK_NV(DT_F32, false);
    else MXK_NV(DT_BF16, false);
  }
#undef MXK_NV
  return hipGetLastError();
}

}  // namespace mxk
