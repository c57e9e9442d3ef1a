// gemm_nvpipe.hip -- NVFP4 GEMM C = (A * B^T) * S_A * S_B, plain or grouped
// over experts with an optional row gather of A, on the DMA pipeline of
// device/pipe.h ("Microscaling (MX) and block-scaled 4-bit formats", section
// "NVFP4": E2M1 elements, an E4M3 scale per 16, an FP32 scale per tensor;
// "Thinking Machines ... Inkling 2 Small", section "A precision choice for
// each stage": NVFP4 forward in the expert layers).
//
// gfx950's scaled matrix instruction takes E8M0 scales per 32 elements, and
// an E4M3 block scale is not a power of two, so every element is multiplied
// by its block scale before a plain 16-bit instruction.  e2m1 * e4m3 has at
// most 2 + 4 significant bits and lies in [2^-10, 2880], so it is exact in
// FP16, and v_mfma_f32_32x32x16_f16 sums exact products in FP32.  The
// conversion splits the block scale s = 2^e * mu: v_cvt_scalef32_pk_f16_fp4
// applies 2^e (it uses only the exponent of its FP32 scale operand) and one
// v_pk_mul_f16 applies mu to two elements -- 8 VALU instructions per 8
// elements.  A 2 KB LDS table maps each E4M3 code to (2^e as FP32 bits, mu
// pair as FP16 bits): normal codes 2^(c/8 - 7) * (1 + (c%8)/8), subnormal
// codes c * 2^-9 as (2^-9, c) -- both exact -- and code 0 gives mu = 0.
//
// Stages: the FP4 codes of 256 A and 256 B rows, 128 bytes (256 elements)
// per row and step, land in LDS by global_load_lds exactly as in the MX
// pipelined kernel (XOR-swizzled 16-byte chunks, two stages), and the
// step's 16 E4M3 bytes per row go to a rotating scale buffer two steps ahead.
// Within a step, slice q (64 elements) gives lane (r = l mod 32, g = l / 32)
// chunk 2q + g of its row (32 elements, two NVFP4 blocks); unit m (0..3)
// of the slice takes the lane's code dword m (8 elements of block m / 2) and
// feeds 16 instructions.  A and B use the same assignment of K positions to
// (instruction, lane group, element), so every block's products are summed.
//
// Per step: 16 windows of 16 instructions.  Window u converts unit u+1; the
// code dwords of the next slice arrive two units at a time (8-byte reads),
// units 0-1 in window 4q+1 and units 2-3 in window 4q+3, each into the
// registers of two units already converted; the scale codes of the next
// slice are read in its window 4q+1 and looked up in 4q+2.  The barrier of
// the step follows window 13; the next stage's reads (windows 14 and 15) and
// the refill DMAs of the stage just consumed come after it.  Each workgroup
// owns a 256x256 output tile of one group.
#include <atomic>

#include "../device/codec.h"
#include "../device/gemm_common.h"
#include "../device/pipe.h"
#include "../launch.h"

namespace mxk {

namespace {

typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
// (FP32 bits of 2^e, mu pair as two FP16).  A struct rather than a vector
// type: hipcc miscompiles __builtin_bit_cast of an ext_vector_type element
// (it reads element 0).
struct TabE {
  uint32_t x, mu;
};

constexpr int kStepK = 256;                   // K elements per step
constexpr int kTabBase = kSmemBytes;          // E4M3 table: 256 x 8 bytes
constexpr int kNvSmem = kSmemBytes + 256 * 8;

// table entry of E4M3 magnitude code c
__device__ inline TabE nv_tab_entry(uint32_t c) {
  uint32_t ex, mu;
  if (c >= 8u) {
    ex = (c >> 3) + 120u;
    mu = 0x3C00u | ((c & 7u) << 7);
  } else {
    ex = 118u;  // 2^-9
    mu = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(float)c);  // exact, 0 for c = 0
  }
  return TabE{ex << 23, mu | (mu << 16)};
}

// 8 FP16 values (element 2k in the low half of word k) of the 8 codes in w
__device__ inline u4 nv_conv(uint32_t w, TabE tab) {
  const float X = u2f(tab.x);
  const v2h mu = __builtin_bit_cast(v2h, tab.mu);
  u4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, X, 0) * mu);
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, X, 1) * mu);
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, X, 2) * mu);
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, X, 3) * mu);
  return o;
}

struct NvState {
  uint32_t raw[8][4];  // [A 0..3, B 4..7][unit of the slice]: the lane's code dwords
  u4 cv[2][8];         // [unit parity]: FP16 fragments
  uint32_t code[8];    // the two scale codes (blocks 2c, 2c+1) of a slice
  TabE tab[2][8][2];     // [slice parity][fragment][block of the chunk]
};

__device__ inline uint32_t frag_row(int t, uint32_t wm, uint32_t wn, uint32_t lr) {
  return t < 4 ? wm * 128 + t * 32 + lr : kTile + wn * 128 + (t - 4) * 32 + lr;
}

// code dwords 2h, 2h+1 of chunk 2q + g of each fragment row, one 8-byte read
// each (a 4-byte read per dword met 4-way bank conflicts: 32 rows of one
// 16-byte column fall on 16 distinct 4-byte banks; 8-byte reads halve that)
__device__ inline void read_half(const uint8_t* __restrict__ L, uint32_t q, int h, uint32_t wm, uint32_t wn,
                                 uint32_t lr, uint32_t lg, uint32_t (&raw)[8][4]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint2 v = *reinterpret_cast<const uint2*>(L + chunk_off(frag_row(t, wm, wn, lr), 2 * q + lg) + 8 * h);
    raw[t][2 * h] = v.x;
    raw[t][2 * h + 1] = v.y;
  }
}

// scale codes of blocks 2c, 2c+1 (c = 2q + g) of step `step` for each fragment row
__device__ inline void read_codes(const uint8_t* __restrict__ smem, uint32_t step, uint32_t q, uint32_t wm,
                                  uint32_t wn, uint32_t lr, uint32_t lg, uint32_t (&code)[8]) {
  const uint8_t* LS = smem + kScaleBase + (step % kScaleBufs) * kScaleBuf;
#pragma unroll
  for (int t = 0; t < 8; ++t)
    code[t] = *reinterpret_cast<const uint16_t*>(LS + frag_row(t, wm, wn, lr) * kScaleRow + 2 * (2 * q + lg));
}

__device__ inline void lookup(const uint8_t* __restrict__ smem, const uint32_t (&code)[8], TabE (&tab)[8][2]) {
#pragma unroll
  for (int t = 0; t < 8; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      tab[t][h] = *reinterpret_cast<const TabE*>(smem + kTabBase + ((code[t] >> (8 * h)) & 0xFFu) * 8);
}

__device__ inline void conv_unit(const uint32_t (&raw)[8][4], int m, const TabE (&tab)[8][2], u4 (&cv)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) cv[t] = nv_conv(raw[t][m], tab[t][m / 2]);
}

__device__ inline void mfma_f16_16(const u4 (&f)[8], v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, f[i]),
                                                         __builtin_bit_cast(v8h, f[4 + j]), acc[i][j], 0, 0, 0);
}

// Window U of step st (see the file comment).
template <int U, bool SWITCH, bool DMA>
__device__ inline void nv_window(const PipeCtx& x, uint8_t* __restrict__ smem, uint32_t st, uint32_t wm,
                                 uint32_t wn, uint32_t lr, uint32_t lg, NvState& s, v16f (&acc)[4][4]) {
  constexpr int kConvValu = 8 * 8;
  uint8_t* cur = smem + (st & 1u) * kStageBytes;
  uint8_t* nxt = smem + ((st + 1u) & 1u) * kStageBytes;
  // unit U+1: same step, or (U = 15) the next step's first unit
  constexpr bool kConvNext = U < 15 || SWITCH;
  // lookup of the next stage's first slice happens in window 15, before its use
  if constexpr (U == 15 && SWITCH) {
    lookup(smem, s.code, s.tab[0]);
  }
  if constexpr (kConvNext) conv_unit(s.raw, (U + 1) % 4, s.tab[((U + 1) / 4) % 2], s.cv[(U + 1) % 2]);
  // code dwords of the next slice, two at a time into the registers of the
  // two units already converted: dwords 0-1 in window 4q+1, 2-3 in 4q+3
  // (the next step's first slice after the barrier, in windows 14 and 15)
  constexpr bool kHalf0 = (U % 4 == 1 && U < 12) || (U == 14 && SWITCH);
  constexpr bool kHalf1 = (U % 4 == 3 && U < 12) || (U == 15 && SWITCH);
  if constexpr (kHalf0 || kHalf1) {
    if constexpr (U < 12) read_half(cur, U / 4 + 1, kHalf1 ? 1 : 0, wm, wn, lr, lg, s.raw);
    else read_half(nxt, 0, kHalf1 ? 1 : 0, wm, wn, lr, lg, s.raw);
  }
  // scale codes and table entries of the next slice
  if constexpr (U % 4 == 1 && U < 12) {
    read_codes(smem, st, U / 4 + 1, wm, wn, lr, lg, s.code);
  }
  if constexpr (U % 4 == 2 && U < 12) {
    lookup(smem, s.code, s.tab[(U / 4 + 1) % 2]);
  }
  if constexpr (U == 14 && SWITCH) {
    read_codes(smem, st + 1, 0, wm, wn, lr, lg, s.code);
  }
  if constexpr (DMA && U == 14) {
    issue_stage(x, st + 2, cur);
  }
  if constexpr (DMA && U == 15) {
    issue_scales(x, smem, st + 2, (st + 2) % kScaleBufs, 0);
    issue_scales(x, smem, st + 2, (st + 2) % kScaleBufs, 1);
  }
  mfma_f16_16(s.cv[U % 2], acc);
  constexpr int kRaw = (kHalf0 || kHalf1) ? 8 : 0;
  constexpr int kCodes = ((U % 4 == 1 && U < 12) || (U == 14 && SWITCH)) ? 8 : 0;
  constexpr int kLook = ((U % 4 == 2 && U < 12) || (U == 15 && SWITCH)) ? 16 : 0;
  spread_front<kConvNext ? kConvValu : 0, kRaw + kCodes + kLook, DMA ? (U == 14 ? 16 : (U == 15 ? 2 : 0)) : 0>();
  sched_fence();
  if constexpr (U == 13 && SWITCH) {
    // this wave's DMAs of stage st+1 (and its scales) have landed; after the
    // barrier every wave's have, and every wave is done reading stage st
    wait_vmcnt<0>();
    dma_barrier();
    sched_fence();
  }
}

template <int U, bool SWITCH, bool DMA>
__device__ inline void nv_windows(const PipeCtx& x, uint8_t* __restrict__ smem, uint32_t st, uint32_t wm,
                                  uint32_t wn, uint32_t lr, uint32_t lg, NvState& s, v16f (&acc)[4][4]) {
  if constexpr (U < 16) {
    nv_window<U, SWITCH, DMA>(x, smem, st, wm, wn, lr, lg, s, acc);
    nv_windows<U + 1, SWITCH, DMA>(x, smem, st, wm, wn, lr, lg, s, acc);
  }
}

// One workgroup per CU (256 accumulator registers per lane).
template <int CDT, bool GATHER>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_nv_pipe(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const float* __restrict__ a_ts,
    const int32_t* __restrict__ row_index, int64_t a_rows, int64_t R, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, const float* __restrict__ b_ts, int32_t groups,
    const int64_t* __restrict__ offsets, int64_t N, int64_t K, void* __restrict__ C, int64_t ldc,
    uint32_t tiles_n, uint32_t tiles_m_bound, uint32_t vec) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  // workgroup -> (n tile, m tile over all groups); ids on one XCD (id mod 8)
  // are adjacent
  uint32_t id = blockIdx.x;
  const uint32_t total = tiles_n * tiles_m_bound;
  if ((total & 7u) == 0) id = (id & 7u) * (total >> 3) + (id >> 3);
  const int64_t tile = id / tiles_n;
  const int64_t n0 = (int64_t)(id % tiles_n) * kTile;
  int64_t g = -1, g_lo = 0, g_hi = 0;
  if (offsets == nullptr) {
    if (tile * kTile < R) {
      g = 0;
      g_lo = tile * kTile;
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
      const int64_t nt = (hi - lo + kTile - 1) / kTile;
      if (tile < acc + nt) {
        g = e;
        g_lo = lo + (tile - acc) * kTile;
        g_hi = hi;
        break;
      }
      acc += nt;
    }
  }
  if (g < 0) return;  // surplus workgroup (uniform across the block)

  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t m0 = g_lo;
  const int64_t rowbytes = K / 2, kb = K / 16;
  const uint32_t steps = (uint32_t)(K / kStepK);
  const uint8_t* Bg = B + g * N * rowbytes;
  const uint8_t* SBg = SB + g * N * kb;
  auto src_row = [&](int64_t rr) -> int64_t {  // routed row (clamped to the group) -> A row
    rr = rr < g_hi ? rr : g_hi - 1;
    if constexpr (GATHER) {
      int64_t s = row_index[rr];
      s = s < 0 ? 0 : s;
      return s < a_rows ? s : a_rows - 1;
    } else {
      return rr;
    }
  };

  // E4M3 decode table (published to the other waves by the prologue barrier)
  *reinterpret_cast<TabE*>(smem + kTabBase + t * 8) = nv_tab_entry(t);

  PipeCtx x;
  x.wid = __builtin_amdgcn_readfirstlane(wid);
  x.nper = steps;  // one scale period (16 bytes per row) per step
  const bool waveA = wid < 2;
  x.cbase = waveA ? A : Bg;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t r = 8u * (16u * wid + i) + (lane >> 3);
    const uint32_t c = (lane & 7u) ^ swz(r);
    int64_t grow;
    if (waveA) {
      grow = src_row(m0 + (r & (kTile - 1)));
    } else {
      grow = n0 + (r & (kTile - 1));
      grow = grow < N ? grow : N - 1;
    }
    x.coff[i] = (uint32_t)(grow * rowbytes) + 16u * c;
  }
  x.sA = SA;
  x.sB = SBg;
  {
    const int64_t ga = src_row(m0 + 64 * wid + lane);
    int64_t gb = n0 + 64 * wid + lane;
    gb = gb < N ? gb : N - 1;
    x.soffA = (uint32_t)(ga * kb);
    x.soffB = (uint32_t)(gb * kb);
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  issue_stage(x, 0, smem);
  issue_scales(x, smem, 0, 0, 0);
  issue_scales(x, smem, 0, 0, 1);
  issue_scales(x, smem, 1, 1, 0);
  issue_scales(x, smem, 1, 1, 1);
  if (steps > 1) {
    issue_stage(x, 1, smem + kStageBytes);
    wait_vmcnt<16>();  // stage 0 and the scales of steps 0 and 1
  } else {
    wait_vmcnt<0>();
  }
  dma_barrier();
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  NvState s;
  read_codes(smem, 0, 0, wm, wn, lr, lg, s.code);
  lookup(smem, s.code, s.tab[0]);
  read_half(smem, 0, 0, wm, wn, lr, lg, s.raw);
  read_half(smem, 0, 1, wm, wn, lr, lg, s.raw);
  conv_unit(s.raw, 0, s.tab[0], s.cv[0]);
  sched_fence();
  uint32_t st = 0;
  for (; st + 2 < steps; ++st) nv_windows<0, true, true>(x, smem, st, wm, wn, lr, lg, s, acc);
  if (st + 1 < steps) {
    nv_windows<0, true, false>(x, smem, st, wm, wn, lr, lg, s, acc);
    ++st;
  }
  nv_windows<0, false, false>(x, smem, st, wm, wn, lr, lg, s, acc);

  const float sab = *a_ts * b_ts[g];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] *= sab;
  // epilogue: LDS is free once every wave is past its last read
  dma_barrier();
  store_tile<CDT>(smem, acc, C, ldc, g_hi, N, m0 + wm * 128, n0 + wn * 128, vec != 0, wid, lane);
}

template <int CDT, bool GATHER>
hipError_t launch_nv(const uint8_t* a, const uint8_t* sa, const float* ats, const int32_t* ri, int64_t a_rows,
                     int64_t R, const uint8_t* b, const uint8_t* sb, const float* bts, int32_t groups,
                     const int64_t* off, int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const uint32_t tn = (uint32_t)((N + kTile - 1) / kTile);
  const uint32_t tmb = (uint32_t)((R + kTile - 1) / kTile + (off ? groups : 0));
  auto kern = k_gemm_nv_pipe<CDT, GATHER>;
  // the dynamic LDS limit is raised once per device
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kNvSmem);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int64_t eb = CDT == DT_F32 ? 4 : 2;
  const uint32_t vec = ((reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * eb) % 16 == 0) ? 1u : 0u;
  hipLaunchKernelGGL(kern, dim3(tn * tmb), dim3(256), kNvSmem, s, a, sa, ats, ri, a_rows, R, b, sb, bts, groups,
                     off, N, K, C, ldc, tn, tmb, vec);
  return hipGetLastError();
}

}  // namespace

bool gemm_nvfp4_pipe_fits(int64_t a_rows, int64_t R, int64_t N, int64_t K) {
  // K in whole steps; 32-bit byte offsets within A and within one expert's B
  return K >= kStepK && K % kStepK == 0 && a_rows * (K / 2) < ((int64_t)1 << 32) - 4096 &&
         N * (K / 2) < ((int64_t)1 << 32) - 4096 && R * N >= (int64_t)kTile * kTile * 64;
}

hipError_t launch_gemm_nvfp4_pipe(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                                  const int32_t* row_index, int64_t a_rows, int64_t routed_rows,
                                  const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                                  int32_t groups, const int64_t* offsets, int64_t N, int64_t K, void* C,
                                  int cdt, int64_t ldc, hipStream_t s) {
#define MXK_NVP(D, G)                                                                                       \
  launch_nv<D, G>(a_codes, a_scales, a_ts, row_index, a_rows, routed_rows, b_codes, b_scales, b_ts, groups, \
                  offsets, N, K, C, ldc, s)
  if (row_index) return cdt == DT_F32 ? MXK_NVP(DT_F32, true) : MXK_NVP(DT_BF16, true);
  return cdt == DT_F32 ? MXK_NVP(DT_F32, false) : MXK_NVP(DT_BF16, false);
#undef MXK_NVP
}

}  // namespace mxk
