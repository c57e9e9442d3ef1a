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
// The FP4 form of this instruction runs at twice the FP8 rate; the 16x16x128
// FP4 form only at the FP8 rate (measured), so 32x32x64 is used.
//
// MXFP4 is exact on this instruction (FP32 accumulation of exact products).
// The FP8 variant is the hardware-native MXFP8 path: gfx950 sums the FP8
// products of each 8-element group in a narrow aligned window (about 14 bits
// below the group's largest product) before FP32 accumulation, so it does not
// meet a 1e-5 relative bound in general; the exact MXFP8 GEMM is the
// BF16-staged kernel in gemm_staged.hip.
//
// Pipelined kernel (K a multiple of the step): 256 threads (4 waves, 2x2), a
// 256x256 C tile per workgroup, 128x128 per wave (4x4 instruction tiles, 256
// accumulator registers), one workgroup per CU.  Each K step moves one
// 128-byte segment per row (FP4: 256 elements, four instruction slices; FP8:
// 128 elements, two) plus the row's scale bytes of the step, straight from
// global memory into LDS with global_load_lds (no register staging), two
// stage buffers deep.  Full 128-byte segments stream markedly faster than
// half lines (measured).  The 16-byte chunks of a row are XOR-swizzled by
// ((row >> 1) & 7), so fragment reads of 16 consecutive rows hit distinct
// bank groups.  Slice fragments are double-buffered in registers; a wave waits for
// the next stage and joins the one barrier of the step just before the last
// slice's matrix instructions, so the refill of the stage just consumed and
// the first reads of the next stage overlap that slice.  The epilogue
// stages each wave's accumulator tile through LDS and writes C rows with
// 16-byte stores.  Workgroup -> tile mapping keeps the tiles of one XCD
// (workgroups are dealt round-robin over the 8 XCDs) adjacent in M and N for
// L2 reuse.
//
// A simple kernel (register-staged, 128x128 tiles, any K % 32 == 0) covers
// shapes the pipelined one does not take.
#include <atomic>

#include "../device/codec.h"
#include "../device/gemm_common.h"
#include "../device/pipe.h"
#include "../launch.h"

namespace mxk {

namespace {


template <int FMT>
struct StepCfg {
  static constexpr int kKElems = FMT == FMT_MXFP8 ? 64 : 128;  // K elements per step
  static constexpr int kInstr = FMT == FMT_MXFP8 ? 1 : 2;      // instructions per step
  static constexpr int kBlocks = kKElems / 32;                 // scale bytes per row per step
};


template <int CDT>
__device__ inline void store_c(void* C, int64_t ldc, int64_t row, int64_t col, float v) {
  if constexpr (CDT == DT_F32) static_cast<float*>(C)[row * ldc + col] = v;
  else static_cast<uint16_t*>(C)[row * ldc + col] = f32_to_bf16(v);
}

// ---------------------------------------------------------------------------
// pipelined kernel (stage layout and DMA helpers: device/pipe.h)
// ---------------------------------------------------------------------------
// K slices (64-element instructions) per step and scale dwords per row
template <int FMT>
struct PipeCfg {
  static constexpr int kSlices = FMT == FMT_MXFP8 ? 2 : 4;
  static constexpr int kKElems = FMT == FMT_MXFP8 ? 128 : 256;
  static constexpr int kScaleDw = FMT == FMT_MXFP8 ? 1 : 2;      // scale dwords per row and step
  static constexpr int kPeriod = kScaleRow / (4 * kScaleDw);       // steps per scale period
};

// Fragments of one K slice for one wave (16 bytes per operand tile; FP8 keeps
// the lane's second 16 bytes in the *hi arrays).
template <int FMT>
struct Slice {
  u4 a[4], b[4];
  u4 ahi[FMT == FMT_MXFP8 ? 4 : 1], bhi[FMT == FMT_MXFP8 ? 4 : 1];
};

template <int FMT>
__device__ inline void load_slice(const uint8_t* __restrict__ L, uint32_t q, uint32_t wm, uint32_t wn,
                                  uint32_t lr, uint32_t lg, Slice<FMT>& f) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t r = t < 4 ? wm * 128 + t * 32 + lr : kTile + wn * 128 + (t - 4) * 32 + lr;
    if constexpr (FMT == FMT_MXFP8) {
      const u4 x0 = *reinterpret_cast<const u4*>(L + chunk_off(r, 4 * q + lg));
      const u4 x1 = *reinterpret_cast<const u4*>(L + chunk_off(r, 4 * q + 2 + lg));
      if (t < 4) { f.a[t] = x0; f.ahi[t] = x1; }
      else { f.b[t - 4] = x0; f.bhi[t - 4] = x1; }
    } else {
      const u4 x0 = *reinterpret_cast<const u4*>(L + chunk_off(r, 2 * q + lg));
      if (t < 4) f.a[t] = x0;
      else f.b[t - 4] = x0;
    }
  }
}

// raw scale dwords of the wave's rows for one stage
struct Scales {
  uint32_t a[2][4], b[2][4];
};
// Scale dwords of step `step` for the wave's rows (FP4: two per row, one
// 64-bit read; FP8: one).
template <int FMT>
__device__ inline void load_scales(const uint8_t* __restrict__ smem, uint32_t step, uint32_t wm,
                                   uint32_t wn, uint32_t lr, Scales& s) {
  constexpr uint32_t P = PipeCfg<FMT>::kPeriod;
  const uint8_t* LS = smem + kScaleBase + ((step / P) % kScaleBufs) * kScaleBuf +
                      (step % P) * (4 * PipeCfg<FMT>::kScaleDw);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t ra = wm * 128 + i * 32 + lr, rb = kTile + wn * 128 + i * 32 + lr;
    if constexpr (FMT == FMT_MXFP8) {
      s.a[0][i] = *reinterpret_cast<const uint32_t*>(LS + ra * kScaleRow);
      s.b[0][i] = *reinterpret_cast<const uint32_t*>(LS + rb * kScaleRow);
    } else {
      const uint2 va = *reinterpret_cast<const uint2*>(LS + ra * kScaleRow);
      const uint2 vb = *reinterpret_cast<const uint2*>(LS + rb * kScaleRow);
      s.a[0][i] = va.x; s.a[1][i] = va.y;
      s.b[0][i] = vb.x; s.b[1][i] = vb.y;
    }
  }
}

__device__ inline v8i widen(u4 lo, u4 hi) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}
__device__ inline v8i widen4(u4 lo) {
  return v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
}

// Scale dwords shifted so that byte 0 / byte 2 (selected by opsel) are
// this lane's K-blocks: lane group lg (lanes 32..63) takes the odd blocks.
__device__ inline void shift_scales(const Scales& in, uint32_t lg, Scales& out) {
#pragma unroll
  for (int d = 0; d < 2; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out.a[d][i] = in.a[d][i] >> (8 * lg);
      out.b[d][i] = in.b[d][i] >> (8 * lg);
    }
}

// 16 MFMAs of K slice q with pre-shifted scales.  The lane's scale byte for
// slice q is byte (2q + lg) of the step's scale bytes: dword (2q + lg) / 4,
// after the shift by lg bytes selected by opsel = 2 * (q % 2) (FP4), or
// opsel = 2q (FP8, one dword per step).
// Matrix-instruction element types (cbsz / blgp) of A and B: FP8 E4M3 0,
// E5M2 1 (MX_GEMM_FP8_NATIVE pairs), FP4 4.
template <int FMT>
constexpr int kType = FMT == FMT_MXFP8 ? 0 : 4;

template <int FMT, int Q, int TA, int TB>
__device__ inline void mfma_slice(const Slice<FMT>& f, const Scales& sh, v16f (&acc)[4][4]) {
  constexpr int D = FMT == FMT_MXFP8 ? 0 : Q / 2;
  constexpr int OPSEL = FMT == FMT_MXFP8 ? 2 * Q : 2 * (Q % 2);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (FMT == FMT_MXFP8)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen(f.a[i], f.ahi[i]), widen(f.b[j], f.bhi[j]), acc[i][j], TA, TB, OPSEL, (int)sh.a[D][i], OPSEL, (int)sh.b[D][j]);
      else
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(widen4(f.a[i]), widen4(f.b[j]), acc[i][j], 4, 4, OPSEL, (int)sh.a[D][i], OPSEL, (int)sh.b[D][j]);
    }
}

// Register state of the pipeline: slice fragments (double-buffered), the
// scale dwords of the current and the next stage, and the current ones
// shifted for this lane.
template <int FMT>
struct PipeState {
  Slice<FMT> s[PipeCfg<FMT>::kSlices];  // one buffer per slice of a step
  Scales sc, scn, sh;
};

// One K step.  SWITCH: a next stage exists; DMA: refill the buffer of the
// stage being consumed with stage st + 2.
//
// FP4 (four slices, one fragment buffer each):
//   W0: MFMAs of slice 0 | LDS reads of slices 1 and 2
//   W1: MFMAs of slice 1 | LDS reads of slice 3
//   wait for this wave's DMAs of stage st+1; barrier (every wave holds all
//   of stage st in registers and stage st+1 has landed)
//   W2: MFMAs of slice 2 | DMAs of stage st+2 into the buffer just released
//   W3: MFMAs of slice 3 | LDS reads of stage st+1's scales and slice 0
// FP8 (two slices):
//   W0: MFMAs of slice 0 | LDS reads of slice 1
//   wait; barrier
//   W1: MFMAs of slice 1 | DMAs of stage st+2, reads of st+1's scales and
//       slice 0
// Spreading the DMAs over matrix work keeps their issue from stalling it.
template <int FMT, bool SWITCH, bool DMA, int TA, int TB>
__device__ inline void pipe_step(const PipeCtx& x, uint8_t* __restrict__ smem, uint32_t st,
                                 uint32_t wm, uint32_t wn, uint32_t lr, uint32_t lg,
                                 PipeState<FMT>& ps, v16f (&acc)[4][4]) {
  uint8_t* cur = smem + (st & 1u) * kStageBytes;
  uint8_t* nxt = smem + ((st + 1u) & 1u) * kStageBytes;
  // the scale reads precede slice 0's reads: waiting for them leaves those
  // in flight
  shift_scales(ps.sc, lg, ps.sh);
  sched_fence();
  if constexpr (FMT == FMT_MXFP4) {
    load_slice<FMT>(cur, 1, wm, wn, lr, lg, ps.s[1]);
    load_slice<FMT>(cur, 2, wm, wn, lr, lg, ps.s[2]);
    mfma_slice<FMT, 0, TA, TB>(ps.s[0], ps.sh, acc);
    interleave<8, 0, 2>();
    sched_fence();
    load_slice<FMT>(cur, 3, wm, wn, lr, lg, ps.s[3]);
    mfma_slice<FMT, 1, TA, TB>(ps.s[1], ps.sh, acc);
    interleave<8, 0, 1>();
    sched_fence();
    if constexpr (SWITCH) {
      wait_vmcnt<0>();
      dma_barrier();
      sched_fence();
      if constexpr (DMA) {
        issue_stage(x, st + 2, cur);
        const uint32_t q = st / PipeCfg<FMT>::kPeriod + 2;
        issue_scales(x, smem, q, q % kScaleBufs, st & 1u);
      }
      mfma_slice<FMT, 2, TA, TB>(ps.s[2], ps.sh, acc);
      interleave<16, 1, 0>();
      sched_fence();
      load_scales<FMT>(smem, st + 1, wm, wn, lr, ps.scn);
      load_slice<FMT>(nxt, 0, wm, wn, lr, lg, ps.s[0]);
      mfma_slice<FMT, 3, TA, TB>(ps.s[3], ps.sh, acc);
      interleave<8, 0, 3>();
      sched_fence();
      ps.sc = ps.scn;
    } else {
      mfma_slice<FMT, 2, TA, TB>(ps.s[2], ps.sh, acc);
      mfma_slice<FMT, 3, TA, TB>(ps.s[3], ps.sh, acc);
      sched_fence();
    }
  } else {
    load_slice<FMT>(cur, 1, wm, wn, lr, lg, ps.s[1]);
    mfma_slice<FMT, 0, TA, TB>(ps.s[0], ps.sh, acc);
    interleave<8, 0, 2>();
    sched_fence();
    if constexpr (SWITCH) {
      wait_vmcnt<0>();
      dma_barrier();
      sched_fence();
      if constexpr (DMA) {
        issue_stage(x, st + 2, cur);
        const uint32_t q = st / PipeCfg<FMT>::kPeriod + 2;
        issue_scales(x, smem, q, q % kScaleBufs, st & 1u);
      }
      load_scales<FMT>(smem, st + 1, wm, wn, lr, ps.scn);
      load_slice<FMT>(nxt, 0, wm, wn, lr, lg, ps.s[0]);
      mfma_slice<FMT, 1, TA, TB>(ps.s[1], ps.sh, acc);
      interleave<12, 2, 2>();
      sched_fence();
      ps.sc = ps.scn;
    } else {
      mfma_slice<FMT, 1, TA, TB>(ps.s[1], ps.sh, acc);
      sched_fence();
    }
  }
}

// One workgroup per CU (256 accumulator registers per lane).
template <int FMT, int CDT, int TA = kType<FMT>, int TB = kType<FMT>>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx_pipe(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t vec) {
  using PC = PipeCfg<FMT>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * kTile, n0 = (int64_t)tni * kTile;
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t rowbytes = FMT == FMT_MXFP8 ? K : K / 2;
  const int64_t kblocks = K / 32;
  const uint32_t steps = (uint32_t)(K / PC::kKElems);

  // Code instruction i of wave w: LDS row r = 8*(16w+i) + lane/8, physical
  // chunk p = lane%8 holding logical chunk p ^ swz(r).  Rows past M / N read
  // the last valid row (their results are not stored).
  PipeCtx x;
  x.wid = __builtin_amdgcn_readfirstlane(wid);  // wave-uniform: LDS bases in scalar registers
  x.nper = steps / PC::kPeriod;
  const bool waveA = wid < 2;
  x.cbase = waveA ? A : B;
  const int64_t lim = waveA ? M : N;
  const int64_t row0 = waveA ? m0 : n0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t r = 8u * (16u * wid + i) + (lane >> 3);
    const uint32_t c = (lane & 7u) ^ swz(r);
    int64_t grow = row0 + (r & (kTile - 1));
    grow = grow < lim ? grow : lim - 1;
    x.coff[i] = (uint32_t)(grow * rowbytes) + 16u * c;
  }
  x.sA = SA;
  x.sB = SB;
  {
    int64_t ga = m0 + 64 * wid + lane, gb = n0 + 64 * wid + lane;
    ga = ga < M ? ga : M - 1;
    gb = gb < N ? gb : N - 1;
    x.soffA = (uint32_t)(ga * kblocks);
    x.soffB = (uint32_t)(gb * kblocks);
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Two LDS stages.  Within stage st the K slices run with their fragments
  // double-buffered in registers; before the last slice of stage st the wave
  // waits for stage st+1's DMAs and joins the barrier (all waves then hold
  // every fragment of stage st, so its buffer is refilled with stage st+2)
  // and starts reading stage st+1's first slice.  The loop body has no
  // branch (the last two steps are peeled), so the matrix instructions stay
  // where they are written.
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  issue_stage(x, 0, smem);
  issue_scales(x, smem, 0, 0, 0);
  issue_scales(x, smem, 0, 0, 1);
  issue_scales(x, smem, 1, 1, 0);
  issue_scales(x, smem, 1, 1, 1);
  if (steps > 1) {
    issue_stage(x, 1, smem + kStageBytes);
    wait_vmcnt<16>();  // stage 0 and the first two scale periods
  } else {
    wait_vmcnt<0>();
  }
  dma_barrier();
  PipeState<FMT> ps;
  load_scales<FMT>(smem, 0, wm, wn, lr, ps.sc);
  load_slice<FMT>(smem, 0, wm, wn, lr, lg, ps.s[0]);
  uint32_t st = 0;
  for (; st + 2 < steps; ++st) pipe_step<FMT, true, true, TA, TB>(x, smem, st, wm, wn, lr, lg, ps, acc);
  if (st + 1 < steps) {
    pipe_step<FMT, true, false, TA, TB>(x, smem, st, wm, wn, lr, lg, ps, acc);
    ++st;
  }
  pipe_step<FMT, false, false, TA, TB>(x, smem, st, wm, wn, lr, lg, ps, acc);

  // epilogue: LDS is free once every wave is past its last fragment read
  dma_barrier();
  store_tile<CDT>(smem, acc, C, ldc, M, N, m0 + wm * 128, n0 + wn * 128, vec != 0, wid, lane);
}

template <int FMT, int CDT, int TA = kType<FMT>, int TB = kType<FMT>>
hipError_t launch_pipe(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                       int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const uint32_t tm = (uint32_t)((M + kTile - 1) / kTile), tn = (uint32_t)((N + kTile - 1) / kTile);
  const size_t smem = (size_t)kSmemBytes;
  auto kern = k_gemm_mx_pipe<FMT, CDT, TA, TB>;
  // The dynamic LDS limit is raised once per device (bit d of a mask), so
  // that later launches -- including those recorded into a HIP graph --
  // make no call beyond the launch itself.
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  // 16-byte row stores need a 16-byte aligned C and row pitch
  const int64_t eb = CDT == DT_F32 ? 4 : 2;
  const uint32_t vec = ((reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * eb) % 16 == 0) ? 1u : 0u;
  hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(256), smem, s, a, sa, b, sb, M, N, K, C, ldc, tm, tn, vec);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// exact MXFP8: the same DMA pipeline feeding the BF16 instruction
// ---------------------------------------------------------------------------
// gfx950's FP8 instruction is not exact (see above), so the exact MXFP8 GEMM
// contracts on v_mfma_f32_32x32x16_bf16: E4M3 * 2^(c-127) is exact in BF16
// for scale codes c in [3, 246].  The FP8 stages land in LDS exactly as for
// the native kernel.  For each 32-element K-block b of a step, lane
// (r = l mod 32, g = l / 32) reads its row's 16-byte chunk 2b + g (the FP8
// fragment read, conflict-free under the swizzle), converts it with the
// block's scale (v_cvt_scalef32_pk_bf16_fp8 scales by the exponent of its
// FP32 operand, i.e. by the E8M0 value) and feeds two BF16 instructions:
// chunk bytes 0..7, then 8..15.  A and B use the same assignment of K
// positions to (instruction, lane group, element), so each instruction sums
// exactly the products of its 16 positions and every block's 32 products are
// summed.  Conversion costs two VALU instructions per matrix instruction and
// runs between them; reads and conversions run one half-block ahead.
//
// Scale codes 0 (2^-127, an FP32 subnormal the converter does not take as a
// scale) and 255 (NaN) are not converted correctly here: the launcher follows
// this kernel with the staged kernel in fix-up mode, which recomputes
// exactly every output tile whose operand rows hold such a code.

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf_x __attribute__((ext_vector_type(2)));

// 8 BF16 values (element 2k in the low half of word k) from the 8 FP8 codes
// in w0, w1, scaled by E8M0 code c (1 .. 254).
// F: the element type of the codes -- FMT_MXFP8 (E4M3), FMT_MXFP8_E5M2
// (v_cvt_scalef32_pk_bf16_bf8) or FMT_MXINT8.  INT8 code k (two's
// complement) means k * 2^-6: with u = k + 128 (the byte with its top bit
// flipped), u * X' - 128 X' = k X' exactly (X' = 2^(c-133)), a value of at
// most 8 significant bits, so its top 16 bits are its exact BF16 whenever it
// is a normal BF16 value (scale codes 7 .. 254).
template <int F>
__device__ inline u4 conv8(uint32_t w0, uint32_t w1, uint32_t c) {
  const float X = u2f(c << 23);
  u4 o;
  if constexpr (F == FMT_MXINT8) {
    const float Xs = X * 0.015625f, off = -128.0f * Xs;  // both exact
    const uint32_t u[2] = {w0 ^ 0x80808080u, w1 ^ 0x80808080u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t wd = u[k >> 1], sh = 16 * (k & 1);
      const float lo = __builtin_fmaf((float)((wd >> sh) & 0xFFu), Xs, off);
      const float hi = __builtin_fmaf((float)((wd >> (sh + 8)) & 0xFFu), Xs, off);
      // both exact in BF16: the pack's rounding changes nothing
      o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v2f{lo, hi}, v2bf_x));
    }
  } else if constexpr (F == FMT_MXFP8_E5M2) {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, X, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w0, X, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, X, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8(w1, X, true));
  } else {
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, X, false));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, X, true));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, X, false));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, X, true));
  }
  return o;
}

// Register state: raw chunks of two blocks, the converted halves, and the
// scale dwords (byte b: block b of the step) of the current and next step.
struct XState {
  u4 raw[2][8];  // [block parity][A 0..3, B 4..7]
  u4 lo[8], hi[8];
  uint32_t sc[8], scn[8];
};

__device__ inline void read_raw(const uint8_t* __restrict__ L, uint32_t b, uint32_t wm, uint32_t wn,
                                uint32_t lr, uint32_t lg, u4 (&raw)[8]) {
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const uint32_t r = t < 4 ? wm * 128 + t * 32 + lr : kTile + wn * 128 + (t - 4) * 32 + lr;
    raw[t] = *reinterpret_cast<const u4*>(L + chunk_off(r, 2 * b + lg));
  }
}

// half H (0: chunk bytes 0..7, 1: 8..15) of block b (scale byte b); FA / FB:
// the element types of A (tiles 0..3) and B (tiles 4..7)
template <int H, int BA, int BB>
__device__ inline void conv_half(const u4 (&raw)[8], const uint32_t (&sc)[8], uint32_t b, u4 (&out)[8]) {
#pragma unroll
  for (int t = 0; t < 4; ++t) out[t] = conv8<BA>(raw[t][2 * H], raw[t][2 * H + 1], (sc[t] >> (8 * b)) & 0xFFu);
#pragma unroll
  for (int t = 4; t < 8; ++t) out[t] = conv8<BB>(raw[t][2 * H], raw[t][2 * H + 1], (sc[t] >> (8 * b)) & 0xFFu);
}

__device__ inline void mfma_bf16_16(const u4 (&f)[8], v16f (&acc)[4][4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, f[i]),
                                                          __builtin_bit_cast(v8bf, f[4 + j]), acc[i][j], 0, 0, 0);
}

__device__ inline void load_scales_x(const uint8_t* __restrict__ smem, uint32_t step, uint32_t wm, uint32_t wn,
                                     uint32_t lr, uint32_t (&s)[8]) {
  Scales t;
  load_scales<FMT_MXFP8>(smem, step, wm, wn, lr, t);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[i] = t.a[0][i];
    s[4 + i] = t.b[0][i];
  }
}

// One K step (4 blocks, 8 half-block windows of 16 instructions):
//   H0 b0 lo | convert b0 hi              H1 b0 hi | convert b1 lo, read b2
//   H2 b1 lo | convert b1 hi              H3 b1 hi | convert b2 lo, read b3
//   wait for this wave's DMAs of stage st+1; barrier
//   H4 b2 lo | convert b2 hi, DMAs        H5 b2 hi | convert b3 lo, read b0',
//                                                     scales of st+1
//   H6 b3 lo | convert b3 hi              H7 b3 hi | convert b0' lo, read b1'
// (primes: stage st+1).  SWITCH: a next stage exists; DMA: refill the buffer
// just consumed with stage st+2.
template <bool SWITCH, bool DMA, int BA, int BB>
__device__ inline void exact_step(const PipeCtx& x, uint8_t* __restrict__ smem, uint32_t st, uint32_t wm,
                                  uint32_t wn, uint32_t lr, uint32_t lg, XState& xs, v16f (&acc)[4][4]) {
  uint8_t* cur = smem + (st & 1u) * kStageBytes;
  uint8_t* nxt = smem + ((st + 1u) & 1u) * kStageBytes;
  // VALU per conversion window (FP8: 32 conversions + scale bytes; INT8 about
  // 11 per 4 elements)
  constexpr int CV = (BA == FMT_MXINT8 ? 90 : 20) + (BB == FMT_MXINT8 ? 90 : 20);
  // H0
  conv_half<1, BA, BB>(xs.raw[0], xs.sc, 0, xs.hi);
  mfma_bf16_16(xs.lo, acc);
  spread_x<CV, 0, 0>();
  sched_fence();
  // H1
  conv_half<0, BA, BB>(xs.raw[1], xs.sc, 1, xs.lo);
  read_raw(cur, 2, wm, wn, lr, lg, xs.raw[0]);
  mfma_bf16_16(xs.hi, acc);
  spread_x<CV, 8, 0>();
  sched_fence();
  // H2
  conv_half<1, BA, BB>(xs.raw[1], xs.sc, 1, xs.hi);
  mfma_bf16_16(xs.lo, acc);
  spread_x<CV, 0, 0>();
  sched_fence();
  // H3
  conv_half<0, BA, BB>(xs.raw[0], xs.sc, 2, xs.lo);
  read_raw(cur, 3, wm, wn, lr, lg, xs.raw[1]);
  mfma_bf16_16(xs.hi, acc);
  spread_x<CV, 8, 0>();
  sched_fence();
  if constexpr (SWITCH) {
    wait_vmcnt<0>();
    dma_barrier();
    sched_fence();
  }
  // H4
  if constexpr (DMA) {
    issue_stage(x, st + 2, cur);
    const uint32_t q = st / PipeCfg<FMT_MXFP8>::kPeriod + 2;
    issue_scales(x, smem, q, q % kScaleBufs, st & 1u);
  }
  conv_half<1, BA, BB>(xs.raw[0], xs.sc, 2, xs.hi);
  mfma_bf16_16(xs.lo, acc);
  spread_x<CV, 0, DMA ? 17 : 0>();
  sched_fence();
  // H5
  conv_half<0, BA, BB>(xs.raw[1], xs.sc, 3, xs.lo);
  if constexpr (SWITCH) {
    read_raw(nxt, 0, wm, wn, lr, lg, xs.raw[0]);
    load_scales_x(smem, st + 1, wm, wn, lr, xs.scn);
  }
  mfma_bf16_16(xs.hi, acc);
  spread_x<CV, SWITCH ? 12 : 0, 0>();
  sched_fence();
  // H6
  conv_half<1, BA, BB>(xs.raw[1], xs.sc, 3, xs.hi);
  mfma_bf16_16(xs.lo, acc);
  spread_x<CV, 0, 0>();
  sched_fence();
  // H7
  if constexpr (SWITCH) {
    conv_half<0, BA, BB>(xs.raw[0], xs.scn, 0, xs.lo);
    read_raw(nxt, 1, wm, wn, lr, lg, xs.raw[1]);
  }
  mfma_bf16_16(xs.hi, acc);
  spread_x<SWITCH ? CV : 0, SWITCH ? 8 : 0, 0>();
  sched_fence();
  if constexpr (SWITCH) {
#pragma unroll
    for (int t = 0; t < 8; ++t) xs.sc[t] = xs.scn[t];
  }
}

template <int CDT, int BA, int BB>
__device__ inline void exact_body(const PipeCtx& x, uint8_t* __restrict__ smem, uint32_t steps, uint32_t wm,
                                  uint32_t wn, uint32_t lr, uint32_t lg, uint32_t wid, uint32_t lane,
                                  void* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t m0,
                                  int64_t n0, uint32_t vec) {
  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  XState xs;
  load_scales_x(smem, 0, wm, wn, lr, xs.sc);
  read_raw(smem, 0, wm, wn, lr, lg, xs.raw[0]);
  read_raw(smem, 1, wm, wn, lr, lg, xs.raw[1]);
  conv_half<0, BA, BB>(xs.raw[0], xs.sc, 0, xs.lo);
  sched_fence();
  uint32_t st = 0;
  for (; st + 2 < steps; ++st) exact_step<true, true, BA, BB>(x, smem, st, wm, wn, lr, lg, xs, acc);
  if (st + 1 < steps) {
    exact_step<true, false, BA, BB>(x, smem, st, wm, wn, lr, lg, xs, acc);
    ++st;
  }
  exact_step<false, false, BA, BB>(x, smem, st, wm, wn, lr, lg, xs, acc);
  dma_barrier();
  store_tile<CDT>(smem, acc, C, ldc, M, N, m0 + wm * 128, n0 + wn * 128, vec != 0, wid, lane);
}

template <int CDT, int BA, int BB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx8_exact(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ C,
    int64_t ldc, uint32_t tiles_m, uint32_t tiles_n, uint32_t vec) {
  using PC = PipeCfg<FMT_MXFP8>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * kTile, n0 = (int64_t)tni * kTile;
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t rowbytes = K;
  const int64_t kblocks = K / 32;
  const uint32_t steps = (uint32_t)(K / PC::kKElems);

  PipeCtx x;
  x.wid = __builtin_amdgcn_readfirstlane(wid);
  x.nper = steps / PC::kPeriod;
  const bool waveA = wid < 2;
  x.cbase = waveA ? A : B;
  const int64_t lim = waveA ? M : N;
  const int64_t row0 = waveA ? m0 : n0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t r = 8u * (16u * wid + i) + (lane >> 3);
    const uint32_t c = (lane & 7u) ^ swz(r);
    int64_t grow = row0 + (r & (kTile - 1));
    grow = grow < lim ? grow : lim - 1;
    x.coff[i] = (uint32_t)(grow * rowbytes) + 16u * c;
  }
  x.sA = SA;
  x.sB = SB;
  {
    int64_t ga = m0 + 64 * wid + lane, gb = n0 + 64 * wid + lane;
    ga = ga < M ? ga : M - 1;
    gb = gb < N ? gb : N - 1;
    x.soffA = (uint32_t)(ga * kblocks);
    x.soffB = (uint32_t)(gb * kblocks);
  }
  issue_stage(x, 0, smem);
  issue_scales(x, smem, 0, 0, 0);
  issue_scales(x, smem, 0, 0, 1);
  issue_scales(x, smem, 1, 1, 0);
  issue_scales(x, smem, 1, 1, 1);
  if (steps > 1) issue_stage(x, 1, smem + kStageBytes);
  if (steps > 1) {
    wait_vmcnt<16>();  // stage 0 and the first two scale periods
  } else {
    wait_vmcnt<0>();
  }
  dma_barrier();
  exact_body<CDT, BA, BB>(x, smem, steps, wm, wn, lane & 31u, lane >> 5, wid, lane, C, ldc, M, N, m0, n0, vec);
}

template <int CDT, int BA, int BB>
hipError_t launch_exact(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb,
                        int64_t M, int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const uint32_t tm = (uint32_t)((M + kTile - 1) / kTile), tn = (uint32_t)((N + kTile - 1) / kTile);
  const size_t smem = (size_t)kSmemBytes;
  auto kern = k_gemm_mx8_exact<CDT, BA, BB>;
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  const int64_t eb = CDT == DT_F32 ? 4 : 2;
  const uint32_t vec = ((reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * eb) % 16 == 0) ? 1u : 0u;
  hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(256), smem, s, a, sa, b, sb, M, N, K, C, ldc, tm, tn, vec);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// simple kernel: register-staged double buffer, 128x128 tiles, any K % 32
// ---------------------------------------------------------------------------
constexpr int kPitchS = 80;  // LDS bytes per row: 64 code bytes, 4 scale bytes, pad

template <int FMT, int CDT, int TA = kType<FMT>, int TB = kType<FMT>>
__global__ __launch_bounds__(256) void k_gemm_mx_simple(const uint8_t* __restrict__ A,
                                                        const uint8_t* __restrict__ SA,
                                                        const uint8_t* __restrict__ B,
                                                        const uint8_t* __restrict__ SB, int64_t M,
                                                        int64_t N, int64_t K, void* __restrict__ C,
                                                        int64_t ldc, uint32_t tiles_m,
                                                        uint32_t tiles_n) {
  using SC = StepCfg<FMT>;
  constexpr int BM = 128, BN = 128, kRows = BM + BN;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kRows * kPitchS];
  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * BM, n0 = (int64_t)tni * BN;
  const uint32_t t = threadIdx.x;
  const uint32_t lane = t & 63u, wid = t >> 6;
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const int64_t rowbytes = FMT == FMT_MXFP8 ? K : K / 2;
  const int64_t kblocks = K / 32;
  const int64_t steps = (K + SC::kKElems - 1) / SC::kKElems;

  uint4 reg[4];
  uint32_t sreg = 0;
  auto load_step = [&](int64_t step) {
    const int64_t kb = step * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p = t + 256u * j;
      const uint32_t r = p >> 2;
      const bool isA = r < (uint32_t)BM;
      const int64_t grow = isA ? m0 + r : n0 + (r - BM);
      const int64_t off = kb + (p & 3u) * 16;
      reg[j] = (grow < (isA ? M : N) && off < rowbytes)
                   ? *reinterpret_cast<const uint4*>((isA ? A : B) + grow * rowbytes + off)
                   : make_uint4(0, 0, 0, 0);
    }
    const bool isA = t < (uint32_t)BM;
    const int64_t grow = isA ? m0 + t : n0 + (t - BM);
    const int64_t b0 = step * SC::kBlocks;
    uint32_t w = 0;
    if (grow < (isA ? M : N))
      for (int i = 0; i < SC::kBlocks; ++i)
        if (b0 + i < kblocks) w |= (uint32_t)(isA ? SA : SB)[grow * kblocks + b0 + i] << (8 * i);
    sreg = w;
  };
  auto store_step = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t p = t + 256u * j;
      *reinterpret_cast<uint4*>(&lds[buf][(p >> 2) * kPitchS + (p & 3u) * 16]) = reg[j];
    }
    *reinterpret_cast<uint32_t*>(&lds[buf][t * kPitchS + 64]) = sreg;
  };

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
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
    uint32_t sa[2], sb[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      sa[i] = *reinterpret_cast<const uint32_t*>(L + (wm * 64 + i * 32 + lr) * kPitchS + 64) >> (8 * lg);
      sb[i] = *reinterpret_cast<const uint32_t*>(L + (BM + wn * 64 + i * 32 + lr) * kPitchS + 64) >> (8 * lg);
    }
#pragma unroll
    for (int ins = 0; ins < SC::kInstr; ++ins) {
      v8i af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const uint8_t* ra = L + (wm * 64 + i * 32 + lr) * kPitchS;
        const uint8_t* rb = L + (BM + wn * 64 + i * 32 + lr) * kPitchS;
        if constexpr (FMT == FMT_MXFP8) {
          const uint4 a0 = *reinterpret_cast<const uint4*>(ra + 16 * lg), a1 = *reinterpret_cast<const uint4*>(ra + 32 + 16 * lg);
          const uint4 b0 = *reinterpret_cast<const uint4*>(rb + 16 * lg), b1 = *reinterpret_cast<const uint4*>(rb + 32 + 16 * lg);
          af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          bf[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, (int)b1.x, (int)b1.y, (int)b1.z, (int)b1.w};
        } else {
          const uint4 a0 = *reinterpret_cast<const uint4*>(ra + ins * 32 + 16 * lg);
          const uint4 b0 = *reinterpret_cast<const uint4*>(rb + ins * 32 + 16 * lg);
          af[i] = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, 0, 0, 0, 0};
          bf[i] = v8i{(int)b0.x, (int)b0.y, (int)b0.z, (int)b0.w, 0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if constexpr (FMT == FMT_MXFP8)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], TA, TB, 0, (int)sa[i], 0, (int)sb[j]);
          else if (ins == 0)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 0, (int)sa[i], 0, (int)sb[j]);
          else
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[i], bf[j], acc[i][j], 4, 4, 2, (int)sa[i], 2, (int)sb[j]);
        }
    }
    if (st + 1 < steps) store_step(buf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + lr;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (v / 4) + 4 * lg + (v % 4);
        if (row < M && col < N) store_c<CDT>(C, ldc, row, col, acc[i][j][v]);
      }
    }
}

template <int FMT, int CDT, int TA = kType<FMT>, int TB = kType<FMT>>
hipError_t run(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
               int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  const int64_t rb = FMT == FMT_MXFP8 ? K : K / 2;
  const bool fits32 = (M > N ? M : N) * rb < ((int64_t)1 << 32) - 4096;
  // K a multiple of 512: whole steps and whole 16-byte scale periods per row
  const bool pipe = fits32 && K > 0 && (K % 512 == 0) &&
                    M * N >= (int64_t)kTile * kTile * 128;
  hipError_t e;
  if (pipe) {
    e = launch_pipe<FMT, CDT, TA, TB>(a, sa, b, sb, M, N, K, C, ldc, s);
  } else {
    const uint32_t tm = (uint32_t)((M + 127) / 128), tn = (uint32_t)((N + 127) / 128);
    hipLaunchKernelGGL((k_gemm_mx_simple<FMT, CDT, TA, TB>), dim3(tm * tn), dim3(256), 0, s, a, sa, b, sb,
                       M, N, K, C, ldc, tm, tn);
    e = hipGetLastError();
  }
  if (e != hipSuccess || FMT != FMT_MXFP4) return e;
  // MXFP4 x MXFP4: the scaled instruction is exact while every product is a
  // multiple of 2^-149, i.e. c_A + c_B >= 107 (E2M1 elements are multiples
  // of 2^-1).  Tiles whose operands hold a code below 54 (or 255) are
  // recomputed by the generic kernel's fix-up mode.
  return launch_gemm_mx_any(FMT_MXFP4, a, sa, FMT_MXFP4, b, sb, M, N, K, C, CDT, ldc, s, 54u, 254u);
}

}  // namespace

bool gemm_mxfp8_exact_pipe_fits(int64_t M, int64_t N, int64_t K) {
  const bool fits32 = (M > N ? M : N) * K < ((int64_t)1 << 32) - 4096;
  return fits32 && K > 0 && (K % 512 == 0) && M * N >= (int64_t)kTile * kTile * 128;
}

hipError_t launch_gemm_mxfp8_exact_pipe(const uint8_t* a_codes, const uint8_t* a_scales,
                                        const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                        int64_t N, int64_t K, void* C, int cdt, int64_t ldc,
                                        hipStream_t s, int fa, int fb) {
#define MXK_X(A_, B_)                                                                                \
  if (fa == A_ && fb == B_)                                                                          \
    return cdt == DT_F32 ? launch_exact<DT_F32, A_, B_>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s) \
                         : launch_exact<DT_BF16, A_, B_>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
  MXK_X(FMT_MXFP8, FMT_MXFP8)
  MXK_X(FMT_MXFP8_E5M2, FMT_MXFP8)
  MXK_X(FMT_MXFP8, FMT_MXFP8_E5M2)
  MXK_X(FMT_MXFP8_E5M2, FMT_MXFP8_E5M2)
  MXK_X(FMT_MXINT8, FMT_MXINT8)
  MXK_X(FMT_MXINT8, FMT_MXFP8)
  MXK_X(FMT_MXFP8, FMT_MXINT8)
  MXK_X(FMT_MXINT8, FMT_MXFP8_E5M2)
  MXK_X(FMT_MXFP8_E5M2, FMT_MXINT8)
#undef MXK_X
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_mx(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                          int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s, int fa, int fb) {
  if (M == 0 || N == 0) return hipSuccess;
  if (fmt == FMT_MXFP8 && (fa == FMT_MXFP8_E5M2 || fb == FMT_MXFP8_E5M2)) {
    // FP8 pairs with E5M2 on the scaled FP8 instruction (element types 1 / 0)
#define MXK_N8(A_, B_)                                                                               \
  if ((fa == FMT_MXFP8_E5M2) == (A_ == 1) && (fb == FMT_MXFP8_E5M2) == (B_ == 1))                      \
    return cdt == DT_F32 ? run<FMT_MXFP8, DT_F32, A_, B_>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s) \
                         : run<FMT_MXFP8, DT_BF16, A_, B_>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
    MXK_N8(1, 0)
    MXK_N8(0, 1)
    MXK_N8(1, 1)
#undef MXK_N8
  }
  if (fmt == FMT_MXFP8)
    return cdt == DT_F32 ? run<FMT_MXFP8, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                         : run<FMT_MXFP8, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
  return cdt == DT_F32 ? run<FMT_MXFP4, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                       : run<FMT_MXFP4, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
}

}  // namespace mxk
