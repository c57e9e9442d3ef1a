// gemm_f6.hip -- block-scaled GEMM C = A * B^T for MX pairs with an FP6
// operand (MXFP6 E2M3 or E3M2 against E2M3, E3M2 or E2M1; row layout) on
// gfx950's scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 (E3M2 x
// E3M2 on the BF16 instruction)
// ("Microscaling (MX) and block-scaled 4-bit formats", section "Hardware and
// kernels": the block scales are applied inside the matrix instruction;
// "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier", section "The OCP
// Microscaling (MX) spec": the FP6 element types).
//
// Exactness (measured on gfx950 against exactly summed products, random and
// adversarial codes): for these pairs the instruction forms the exact sum of
// its 64 products and rounds it once into the FP32 accumulator, as for FP4 x
// FP4.  E3M2 x E3M2, whose products span 18 bits, is summed in a narrower
// window (errors up to ~1e-4 of sum|a*b|), so this kernel decodes that pair
// to BF16 instead (see mfma_slice).  Like
// every scaled-instruction path, partial sums in FP32's subnormal range are
// flushed, so exactness needs the products of each block pair to stay above
// 2^-126 (combined scale codes c_a + c_b >= 135 suffice for every pair).
//
// Operand registers (measured): lane l holds K-block l / 32 of row l mod 32,
// as the block's packed bytes verbatim -- FP6 24 bytes with element i at bits
// 6 i, FP4 16 bytes with element i in nibble i -- and the lane's E8M0 scale
// byte (selected by opsel) is that block's.
//
// Workgroup: 256 threads (2 x 2 waves), a 256 x 256 C tile, each wave 128 x
// 128 (4 x 4 instruction tiles, 256 accumulator registers), one workgroup
// per CU.  A K step is 128 elements (two instruction slices).  Each row's
// segment of the step (FP6 96 bytes = 6 chunks of 16 bytes, FP4 64 bytes =
// 4 chunks) is copied straight from global memory into LDS with
// global_load_lds (64 lanes x 16 bytes per instruction, each lane one chunk,
// so consecutive lanes read consecutive bytes of a row), three stages deep.
// In LDS a row's chunks sit in a rotated order -- chunk c of row r in slot
// (c + f(r)) mod 6 (FP6, f(r) = (r >> 3) & 3) or mod 4 (FP4, f(r) = (r >> 2)
// & 3) -- so that the 16 lanes served together by a 16-byte LDS read, which
// hold 16 consecutive rows, hit 16 distinct bank groups.  A lane's FP6 block
// (24 bytes) spans two chunks; it reads both whole chunks and keeps its 24
// bytes (8-byte reads of a 96-byte pitch would conflict two ways).  The
// scale bytes of the 512 rows travel per period of 4 steps (16 bytes per row,
// so a row's scale line is touched once per period instead of once per step) into two buffers behind the code stages (LDS: 160 KB for FP6 x
// FP6; K % 512 == 0).  The loop's only vector-memory operations are these
// copies, and a counted wait bounds them.  Each step's barrier sits between its two
// slices: slice 1 is read while slice 0's instructions run, and the next
// stage's scales and slice 0 while slice 1's run, with the copy of stage
// st+3 into the buffer just released.
//
// Measured at 4096^3 (E2M3 x E2M3): the copies alone take 58 us, the matrix
// instructions alone 36 us, the whole kernel 83 us.  A 96-byte segment is not
// aligned to the 128-byte cache lines, so a step touches ~1.75 lines per row
// (the 128-byte segments of the MXFP4 pipeline touch one); aligned 384-byte
// steps would need 192 KB of LDS per stage pair.
#include <atomic>

#include "../device/codec.h"
#include "../device/gemm_common.h"
#include "../device/pipe.h"
#include "../launch.h"

namespace mxk {

namespace {

// matrix-instruction element type codes (cbsz / blgp)
constexpr int kE2M3 = 2, kE3M2 = 3, kE2M1 = 4;

template <int T>
struct F6Op {
  static constexpr int kBits = T == kE2M1 ? 4 : 6;
  static constexpr int kChunks = kBits;          // 16-byte chunks per row and step (128 elements)
  static constexpr int kFrag = 64 * 4 * kBits;   // one 32-row x 64-element fragment
  static constexpr int kStage = 2 * 8 * kFrag;   // 2 slices x 8 row tiles = 256 rows x 16 kBits bytes
};

// LDS slot of chunk c of a row whose rotation is f.
template <int T>
__device__ inline uint32_t slot_of(uint32_t c, uint32_t f) {
  constexpr uint32_t n = F6Op<T>::kChunks;
  const uint32_t s = c + f;
  return s >= n ? s - n : s;
}
template <int T>
__device__ inline uint32_t rot_of(uint32_t r) {
  return T == kE2M1 ? (r >> 2) & 3u : (r >> 3) & 3u;
}

// DMA instructions per wave and stage: the stage holds 256 rows of A then
// 256 rows of B, i.e. 4 * (chunks_A + chunks_B) instructions of 1 KB.
// The scales travel per period of 4 steps (512 K elements): 16 bytes of each
// of the 512 rows (A then B), 8 DMAs of 64 lanes x 16 bytes (two per wave),
// into two buffers after the three code stages.
template <int TA, int TB>
struct Dma {
  static constexpr int kA = 4 * F6Op<TA>::kChunks;
  static constexpr int kPerWave = (kA + 4 * F6Op<TB>::kChunks) / 4;  // code DMAs per wave and step
  static constexpr uint32_t kStage = F6Op<TA>::kStage + F6Op<TB>::kStage;
  static constexpr uint32_t kScaleBase = 3 * kStage;
  static constexpr uint32_t kScaleBuf = 512 * 16;
  static constexpr uint32_t kLds = kScaleBase + 2 * kScaleBuf;
};

// Per-lane copy plan: instruction i of wave w fills stage bytes
// 1024 (w * kPerWave + i) ..; its lane l writes chunk slot P = 64 (w kPerWave
// + i) + l, which is slot P mod n of row P / n of A (or of B past A's
// slots) and holds that row's chunk (slot - f(row)) mod n.
template <int TA, int TB>
struct CopyPlan {
  const uint8_t* src[Dma<TA, TB>::kPerWave];  // step-0 global address of the lane's chunk
  const uint8_t* ssrc[2];                      // period-0 address of the lane's scale bytes
};

template <int T>
__device__ inline const uint8_t* chunk_src(const uint8_t* X, int64_t row0, int64_t rows, int64_t rowbytes,
                                           uint32_t P) {
  constexpr uint32_t n = F6Op<T>::kChunks;
  const uint32_t r = P / n, s = P - r * n, f = rot_of<T>(r);
  const uint32_t c = s >= f ? s - f : s + n - f;
  int64_t g = row0 + r;
  g = g < rows ? g : rows - 1;  // rows past the matrix repeat its last row (not stored)
  return X + g * rowbytes + 16 * c;
}

template <int TA, int TB>
__device__ inline void issue_dma(const CopyPlan<TA, TB>& p, uint32_t wid, uint32_t step, uint8_t* stage) {
  using D = Dma<TA, TB>;
#pragma unroll
  for (int i = 0; i < D::kPerWave; ++i) {
    const uint32_t g = wid * D::kPerWave + i;
    const uint32_t seg = g < (uint32_t)D::kA ? 16u * F6Op<TA>::kBits : 16u * F6Op<TB>::kBits;
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.src[i] + (size_t)step * seg), (lds_ptr_t)(stage + 1024u * g),
                                     16, 0, 0);
  }
}

// Scale bytes of period `per` (steps 4 per .. 4 per + 3) into scale buffer buf:
// row r's 16 bytes at 16 r.
template <int TA, int TB>
__device__ inline void issue_scale_dma(const CopyPlan<TA, TB>& p, uint32_t wid, uint32_t per, uint8_t* smem,
                                       uint32_t buf) {
  using D = Dma<TA, TB>;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    __builtin_amdgcn_global_load_lds((gbl_ptr_t)(p.ssrc[j] + 16u * per),
                                     (lds_ptr_t)(smem + D::kScaleBase + buf * D::kScaleBuf + 1024u * (2u * wid + j)),
                                     16, 0, 0);
}

// Raw fragment chunks of this lane for one slice q: its K-block is b = 2q +
// lg.  FP4: chunk b.  FP6: block 2q = chunk 3q + the low half of chunk 3q+1,
// block 2q+1 = the high half of chunk 3q+1 + chunk 3q+2; the lane reads
// chunks 3q + lg and 3q + 1 + lg whole (p and q below).
template <int T>
struct RawFrag {
  u4 p, q;  // q: FP6 only
};
template <int TA, int TB>
struct RawSlice {
  RawFrag<TA> a[4];
  RawFrag<TB> b[4];
};

template <int T>
__device__ inline void read_raw(const uint8_t* stage, uint32_t q, uint32_t rt, uint32_t lr, uint32_t lg,
                                RawFrag<T>& f) {
  constexpr uint32_t seg = 16u * F6Op<T>::kBits;
  const uint8_t* row = stage + (32u * rt + lr) * seg;
  const uint32_t r = rot_of<T>(lr);
  if constexpr (T == kE2M1) {
    f.p = *reinterpret_cast<const u4*>(row + 16u * slot_of<T>(2u * q + lg, r));
  } else {
    f.p = *reinterpret_cast<const u4*>(row + 16u * slot_of<T>(3u * q + lg, r));
    f.q = *reinterpret_cast<const u4*>(row + 16u * slot_of<T>(3u * q + 1u + lg, r));
  }
}

template <int TA, int TB>
__device__ inline void read_slice(const uint8_t* stage, uint32_t q, uint32_t wm, uint32_t wn, uint32_t lr,
                                  uint32_t lg, RawSlice<TA, TB>& s) {
#pragma unroll
  for (int i = 0; i < 4; ++i) read_raw<TA>(stage, q, wm * 4 + i, lr, lg, s.a[i]);
#pragma unroll
  for (int j = 0; j < 4; ++j) read_raw<TB>(stage + F6Op<TA>::kStage, q, wn * 4 + j, lr, lg, s.b[j]);
}

// The instruction operand: FP4 the chunk; FP6 the lane's 24 bytes (lane
// group 0: p, low half of q; lane group 1: high half of p, q).
template <int T>
__device__ inline v8i operand(const RawFrag<T>& f, bool h) {
  if constexpr (T == kE2M1) {
    return v8i{(int)f.p[0], (int)f.p[1], (int)f.p[2], (int)f.p[3], 0, 0, 0, 0};
  } else {
    const u4 P = f.p, Q = f.q;
    return v8i{(int)(h ? P[2] : P[0]), (int)(h ? P[3] : P[1]), (int)(h ? Q[0] : P[2]),
               (int)(h ? Q[1] : P[3]), (int)(h ? Q[2] : Q[0]), (int)(h ? Q[3] : Q[1]), 0, 0};
  }
}

// The lane's scale dwords of a step (A rows, B rows), shifted so that byte
// 0 / 2 (opsel) is the lane group's block of slice 0 / 1.
struct StepScales {
  uint32_t a[4], b[4];
};
template <int TA, int TB>
__device__ inline void read_scales(const uint8_t* smem, uint32_t step, uint32_t wm, uint32_t wn, uint32_t lr,
                                   uint32_t lg, StepScales& sc) {
  using D = Dma<TA, TB>;
  const uint8_t* S = smem + D::kScaleBase + ((step >> 2) & 1u) * D::kScaleBuf + 4u * (step & 3u);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sc.a[i] = *reinterpret_cast<const uint32_t*>(S + 16u * (wm * 128 + 32 * i + lr)) >> (8u * lg);
    sc.b[i] = *reinterpret_cast<const uint32_t*>(S + 16u * (256 + wn * 128 + 32 * i + lr)) >> (8u * lg);
  }
}

// E3M2 x E3M2 is not summed exactly by the scaled instruction.  Its operands
// are decoded instead: each lane's 24-byte block times its E8M0 scale becomes
// 32 BF16 values with one v_cvt_scalef32_pk32_bf16_bf6 (exact while the
// scaled values are normal BF16 values: scale codes 5 .. 250), which feed
// four v_mfma_f32_32x32x16_bf16.  Instruction k takes elements 8k .. 8k+7 of
// every lane's block, the same positions for A and B, so the 64 products of
// the slice are each summed once (exact products, FP32 accumulation).
typedef __bf16 v8bf_t __attribute__((ext_vector_type(8)));
typedef __bf16 v32bf_t __attribute__((ext_vector_type(32)));
typedef unsigned int v6u_t __attribute__((ext_vector_type(6)));
struct Bf16Block {
  v8bf_t k[4];
};

__device__ inline Bf16Block decode_bf6(const v8i& o, uint32_t code) {
  const v6u_t w = {(unsigned)o[0], (unsigned)o[1], (unsigned)o[2], (unsigned)o[3], (unsigned)o[4], (unsigned)o[5]};
  const v32bf_t r = __builtin_amdgcn_cvt_scalef32_pk32_bf16_bf6(w, u2f(code << 23));
  return __builtin_bit_cast(Bf16Block, r);
}

template <int TA, int TB, int Q>
__device__ inline void mfma_slice(const RawSlice<TA, TB>& s, const StepScales& sc, bool h, v16f (&acc)[4][4]) {
  if constexpr (TA == kE3M2 && TB == kE3M2) {
    Bf16Block bd[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bd[j] = decode_bf6(operand<TB>(s.b[j], h), (sc.b[j] >> (16 * Q)) & 0xFFu);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const Bf16Block ad = decode_bf6(operand<TA>(s.a[i], h), (sc.a[i] >> (16 * Q)) & 0xFFu);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int k = 0; k < 4; ++k)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ad.k[k], bd[j].k[k], acc[i][j], 0, 0, 0);
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const v8i a = operand<TA>(s.a[i], h);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, operand<TB>(s.b[j], h), acc[i][j], TA, TB,
                                                                  2 * Q, (int)sc.a[i], 2 * Q, (int)sc.b[j]);
  }
}

template <int TA, int TB, int CDT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_gemm_mx_f6(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ SA, const uint8_t* __restrict__ B,
    const uint8_t* __restrict__ SB, int64_t M, int64_t N, int64_t K, void* __restrict__ C, int64_t ldc,
    uint32_t tiles_m, uint32_t tiles_n, uint32_t vec) {
  using D = Dma<TA, TB>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint32_t tmi, tni;
  tile_of(blockIdx.x, tiles_m, tiles_n, &tmi, &tni);
  const int64_t m0 = (int64_t)tmi * 256, n0 = (int64_t)tni * 256;
  const uint32_t t = threadIdx.x, lane = t & 63u;
  const uint32_t wid = __builtin_amdgcn_readfirstlane(t >> 6);
  const uint32_t wm = wid >> 1, wn = wid & 1u;
  const uint32_t lr = lane & 31u, lg = lane >> 5;
  const uint32_t steps = (uint32_t)(K / 128);
  const int64_t kb = K / 32;

  CopyPlan<TA, TB> plan;
#pragma unroll
  for (int i = 0; i < D::kPerWave; ++i) {
    const uint32_t P = 64u * (wid * D::kPerWave + i) + lane;
    const uint32_t PA = 256u * F6Op<TA>::kChunks;
    plan.src[i] = P < PA ? chunk_src<TA>(A, m0, M, K * F6Op<TA>::kBits / 8, P)
                         : chunk_src<TB>(B, n0, N, K * F6Op<TB>::kBits / 8, P - PA);
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // scale DMA j of this wave: rows 64 (2 wid + j) + lane of the 512 (A rows, then B rows)
    const uint32_t rr = 64u * (2u * wid + j) + lane;
    int64_t g = rr < 256 ? m0 + rr : n0 + (rr - 256);
    const int64_t lim = rr < 256 ? M : N;
    g = g < lim ? g : lim - 1;
    plan.ssrc[j] = (rr < 256 ? SA : SB) + g * kb;
  }

  v16f acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // Three code stages.  Issue order (vmcnt counts in order): scales of period
  // 0, code stages 0, 1, 2; then in step st (after the step's barrier) code
  // stage st+3 into the buffer of stage st, and in every 4th step the scales
  // of the next period into the scale buffer of the period before.  In step st
  // the wave waits until at most kPerWave issues are in flight, so stage st+1
  // (issued before stage st+2) and every scale copy issued before stage st+2
  // have landed; the next period's scales are issued 3 steps before their
  // first read, ahead of two code stages.  The barrier also means that every
  // wave has read all of stage st and of the period before's scales.  Copies
  // past the end reload the last step / period into buffers nobody reads.
  constexpr int NI = D::kPerWave;
  const uint32_t nper = steps >> 2;
  const bool h = lg != 0;
  issue_scale_dma<TA, TB>(plan, wid, 0, smem, 0);
  issue_dma<TA, TB>(plan, wid, 0, smem);
  issue_dma<TA, TB>(plan, wid, steps > 1 ? 1 : 0, smem + D::kStage);
  issue_dma<TA, TB>(plan, wid, steps > 2 ? 2 : steps - 1, smem + 2 * D::kStage);
  wait_vmcnt<2 * NI>();
  dma_barrier();
  sched_fence();
  RawSlice<TA, TB> f0, f1;
  StepScales sc, scn;
  read_scales<TA, TB>(smem, 0, wm, wn, lr, lg, sc);
  read_slice<TA, TB>(smem, 0, wm, wn, lr, lg, f0);

  uint32_t cur = 0;  // buffer of step st (st mod 3)
  for (uint32_t st = 0; st < steps; ++st) {
    const uint8_t* stage = smem + cur * D::kStage;
    const uint32_t nb = cur == 2 ? 0 : cur + 1;  // buffer of step st + 1
    const uint8_t* next = smem + nb * D::kStage;
    sched_fence();
    read_slice<TA, TB>(stage, 1, wm, wn, lr, lg, f1);
    mfma_slice<TA, TB, 0>(f0, sc, h, acc);
    interleave<16, 0, 1>();
    sched_fence();
    wait_vmcnt<NI>();
    dma_barrier();
    sched_fence();
    const uint32_t n3 = st + 3 < steps ? st + 3 : steps - 1;
    issue_dma<TA, TB>(plan, wid, n3, smem + cur * D::kStage);
    if ((st & 3u) == 0) {
      const uint32_t p1 = (st >> 2) + 1;
      issue_scale_dma<TA, TB>(plan, wid, p1 < nper ? p1 : nper - 1, smem, p1 & 1u);
    }
    read_scales<TA, TB>(smem, st + 1, wm, wn, lr, lg, scn);
    read_slice<TA, TB>(next, 0, wm, wn, lr, lg, f0);
    mfma_slice<TA, TB, 1>(f1, sc, h, acc);
    interleave<NI, 1, 2>();
    sched_fence();
    sc = scn;
    cur = nb;
  }
  // the clamped copies of the last steps may still be landing in LDS, which
  // the epilogue reuses
  wait_vmcnt<0>();
  __syncthreads();

  store_tile<CDT>(smem, acc, C, ldc, M, N, m0 + wm * 128, n0 + wn * 128, vec != 0, wid, lane);
}

template <int TA, int TB, int CDT>
hipError_t launch_f6(const uint8_t* a, const uint8_t* sa, const uint8_t* b, const uint8_t* sb, int64_t M,
                     int64_t N, int64_t K, void* C, int64_t ldc, hipStream_t s) {
  constexpr int kStages = Dma<TA, TB>::kLds;
  constexpr int kEpi = 4 * 64 * (128 * (CDT == DT_F32 ? 4 : 2) + 16);  // store_tile staging
  constexpr int kLds = kStages > kEpi ? kStages : kEpi;
  static_assert(kLds <= 160 * 1024, "LDS budget");
  auto kern = k_gemm_mx_f6<TA, TB, CDT>;
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t)1 << dev : 0;
  if (!bit || !(attr_done.load(std::memory_order_acquire) & bit)) {
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLds);
    if (e != hipSuccess) return e;
    attr_done.fetch_or(bit, std::memory_order_acq_rel);
  }
  const uint32_t tm = (uint32_t)((M + 255) / 256), tn = (uint32_t)((N + 255) / 256);
  const int64_t eb = CDT == DT_F32 ? 4 : 2;
  const uint32_t vec = ((reinterpret_cast<uintptr_t>(C) & 15u) == 0 && (ldc * eb) % 16 == 0) ? 1u : 0u;
  hipLaunchKernelGGL(kern, dim3(tm * tn), dim3(256), kLds, s, a, sa, b, sb, M, N, K, C, ldc, tm, tn, vec);
  return hipGetLastError();
}

// library format -> instruction type code (-1: not an FP6/FP4 type)
int f6_type(int fmt) {
  return fmt == FMT_MXFP6_E2M3 ? kE2M3 : fmt == FMT_MXFP6_E3M2 ? kE3M2 : fmt == FMT_MXFP4 ? kE2M1 : -1;
}

}  // namespace

bool gemm_mx_f6_fits(int fa, int fb, int64_t M, int64_t N, int64_t K) {
  const int ta = f6_type(fa), tb = f6_type(fb);
  if (ta < 0 || tb < 0) return false;
  if (ta == kE2M1 && tb == kE2M1) return false;  // MXFP4 x MXFP4 has its own kernels
  if (K % 512 != 0 || K <= 0) return false;
  // 32-bit tile count; 64-bit addressing elsewhere
  return (uint64_t)((M + 255) / 256) * (uint64_t)((N + 255) / 256) <= 0x7FFFFFFFull;
}

hipError_t launch_gemm_mx_f6(int fa, const uint8_t* a_codes, const uint8_t* a_scales, int fb,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                             int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s) {
  if (!gemm_mx_f6_fits(fa, fb, M, N, K)) return hipErrorInvalidValue;
  if (M == 0 || N == 0) return hipSuccess;
  const int ta = f6_type(fa), tb = f6_type(fb);
  if (ta == kE3M2 && tb == kE3M2) {
    // decoded to BF16 (see mfma_slice), exact for scale codes 5 .. 250 whose
    // products are normal FP32 values (c_A + c_B >= 128 + 4 + 4: codes of at
    // least 68); the tiles whose operands hold another code are recomputed
    // by the generic kernel's fix-up mode
    const hipError_t e = cdt == DT_F32
                             ? launch_f6<kE3M2, kE3M2, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s)
                             : launch_f6<kE3M2, kE3M2, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
    if (e != hipSuccess) return e;
    return launch_gemm_mx_any(fa, a_codes, a_scales, fb, b_codes, b_scales, M, N, K, C, cdt, ldc, s, 68u, 250u);
  }
  hipError_t e = hipErrorInvalidValue;
#define MXK_F6(A_, B_)                                                                                   \
  if (ta == A_ && tb == B_)                                                                              \
    e = cdt == DT_F32 ? launch_f6<A_, B_, DT_F32>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s) \
                      : launch_f6<A_, B_, DT_BF16>(a_codes, a_scales, b_codes, b_scales, M, N, K, C, ldc, s);
  MXK_F6(kE2M3, kE2M3)
  MXK_F6(kE2M3, kE3M2)
  MXK_F6(kE3M2, kE2M3)
  MXK_F6(kE2M3, kE2M1)
  MXK_F6(kE2M1, kE2M3)
  MXK_F6(kE3M2, kE2M1)
  MXK_F6(kE2M1, kE3M2)
#undef MXK_F6
  if (e != hipSuccess) return e;
  // The scaled instruction rounds the exact sum of its products once into
  // FP32, so it is exact while every product is a multiple of 2^-149:
  // c_A + c_B >= 105 + g(A) + g(B), with elements multiples of 2^-g (E2M3 3,
  // E3M2 4, E2M1 1).  Tiles whose operands hold a code below half of that
  // (or 255) are recomputed by the generic kernel's fix-up mode.
  auto grid = [](int t) { return t == kE2M3 ? 3u : (t == kE3M2 ? 4u : 1u); };
  const uint32_t thr = 105u + grid(ta) + grid(tb);
  return launch_gemm_mx_any(fa, a_codes, a_scales, fb, b_codes, b_scales, M, N, K, C, cdt, ldc, s,
                            (thr + 1u) / 2u, 254u);
}

}  // namespace mxk
