// api.cpp -- the C ABI declared in include/mx.h: argument checks (no HIP call
// before they pass), dispatch to the kernel launchers, status mapping.
#include "../../include/mx.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "device/codec.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool valid_fmt(int32_t f) { return f >= MX_MXFP8_E4M3 && f <= MX_MXFP6_E2M3; }
// the formats every kernel takes; the other MX element types are quantized,
// decoded and (E5M2) multiplied natively, see include/mx.h
bool core_fmt(int32_t f) { return f == MX_MXFP8_E4M3 || f == MX_MXFP4_E2M1 || f == MX_NVFP4; }
int64_t code_bits(int32_t f) {
  switch (f) {
    case MX_MXFP4_E2M1:
    case MX_NVFP4: return 4;
    case MX_MXFP6_E3M2:
    case MX_MXFP6_E2M3: return 6;
    default: return 8;
  }
}
bool valid_dt(int32_t d) { return d == MX_BF16 || d == MX_F32; }
int64_t dt_bytes(int32_t d) { return d == MX_BF16 ? 2 : 4; }
int64_t block_of(int32_t f) { return f == MX_NVFP4 ? 16 : 32; }

mx_status hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// The product over an empty K: C = 0.
mx_status zero_product(void* C, int32_t cdt, int64_t ldc, int64_t M, int64_t N, mx_stream stream) {
  return hip_status(mxk::launch_zero_matrix(C, cdt == MX_F32 ? mxk::DT_F32 : mxk::DT_BF16, ldc, M, N,
                                            reinterpret_cast<hipStream_t>(stream)));
}

// Checks the descriptor of a quantized tensor of logical shape [rows, cols].
// The tiled layout is MX-only with rows % 32 == 0 and cols % 1024 == 0.
mx_status check_tensor(const mx_tensor* t, int64_t rows, int64_t cols) {
  if (!t) return MX_ERR_NULL;
  if (!valid_fmt(t->fmt)) return MX_ERR_FORMAT;
  if (t->layout != MX_LAYOUT_ROWS && t->layout != MX_LAYOUT_TILED) return MX_ERR_FORMAT;
  if (t->rows != rows || t->cols != cols || rows < 0 || cols < 0) return MX_ERR_SHAPE;
  if (cols % block_of(t->fmt)) return MX_ERR_SHAPE;
  if (t->layout == MX_LAYOUT_TILED) {
    if (t->fmt != MX_MXFP8_E4M3 && t->fmt != MX_MXFP4_E2M1 && t->fmt != MX_MXFP8_E5M2)
      return MX_ERR_UNSUPPORTED;
    if (rows % 32 || cols % 1024) return MX_ERR_SHAPE;
  }
  if (rows * cols > 0) {
    if (!t->codes || !t->scales) return MX_ERR_NULL;
    if (!aligned16(t->codes) || !aligned16(t->scales)) return MX_ERR_ALIGN;
  }
  if (t->fmt == MX_NVFP4) {
    if (!t->tensor_scale) return MX_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(t->tensor_scale) & 3u) return MX_ERR_ALIGN;
  }
  return MX_OK;
}

// Output matrices written element by element only need element alignment.
mx_status check_output(const void* p, int32_t dt, int64_t rows, int64_t cols, int64_t ld) {
  if (!valid_dt(dt)) return MX_ERR_FORMAT;
  if (rows < 0 || cols < 0 || ld < cols) return MX_ERR_SHAPE;
  if (rows * cols == 0) return MX_OK;
  if (!p) return MX_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(p) % dt_bytes(dt)) return MX_ERR_ALIGN;
  return MX_OK;
}

mx_status check_matrix(const void* p, int32_t dt, int64_t rows, int64_t cols, int64_t ld) {
  if (!valid_dt(dt)) return MX_ERR_FORMAT;
  if (rows < 0 || cols < 0 || ld < cols) return MX_ERR_SHAPE;
  if (rows * cols == 0) return MX_OK;
  if (!p) return MX_ERR_NULL;
  if (!aligned16(p) || (ld * dt_bytes(dt)) % 16) return MX_ERR_ALIGN;
  return MX_OK;
}

}  // namespace

extern "C" {

size_t mx_codes_bytes(int32_t fmt, int64_t rows, int64_t cols) {
  if (!valid_fmt(fmt) || rows < 0 || cols < 0) return 0;
  return (size_t)(rows * (cols * code_bits(fmt) / 8));
}

size_t mx_scales_bytes(int32_t fmt, int64_t rows, int64_t cols) {
  if (!valid_fmt(fmt) || rows < 0 || cols < 0) return 0;
  return (size_t)(rows * (cols / block_of(fmt)));
}

uint16_t mx_rht_signs(uint64_t seed) {
  mxk::u32x4 w = mxk::philox4x32_10(0u, 0u, 0u, 1u, (uint32_t)seed, (uint32_t)(seed >> 32));
  return (uint16_t)(w.x & 0xFFFFu);
}

const char* mx_status_string(int32_t s) {
  switch (s) {
    case MX_OK: return "ok";
    case MX_ERR_NULL: return "required pointer is NULL";
    case MX_ERR_SHAPE: return "inconsistent or unsupported shape";
    case MX_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case MX_ERR_FORMAT: return "unknown format, dtype or rounding mode";
    case MX_ERR_UNSUPPORTED: return "unsupported combination";
    case MX_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

namespace {
// Checks the arguments of one quantization and fills its kernel arguments.
mx_status make_quant_args(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ld_x,
                          const mx_tensor* out, int32_t rnd, mx_rng rng, uint32_t flags,
                          uint16_t rht_sign_mask, float* amax, mxk::QuantArgs* a, bool* empty) {
  *empty = false;
  if (!out) return MX_ERR_NULL;
  if (rnd != MX_RNE && rnd != MX_SR) return MX_ERR_FORMAT;
  if (flags & ~(MX_FLAG_RHT16 | MX_FLAG_AMAX_GIVEN | MX_FLAG_SCALE_CEIL | MX_FLAG_FOUR_OVER_SIX |
                MX_FLAG_BLOCK_2D))
    return MX_ERR_UNSUPPORTED;
  mx_status st = check_matrix(x, xdt, rows, cols, ld_x);
  if (st != MX_OK) return st;
  st = check_tensor(out, rows, cols);
  if (st != MX_OK) return st;
  const bool nv = out->fmt == MX_NVFP4;
  if ((flags & MX_FLAG_SCALE_CEIL) && nv) return MX_ERR_UNSUPPORTED;
  if ((flags & (MX_FLAG_FOUR_OVER_SIX | MX_FLAG_BLOCK_2D)) && !nv) return MX_ERR_UNSUPPORTED;
  if ((flags & MX_FLAG_FOUR_OVER_SIX) && (rnd != MX_RNE || (flags & MX_FLAG_BLOCK_2D)))
    return MX_ERR_UNSUPPORTED;
  if (out->fmt == MX_NVFP4) {
    if (!amax) return MX_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(amax) & 3u) return MX_ERR_ALIGN;
  } else if (flags & MX_FLAG_AMAX_GIVEN) {
    return MX_ERR_UNSUPPORTED;
  }
  if (rows * cols == 0 && out->fmt != MX_NVFP4) {
    *empty = true;
    return MX_OK;
  }
  a->x = x;
  a->xdt = xdt;
  a->rows = rows;
  a->cols = cols;
  a->ld_x = ld_x;
  a->fmt = out->fmt;
  a->codes = static_cast<uint8_t*>(out->codes);
  a->scales = out->scales;
  a->tensor_scale = out->tensor_scale;
  a->amax = amax;
  a->sr = rnd == MX_SR;
  a->seed = rng.seed;
  a->counter = rng.counter;
  a->rht = (flags & MX_FLAG_RHT16) != 0;
  a->sign_mask = rht_sign_mask;
  a->amax_given = (flags & MX_FLAG_AMAX_GIVEN) != 0;
  a->tiled = out->layout == MX_LAYOUT_TILED;
  a->ceil = (flags & MX_FLAG_SCALE_CEIL) != 0;
  a->four6 = (flags & MX_FLAG_FOUR_OVER_SIX) != 0;
  a->block2d = (flags & MX_FLAG_BLOCK_2D) != 0;
  return MX_OK;
}
}  // namespace

mx_status mx_quantize(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ld_x,
                      const mx_tensor* out, int32_t rnd, mx_rng rng, uint32_t flags,
                      uint16_t rht_sign_mask, float* amax, mx_stream stream) {
  mxk::QuantArgs a;
  bool empty = false;
  const mx_status st = make_quant_args(x, xdt, rows, cols, ld_x, out, rnd, rng, flags, rht_sign_mask, amax,
                                       &a, &empty);
  if (st != MX_OK || empty) return st;
  return hip_status(mxk::launch_quantize(a, reinterpret_cast<hipStream_t>(stream)));
}

namespace {
// mx_quantize_batch's work.  With slots != NULL, job i's amax slot is
// slots + i instead of jobs[i].amax.
mx_status quantize_batch(const mx_quantize_job* jobs, int32_t count, float* slots, mx_stream stream) {
  if (count < 0) return MX_ERR_SHAPE;
  if (count == 0) return MX_OK;
  if (!jobs) return MX_ERR_NULL;
  auto slot = [&](int32_t i) { return slots ? slots + i : jobs[i].amax; };
  // every job is checked before anything is enqueued
  for (int32_t i = 0; i < count; ++i) {
    const mx_quantize_job& j = jobs[i];
    mxk::QuantArgs a;
    bool empty = false;
    const mx_status st = make_quant_args(j.x, j.xdt, j.rows, j.cols, j.ld_x, j.out, j.rnd, j.rng, j.flags,
                                         j.rht_sign_mask, slot(i), &a, &empty);
    if (st != MX_OK) return st;
  }
  constexpr int kChunk = 64;  // then built and launched kChunk at a time
  mxk::QuantArgs args[kChunk];
  for (int32_t i0 = 0; i0 < count; i0 += kChunk) {
    int n = 0;
    const int32_t i1 = count - i0 < kChunk ? count : i0 + kChunk;
    for (int32_t i = i0; i < i1; ++i) {
      const mx_quantize_job& j = jobs[i];
      bool empty = false;
      const mx_status st = make_quant_args(j.x, j.xdt, j.rows, j.cols, j.ld_x, j.out, j.rnd, j.rng, j.flags,
                                           j.rht_sign_mask, slot(i), &args[n], &empty);
      if (st != MX_OK) return st;
      if (!empty) ++n;
    }
    const mx_status st = hip_status(mxk::launch_quantize_batch(args, n, reinterpret_cast<hipStream_t>(stream)));
    if (st != MX_OK) return st;
  }
  return MX_OK;
}
}  // namespace

mx_status mx_quantize_batch(const mx_quantize_job* jobs, int32_t count, mx_stream stream) {
  return quantize_batch(jobs, count, nullptr, stream);
}

// The amax slots of mx_quantize_batch_noalloc: one FP32 per job, one copy per
// device.  Host code never uses this name as an address (on the host it is
// only a stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, once per device, and is kept in g_scratch.
static __device__ __align__(256) float scratch[MX_NOALLOC_MAX_JOBS];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices];  // device address of `scratch` on each device

// The scratch address on the current device (looked up on first use).
mx_status scratch_of_current_device(float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MX_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MX_ERR_HIP;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return MX_OK;
}
}  // namespace

mx_status mx_quantize_batch_noalloc(const mx_quantize_job* jobs, int32_t count, mx_stream stream) {
  if (count < 0 || count > MX_NOALLOC_MAX_JOBS) return MX_ERR_SHAPE;
  if (count == 0) return MX_OK;
  if (!jobs) return MX_ERR_NULL;
  for (int32_t i = 0; i < count; ++i)
    if (jobs[i].amax || (jobs[i].flags & MX_FLAG_AMAX_GIVEN)) return MX_ERR_UNSUPPORTED;
  if (stream) {
    int cur = -1, sdev = -1;
    if (hipGetDevice(&cur) != hipSuccess || hipStreamGetDevice(reinterpret_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return MX_ERR_HIP;
    if (cur != sdev) return MX_ERR_UNSUPPORTED;
  }
  float* slots = nullptr;
  const mx_status st = scratch_of_current_device(&slots);
  if (st != MX_OK) return st;
  return quantize_batch(jobs, count, slots, stream);
}

mx_status mx_amax(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ld_x,
                  uint32_t flags, uint16_t rht_sign_mask, float* amax, mx_stream stream) {
  if (flags & ~MX_FLAG_RHT16) return MX_ERR_UNSUPPORTED;
  mx_status st = check_matrix(x, xdt, rows, cols, ld_x);
  if (st != MX_OK) return st;
  if (!amax) return MX_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(amax) & 3u) return MX_ERR_ALIGN;
  if (cols % 16) return MX_ERR_SHAPE;
  return hip_status(mxk::launch_amax(x, xdt, rows, cols, ld_x, (flags & MX_FLAG_RHT16) != 0,
                                     rht_sign_mask, amax, reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_dequantize(const mx_tensor* in, void* y, int32_t ydt, int64_t ld_y, uint32_t flags,
                        uint16_t rht_sign_mask, mx_stream stream) {
  if (!in) return MX_ERR_NULL;
  if (flags & ~MX_FLAG_RHT16) return MX_ERR_UNSUPPORTED;
  mx_status st = check_tensor(in, in->rows, in->cols);
  if (st != MX_OK) return st;
  st = check_matrix(y, ydt, in->rows, in->cols, ld_y);
  if (st != MX_OK) return st;
  if (in->rows * in->cols == 0) return MX_OK;
  return hip_status(mxk::launch_dequantize(in->fmt, static_cast<const uint8_t*>(in->codes),
                                           in->scales, in->tensor_scale, in->rows, in->cols, y,
                                           ydt, ld_y, (flags & MX_FLAG_RHT16) != 0, rht_sign_mask,
                                           in->layout == MX_LAYOUT_TILED,
                                           reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_requant_transpose(const mx_tensor* src, const void* x_bf16, int64_t ld_x,
                               int64_t rows, int64_t cols, const mx_tensor* out, int32_t rnd,
                               mx_rng rng, mx_stream stream) {
  if (!out) return MX_ERR_NULL;
  if ((src == nullptr) == (x_bf16 == nullptr)) return MX_ERR_NULL;
  if (rnd != MX_RNE && rnd != MX_SR) return MX_ERR_FORMAT;
  if (rows < 0 || cols < 0) return MX_ERR_SHAPE;
  if (rows % 32 || cols % 16) return MX_ERR_SHAPE;
  if (src) {
    mx_status st = check_tensor(src, rows, cols);
    if (st != MX_OK) return st;
    if (src->fmt != MX_NVFP4 || src->layout != MX_LAYOUT_ROWS) return MX_ERR_UNSUPPORTED;
  } else {
    mx_status st = check_matrix(x_bf16, MX_BF16, rows, cols, ld_x);
    if (st != MX_OK) return st;
  }
  mx_status st = check_tensor(out, cols, rows);
  if (st != MX_OK) return st;
  if (out->fmt != MX_MXFP8_E4M3 || out->layout != MX_LAYOUT_ROWS) return MX_ERR_UNSUPPORTED;
  if (rows * cols == 0) return MX_OK;
  return hip_status(mxk::launch_requant_transpose(
      src ? static_cast<const uint8_t*>(src->codes) : nullptr, src ? src->scales : nullptr,
      src ? src->tensor_scale : nullptr, static_cast<const uint16_t*>(x_bf16), ld_x, rows, cols,
      static_cast<uint8_t*>(out->codes), out->scales, rnd == MX_SR, rng.seed, rng.counter,
      reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_hadamard16(const void* x, int32_t xdt, void* y, int32_t ydt, int64_t rows,
                        int64_t cols, uint16_t sign_mask, int32_t inverse, mx_stream stream) {
  mx_status st = check_matrix(x, xdt, rows, cols, cols);
  if (st != MX_OK) return st;
  st = check_matrix(y, ydt, rows, cols, cols);
  if (st != MX_OK) return st;
  if (cols % 16) return MX_ERR_SHAPE;
  if (rows * cols == 0) return MX_OK;
  if (x == y && xdt != ydt) return MX_ERR_UNSUPPORTED;
  return hip_status(mxk::launch_hadamard16(x, xdt, y, ydt, rows, cols, sign_mask, inverse != 0,
                                           reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_error_stats(const void* x, int32_t xdt, int64_t ld_x, const float* y, int64_t ld_y, int64_t rows,
                         int64_t cols, double* stats, mx_stream stream) {
  if (!stats) return MX_ERR_NULL;
  if (!aligned16(stats)) return MX_ERR_ALIGN;
  mx_status st = check_matrix(x, xdt, rows, cols, ld_x);
  if (st != MX_OK) return st;
  st = check_matrix(y, MX_F32, rows, cols, ld_y);
  if (st != MX_OK) return st;
  if (cols % 8) return MX_ERR_SHAPE;
  return hip_status(mxk::launch_error_stats(x, xdt, ld_x, y, ld_y, rows, cols, stats,
                                            reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_gemm_ex(const mx_tensor* A, const mx_tensor* B, void* C, int32_t cdt, int64_t ldc,
                     uint32_t flags, mx_stream stream) {
  if (!A || !B) return MX_ERR_NULL;
  if (flags & ~MX_GEMM_FP8_NATIVE) return MX_ERR_UNSUPPORTED;
  mx_status st = check_tensor(A, A->rows, A->cols);
  if (st != MX_OK) return st;
  st = check_tensor(B, B->rows, B->cols);
  if (st != MX_OK) return st;
  const bool fp8a = A->fmt == MX_MXFP8_E4M3 || A->fmt == MX_MXFP8_E5M2;
  const bool fp8b = B->fmt == MX_MXFP8_E4M3 || B->fmt == MX_MXFP8_E5M2;
  if (A->layout == MX_LAYOUT_TILED && B->layout == MX_LAYOUT_TILED && fp8a && fp8b &&
      (A->fmt == MX_MXFP8_E5M2 || B->fmt == MX_MXFP8_E5M2)) {
    // FP8 pairs with E5M2 in the tile layout: the scaled FP8 instruction
    if (!(flags & MX_GEMM_FP8_NATIVE)) return MX_ERR_UNSUPPORTED;
    if (A->cols != B->cols) return MX_ERR_SHAPE;
    st = check_output(C, cdt, A->rows, B->rows, ldc);
    if (st != MX_OK) return st;
    if (A->rows * B->rows == 0) return MX_OK;
    if (A->cols == 0) return zero_product(C, cdt, ldc, A->rows, B->rows, stream);
    return hip_status(mxk::launch_gemm_mx_tiled(A->fmt, static_cast<const uint8_t*>(A->codes), A->scales,
                                                static_cast<const uint8_t*>(B->codes), B->scales, A->rows,
                                                B->rows, A->cols, C, cdt, ldc,
                                                reinterpret_cast<hipStream_t>(stream), B->fmt));
  }
  if (A->fmt != B->fmt || !core_fmt(A->fmt)) {
    // mixed formats or the other MX element types: every MX (E8M0) pair, row
    // layout, exact BF16 staging
    if (A->fmt == MX_NVFP4 || B->fmt == MX_NVFP4) return MX_ERR_UNSUPPORTED;
    // MX_GEMM_FP8_NATIVE: FP8 pairs (E4M3 / E5M2) only
    if (flags && !(fp8a && fp8b)) return MX_ERR_UNSUPPORTED;
    if (A->layout != MX_LAYOUT_ROWS || B->layout != MX_LAYOUT_ROWS) return MX_ERR_UNSUPPORTED;
    if (A->cols != B->cols || A->cols % 32) return MX_ERR_SHAPE;
    st = check_output(C, cdt, A->rows, B->rows, ldc);
    if (st != MX_OK) return st;
    if (A->rows * B->rows == 0) return MX_OK;
    if (A->cols == 0) return zero_product(C, cdt, ldc, A->rows, B->rows, stream);
    if (flags)  // row-layout FP8 pairs with E5M2 on the scaled FP8 instruction
      return hip_status(mxk::launch_gemm_mx(mxk::FMT_MXFP8, static_cast<const uint8_t*>(A->codes), A->scales,
                                            static_cast<const uint8_t*>(B->codes), B->scales, A->rows, B->rows,
                                            A->cols, C, cdt, ldc, reinterpret_cast<hipStream_t>(stream), A->fmt,
                                            B->fmt));
    const bool b8a = fp8a || A->fmt == MX_MXINT8, b8b = fp8b || B->fmt == MX_MXINT8;
    if (b8a && b8b && mxk::gemm_mxfp8_exact_pipe_fits(A->rows, B->rows, A->cols))
      // pairs of 8-bit MX types (E4M3, E5M2, INT8) other than E4M3 x E4M3:
      // the exact 8-bit pipeline (BF16 instruction)
      return hip_status(mxk::launch_gemm_mxfp8_exact(static_cast<const uint8_t*>(A->codes), A->scales,
                                                     static_cast<const uint8_t*>(B->codes), B->scales, A->rows,
                                                     B->rows, A->cols, C, cdt, ldc,
                                                     reinterpret_cast<hipStream_t>(stream), A->fmt, B->fmt));
    if (mxk::gemm_mx_f6_fits(A->fmt, B->fmt, A->rows, B->rows, A->cols))
      return hip_status(mxk::launch_gemm_mx_f6(A->fmt, static_cast<const uint8_t*>(A->codes), A->scales,
                                               B->fmt, static_cast<const uint8_t*>(B->codes), B->scales,
                                               A->rows, B->rows, A->cols, C, cdt, ldc,
                                               reinterpret_cast<hipStream_t>(stream)));
    {
      // the generic kernel decodes to BF16: a tile is computed as it is when
      // every code lies in the conversions' exact range and every pair of
      // codes puts the products at normal FP32 values (c_A + c_B >= 128 +
      // g_A + g_B, elements multiples of 2^-g), else with shifted codes
      auto grid = [](int32_t f) {
        return f == MX_MXFP8_E4M3 ? 9u : f == MX_MXFP8_E5M2 ? 16u : f == MX_MXINT8 ? 6u
               : f == MX_MXFP6_E3M2 ? 4u : f == MX_MXFP6_E2M3 ? 3u : 1u;
      };
      const uint32_t lo = (128u + grid(A->fmt) + grid(B->fmt) + 1u) / 2u;
      const uint32_t hi = (A->fmt == MX_MXINT8 && B->fmt == MX_MXINT8) ? 254u : 239u;
      return hip_status(mxk::launch_gemm_mx_any(A->fmt, static_cast<const uint8_t*>(A->codes), A->scales,
                                                B->fmt, static_cast<const uint8_t*>(B->codes), B->scales,
                                                A->rows, B->rows, A->cols, C, cdt, ldc,
                                                reinterpret_cast<hipStream_t>(stream), lo, hi, true));
    }
  }
  if ((flags & MX_GEMM_FP8_NATIVE) && A->fmt != MX_MXFP8_E4M3) return MX_ERR_UNSUPPORTED;
  if (A->cols != B->cols || A->cols % 32) return MX_ERR_SHAPE;
  const bool tiled = A->layout == MX_LAYOUT_TILED;
  if ((B->layout == MX_LAYOUT_TILED) != tiled) return MX_ERR_UNSUPPORTED;
  // tiled MXFP8 only has the native-FP8 kernel
  if (tiled && A->fmt == MX_MXFP8_E4M3 && !(flags & MX_GEMM_FP8_NATIVE)) return MX_ERR_UNSUPPORTED;
  const int64_t M = A->rows, N = B->rows, K = A->cols;
  st = check_output(C, cdt, M, N, ldc);
  if (st != MX_OK) return st;
  if (M * N == 0) return MX_OK;
  if (K == 0) return zero_product(C, cdt, ldc, M, N, stream);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const uint8_t* ac = static_cast<const uint8_t*>(A->codes);
  const uint8_t* bc = static_cast<const uint8_t*>(B->codes);
  if (tiled)
    return hip_status(mxk::launch_gemm_mx_tiled(A->fmt, ac, A->scales, bc, B->scales, M, N, K, C,
                                                cdt, ldc, s, B->fmt));
  switch (A->fmt) {
    case MX_NVFP4:
      // one group covering all rows (no offsets array needed)
      return hip_status(mxk::launch_gemm_nvfp4(ac, A->scales, A->tensor_scale, nullptr, M, M, bc,
                                               B->scales, B->tensor_scale, 1, nullptr, N, K, C,
                                               cdt, ldc, s));
    case MX_MXFP8_E4M3:
      if (flags & MX_GEMM_FP8_NATIVE)
        return hip_status(mxk::launch_gemm_mx(A->fmt, ac, A->scales, bc, B->scales, M, N, K, C,
                                              cdt, ldc, s));
      return hip_status(mxk::launch_gemm_mxfp8_exact(ac, A->scales, bc, B->scales, M, N, K, C,
                                                     cdt, ldc, s));
    default:
      return hip_status(mxk::launch_gemm_mx(A->fmt, ac, A->scales, bc, B->scales, M, N, K, C, cdt,
                                            ldc, s));
  }
}

mx_status mx_gemm_quantize(const mx_tensor* A, const mx_tensor* B, const mx_tensor* out,
                           int32_t rnd, mx_rng rng, uint32_t flags, mx_stream stream) {
  if (!A || !B || !out) return MX_ERR_NULL;
  if (rnd != MX_RNE && rnd != MX_SR) return MX_ERR_FORMAT;
  if (flags & ~(MX_GEMM_FP8_NATIVE | MX_FLAG_SCALE_CEIL)) return MX_ERR_UNSUPPORTED;
  mx_status st = check_tensor(A, A->rows, A->cols);
  if (st != MX_OK) return st;
  st = check_tensor(B, B->rows, B->cols);
  if (st != MX_OK) return st;
  if (A->fmt != B->fmt || A->layout != MX_LAYOUT_TILED || B->layout != MX_LAYOUT_TILED)
    return MX_ERR_UNSUPPORTED;
  if (A->fmt == MX_MXFP8_E4M3 ? !(flags & MX_GEMM_FP8_NATIVE) : (flags & MX_GEMM_FP8_NATIVE) != 0)
    return MX_ERR_UNSUPPORTED;
  if (A->cols != B->cols) return MX_ERR_SHAPE;
  const int64_t M = A->rows, N = B->rows, K = A->cols;
  st = check_tensor(out, M, N);
  if (st != MX_OK) return st;
  if (out->fmt != MX_MXFP8_E4M3 && out->fmt != MX_MXFP4_E2M1 && out->fmt != MX_MXFP8_E5M2)
    return MX_ERR_UNSUPPORTED;
  if (K == 0) return MX_ERR_SHAPE;
  if (M * N == 0) return MX_OK;
  return hip_status(mxk::launch_gemm_mx_tiled_quant(
      A->fmt, static_cast<const uint8_t*>(A->codes), A->scales,
      static_cast<const uint8_t*>(B->codes), B->scales, M, N, K, out->fmt,
      out->layout == MX_LAYOUT_TILED, static_cast<uint8_t*>(out->codes), out->scales, rnd == MX_SR,
      rng.seed, rng.counter, (flags & MX_FLAG_SCALE_CEIL) != 0, reinterpret_cast<hipStream_t>(stream)));
}

mx_status mx_gemm_quantize_a(const void* A, int64_t lda, int64_t M, int32_t a_fmt, int32_t rnd, mx_rng rng,
                             const mx_tensor* B, void* C, int32_t cdt, int64_t ldc, const mx_tensor* a_out,
                             mx_stream stream) {
  if (!B) return MX_ERR_NULL;
  if (rnd != MX_RNE && rnd != MX_SR) return MX_ERR_FORMAT;
  if (a_fmt != MX_MXFP8_E4M3 && a_fmt != MX_MXFP4_E2M1) return MX_ERR_UNSUPPORTED;
  mx_status st = check_tensor(B, B->rows, B->cols);
  if (st != MX_OK) return st;
  if ((B->fmt != MX_MXFP8_E4M3 && B->fmt != MX_MXFP4_E2M1) || B->layout != MX_LAYOUT_ROWS)
    return MX_ERR_UNSUPPORTED;
  const int64_t N = B->rows, K = B->cols;
  if (M < 0 || K % 32 || K == 0) return MX_ERR_SHAPE;
  st = check_matrix(A, MX_BF16, M, K, lda);
  if (st != MX_OK) return st;
  st = check_output(C, cdt, M, N, ldc);
  if (st != MX_OK) return st;
  if (a_out) {
    st = check_tensor(a_out, M, K);
    if (st != MX_OK) return st;
    if (a_out->fmt != a_fmt || a_out->layout != MX_LAYOUT_ROWS) return MX_ERR_UNSUPPORTED;
  }
  if (M * N == 0) return MX_OK;
  const hipError_t e = mxk::launch_gemm_quantize_a(
      a_fmt, static_cast<const uint16_t*>(A), lda, static_cast<const uint8_t*>(B->codes), B->scales, B->fmt, M, N,
      K, C, cdt, ldc, a_out ? static_cast<uint8_t*>(a_out->codes) : nullptr, a_out ? a_out->scales : nullptr,
      rnd == MX_SR, rng.seed, rng.counter, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess || !a_out) return hip_status(e);
  // With Q(A) written out, the tiles whose codes could pair below normal
  // FP32 products (c_A + c_B < 128 + g_A + g_B; E4M3 9, E2M1 1) or lie
  // outside the decode's exact range are recomputed from Q(A) and B.
  const uint32_t ga = a_fmt == MX_MXFP8_E4M3 ? 9u : 1u, gb = B->fmt == MX_MXFP8_E4M3 ? 9u : 1u;
  return hip_status(mxk::launch_gemm_mx_any(a_fmt, static_cast<const uint8_t*>(a_out->codes), a_out->scales,
                                            B->fmt, static_cast<const uint8_t*>(B->codes), B->scales, M, N, K, C,
                                            cdt, ldc, reinterpret_cast<hipStream_t>(stream),
                                            (128u + ga + gb + 1u) / 2u, 239u, false));
}

mx_status mx_gemm(const mx_tensor* A, const mx_tensor* B, void* C, int32_t cdt, int64_t ldc,
                  mx_stream stream) {
  return mx_gemm_ex(A, B, C, cdt, ldc, 0u, stream);
}

mx_status mx_gemm_grouped(const mx_tensor* A, const int32_t* row_index, int64_t routed_rows,
                          const mx_tensor* B, int32_t num_groups, const int64_t* group_offsets,
                          void* C, int32_t cdt, int64_t ldc, mx_stream stream) {
  if (!A || !B) return MX_ERR_NULL;
  if (num_groups < 1) return MX_ERR_SHAPE;
  mx_status st = check_tensor(A, A->rows, A->cols);
  if (st != MX_OK) return st;
  st = check_tensor(B, B->rows, B->cols);
  if (st != MX_OK) return st;
  if (A->fmt != MX_NVFP4 || B->fmt != MX_NVFP4) return MX_ERR_UNSUPPORTED;
  if (A->cols != B->cols || A->cols % 32) return MX_ERR_SHAPE;
  if (B->rows % num_groups) return MX_ERR_SHAPE;
  if (routed_rows < 0) return MX_ERR_SHAPE;
  if (!row_index && routed_rows != A->rows) return MX_ERR_SHAPE;
  if (row_index && routed_rows > 0 && A->rows == 0) return MX_ERR_SHAPE;  // no row to gather
  if (!group_offsets) return MX_ERR_NULL;
  const int64_t N = B->rows / num_groups, K = A->cols;
  st = check_output(C, cdt, routed_rows, N, ldc);
  if (st != MX_OK) return st;
  if (routed_rows * N == 0) return MX_OK;
  if (K == 0) return zero_product(C, cdt, ldc, routed_rows, N, stream);
  return hip_status(mxk::launch_gemm_nvfp4(
      static_cast<const uint8_t*>(A->codes), A->scales, A->tensor_scale, row_index, A->rows, routed_rows,
      static_cast<const uint8_t*>(B->codes), B->scales, B->tensor_scale, num_groups,
      group_offsets, N, K, C, cdt, ldc, reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
