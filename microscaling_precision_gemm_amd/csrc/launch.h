// launch.h -- internal launchers between the C ABI (api.cpp) and the kernels.
// Arguments are already validated when these run.  Each returns the HIP error
// of its launch(es).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mxk {

// MX formats: FP8 E4M3, FP4 E2M1, NVFP4, then the other MX element types
// (INT8 with 6 fraction bits, FP8 E5M2, FP6 E3M2 and E2M3), all with E8M0
// scales per 32 except NVFP4.
enum Fmt {
  FMT_MXFP8 = 1,
  FMT_MXFP4 = 2,
  FMT_NVFP4 = 3,
  FMT_MXINT8 = 4,
  FMT_MXFP8_E5M2 = 5,
  FMT_MXFP6_E3M2 = 6,
  FMT_MXFP6_E2M3 = 7
};
enum DType { DT_BF16 = 0, DT_F32 = 1 };

struct QuantArgs {
  const void* x;
  int xdt;
  int64_t rows, cols, ld_x;
  int fmt;
  uint8_t* codes;
  uint8_t* scales;
  float* tensor_scale;  // NVFP4
  float* amax;          // NVFP4
  bool sr;
  uint64_t seed, counter;
  bool rht;
  uint32_t sign_mask;
  bool amax_given;
  bool tiled;  // codes and scales in the matrix-instruction tile layout
  bool ceil;     // MX: ceil (no-saturation) scale rule
  bool four6;    // NVFP4: Four Over Six block-scale choice (round-to-nearest)
  bool block2d;  // NVFP4: one block scale per 16 x 16 tile
};

hipError_t launch_quantize(const QuantArgs& a, hipStream_t s);

// Up to kMaxBatch tile-layout MX quantizations in one launch.
constexpr int kMaxBatch = 4;
struct QuantBatch {
  QuantArgs job[kMaxBatch];
  int64_t first[kMaxBatch + 1];  // first wave of each job; first[n] = total
  int n;
};
// Up to kMaxNvBatch NVFP4 quantizations per launch (and per pass).
constexpr int kMaxNvBatch = 16;
struct NvBatch {
  QuantArgs job[kMaxNvBatch];
  int64_t first[kMaxNvBatch + 1];  // first workgroup of each job; first[n] = total
  int n;
};
// Quantize n tensors: one launch per group of up to kMaxBatch consecutive
// jobs that are tile-layout MX with the same format, input dtype, rounding
// and transform; one launch per pass (amax, encode) for up to kMaxNvBatch
// consecutive NVFP4 jobs with the same input dtype, rounding, transform and
// variant; any other job is launched on its own.  Same results as n
// launch_quantize calls in order.
hipError_t launch_quantize_batch(const QuantArgs* a, int n, hipStream_t s);
hipError_t launch_amax(const void* x, int xdt, int64_t rows, int64_t cols, int64_t ld_x, bool rht,
                       uint32_t sign_mask, float* amax, hipStream_t s);
hipError_t launch_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales,
                             const float* tensor_scale, int64_t rows, int64_t cols, void* y,
                             int ydt, int64_t ld_y, bool rht, uint32_t sign_mask, bool tiled,
                             hipStream_t s);
// Round-trip error statistics of y (FP32) against x (stats.hip): stats[0..3]
// = sum (y-x)^2, sum x^2, sum (y-x), max |y-x| (device doubles, overwritten).
hipError_t launch_error_stats(const void* x, int xdt, int64_t ld_x, const float* y, int64_t ld_y, int64_t rows,
                              int64_t cols, double* stats, hipStream_t s);
// C = 0 over rows x cols (BF16 or FP32, row pitch ldc elements; stats.hip):
// a GEMM's result when K is 0.  A kernel, not a memset, so that the call
// stays capturable in a graph.
hipError_t launch_zero_matrix(void* c, int cdt, int64_t ldc, int64_t rows, int64_t cols, hipStream_t s);
hipError_t launch_hadamard16(const void* x, int xdt, void* y, int ydt, int64_t rows, int64_t cols,
                             uint32_t sign_mask, bool inverse, hipStream_t s);
hipError_t launch_requant_transpose(const uint8_t* src_codes, const uint8_t* src_scales,
                                    const float* src_tensor_scale, const uint16_t* x_bf16,
                                    int64_t ld_x, int64_t rows, int64_t cols, uint8_t* codes,
                                    uint8_t* scales, bool sr, uint64_t seed, uint64_t counter,
                                    hipStream_t s);
// fmt FMT_MXFP8 runs on the scaled FP8 instruction; fa / fb (FMT_MXFP8 or
// FMT_MXFP8_E5M2) then give the element types of A and B.
hipError_t launch_gemm_mx(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                          const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                          int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s,
                          int fa = FMT_MXFP8, int fb = FMT_MXFP8);
// A and B in the tiled layout (M, N multiples of 32, K of 1024)
// C = A * B^T for any pair of MX formats (E8M0 scales; row layout), exact
// BF16 staging (gemm_any.hip).
// fix_lo > 0: the 128 x 128 tiles whose operand rows hold a scale code
// outside [fix_lo, fix_hi] are computed with the codes shifted into the exact
// range where one shift per operand allows; the others are computed as they
// are when `every`, else left as they are (the fix-up pass behind another
// kernel).
hipError_t launch_gemm_mx_any(int fa, const uint8_t* a_codes, const uint8_t* a_scales, int fb,
                              const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                              int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s, uint32_t fix_lo = 0,
                              uint32_t fix_hi = 254, bool every = false);
// MX pairs with an FP6 operand (E2M3/E3M2 against E2M3/E3M2/E2M1, not E3M2 x
// E3M2) on the scaled FP6/FP4 instruction (gemm_f6.hip); shapes it takes.
bool gemm_mx_f6_fits(int fa, int fb, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_mx_f6(int fa, const uint8_t* a_codes, const uint8_t* a_scales, int fb,
                             const uint8_t* b_codes, const uint8_t* b_scales, int64_t M, int64_t N,
                             int64_t K, void* C, int cdt, int64_t ldc, hipStream_t s);
// C = A * B^T of tile-layout MX operands, written quantized along its rows
// (MX format ofmt, row or tile layout) by the GEMM's epilogue.
// C = Q(A) * B^T with A (BF16, row pitch lda) quantized to afmt (FMT_MXFP8 or
// FMT_MXFP4) inside the GEMM; B in bfmt (FMT_MXFP8 or FMT_MXFP4), row layout;
// a_codes / a_scales (both or neither): Q(A) written out, row layout.
hipError_t launch_gemm_quantize_a(int afmt, const uint16_t* a, int64_t lda, const uint8_t* b_codes,
                                  const uint8_t* b_scales, int bfmt, int64_t M, int64_t N, int64_t K, void* C,
                                  int cdt, int64_t ldc, uint8_t* a_codes, uint8_t* a_scales, bool sr,
                                  uint64_t seed, uint64_t counter, hipStream_t s);
hipError_t launch_gemm_mx_tiled_quant(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                      const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                      int64_t N, int64_t K, int ofmt, bool otiled, uint8_t* codes,
                                      uint8_t* scales, bool sr, uint64_t seed, uint64_t counter,
                                      bool ceil, hipStream_t s);
hipError_t launch_gemm_mx_tiled(int fmt, const uint8_t* a_codes, const uint8_t* a_scales,
                                const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                int64_t N, int64_t K, void* C, int cdt, int64_t ldc,
                                hipStream_t s, int fmt_b);
// exact MXFP8 on the DMA pipeline (BF16 instruction); shapes it takes
bool gemm_mxfp8_exact_pipe_fits(int64_t M, int64_t N, int64_t K);
// fa / fb: element types FMT_MXFP8 (E4M3), FMT_MXFP8_E5M2 or FMT_MXINT8, any
// pair
hipError_t launch_gemm_mxfp8_exact_pipe(const uint8_t* a_codes, const uint8_t* a_scales,
                                        const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                        int64_t N, int64_t K, void* C, int cdt, int64_t ldc,
                                        hipStream_t s, int fa = FMT_MXFP8, int fb = FMT_MXFP8);
// fa / fb: FMT_MXFP8 (E4M3), FMT_MXFP8_E5M2 or FMT_MXINT8, any pair; pairs
// other than E4M3 x E4M3 need gemm_mxfp8_exact_pipe_fits
hipError_t launch_gemm_mxfp8_exact(const uint8_t* a_codes, const uint8_t* a_scales,
                                   const uint8_t* b_codes, const uint8_t* b_scales, int64_t M,
                                   int64_t N, int64_t K, void* C, int cdt, int64_t ldc,
                                   hipStream_t s, int fa = FMT_MXFP8, int fb = FMT_MXFP8);
// a_rows: rows of the A source (row_index entries are clamped to it)
hipError_t launch_gemm_nvfp4(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                             const int32_t* row_index, int64_t a_rows, int64_t routed_rows,
                             const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                             int32_t groups, const int64_t* offsets, int64_t N, int64_t K,
                             void* C, int cdt, int64_t ldc, hipStream_t s);

// NVFP4 on the DMA pipeline (FP16 instruction); shapes it takes
bool gemm_nvfp4_pipe_fits(int64_t a_rows, int64_t R, int64_t N, int64_t K);
hipError_t launch_gemm_nvfp4_pipe(const uint8_t* a_codes, const uint8_t* a_scales, const float* a_ts,
                                  const int32_t* row_index, int64_t a_rows, int64_t routed_rows,
                                  const uint8_t* b_codes, const uint8_t* b_scales, const float* b_ts,
                                  int32_t groups, const int64_t* offsets, int64_t N, int64_t K, void* C,
                                  int cdt, int64_t ldc, hipStream_t s);

}  // namespace mxk
