/*
 * mx.h -- C ABI of the block-scaled (microscaling) quantization and GEMM
 * library for AMD Instinct MI355X (gfx950).
 *
 * What the library computes follows these web pages (cited by title and
 * section):
 *   "Microscaling (MX) and block-scaled 4-bit formats"           [MXF]
 *   "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier"              [FP4]
 *   "Thinking Machines ... Inkling 2 Small: end-to-end 4-bit training"  [INK]
 *   "LMSYS and humans& ... MXFP8 and NVFP4 RL recipes in Miles"   [MIL]
 *
 * Formats (mx_format):
 *   MX_MXFP8_E4M3  32 consecutive E4M3 elements share one E8M0 power-of-two
 *                  scale; one-dimensional blocks along a row ([MIL] "Recipe 1:
 *                  End-to-end MXFP8"; [MXF] "The idea").
 *   MX_MXFP4_E2M1  32 E2M1 elements + one E8M0 scale, 4.25 bits per element
 *                  ([MXF] "Microscaling"; [FP4] format table).
 *   MX_NVFP4       16 E2M1 elements + one E4M3 scale, plus one FP32 scale per
 *                  tensor ([MXF] "NVFP4"; [FP4] format table).
 *   The other MX element types ([MXF] "The idea"; [FP4] "The OCP
 *   Microscaling (MX) spec"), 32 elements + one E8M0 scale, bits as the OCP
 *   definitions give them:
 *   MX_MXINT8      8-bit two's complement with 6 fraction bits (-2 .. 127/64);
 *                  with MX_FLAG_RHT16 this is also the block-scaled "S2F6"
 *                  combine codec ([INK] "Why communication became the next
 *                  bottleneck": 8.25 bits per value).
 *   MX_MXFP8_E5M2  E5M2 (bias 15, largest finite 57344; the encoder saturates).
 *   MX_MXFP6_E3M2, MX_MXFP6_E2M3  FP6 (largest 28 / 7.5), packed 4 elements in
 *                  3 bytes: element c of a row at bits 6c .. 6c+5 of the row's
 *                  little-endian bit string.
 *   They are taken by mx_quantize, mx_amax and mx_dequantize, and as GEMM
 *   operands by mx_gemm / mx_gemm_ex (row layout, no flags), also mixed with
 *   MXFP8 E4M3 or MXFP4 (any pair of MX formats: A->fmt may differ from
 *   B->fmt).  MX_MXFP8_E5M2 also has the tile layout; a tiled pair of E4M3 /
 *   E5M2 operands with at least one E5M2 runs on the scaled FP8 instruction
 *   with MX_GEMM_FP8_NATIVE (that flag's bound).
 *
 * Conventions shared by every call:
 *   - Pointers are device pointers (HIP), except the mx_tensor descriptor
 *     itself and the arguments documented as host values.
 *   - Ownership: the caller allocates and frees every buffer.  The library
 *     never allocates, frees or synchronizes; its one device array (1 KiB per
 *     device, the amax slots of mx_quantize_batch_noalloc) is static.
 *   - Execution: every call enqueues work on `stream` (NULL = the default
 *     stream) and returns before the work has run.  Buffers must stay alive
 *     until the stream reaches the work.  Calls are thread-safe; the only
 *     state the library keeps is a per-device flag recording that a kernel's
 *     dynamic LDS limit has been raised (set on first use, idempotent) and,
 *     per device, the address of that static array (looked up on first use).
 *   - Errors: arguments are checked on the host before anything is enqueued
 *     (no HIP call happens on a failed check).  A failed check returns
 *     MX_ERR_NULL / MX_ERR_SHAPE / MX_ERR_ALIGN / MX_ERR_FORMAT /
 *     MX_ERR_UNSUPPORTED; a failed launch returns MX_ERR_HIP.  Nothing aborts.
 *   - Alignment: device pointers to inputs and to code/scale arrays must be
 *     16-byte aligned and leading dimensions must keep every row 16-byte
 *     aligned; GEMM outputs only need element alignment.
 */
#ifndef MX_H_
#define MX_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as hipStream_t. */
typedef struct ihipStream_t* mx_stream;

typedef enum {
  MX_OK = 0,
  MX_ERR_NULL = 1,        /* a required pointer is NULL */
  MX_ERR_SHAPE = 2,       /* sizes inconsistent or not a multiple of the block */
  MX_ERR_ALIGN = 3,       /* pointer or leading dimension misaligned */
  MX_ERR_FORMAT = 4,      /* unknown format, dtype or rounding mode */
  MX_ERR_UNSUPPORTED = 5, /* valid values in a combination the library does not offer */
  MX_ERR_HIP = 6          /* the HIP runtime rejected a launch */
} mx_status;

typedef enum {
  MX_MXFP8_E4M3 = 1,
  MX_MXFP4_E2M1 = 2,
  MX_NVFP4 = 3,
  MX_MXINT8 = 4,
  MX_MXFP8_E5M2 = 5,
  MX_MXFP6_E3M2 = 6,
  MX_MXFP6_E2M3 = 7
} mx_format;

/* Rounding of elements: round-to-nearest, ties to the even code, or
 * stochastic rounding ([MXF] "Open points"; glossary "stochastic rounding";
 * [INK] "A precision choice for each stage").  Out-of-range elements
 * saturate to the largest finite value under both modes. */
typedef enum { MX_RNE = 0, MX_SR = 1 } mx_round;

typedef enum { MX_BF16 = 0, MX_F32 = 1 } mx_dtype;

/* Counter-based random stream for stochastic rounding (host struct, passed by
 * value).  Output element n (row-major linear index in the *output* tensor)
 * uses 16 bits of Philox-4x32-10 (Salmon et al., SC'11) with key = seed and
 * counter = (counter + n/8) in the low two words, so results are a pure
 * function of (input, seed, counter).  A caller that wants disjoint streams
 * advances `counter` by ceil(numel / 8) per call. */
typedef struct {
  uint64_t seed;
  uint64_t counter;
} mx_rng;

/* One quantized matrix, logical shape [rows, cols], blocks along cols.
 * (host struct; the pointers inside are device pointers)
 *   codes   8-bit elements (MXFP8 E4M3 / E5M2, MXINT8): uint8 [rows, cols],
 *           one code per element.
 *           FP4 formats: uint8 [rows, cols/2], element 2j in the low nibble
 *           and element 2j+1 in the high nibble of byte j.
 *           FP6 formats: uint8 [rows, 3 cols / 4], see MX_MXFP6_*.
 *   scales  uint8 [rows, cols/32] E8M0 codes (MX formats) or
 *           uint8 [rows, cols/16] E4M3 codes (NVFP4), row-major.
 *   tensor_scale  NVFP4 only: FP32 S, the per-tensor decode multiplier
 *           (x ~ e2m1 * e4m3 * S); NULL for MX formats.  For the stacked
 *           weights of mx_gemm_grouped it points to one S per group.
 * Rows are dense: the row pitch is the row's code bytes.
 *
 * layout (mx_layout) selects how the code and scale bytes are ordered:
 *   MX_LAYOUT_ROWS   the row-major arrays above (every format, every call).
 *   MX_LAYOUT_TILED  matrix-instruction tiles (MXFP8 E4M3 / E5M2 and MXFP4;
 *           rows % 32 == 0 and cols % 1024 == 0).  Same byte counts as
 *           MX_LAYOUT_ROWS.
 *     codes: the [rows, row_bytes] code matrix is cut into tiles of 32 rows x
 *           128 bytes (256 FP4 or 128 FP8 elements); tile (T, t) (rows 32T..,
 *           code bytes 128t..) is 4096 contiguous bytes at byte offset
 *           (T * row_bytes / 128 + t) * 4096, and within it the 16-byte chunk
 *           c (bytes 16c .. 16c+15 of the tile row) of tile row r is at
 *           (c / 2) * 1024 + ((c % 2) * 32 + r) * 16.
 *     scales: tiles of 32 rows x 32 blocks (1024 elements); tile (T, g) is
 *           1024 contiguous bytes at (T * cols / 1024 + g) * 1024, and the
 *           scale of block b (0..31 within the tile) of tile row r is byte
 *           ((b % 2) * 32 + r) * 16 + b / 2.
 *     (One 1024-byte run of a code tile is exactly the operand fragment a
 *     wavefront loads for a 32 x 64-element matrix instruction, and lane
 *     (b % 2) * 32 + r finds all the scales it applies in one 16-byte word.)
 *   Accepted by mx_quantize (output), mx_dequantize (input) and mx_gemm /
 *   mx_gemm_ex (both operands tiled; MXFP8 then needs MX_GEMM_FP8_NATIVE);
 *   other calls return MX_ERR_UNSUPPORTED for a tiled tensor. */
typedef enum { MX_LAYOUT_ROWS = 0, MX_LAYOUT_TILED = 1 } mx_layout;

typedef struct {
  int32_t fmt;    /* mx_format */
  int32_t layout; /* mx_layout */
  int64_t rows;
  int64_t cols;
  void* codes;
  uint8_t* scales;
  float* tensor_scale;
} mx_tensor;

#define MX_FLAG_RHT16 1u      /* apply the 16-point random Hadamard transform first */
#define MX_FLAG_AMAX_GIVEN 2u /* NVFP4: *amax already holds max|x| (after RHT if set) */
#define MX_FLAG_SCALE_CEIL 4u    /* MX: the smallest scale that saturates no element */
#define MX_FLAG_FOUR_OVER_SIX 8u /* NVFP4, RNE: per block, map the max to 4 or 6 */
#define MX_FLAG_BLOCK_2D 16u     /* NVFP4: one block scale per 16 x 16 tile */

/* Bytes of the code and scale arrays of a [rows, cols] tensor ([MXF]
 * "Microscaling": 8 bits per 32 elements; [FP4] format table).  Returns 0 for
 * an invalid format.  Host function, no device work. */
size_t mx_codes_bytes(int32_t fmt, int64_t rows, int64_t cols);
size_t mx_scales_bytes(int32_t fmt, int64_t rows, int64_t cols);

/* 16 random signs of the Hadamard transform for a seed: bit j set = negate
 * element j of every 16-group.  Taken from Philox-4x32-10 with key = seed and
 * counter (0, 0, 0, 1), a counter no element draw uses.  Host function. */
uint16_t mx_rht_signs(uint64_t seed);

/* Quantize x [rows, cols] (row pitch ld_x elements, dtype xdt) along cols
 * into `out` (fmt, rows, cols and pointers filled in by the caller).
 *
 * MX formats ([MXF] "Microscaling", "The idea"): per 32-block, the shared
 * scale is X = 2^e with e = floor(log2 max|x|) - emax (emax = 8 for E4M3, 2
 * for E2M1), clamped to [-127, 127]; an all-zero block gets e = -127; a block
 * holding NaN or Inf gets the NaN scale code 0xFF and element codes 0.
 * Elements are x / X rounded (rnd) and saturated.
 *
 * NVFP4 ([MXF] "NVFP4"; [FP4] format table): T = max|x| over the tensor,
 * S = T / 2688 (S = 1 when T = 0); per 16-block sb = E4M3 round-to-nearest of
 * max|x| / (6 S); elements x * (1 / (dec(sb) * S)) rounded to E2M1 (rnd),
 * saturating at +-6; blocks whose sb decodes to 0, and zero elements (also
 * where a tiny S makes the reciprocal +Inf), store +-0.  All steps are FP32,
 * one rounding each, in that order.  `amax` (device, one float) is required: with
 * MX_FLAG_AMAX_GIVEN it is read, otherwise T is computed into it first (two
 * passes over x).  Inputs must be finite.
 *
 * MX_FLAG_RHT16 ([MXF] "NVFP4": random Hadamard transforms bound block
 * outliers): each 16-group of a row is first mapped to
 * y = (1/4) H16 D x in FP32 (see mx_hadamard16) and y is quantized.
 *
 * Variants (the stored format is unchanged, so every consumer reads them):
 *   MX_FLAG_SCALE_CEIL (MX formats; [FP4] "The two Blackwell formats: MXFP4
 *     vs NVFP4": a power-of-two scale either wastes range or saturates the
 *     block maximum): e is the smallest integer in [-127, 127] with
 *     max|x| <= g_max * 2^e (g_max = 448 for E4M3, 6 for E2M1), so no
 *     element saturates.
 *   MX_FLAG_FOUR_OVER_SIX (NVFP4 with MX_RNE; [INK] "A precision choice for
 *     each stage": a choice between block scales that lowers the
 *     quantization error): each block is encoded with sb from
 *     max|x| / (6 S) and from max|x| / (4 S); the encoding whose decoded
 *     values have the smaller squared error is kept, the first (6) on a tie.
 *     The error is the exact sum over the 16 elements of
 *     (x - fp32(e2m1 * e4m3 * S))^2, with no rounding, so the choice does
 *     not depend on an order of summation.
 *   MX_FLAG_BLOCK_2D (NVFP4; [MXF] "NVFP4": two-dimensional weight
 *     quantisation): one block scale per tile of 16 rows x 16 columns (the
 *     last band of rows may be shorter), from the tile's max|x|, stored in
 *     each of its rows; the quantized values of x^T are then the transpose of
 *     those of x.  Not combined with MX_FLAG_FOUR_OVER_SIX.
 * Other combinations return MX_ERR_UNSUPPORTED.
 *
 * Requirements: cols % 32 == 0 (MX) or % 16 == 0 (NVFP4); out->rows == rows.
 * SR stream: see mx_rng. */
mx_status mx_quantize(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ld_x,
                      const mx_tensor* out, int32_t rnd, mx_rng rng, uint32_t flags,
                      uint16_t rht_sign_mask, float* amax, mx_stream stream);

/* Several quantizations in one call: jobs[i] holds the arguments of one
 * mx_quantize call, and the result is that of calling mx_quantize on jobs[0],
 * jobs[1], ... in order on `stream`.  Consecutive jobs that write MXFP8 or
 * MXFP4 in the tile layout with the same format, input dtype, rounding and
 * MX_FLAG_RHT16 setting are quantized by one kernel launch (up to 4 per
 * launch), which saves the launch gaps and the ramp of small tensors.
 * Consecutive NVFP4 jobs with the same input dtype, rounding, flags and sign
 * mask, and no amax or tensor-scale slot in common (a given amax may be
 * shared), share each pass (up to 16 per launch): one launch clears their
 * amax slots, one computes every amax, one encodes -- the expert weights of
 * a mixture-of-experts layer in three launches instead of 2 per expert.
 * Other jobs are launched one by one.  Every job is checked before anything is
 * enqueued; the first failing job's status is returned.  No job's input may
 * be written by an earlier job of the same call.  `jobs` is a host array;
 * `out` points to a host descriptor. */
typedef struct {
  const void* x;
  int32_t xdt;
  int64_t rows, cols, ld_x;
  const mx_tensor* out;
  int32_t rnd;
  mx_rng rng;
  uint32_t flags;
  uint16_t rht_sign_mask;
  float* amax;
} mx_quantize_job;
mx_status mx_quantize_batch(const mx_quantize_job* jobs, int32_t count, mx_stream stream);

/* Per-tensor amax of x (after the Hadamard transform when MX_FLAG_RHT16 is
 * set) into *amax (device float, overwritten).  The first pass of NVFP4
 * quantization ([MXF] "NVFP4": second-level per-tensor scale). */
mx_status mx_amax(const void* x, int32_t xdt, int64_t rows, int64_t cols, int64_t ld_x,
                  uint32_t flags, uint16_t rht_sign_mask, float* amax, mx_stream stream);

/* Decode `in` into y [rows, cols] (row pitch ld_y, dtype ydt): MX elements
 * times 2^(c-127); NVFP4 as fp32(e2m1 * e4m3 * S) ([MXF] glossary "scale
 * factor": multiplied back after).  With MX_FLAG_RHT16 the inverse Hadamard
 * transform (same signs) is applied to the FP32 values before output.  BF16
 * output rounds to nearest even. */
mx_status mx_dequantize(const mx_tensor* in, void* y, int32_t ydt, int64_t ld_y, uint32_t flags,
                        uint16_t rht_sign_mask, mx_stream stream);

/* Round-trip error statistics of a decoded tensor y against its source x
 * (measurement support for the decode row; [MXF] "NVFP4": random Hadamard
 * transforms bound block outliers and stochastic rounding keeps gradients
 * unbiased; glossary "stochastic rounding": the expected value is
 * preserved).  x: [rows, cols] BF16 or FP32 (xdt), row pitch ld_x; y:
 * [rows, cols] FP32, row pitch ld_y (e.g. mx_dequantize's output).  Writes
 * four FP64 values to stats (device, 16-byte aligned): sum (y - x)^2,
 * sum x^2, sum (y - x), max |y - x|, each term formed in FP64; relative RMSE
 * = sqrt(stats[0] / stats[1]), mean error (bias) = stats[2] / (rows * cols).
 * The sums are accumulated with atomics, so their last bits may differ from
 * call to call.  cols % 8 == 0; 16-byte aligned rows.  The stats buffer is
 * cleared by a kernel on the stream first (no memset).  Errors:
 * MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_FORMAT, MX_ERR_HIP. */
mx_status mx_error_stats(const void* x, int32_t xdt, int64_t ld_x, const float* y, int64_t ld_y, int64_t rows,
                         int64_t cols, double* stats, mx_stream stream);

/* Backward-pass requantization ([INK] "A precision choice for each stage":
 * dequantize saved values, transpose at higher precision, stochastically
 * re-quantize to MXFP8).  Source [rows, cols]: either an NVFP4 tensor `src`
 * (x = fp32(e2m1 * e4m3 * S)) or a BF16 matrix x_bf16 with row pitch ld_x
 * (exactly one of the two is non-NULL).  Output `out`: MXFP8 E4M3 of the
 * transpose, logical [cols, rows], 32-blocks along its rows (the source row
 * axis).  The SR index of an element is its position in the output.
 * Requirements: rows % 32 == 0, cols % 16 == 0, out->fmt == MX_MXFP8_E4M3. */
mx_status mx_requant_transpose(const mx_tensor* src, const void* x_bf16, int64_t ld_x,
                               int64_t rows, int64_t cols, const mx_tensor* out, int32_t rnd,
                               mx_rng rng, mx_stream stream);

/* Standalone 16-point random Hadamard transform along rows of x [rows, cols]
 * (dense rows): y = (1/4) H16 D x per 16-group, H16 the Sylvester Hadamard
 * matrix in natural order, D = diag of the signs in sign_mask, evaluated in
 * FP32 as butterfly stages of stride 1, 2, 4, 8.  inverse != 0 applies the
 * stages, the 1/4 factor, then the signs (x = D H16 y / 4).  ([MXF] "NVFP4";
 * [INK] "Why communication became the next bottleneck".)  cols % 16 == 0;
 * x and y may not overlap unless x == y with xdt == ydt. */
mx_status mx_hadamard16(const void* x, int32_t xdt, void* y, int32_t ydt, int64_t rows,
                        int64_t cols, uint16_t sign_mask, int32_t inverse, mx_stream stream);

/* Block-scaled GEMM C = A * B^T ([MXF] "Hardware and kernels": the block
 * scales are applied inside the matrix multiply).  A is [M, K], B is [N, K]
 * (both quantized along K), C is [M, N] row-major with row pitch ldc in
 * dtype cdt (FP32, or BF16 rounded to nearest even).  The result is the
 * FP32-accumulated sum of the exact products of the decoded operands:
 *   MXFP4  scaled FP4 matrix instructions (E8M0 scales inside the instruction);
 *   MXFP8  E4M3 * 2^(c-127) converted to exact BF16 (exact for scale codes c
 *          in [3, 246]), BF16 matrix instructions, whose products must be
 *          normal FP32 values (c_A + c_B >= 146); a fix-up pass recomputes
 *          every tile holding a code outside [73, 246] with each operand's
 *          codes shifted by one power of two per tile so that both hold
 *          (exact unless a tile's codes span more than the range on one
 *          side); code 255 gives NaN in its rows / columns;
 *   NVFP4  e2m1 * e4m3 converted to exact FP16, FP16 matrix instructions
 *          (BF16 for shapes too small for the pipelined kernel), the FP32
 *          result multiplied by S_A * S_B.
 *   FP6 pairs (E2M3 or E3M2 against E2M3, E3M2 or MXFP4, not E3M2 x E3M2),
 *          K % 512 == 0: scaled FP6/FP4 matrix instructions, which form the
 *          exact sum of each instruction's 64 products (measured on gfx950).
 *          E3M2 x E3M2, which that instruction sums in a narrower window, is
 *          decoded to exact BF16 in the same kernel (scale codes 68 .. 250,
 *          where the decode is exact and the products are normal FP32
 *          values; tiles with other codes recomputed by the generic kernel
 *          with shifted codes, as for MXFP8).
 *   Other pairs of 8-bit types (E4M3, E5M2, INT8: E5M2 x E4M3, INT8 x INT8,
 *          INT8 x E4M3, ...) where the MXFP8 pipeline fits (K % 512 == 0,
 *          M * N >= 2^23): as MXFP8, each element times its scale converted to BF16,
 *          exact for scale codes c in [17, 239] (E5M2) and [7, 254] (INT8)
 *          with normal FP32 products (c_A + c_B >= 128 + g_A + g_B, g
 *          below); tiles holding a code below half of that bound or outside
 *          the range are recomputed as for MXFP8.
 *   Other MX pairs (8-bit types mixed with FP6 or FP4, FP6 and 8-bit pairs
 *          at other shapes): every element times its scale decoded to exact
 *          BF16, BF16 matrix instructions; a tile holding a code below half
 *          of 128 + g_A + g_B, or outside the decode's exact range, is
 *          computed with shifted codes as in the MXFP8 fix-up.
 * The scaled matrix instructions (MXFP4, FP6 pairs, MX_GEMM_FP8_NATIVE) form
 * the exact sum of their scaled products and round it once into FP32,
 * subnormals included (measured), so the bound holds while every product is
 * a multiple of 2^-149: an element of type X is a multiple of 2^-g(X) (E2M1
 * 1, E2M3 3, E3M2 4, E4M3 9, E5M2 16), which gives c_A + c_B >= 105 + g(A) +
 * g(B) (MXFP4 pairs 107).  The tile-layout paths (MXFP4 and native FP8 on
 * MX_LAYOUT_TILED operands, mx_gemm_quantize) detect tiles whose scale codes
 * could pair below that and compute them again with raised codes; the
 * row-layout MXFP4 and FP6-pair kernels are followed by a fix-up pass that
 * recomputes every tile holding a code below half of that bound (rounded
 * up) with shifted codes.  So every path meets the bound for every finite
 * code whose tile one shift per operand fits into range.  Scale code 255
 * (NaN) gives NaN in exactly the output rows / columns whose blocks carry it.
 * Requirements: A->fmt == B->fmt, or both MX formats (E8M0 scales) in the
 * row layout; A->cols == B->cols == K; K % 32 == 0.  M == 0 or N == 0
 * enqueues nothing; K == 0 (an empty sum) writes C = 0. */
mx_status mx_gemm(const mx_tensor* A, const mx_tensor* B, void* C, int32_t cdt, int64_t ldc,
                  mx_stream stream);

/* mx_gemm with options.  MX_GEMM_FP8_NATIVE (FP8 pairs: MXFP8 E4M3 and E5M2,
 * mixed too, row or tile layout) runs the product on gfx950's scaled FP8
 * matrix instruction instead.  That instruction sums the
 * products of each 8-element K group in a window about 14 bits below the
 * group's largest product before FP32 accumulation, so its error can reach
 * about 2^-13 * sum|a*b| (measured), outside the 1e-5 bound mx_gemm meets;
 * in exchange it runs at the FP8 matrix rate. */
#define MX_GEMM_FP8_NATIVE 1u
mx_status mx_gemm_ex(const mx_tensor* A, const mx_tensor* B, void* C, int32_t cdt, int64_t ldc,
                     uint32_t flags, mx_stream stream);

/* Block-scaled GEMM whose product leaves the kernel already quantized
 * ([MXF] "Open points": fused quantize-and-GEMM kernels, since computing block
 * scales is memory traffic of its own).  C = A * B^T [M, N] as mx_gemm_ex
 * computes it in FP32 (tile-layout operands: MXFP4, or MXFP8 with
 * MX_GEMM_FP8_NATIVE and that flag's bound), then quantized along its rows
 * exactly as mx_quantize quantizes an FP32 matrix: 32-column blocks, E8M0
 * floor rule (or MX_FLAG_SCALE_CEIL), rounding rnd, SR draws indexed by the
 * element's row-major position in C.  The FP32 product is never stored: since
 * it is fixed only to within the GEMM's bound, codes and scales are too (a
 * value near a rounding or scale boundary may land on either side).
 * `out` is MXFP8 (E4M3, or E5M2 -- the usual gradient format) or MXFP4 with
 * rows = M and cols = N, in the row layout or
 * the tile layout (then M % 32 == 0 and N % 1024 == 0), so it can be the A
 * operand of the next product.  flags: MX_GEMM_FP8_NATIVE,
 * MX_FLAG_SCALE_CEIL; anything else returns MX_ERR_UNSUPPORTED, as do
 * row-layout operands and an NVFP4 output (its tensor scale needs the whole
 * product first).  K == 0 returns MX_ERR_SHAPE.  Cost (4096^3 MXFP4,
 * measured): 42 us fused against 48 us for mx_gemm into a BF16 buffer
 * followed by mx_quantize with MX_RNE, 48 against 52 us with MX_SR. */
mx_status mx_gemm_quantize(const mx_tensor* A, const mx_tensor* B, const mx_tensor* out,
                           int32_t rnd, mx_rng rng, uint32_t flags, mx_stream stream);

/* Block-scaled GEMM whose A operand is quantized inside the GEMM's prologue
 * ([MXF] "Open points": fused quantize-and-GEMM kernels, since computing block
 * scales is memory traffic of its own).  A: BF16 [M, K] (device, row pitch
 * lda elements, 16-byte aligned rows).  Every 32-element block of A's rows is
 * quantized in the kernel exactly as mx_quantize quantizes A into a_fmt
 * (MX_MXFP8_E4M3 or MX_MXFP4_E2M1, E8M0 floor rule, rounding rnd, SR draws
 * indexed by the element's row-major position in A with the given rng), and
 * C = Q(A) * B^T [M, N] (cdt, row pitch ldc) is the FP32-accumulated sum of
 * the exact products of the decoded operands.  B: MXFP8 E4M3 or MXFP4, row
 * layout, cols == K.  a_out (optional, NULL to skip): receives Q(A) (fmt
 * a_fmt, row layout, [M, K]), e.g. for the backward pass; each block is
 * written once.  Runs on the BF16 matrix instruction after decoding in LDS,
 * which is within the bound while every decoded value is a normal BF16 value
 * (E4M3 codes 3 .. 246; E2M1 2 .. 252) and every product a normal FP32 value
 * (c_A + c_B >= 128 + g_A + g_B, g: E4M3 9, E2M1 1).  With a_out, a fix-up
 * pass recomputes the tiles where a code falls below half of that bound
 * (rounded up) or above 239 from Q(A) and B with shifted codes, as mx_gemm
 * does; without it, codes outside those limits are the caller's to avoid
 * (Q(A)'s codes fall below half of it only for blocks with max |x| < 2^-46).  At 4096^3 it is
 * slower than mx_quantize followed by mx_gemm, because each of the N/256
 * column tiles quantizes its A panel again (measured; the fused product pays
 * only where A must not be written before the GEMM).  Requirements: K % 32
 * == 0, K > 0.  Errors: MX_ERR_NULL, MX_ERR_SHAPE, MX_ERR_ALIGN, MX_ERR_FORMAT,
 * MX_ERR_UNSUPPORTED, MX_ERR_HIP. */
mx_status mx_gemm_quantize_a(const void* A, int64_t lda, int64_t M, int32_t a_fmt, int32_t rnd, mx_rng rng,
                             const mx_tensor* B, void* C, int32_t cdt, int64_t ldc, const mx_tensor* a_out,
                             mx_stream stream);

/* Grouped NVFP4 GEMM for a mixture-of-experts forward pass ([MXF] "NVFP4";
 * [INK] "A precision choice for each stage": NVFP4 forward in the expert
 * layers).  B stacks num_groups expert matrices [N, K] as one NVFP4 tensor of
 * rows = num_groups * N whose tensor_scale points to num_groups floats.
 * group_offsets (device, int64 [num_groups + 1], non-decreasing, first 0, last
 * = number of routed rows R) assigns output rows [off[e], off[e+1]) to expert
 * e.  Being on the device, the offsets are not checked; each range is clamped
 * into [0, R] there, so offsets that break this contract give wrong rows but
 * never a write outside C.  A row source: if row_index is non-NULL (device int32 [R]), routed row r
 * reads A row row_index[r] (A is [tokens, K]; entries outside [0, tokens) are
 * clamped into it); otherwise A has R rows.
 * C is [R, N] (pitch ldc).  C[r, :] = A[src(r)] * B_e^T * S_A * S_B[e].
 * Requirements: A and B NVFP4, K % 32 == 0, num_groups >= 1, `routed_rows`
 * (host) = R, B->rows % num_groups == 0, and with row_index and R > 0, A
 * has at least one row (else MX_ERR_SHAPE).  R == 0 enqueues nothing;
 * K == 0 writes C = 0. */
mx_status mx_gemm_grouped(const mx_tensor* A, const int32_t* row_index, int64_t routed_rows,
                          const mx_tensor* B, int32_t num_groups, const int64_t* group_offsets,
                          void* C, int32_t cdt, int64_t ldc, mx_stream stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * result as mx_quantize_batch(jobs, count, stream), with the amax slot of
 * every NVFP4 job taken from a library-owned device array instead of
 * jobs[i].amax.  Job i uses slot i of that array; the array holds
 * MX_NOALLOC_MAX_JOBS FP32 values (1 KiB) per device, lives until the process
 * ends, and is obtained once per device on the first call made with that
 * device current.  The call allocates nothing and frees nothing.
 * Requirements, on top of mx_quantize_batch's: count <= MX_NOALLOC_MAX_JOBS
 * (else MX_ERR_SHAPE); every jobs[i].amax is NULL and no job sets
 * MX_FLAG_AMAX_GIVEN (else MX_ERR_UNSUPPORTED); `stream` belongs to the
 * current device (else MX_ERR_UNSUPPORTED).  A failure of the symbol lookup
 * returns MX_ERR_HIP.  Every slot a job uses is written by a kernel before it
 * is read, so nothing left by an earlier call leaks into a result.  All calls
 * on one device share the array: calls whose work can overlap on that device
 * (other streams, other threads) race and must be serialized by the
 * caller. */
#define MX_NOALLOC_MAX_JOBS 256
mx_status mx_quantize_batch_noalloc(const mx_quantize_job* jobs, int32_t count, mx_stream stream);

/* Human-readable name of a status code (static string). */
const char* mx_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MX_H_ */
