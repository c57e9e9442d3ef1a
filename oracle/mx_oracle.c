/*
 * mx_oracle.c -- plain, slow CPU oracle for block-scaled (microscaling)
 * quantization and block-scaled GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source, header, table or helper with the
 * HIP library; every number format is decoded from its bit-level definition
 * and every encoder works by searching the decoded alphabet for the nearest
 * value, never by bit tricks.
 *
 * Sources (web pages, cited by title and section):
 *   [MXF]  "Microscaling (MX) and block-scaled 4-bit formats"
 *          sections "The problem", "Microscaling", "The idea", "NVFP4",
 *          "Hardware and kernels", glossary ("scale factor",
 *          "stochastic rounding").
 *   [FP4]  "08 - FP4, MXFP4, NVFP4: The Blackwell Frontier"
 *          sections "Why 4-bit floats at all?" (E2M1 bit layout and code
 *          points), "The two Blackwell formats: MXFP4 vs NVFP4" (format
 *          table), "The OCP Microscaling (MX) spec".
 *   [INK]  "Thinking Machines ... Inkling 2 Small: end-to-end 4-bit training"
 *          section "A precision choice for each stage" (stochastic rounding,
 *          dequantize -> transpose -> stochastic requantize to MXFP8).
 *   [MIL]  "LMSYS and humans& ... MXFP8 and NVFP4 RL recipes in Miles"
 *          section "Recipe 1: End-to-end MXFP8" (32 E4M3 values share one
 *          E8M0 scale, one-dimensional block).
 *   [PHX]  Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as
 *          1, 2, 3", SC'11 -- the Philox-4x32 bijection and key schedule.
 *
 * Where the pages leave a step open, the plainest reading is taken; each such
 * reading is marked READING below.
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fno-fast-math -shared
 * (FP32 expressions must be evaluated exactly as written, one IEEE rounding
 * per operation, no fused multiply-add.)
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define MXO_MXFP8 1
#define MXO_MXFP4 2
#define MXO_NVFP4 3
#define MXO_MXINT8 4      /* 8-bit two's complement, 6 fraction bits (S2F6) */
#define MXO_MXFP8_E5M2 5
#define MXO_MXFP6_E3M2 6
#define MXO_MXFP6_E2M3 7
#define MXO_RNE 0
#define MXO_SR 1

/* Quantizer variants (bits of the `variant` argument). */
#define MXO_V_CEIL 1   /* MX: smallest shared scale that saturates no element */
#define MXO_V_FOUR6 2  /* NVFP4: per block, map the block max to 4 or to 6 */
#define MXO_V_2D 4     /* NVFP4: one block scale per 16 x 16 tile */

/* ------------------------------------------------------------------------ */
/* Element and scale decoders, written from the bit-level definitions.       */
/* ------------------------------------------------------------------------ */

/* E2M1: bits S E E M (bit 3 = sign), exponent bias 1, exponent 0 is
 * subnormal (value = M * 0.5).  [FP4] "Why 4-bit floats at all?" gives the
 * layout and the resulting code points {0, .5, 1, 1.5, 2, 3, 4, 6}; [MXF]
 * "The problem" gives the same non-negative alphabet. */
double mxo_e2m1_decode(uint32_t code) {
  code &= 0xF;
  int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  double mag = (e == 0) ? m * 0.5 : ldexp(1.0 + m / 2.0, e - 1);
  return s ? -mag : mag;
}

/* E4M3 (READING: the OCP "FN" flavour -- bias 7, no infinities, the all-ones
 * exponent-and-mantissa pattern is NaN, largest finite 448).  The pages name
 * E4M3 as the MXFP8 element ([MIL] "Recipe 1") and as the NVFP4 block scale
 * ([MXF] "NVFP4"; [FP4] format table) without giving its bits. */
double mxo_e4m3_decode(uint32_t code) {
  code &= 0xFF;
  int s = (code >> 7) & 1, e = (code >> 3) & 0xF, m = code & 7;
  if (e == 15 && m == 7) return NAN;
  double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
  return s ? -mag : mag;
}

/* E8M0: an unsigned power of two made of exponent bits only, 2^-127..2^127,
 * with one code reserved for NaN ([FP4] "The OCP Microscaling (MX) spec";
 * [MXF] "Microscaling"). */
double mxo_e8m0_decode(uint32_t code) {
  code &= 0xFF;
  if (code == 0xFF) return NAN;
  return ldexp(1.0, (int)code - 127);
}

/* The other MX element types ([MXF] "The idea" and [FP4] "The OCP
 * Microscaling (MX) spec" name FP8 E5M2, FP6 E3M2 and E2M3, and INT8 as MX
 * elements, without their bits).  READING: the OCP definitions --
 *   E5M2: bias 15, IEEE-style, exponent 31 holds Inf (mantissa 0) and NaN;
 *         largest finite 57344.
 *   E3M2: bias 3, no Inf or NaN, largest 28.   E2M3: bias 1, largest 7.5.
 *   INT8: two's complement with an implied scale 2^-6, so -2 .. 127/64.
 * The last is also this reading of the block-scaled "S2F6" 8-bit fixed-point
 * format ([INK] "Why communication became the next bottleneck": 8.25 bits per
 * value, i.e. 8-bit elements with one 8-bit scale per 32). */
static double minifloat(uint32_t code, int ebits, int mbits, int bias, int ieee_top) {
  int s = (code >> (ebits + mbits)) & 1;
  int e = (code >> mbits) & ((1 << ebits) - 1);
  int m = code & ((1 << mbits) - 1);
  double mag;
  if (ieee_top && e == (1 << ebits) - 1) mag = m ? NAN : INFINITY;
  else if (e == 0) mag = ldexp((double)m, 1 - bias - mbits);
  else mag = ldexp(1.0 + ldexp((double)m, -mbits), e - bias);
  return s ? -mag : mag;
}
double mxo_e5m2_decode(uint32_t code) { return minifloat(code & 0xFF, 5, 2, 15, 1); }
double mxo_e3m2_decode(uint32_t code) { return minifloat(code & 0x3F, 3, 2, 3, 0); }
double mxo_e2m3_decode(uint32_t code) { return minifloat(code & 0x3F, 2, 3, 1, 0); }
double mxo_int8_decode(uint32_t code) { return (double)(int8_t)(uint8_t)code / 64.0; }

/* ------------------------------------------------------------------------ */
/* Alphabets: the non-negative finite values of an element format, sorted,  */
/* with their codes.  Built by decoding every code.                          */
/* ------------------------------------------------------------------------ */
typedef struct {
  int n;
  double v[256];
  uint32_t code[256];
  uint32_t sign_bit; /* sign-magnitude formats: the sign bit; 0 for two's complement */
  int twos;          /* two's complement: v holds every value, negative ones included */
} mxo_alphabet;

static mxo_alphabet g_e2m1, g_e4m3, g_e5m2, g_e3m2, g_e2m3, g_int8;
static int g_ready = 0;

static void build_alphabet(mxo_alphabet* a, double (*dec)(uint32_t), int ncodes,
                           uint32_t sign_bit, int twos) {
  a->n = 0;
  a->sign_bit = sign_bit;
  a->twos = twos;
  for (int c = 0; c < ncodes; ++c) {
    if (!twos && (c & sign_bit)) continue; /* non-negative half only */
    double v = dec((uint32_t)c);
    if (isnan(v) || isinf(v)) continue;
    a->v[a->n] = v;
    a->code[a->n] = (uint32_t)c;
    a->n++;
  }
  /* insertion sort by value (codes are already monotone, but do not rely on it) */
  for (int i = 1; i < a->n; ++i) {
    double v = a->v[i];
    uint32_t c = a->code[i];
    int j = i - 1;
    while (j >= 0 && a->v[j] > v) {
      a->v[j + 1] = a->v[j];
      a->code[j + 1] = a->code[j];
      --j;
    }
    a->v[j + 1] = v;
    a->code[j + 1] = c;
  }
}

static void ensure_tables(void) {
  if (g_ready) return;
  build_alphabet(&g_e2m1, mxo_e2m1_decode, 16, 0x8, 0);
  build_alphabet(&g_e4m3, mxo_e4m3_decode, 256, 0x80, 0);
  build_alphabet(&g_e5m2, mxo_e5m2_decode, 256, 0x80, 0);
  build_alphabet(&g_e3m2, mxo_e3m2_decode, 64, 0x20, 0);
  build_alphabet(&g_e2m3, mxo_e2m3_decode, 64, 0x20, 0);
  build_alphabet(&g_int8, mxo_int8_decode, 256, 0, 1);
  g_ready = 1;
}

/* Thread count of the oracle's OpenMP loops (for timing it on one core). */
void mxo_set_threads(int n) { omp_set_num_threads(n > 0 ? n : 1); }
int mxo_get_threads(void) { return omp_get_max_threads(); }

int mxo_init(void) {
  ensure_tables();
  return g_e2m1.n * 1000 + g_e4m3.n;
}

/* Index i with v[i] <= a < v[i+1]; a must be in [0, vmax). */
static int bracket(const mxo_alphabet* al, double a) {
  int lo = 0, hi = al->n - 1; /* invariant v[lo] <= a < v[hi] */
  while (hi - lo > 1) {
    int mid = (lo + hi) / 2;
    if (al->v[mid] <= a) lo = mid;
    else hi = mid;
  }
  return lo;
}

/* Round-to-nearest, ties to the even code (READING of "round-to-nearest",
 * [MXF] "Open points"), saturating to the largest finite value (READING:
 * elements beyond the range saturate), sign preserved, so -0 exists.
 * y must not be NaN. */
static uint32_t encode_rne(const mxo_alphabet* al, double y) {
  if (al->twos) { /* signed list: saturate at both ends, nearest, ties to the even code */
    if (y <= al->v[0]) return al->code[0];
    if (y >= al->v[al->n - 1]) return al->code[al->n - 1];
    int i = bracket(al, y);
    double lo = al->v[i], hi = al->v[i + 1], mid = 0.5 * (lo + hi);
    if (y < mid) return al->code[i];
    if (y > mid) return al->code[i + 1];
    return (al->code[i] & 1) ? al->code[i + 1] : al->code[i];
  }
  uint32_t sign = signbit(y) ? al->sign_bit : 0;
  double a = fabs(y);
  double vmax = al->v[al->n - 1];
  if (a >= vmax) return sign | al->code[al->n - 1];
  int i = bracket(al, a);
  double lo = al->v[i], hi = al->v[i + 1];
  double mid = 0.5 * (lo + hi); /* exact: both are short dyadic numbers */
  uint32_t c;
  if (a < mid) c = al->code[i];
  else if (a > mid) c = al->code[i + 1];
  else c = (al->code[i] & 1) ? al->code[i + 1] : al->code[i];
  return sign | c;
}

/* Stochastic rounding: round up or down at random, with the probability of
 * going up proportional to the distance from the lower neighbour, so the
 * expected value is preserved ([MXF] glossary "stochastic rounding"; [INK]
 * "A precision choice for each stage").
 * READING: 16 random bits r per element; with lo <= a < hi the neighbours and
 * t = (a - lo) * 2^16 / (hi - lo), round up exactly when r < floor(t).
 * P(up) = floor(t)/65536.  Saturate at the largest finite value. */
static uint32_t encode_sr(const mxo_alphabet* al, double y, uint32_t r16) {
  if (al->twos) { /* READING: on the signed value -- up means toward +inf */
    if (y <= al->v[0]) return al->code[0];
    if (y >= al->v[al->n - 1]) return al->code[al->n - 1];
    int i = bracket(al, y);
    double lo = al->v[i], hi = al->v[i + 1];
    if (y == lo) return al->code[i];
    /* t = floor((y - lo) * 2^16 / (hi - lo)), formed as floor(y * S) - lo * S
     * with S = 2^16 / (hi - lo) a power of two: y - lo itself is not exact
     * for a tiny negative y (lo = -1/64), both terms here are. */
    double S = 65536.0 / (hi - lo);
    double ft = floor(y * S) - lo * S;
    return (double)(r16 & 0xFFFF) < ft ? al->code[i + 1] : al->code[i];
  }
  uint32_t sign = signbit(y) ? al->sign_bit : 0;
  double a = fabs(y);
  double vmax = al->v[al->n - 1];
  if (a >= vmax) return sign | al->code[al->n - 1];
  int i = bracket(al, a);
  double lo = al->v[i], hi = al->v[i + 1];
  if (a == lo) return sign | al->code[i];
  double t = (a - lo) * 65536.0 / (hi - lo); /* exact: hi-lo is a power of two */
  double ft = floor(t);
  return sign | ((double)(r16 & 0xFFFF) < ft ? al->code[i + 1] : al->code[i]);
}

uint32_t mxo_e2m1_encode_rne(double y) { ensure_tables(); return encode_rne(&g_e2m1, y); }
uint32_t mxo_e4m3_encode_rne(double y) { ensure_tables(); return encode_rne(&g_e4m3, y); }
uint32_t mxo_e2m1_encode_sr(double y, uint32_t r) { ensure_tables(); return encode_sr(&g_e2m1, y, r); }
uint32_t mxo_e4m3_encode_sr(double y, uint32_t r) { ensure_tables(); return encode_sr(&g_e4m3, y, r); }

/* Element format of an MX format: alphabet, emax (the exponent of the
 * element's largest power of two) and bits per element. */
typedef struct {
  const mxo_alphabet* al;
  int emax, bits;
} mxo_elem;

static int elem_of(int fmt, mxo_elem* e) {
  ensure_tables();
  switch (fmt) {
    case MXO_MXFP8: *e = (mxo_elem){&g_e4m3, 8, 8}; return 0;
    case MXO_MXFP4: *e = (mxo_elem){&g_e2m1, 2, 4}; return 0;
    case MXO_MXINT8: *e = (mxo_elem){&g_int8, 0, 8}; return 0;
    case MXO_MXFP8_E5M2: *e = (mxo_elem){&g_e5m2, 15, 8}; return 0;
    case MXO_MXFP6_E3M2: *e = (mxo_elem){&g_e3m2, 4, 6}; return 0;
    case MXO_MXFP6_E2M3: *e = (mxo_elem){&g_e2m3, 2, 6}; return 0;
    default: return -1;
  }
}

/* Element codes of one MX format (fmt as above): RNE, and SR with r16. */
uint32_t mxo_elem_encode_rne(int fmt, double y) {
  mxo_elem e;
  if (elem_of(fmt, &e)) return 0xFFFFFFFFu;
  return encode_rne(e.al, y);
}
uint32_t mxo_elem_encode_sr(int fmt, double y, uint32_t r) {
  mxo_elem e;
  if (elem_of(fmt, &e)) return 0xFFFFFFFFu;
  return encode_sr(e.al, y, r);
}
double mxo_elem_decode(int fmt, uint32_t code) {
  switch (fmt) {
    case MXO_MXFP8: return mxo_e4m3_decode(code);
    case MXO_MXFP4: return mxo_e2m1_decode(code);
    case MXO_MXINT8: return mxo_int8_decode(code);
    case MXO_MXFP8_E5M2: return mxo_e5m2_decode(code);
    case MXO_MXFP6_E3M2: return mxo_e3m2_decode(code);
    case MXO_MXFP6_E2M3: return mxo_e2m3_decode(code);
    default: return NAN;
  }
}

/* ------------------------------------------------------------------------ */
/* Counter-based random numbers: Philox-4x32 with 10 rounds, from [PHX].     */
/* ------------------------------------------------------------------------ */
static void mul32(uint32_t a, uint32_t b, uint32_t* hi, uint32_t* lo) {
  uint64_t p = (uint64_t)a * (uint64_t)b;
  *hi = (uint32_t)(p >> 32);
  *lo = (uint32_t)p;
}

/* One application of the Philox S-box followed by the word permutation of
 * the 4-word variant: the two multiplied words pass their low halves
 * through, their high halves are xored into the other two words together
 * with the round key.  Multipliers and Weyl key increments as published. */
void mxo_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
  uint32_t k0 = key_in[0], k1 = key_in[1];
  for (int round = 0; round < 10; ++round) {
    uint32_t hi0, lo0, hi1, lo1;
    mul32(M0, c0, &hi0, &lo0);
    mul32(M1, c2, &hi1, &lo1);
    uint32_t n0 = hi1 ^ c1 ^ k0;
    uint32_t n1 = lo1;
    uint32_t n2 = hi0 ^ c3 ^ k1;
    uint32_t n3 = lo0;
    c0 = n0; c1 = n1; c2 = n2; c3 = n3;
    k0 += W0;
    k1 += W1;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* READING (stream layout): key = (seed low word, seed high word); the random
 * value of output element n comes from call number counter + floor(n/8),
 * whose 128-bit counter is (low word, high word, 0, 0); the call's four
 * words give eight 16-bit values, element n taking half (n & 1) of word
 * (n & 7) >> 1, low half first. */
uint32_t mxo_rand16(uint64_t seed, uint64_t counter, uint64_t n) {
  uint64_t c = counter + (n >> 3);
  uint32_t ctr[4] = {(uint32_t)c, (uint32_t)(c >> 32), 0u, 0u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  mxo_philox4x32_10(ctr, key, w);
  uint32_t word = w[(n & 7) >> 1];
  return (word >> (16 * (n & 1))) & 0xFFFFu;
}

/* Element codes of many values at once: y[t] encoded to the element type of
 * MX format `elem` (E4M3 for 1, E2M1 for 2, ...) by round-to-nearest, or by SR with the random value of
 * element index n[t] of the stream (seed, counter).  A loop over the encoders
 * and the stream above, for checks that need many encodings. */
void mxo_encode_elems(int elem, int rnd, const double* y, const uint64_t* n, int64_t count,
                      uint64_t seed, uint64_t counter, uint8_t* codes) {
  mxo_elem el;
  if (elem_of(elem, &el)) return;
  const mxo_alphabet* al = el.al;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t)
    codes[t] = (uint8_t)(rnd == MXO_SR ? encode_sr(al, y[t], mxo_rand16(seed, counter, n[t]))
                                       : encode_rne(al, y[t]));
}

/* READING: the 16 random signs of the Hadamard transform are the low 16 bits
 * of word 0 of the Philox call with counter (0, 0, 0, 1), a counter that no
 * element draw uses (element draws keep the top word 0). */
uint32_t mxo_rht_signs(uint64_t seed) {
  uint32_t ctr[4] = {0u, 0u, 0u, 1u};
  uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
  uint32_t w[4];
  mxo_philox4x32_10(ctr, key, w);
  return w[0] & 0xFFFFu;
}

/* ------------------------------------------------------------------------ */
/* Random Hadamard transform over groups of 16 along a row.                 */
/* READING: y = (1/4) * H16 * D * x, with H16 the Sylvester Hadamard matrix  */
/* in natural order (entry (i,j) = (-1)^popcount(i&j)) and D the diagonal of */
/* signs (bit j of the mask set = negate element j), the same signs for all  */
/* groups.  Evaluated in FP32 as four butterfly stages with strides 1, 2, 4, */
/* 8, then the 1/4 factor; the inverse runs the same stages on y, scales by  */
/* 1/4, then reapplies the signs.  [MXF] "NVFP4" (random Hadamard transforms */
/* to bound block outliers); [INK] "Why communication became the next        */
/* bottleneck" (a random Hadamard rotation spreads outliers).                */
/* ------------------------------------------------------------------------ */
static void hadamard_stages(float v[16]) {
  for (int h = 1; h < 16; h <<= 1) {
    for (int i = 0; i < 16; ++i) {
      if (i & h) continue;
      float a = v[i], b = v[i + h];
      v[i] = a + b;
      v[i + h] = a - b;
    }
  }
}

static void rht16_group(const float* x, float* y, uint32_t mask, int inverse) {
  float v[16];
  if (!inverse) {
    for (int j = 0; j < 16; ++j) v[j] = ((mask >> j) & 1) ? -x[j] : x[j];
    hadamard_stages(v);
    for (int j = 0; j < 16; ++j) y[j] = 0.25f * v[j];
  } else {
    for (int j = 0; j < 16; ++j) v[j] = x[j];
    hadamard_stages(v);
    for (int j = 0; j < 16; ++j) {
      float u = 0.25f * v[j];
      y[j] = ((mask >> j) & 1) ? -u : u;
    }
  }
}

/* Input element types accepted by the oracle. */
#define MXO_IN_BF16 0
#define MXO_IN_F32 1

static float load_elem(const void* x, int dt, int64_t idx) {
  if (dt == MXO_IN_F32) return ((const float*)x)[idx];
  uint32_t bits = (uint32_t)((const uint16_t*)x)[idx] << 16; /* bf16 widens exactly */
  float f;
  memcpy(&f, &bits, 4);
  return f;
}

/* Widen (and optionally Hadamard-rotate) one row into FP32. */
static void load_row(const void* x, int dt, int64_t ld, int64_t r, int64_t cols,
                     int rht, uint32_t mask, float* out) {
  for (int64_t c = 0; c < cols; ++c) out[c] = load_elem(x, dt, r * ld + c);
  if (rht) {
    for (int64_t g = 0; g < cols; g += 16) {
      float tmp[16];
      rht16_group(out + g, tmp, mask, 0);
      memcpy(out + g, tmp, sizeof tmp);
    }
  }
}

void mxo_rht16(const void* x, int xdt, float* y, int64_t rows, int64_t cols, uint32_t mask,
               int inverse) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    float in[16];
    for (int64_t g = 0; g < cols; g += 16) {
      for (int j = 0; j < 16; ++j) in[j] = load_elem(x, xdt, r * cols + g + j);
      rht16_group(in, y + r * cols + g, mask, inverse);
    }
  }
}

/* Code storage of a row: 8-bit elements one per byte; FP4 element 2j in the
 * low nibble of byte j (READING); FP6 (READING: the pages give no packing)
 * element c at bits 6c .. 6c+5 of the row's little-endian bit string, so 4
 * elements fill 3 bytes. */
static void put_code(int bits, uint8_t* row, int64_t c, uint32_t code) {
  if (bits == 8) {
    row[c] = (uint8_t)code;
  } else if (bits == 4) {
    uint8_t* b = &row[c >> 1];
    if (c & 1) *b = (uint8_t)((*b & 0x0F) | (code << 4));
    else *b = (uint8_t)((*b & 0xF0) | code);
  } else {
    for (int k = 0; k < bits; ++k) {
      int64_t bit = c * bits + k;
      uint8_t m = (uint8_t)(1u << (bit & 7));
      if ((code >> k) & 1) row[bit >> 3] |= m;
      else row[bit >> 3] &= (uint8_t)~m;
    }
  }
}
static uint32_t get_code(int bits, const uint8_t* row, int64_t c) {
  if (bits == 8) return row[c];
  if (bits == 4) return (c & 1) ? (row[c >> 1] >> 4) : (row[c >> 1] & 0xF);
  uint32_t code = 0;
  for (int k = 0; k < bits; ++k) {
    int64_t bit = c * bits + k;
    code |= (uint32_t)((row[bit >> 3] >> (bit & 7)) & 1) << k;
  }
  return code;
}

/* ------------------------------------------------------------------------ */
/* MX quantization: 32 consecutive elements along a row share one E8M0      */
/* scale ([MXF] "Microscaling", "The idea"; [MIL] "Recipe 1"; [FP4] format   */
/* table).  A block decodes as v_i = X * P_i (X the shared scale, P_i the    */
/* element), so elements are encoded from x_i / X ([MXF] glossary "scale    */
/* factor": divided by before being squeezed, multiplied back after).        */
/* READING (shared exponent): X = 2^e with e = floor(log2(max|x|)) - emax,   */
/* emax the exponent of the element's largest power of two (E4M3: 8, E2M1:   */
/* 2), clamped to [-127, 127]; scaled values above the element maximum       */
/* saturate.  An all-zero block gets e = -127.  A block holding NaN or Inf   */
/* gets the NaN scale code 0xFF and element codes 0.                         */
/* Variant MXO_V_CEIL ([FP4] "The two Blackwell formats: MXFP4 vs NVFP4": a  */
/* power-of-two scale either wastes range or saturates the block maximum).   */
/* READING: the "no saturation" choice -- e is the smallest integer in       */
/* [-127, 127] with max|x| <= g_max * 2^e (g_max the largest element value), */
/* 127 when there is none; found by trying every e in increasing order.      */
/* ------------------------------------------------------------------------ */
static void mx_encode_block(const float* v, int n, int fmt, int rnd, int ceil_rule,
                            uint64_t seed, uint64_t counter, uint64_t n0, uint8_t* codes_row,
                            int64_t col0, uint8_t* scale_out) {
  mxo_elem el;
  elem_of(fmt, &el);
  const mxo_alphabet* al = el.al;
  const int emax = el.emax;
  double amax = 0.0;
  int bad = 0;
  for (int i = 0; i < n; ++i) {
    if (!isfinite(v[i])) bad = 1;
    double a = fabs((double)v[i]);
    if (a > amax) amax = a;
  }
  uint32_t codes[32];
  if (bad) {
    *scale_out = 0xFF;
    for (int i = 0; i < n; ++i) codes[i] = 0;
  } else {
    int e;
    if (ceil_rule) {
      double gmax = al->v[al->n - 1];
      e = -127;
      while (e < 127 && amax > ldexp(gmax, e)) ++e;
    } else if (amax == 0.0) {
      e = -127;
    } else {
      int E;
      frexp(amax, &E); /* amax = m * 2^E, m in [0.5, 1) -> floor(log2 amax) = E - 1 */
      e = E - 1 - emax;
      if (e < -127) e = -127;
      if (e > 127) e = 127;
    }
    *scale_out = (uint8_t)(e + 127);
    for (int i = 0; i < n; ++i) {
      double y = ldexp((double)v[i], -e); /* exact */
      codes[i] = (rnd == MXO_SR) ? encode_sr(al, y, mxo_rand16(seed, counter, n0 + i))
                                 : encode_rne(al, y);
    }
  }
  for (int i = 0; i < n; ++i) put_code(el.bits, codes_row, col0 + i, codes[i]);
}

static int64_t code_row_bytes(int fmt, int64_t cols) {
  mxo_elem el;
  if (fmt == MXO_NVFP4) return cols / 2;
  if (elem_of(fmt, &el)) return 0;
  return cols * el.bits / 8;
}

int mxo_quantize_mx(const void* x, int xdt, int64_t ld, int64_t rows, int64_t cols, int fmt,
                    int rnd, uint64_t seed, uint64_t counter, int rht, uint32_t mask,
                    int variant, uint8_t* codes, uint8_t* scales) {
  ensure_tables();
  mxo_elem el;
  if (elem_of(fmt, &el) || cols % 32 || (rht && cols % 16)) return -1;
  if (variant & ~MXO_V_CEIL) return -1;
  const int ceil_rule = (variant & MXO_V_CEIL) != 0;
#pragma omp parallel
  {
    float* row = (float*)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      load_row(x, xdt, ld, r, cols, rht, mask, row);
      uint8_t* crow = codes + r * code_row_bytes(fmt, cols);
      for (int64_t b = 0; b < cols / 32; ++b)
        mx_encode_block(row + b * 32, 32, fmt, rnd, ceil_rule, seed, counter,
                        (uint64_t)(r * cols + b * 32), crow, b * 32, &scales[r * (cols / 32) + b]);
    }
    free(row);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* NVFP4: 16 E2M1 elements share one E4M3 scale, plus one FP32 scale per     */
/* tensor that keeps the block scales in range ([MXF] "NVFP4"; [FP4] format  */
/* table and the paragraph under it: "two-level microscaling").              */
/* READING (all FP32, one rounding per operation, in this order):            */
/*   T = max|x| over the tensor (or the caller's amax)                      */
/*   T == 0: S = 1, every block scale code 0, element codes +-0.            */
/*   S  = T / 2688            (2688 = 6 * 448: largest E2M1 x largest E4M3)  */
/*   per 16-block: q = a_b / (6*S);  sb = E4M3 RNE of q (saturating)         */
/*   sb decodes to 0: element codes +-0                                      */
/*   else r = 1 / (dec(sb) * S);  y_i = x_i * r;  E2M1 (RNE or SR) of y_i,   */
/*   saturating (y_i = +-Inf gives +-6); x_i = +-0 gives +-0 even when r is  */
/*   +Inf (0 * Inf has no value).                                            */
/* Stored: codes, block-scale codes, and S (a decode multiplier: x is        */
/* recovered as e2m1 * e4m3 * S).                                            */
/* ------------------------------------------------------------------------ */
float mxo_tensor_amax(const void* x, int xdt, int64_t ld, int64_t rows, int64_t cols, int rht,
                      uint32_t mask) {
  float best = 0.0f;
#pragma omp parallel
  {
    float local = 0.0f;
    float* row = (float*)malloc(sizeof(float) * (size_t)(cols > 0 ? cols : 1));
#pragma omp for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
      load_row(x, xdt, ld, r, cols, rht, mask, row);
      for (int64_t c = 0; c < cols; ++c) {
        float a = fabsf(row[c]);
        if (a > local) local = a;
      }
    }
#pragma omp critical
    if (local > best) best = local;
    free(row);
  }
  return best;
}

/* One 16-element block whose block scale is chosen for the block maximum ab
 * mapped to k (k = 6: the format's rule above).  Writes the 16 codes and
 * returns the block-scale code. */
static uint32_t nv_encode_block(const float* v, float ab, float T, float S, float k, int rnd,
                                uint64_t seed, uint64_t counter, uint64_t n0, uint32_t codes[16]) {
  uint32_t sb = 0;
  float rcp = 0.0f;
  if (T != 0.0f) {
    float d = k * S;
    float q = ab / d;
    sb = encode_rne(&g_e4m3, (double)q);
    float dsb = (float)mxo_e4m3_decode(sb);
    if (dsb != 0.0f) {
      float p = dsb * S;
      rcp = 1.0f / p;
    }
  }
  for (int i = 0; i < 16; ++i) {
    /* READING: a zero element is +-0 also when r overflows to +Inf (S below
     * about 2^-119): 0 * Inf has no value, and every finite r gives +-0. */
    if (rcp == 0.0f || v[i] == 0.0f) {
      codes[i] = signbit(v[i]) ? 0x8u : 0x0u;
    } else {
      float y = v[i] * rcp;
      codes[i] = (rnd == MXO_SR) ? encode_sr(&g_e2m1, (double)y, mxo_rand16(seed, counter, n0 + i))
                                 : encode_rne(&g_e2m1, (double)y);
    }
  }
  return sb;
}

/* Exact squared error of a block against its decoded values, for the Four
 * Over Six choice (MXO_V_FOUR6).  The page asks only for the block scale with
 * the lower quantization error; READING: the error is the sum over the 16
 * elements of (x - xhat)^2, xhat = fp32(e2m1 * e4m3 * S) the decoded value,
 * evaluated EXACTLY (no rounding anywhere), and the two candidates are
 * compared exactly.
 *
 * Every finite FP32 value is an integer multiple of 2^-149 below 2^128, so
 * x - xhat is an integer D times 2^-149 with |D| < 2^278, and (x - xhat)^2 is
 * the integer D^2 < 2^556 times 2^-298.  The sum of 16 such squares is kept as
 * an unsigned integer of FX_LIMBS 64-bit limbs (least significant first). */
#define FX_LIMBS 10
typedef struct { uint64_t w[FX_LIMBS]; } fx_int;

/* |f| * 2^149 as an integer (f finite). */
static void fx_from_f32(float f, fx_int* r) {
  uint32_t b;
  memcpy(&b, &f, 4);
  const uint32_t e = (b >> 23) & 0xFFu, m = b & 0x7FFFFFu;
  /* normal: (m + 2^23) * 2^(e - 150) = (m + 2^23) * 2^(e - 1) * 2^-149;
   * subnormal: m * 2^-149 */
  const uint64_t mant = e ? (uint64_t)(m | 0x800000u) : m;
  const int sh = e ? (int)e - 1 : 0;
  memset(r, 0, sizeof *r);
  r->w[sh / 64] = mant << (sh % 64);
  if (sh % 64 && sh / 64 + 1 < FX_LIMBS) r->w[sh / 64 + 1] = mant >> (64 - sh % 64);
}

static int fx_cmp(const fx_int* a, const fx_int* b) {
  for (int i = FX_LIMBS - 1; i >= 0; --i)
    if (a->w[i] != b->w[i]) return a->w[i] < b->w[i] ? -1 : 1;
  return 0;
}

/* r = a - b, for a >= b */
static void fx_sub(const fx_int* a, const fx_int* b, fx_int* r) {
  uint64_t borrow = 0;
  for (int i = 0; i < FX_LIMBS; ++i) {
    const uint64_t x = a->w[i], y = b->w[i];
    const uint64_t d = x - y - borrow;
    borrow = (x < y) || (x - y < borrow);
    r->w[i] = d;
  }
}

/* r = a + b */
static void fx_add(const fx_int* a, const fx_int* b, fx_int* r) {
  uint64_t carry = 0;
  for (int i = 0; i < FX_LIMBS; ++i) {
    const unsigned __int128 s = (unsigned __int128)a->w[i] + b->w[i] + carry;
    r->w[i] = (uint64_t)s;
    carry = (uint64_t)(s >> 64);
  }
}

/* acc += a * a (a < 2^320, so only its low FX_LIMBS / 2 limbs are nonzero) */
static void fx_add_square(const fx_int* a, fx_int* acc) {
  fx_int p;
  memset(&p, 0, sizeof p);
  for (int i = 0; i < FX_LIMBS / 2; ++i) {
    uint64_t carry = 0;
    for (int j = 0; j < FX_LIMBS / 2; ++j) {
      const unsigned __int128 t = (unsigned __int128)a->w[i] * a->w[j] + p.w[i + j] + carry;
      p.w[i + j] = (uint64_t)t;
      carry = (uint64_t)(t >> 64);
    }
    p.w[i + FX_LIMBS / 2] = carry;
  }
  fx_add(acc, &p, acc);
}

/* The exact error sum of one encoded block (codes, block-scale code sb) as an
 * integer multiple of 2^-298. */
static void nv_block_sq_error(const float* v, const uint32_t codes[16], uint32_t sb, float S,
                              fx_int* err) {
  const double dsb = mxo_e4m3_decode(sb);
  memset(err, 0, sizeof *err);
  for (int j = 0; j < 16; ++j) {
    const double p = mxo_e2m1_decode(codes[j]) * dsb; /* exact: at most 6 significant bits */
    const float xh = (float)p * S;                    /* the decoded FP32 value */
    fx_int a, b, d;
    fx_from_f32(v[j], &a);
    fx_from_f32(xh, &b);
    if (signbit(v[j]) == signbit(xh)) { /* |x - xhat| = ||x| - |xhat|| */
      if (fx_cmp(&a, &b) >= 0) fx_sub(&a, &b, &d);
      else fx_sub(&b, &a, &d);
    } else {
      fx_add(&a, &b, &d);
    }
    fx_add_square(&d, err);
  }
}

/* Sign of (error of encoding a) - (error of encoding b) for one block, both
 * exact (for the tests of this comparison). */
int mxo_nv_sq_error_cmp(const float v[16], const uint8_t ca[16], uint32_t sba, const uint8_t cb[16],
                        uint32_t sbb, float S) {
  uint32_t a[16], b[16];
  for (int j = 0; j < 16; ++j) {
    a[j] = ca[j];
    b[j] = cb[j];
  }
  fx_int ea, eb;
  nv_block_sq_error(v, a, sba, S, &ea);
  nv_block_sq_error(v, b, sbb, S, &eb);
  return fx_cmp(&ea, &eb);
}

/* NVFP4 quantization with the variants:
 *   MXO_V_FOUR6 ([INK] "A precision choice for each stage": for activations
 *     a Four Over Six technique chooses between block scales to lower the
 *     quantization error).
 *     READING: every block is encoded twice, with its maximum mapped to 6
 *     (the rule above) and to 4 (q = a_b / (4 S)); the encoding with the
 *     smaller exact squared error (nv_block_sq_error) is kept, the
 *     6-encoding on a tie.
 *     S is the format's T / 2688 in both, so a 4-candidate whose scale
 *     saturates at 448 simply loses.  Round-to-nearest only.
 *   MXO_V_2D ([MXF] "NVFP4": two-dimensional weight quantisation so forward
 *     and backward passes see consistent values).  READING: one block scale
 *     per tile of 16 rows x 16 columns (the last band of rows may be shorter),
 *     from the maximum over the whole tile, stored in each of the tile's rows
 *     so the tensor keeps the ordinary layout; elements are encoded as above.
 *     The quantized values of the transpose are then the transpose of the
 *     quantized values.
 * The two variants are not combined. */
int mxo_quantize_nvfp4(const void* x, int xdt, int64_t ld, int64_t rows, int64_t cols, int rnd,
                       uint64_t seed, uint64_t counter, int rht, uint32_t mask, int variant,
                       const float* amax_in, uint8_t* codes, uint8_t* scales,
                       float* tensor_scale) {
  ensure_tables();
  if (cols % 16) return -1;
  if (variant & ~(MXO_V_FOUR6 | MXO_V_2D)) return -1;
  if ((variant & MXO_V_FOUR6) && ((variant & MXO_V_2D) || rnd == MXO_SR)) return -1;
  const int four6 = (variant & MXO_V_FOUR6) != 0;
  const int64_t band = (variant & MXO_V_2D) ? 16 : 1;
  float T = amax_in ? *amax_in : mxo_tensor_amax(x, xdt, ld, rows, cols, rht, mask);
  float S = (T == 0.0f) ? 1.0f : T / 2688.0f;
  *tensor_scale = S;
  const int64_t nbands = (rows + band - 1) / band;
#pragma omp parallel
  {
    float* buf = (float*)malloc(sizeof(float) * (size_t)(band * (cols > 0 ? cols : 1)));
#pragma omp for schedule(static)
    for (int64_t t = 0; t < nbands; ++t) {
      const int64_t r0 = t * band;
      const int64_t nr = (rows - r0 < band) ? rows - r0 : band;
      for (int64_t i = 0; i < nr; ++i) load_row(x, xdt, ld, r0 + i, cols, rht, mask, buf + i * cols);
      for (int64_t b = 0; b < cols / 16; ++b) {
        float ab = 0.0f;
        for (int64_t i = 0; i < nr; ++i)
          for (int j = 0; j < 16; ++j) {
            float a = fabsf(buf[i * cols + b * 16 + j]);
            if (a > ab) ab = a;
          }
        for (int64_t i = 0; i < nr; ++i) {
          const int64_t r = r0 + i;
          const float* v = buf + i * cols + b * 16;
          const uint64_t n0 = (uint64_t)(r * cols + b * 16);
          uint32_t c6[16], c4[16];
          uint32_t sb = nv_encode_block(v, ab, T, S, 6.0f, rnd, seed, counter, n0, c6);
          const uint32_t* cw = c6;
          if (four6 && T != 0.0f) {
            uint32_t sb4 = nv_encode_block(v, ab, T, S, 4.0f, rnd, seed, counter, n0, c4);
            fx_int e6, e4;
            nv_block_sq_error(v, c6, sb, S, &e6);
            nv_block_sq_error(v, c4, sb4, S, &e4);
            if (fx_cmp(&e4, &e6) < 0) {
              sb = sb4;
              cw = c4;
            }
          }
          scales[r * (cols / 16) + b] = (uint8_t)sb;
          uint8_t* crow = codes + r * (cols / 2);
          for (int j = 0; j < 16; ++j) {
            int64_t c = b * 16 + j;
            uint8_t* byte = &crow[c >> 1];
            if (c & 1) *byte = (uint8_t)((*byte & 0x0F) | (cw[j] << 4));
            else *byte = (uint8_t)((*byte & 0xF0) | cw[j]);
          }
        }
      }
    }
    free(buf);
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Decoding: multiply each element back by its scale(s).                     */
/* MX: x = P * 2^(c-127).  NVFP4: x = fp32(e2m1 * e4m3 * S); the first       */
/* product is exact, so there is one FP32 rounding.                          */
/* ------------------------------------------------------------------------ */
static double elem_value(int fmt, const uint8_t* codes_row, int64_t c) {
  mxo_elem el;
  elem_of(fmt, &el);
  return mxo_elem_decode(fmt, get_code(el.bits, codes_row, c));
}

void mxo_dequantize(int fmt, const uint8_t* codes, const uint8_t* scales,
                    const float* tensor_scale, int64_t rows, int64_t cols, float* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* crow = codes + r * code_row_bytes(fmt == MXO_NVFP4 ? MXO_MXFP4 : fmt, cols);
    for (int64_t c = 0; c < cols; ++c) {
      if (fmt == MXO_NVFP4) {
        double p = elem_value(MXO_MXFP4, crow, c) *
                   mxo_e4m3_decode(scales[r * (cols / 16) + c / 16]);
        y[r * cols + c] = (float)p * *tensor_scale;
      } else {
        double p = elem_value(fmt, crow, c) * mxo_e8m0_decode(scales[r * (cols / 32) + c / 32]);
        y[r * cols + c] = (float)p; /* exact unless it leaves the FP32 range */
      }
    }
  }
}

/* FP64 values used by the GEMM oracle: the exact product of element and
 * block scale(s), without the NVFP4 tensor scale (applied after the sum). */
void mxo_dequantize_f64(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t rows,
                        int64_t cols, double* y) {
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const uint8_t* crow = codes + r * code_row_bytes(fmt == MXO_NVFP4 ? MXO_MXFP4 : fmt, cols);
    for (int64_t c = 0; c < cols; ++c) {
      if (fmt == MXO_NVFP4)
        y[r * cols + c] =
            elem_value(MXO_MXFP4, crow, c) * mxo_e4m3_decode(scales[r * (cols / 16) + c / 16]);
      else
        y[r * cols + c] =
            elem_value(fmt, crow, c) * mxo_e8m0_decode(scales[r * (cols / 32) + c / 32]);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Backward-pass requantization ([INK] "A precision choice for each stage": */
/* saved values are dequantized, transposed at higher precision, then        */
/* stochastically re-quantized to MXFP8).                                    */
/* READING: "higher precision" is FP32; the output is the transpose          */
/* [cols, rows] in MXFP8 E4M3 with 32-blocks along its rows (the source's    */
/* row axis); the random draw of an element is indexed by its position in    */
/* the transposed output.  The source is an NVFP4 tensor or a BF16 matrix.   */
/* ------------------------------------------------------------------------ */
int mxo_requant_transpose(int src_fmt, const void* src_codes_or_bf16, const uint8_t* src_scales,
                          const float* src_tensor_scale, int64_t rows, int64_t cols, int rnd,
                          uint64_t seed, uint64_t counter, uint8_t* codes, uint8_t* scales) {
  ensure_tables();
  if (rows % 32) return -1;
  float* xt = (float*)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
  if (!xt) return -2;
  /* dequantize to FP32 and transpose */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    for (int64_t c = 0; c < cols; ++c) {
      float v;
      if (src_fmt == MXO_NVFP4) {
        const uint8_t* crow = (const uint8_t*)src_codes_or_bf16 + r * (cols / 2);
        double p = elem_value(MXO_MXFP4, crow, c) *
                   mxo_e4m3_decode(src_scales[r * (cols / 16) + c / 16]);
        v = (float)p * *src_tensor_scale;
      } else {
        v = load_elem(src_codes_or_bf16, MXO_IN_BF16, r * cols + c);
      }
      xt[c * rows + r] = v;
    }
  }
  /* MXFP8 along the new rows */
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < cols; ++r) {
    for (int64_t b = 0; b < rows / 32; ++b)
      mx_encode_block(xt + r * rows + b * 32, 32, MXO_MXFP8, rnd, 0, seed, counter,
                      (uint64_t)(r * rows + b * 32), codes + r * rows, b * 32,
                      &scales[r * (rows / 32) + b]);
  }
  free(xt);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Block-scaled GEMM: C[i,j] = sum_k A[i,k] * B[j,k] over the decoded        */
/* operands, in FP64; the NVFP4 tensor scales multiply the sum at the end.   */
/* Also returns tol[i,j] = 1e-5 * sum_k |A[i,k] * B[j,k]| (same factor).     */
/* ([MXF] "Hardware and kernels": the block scales are applied inside the    */
/* matrix multiply.)  Operands are given as FP64 arrays from                 */
/* mxo_dequantize_f64; A is [M, K] and B is [N, K], both K-contiguous.       */
/* ------------------------------------------------------------------------ */
void mxo_gemm_f64(const double* A, const double* B, int64_t M, int64_t N, int64_t K,
                  double post_scale, double* C, double* tol) {
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t i = 0; i < M; ++i) {
    for (int64_t j = 0; j < N; ++j) {
      double s = 0.0, sa = 0.0;
      for (int64_t k = 0; k < K; ++k) {
        double p = A[i * K + k] * B[j * K + k];
        s += p;
        sa += fabs(p);
      }
      C[i * N + j] = s * post_scale;
      if (tol) tol[i * N + j] = 1e-5 * sa * fabs(post_scale);
    }
  }
}

/* Sampled entries of the same product (for large shapes): entry t is
 * (rows[t], cols[t]). */
void mxo_gemm_f64_sampled(const double* A, const double* B, int64_t K, const int64_t* ri,
                          const int64_t* cj, int64_t count, double post_scale, double* C,
                          double* tol) {
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < count; ++t) {
    const double* a = A + ri[t] * K;
    const double* b = B + cj[t] * K;
    double s = 0.0, sa = 0.0;
    for (int64_t k = 0; k < K; ++k) {
      double p = a[k] * b[k];
      s += p;
      sa += fabs(p);
    }
    C[t] = s * post_scale;
    tol[t] = 1e-5 * sa * fabs(post_scale);
  }
}

/* Byte counts of the stored forms ([MXF] "Microscaling": one 8-bit scale per
 * 32 elements, MXFP4 averaging 4.25 bits; [FP4] format table: NVFP4 4 + 8/16
 * bits plus one FP32 per tensor). */
int64_t mxo_codes_bytes(int fmt, int64_t rows, int64_t cols) {
  return rows * code_row_bytes(fmt, cols);
}
int64_t mxo_scales_bytes(int fmt, int64_t rows, int64_t cols) {
  return fmt == MXO_NVFP4 ? rows * cols / 16 : rows * cols / 32;
}
int64_t mxo_tensor_bytes(int fmt, int64_t rows, int64_t cols) {
  return mxo_codes_bytes(fmt, rows, cols) + mxo_scales_bytes(fmt, rows, cols) +
         (fmt == MXO_NVFP4 ? 4 : 0);
}
