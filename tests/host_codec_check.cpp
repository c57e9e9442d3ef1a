// Host-side exhaustive check of the library's element encoders
// (csrc/device/codec.h, compiled here for the CPU) against the oracle's
// alphabet-search encoders (liboracle.so, loaded at run time).
//   argv[1] = path to liboracle.so
// Prints "FAIL ..." lines for mismatches and "OK <n>" at the end.
#include <dlfcn.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <thread>
#include <vector>

#include "device/codec.h"

typedef uint32_t (*rne_fn)(double);
typedef uint32_t (*sr_fn)(double, uint32_t);
typedef uint32_t (*rand_fn)(uint64_t, uint64_t, uint64_t);

static rne_fn o_e4m3_rne, o_e2m1_rne;
static sr_fn o_e4m3_sr, o_e2m1_sr;
static rand_fn o_rand16;
typedef double (*dec_fn)(uint32_t);
static dec_fn o_e4m3_dec, o_e2m1_dec;
// the other MX element types, by MX format number (4 INT8, 5 E5M2, 6 E3M2, 7 E2M3)
typedef uint32_t (*erne_fn)(int, double);
typedef uint32_t (*esr_fn)(int, double, uint32_t);
typedef double (*edec_fn)(int, uint32_t);
static erne_fn o_elem_rne;
static esr_fn o_elem_sr;
static edec_fn o_elem_dec;

static uint32_t lib_encode(int fmt, float y, bool sr, uint32_t r) {
  switch (fmt) {
    case 4: return mxk::int8_encode(y, sr, r);
    case 5: return mxk::E5M2::encode(y, sr, r);
    case 6: return mxk::E3M2::encode(y, sr, r);
    default: return mxk::E2M3::encode(y, sr, r);
  }
}
static const char* kNames[8] = {"", "", "", "", "int8", "e5m2", "e3m2", "e2m3"};

static std::atomic<long> bad{0};

static void report(const char* what, uint32_t bits, uint32_t r, uint32_t got, uint32_t want) {
  long n = bad.fetch_add(1);
  if (n < 20) printf("FAIL %s y=0x%08x r=%u got=0x%x want=0x%x\n", what, bits, r, got, want);
}

// Exhaustive RNE over every non-negative FP32 pattern up to +Inf (and the
// matching negative pattern for every 64th value).
static void rne_range(uint64_t lo, uint64_t hi) {
  for (uint64_t b = lo; b < hi; ++b) {
    float y = mxk::u2f((uint32_t)b);
    uint32_t g = mxk::e4m3_encode(y, false, 0), w = o_e4m3_rne((double)y);
    if (g != w) report("e4m3_rne", (uint32_t)b, 0, g, w);
    g = mxk::e2m1_encode(y, false, 0);
    w = o_e2m1_rne((double)y);
    if (g != w) report("e2m1_rne", (uint32_t)b, 0, g, w);
    for (int f = 4; f <= 7; ++f) {
      g = lib_encode(f, y, false, 0);
      w = o_elem_rne(f, (double)y);
      if (g != w) report(kNames[f], (uint32_t)b, 0, g, w);
    }
    if ((b & 63) == 0) {
      float ny = -y;
      for (int f = 4; f <= 7; ++f) {
        g = lib_encode(f, ny, false, 0);
        w = o_elem_rne(f, (double)ny);
        if (g != w) report(kNames[f], (uint32_t)b | 0x80000000u, 0, g, w);
      }
      g = mxk::e4m3_encode(ny, false, 0);
      w = o_e4m3_rne((double)ny);
      if (g != w) report("e4m3_rne_neg", (uint32_t)b | 0x80000000u, 0, g, w);
      g = mxk::e2m1_encode(ny, false, 0);
      w = o_e2m1_rne((double)ny);
      if (g != w) report("e2m1_rne_neg", (uint32_t)b | 0x80000000u, 0, g, w);
    }
  }
}

// SR on a pseudo-random sample of y (all binades) with random, boundary and
// threshold random values.
static void sr_range(uint64_t seed, long n) {
  uint64_t s = seed * 0x9E3779B97F4A7C15ull + 1;
  for (long i = 0; i < n; ++i) {
    s ^= s << 13; s ^= s >> 7; s ^= s << 17;
    uint32_t bits = (uint32_t)(s >> 16) & 0x7FFFFFFFu;
    if (bits > 0x7F800000u) bits &= 0x43FFFFFFu;  // keep finite-ish
    if (i & 1) bits = 0x30000000u + (bits % 0x14000000u);  // focus on 2^-31 .. 2^9
    float y = mxk::u2f(bits);
    if (i & 2) y = -y;
    uint32_t rs[6] = {0u, 65535u, (uint32_t)(s & 0xFFFF), (uint32_t)((s >> 20) & 0xFFFF), 0, 0};
    // thresholds: the first r that no longer rounds up, and one below it
    uint32_t t4 = (mxk::f2u(__builtin_fabsf(y)) & 0xFFFFFu) >> 4;
    rs[4] = t4 & 0xFFFF;
    rs[5] = t4 ? (t4 - 1) & 0xFFFF : 0;
    for (int f = 4; f <= 7; ++f) {
      // thresholds of this format: the discarded bits (normal range) or the
      // fraction of the scaled value (subnormal range, INT8)
      float a = __builtin_fabsf(y);
      uint32_t tt = 0;
      if (f == 4) {
        double sc = (double)y * 64.0;
        if (sc > -129.0 && sc < 128.0) tt = (uint32_t)floor((sc - floor(sc)) * 65536.0);
      } else {
        int sh = f == 7 ? 20 : 21;
        tt = (mxk::f2u(a) & ((1u << sh) - 1u)) >> (sh - 16);
      }
      uint32_t fr[6] = {rs[0], rs[1], rs[2], rs[3], tt & 0xFFFF, tt ? (tt - 1) & 0xFFFF : 0};
      for (uint32_t r : fr) {
        uint32_t g = lib_encode(f, y, true, r), w = o_elem_sr(f, (double)y, r);
        if (g != w) report(kNames[f], mxk::f2u(y), r, g, w);
      }
    }
    for (uint32_t r : rs) {
      uint32_t g = mxk::e4m3_encode(y, true, r), w = o_e4m3_sr((double)y, r);
      if (g != w) report("e4m3_sr", mxk::f2u(y), r, g, w);
      g = mxk::e2m1_encode(y, true, r);
      w = o_e2m1_sr((double)y, r);
      if (g != w) report("e2m1_sr", mxk::f2u(y), r, g, w);
    }
  }
}

int main(int argc, char** argv) {
  if (argc < 2) return 2;
  void* h = dlopen(argv[1], RTLD_NOW);
  if (!h) { printf("FAIL dlopen %s\n", dlerror()); return 1; }
  o_e4m3_rne = (rne_fn)dlsym(h, "mxo_e4m3_encode_rne");
  o_e2m1_rne = (rne_fn)dlsym(h, "mxo_e2m1_encode_rne");
  o_e4m3_sr = (sr_fn)dlsym(h, "mxo_e4m3_encode_sr");
  o_e2m1_sr = (sr_fn)dlsym(h, "mxo_e2m1_encode_sr");
  o_rand16 = (rand_fn)dlsym(h, "mxo_rand16");
  o_e4m3_dec = (dec_fn)dlsym(h, "mxo_e4m3_decode");
  o_e2m1_dec = (dec_fn)dlsym(h, "mxo_e2m1_decode");
  o_elem_rne = (erne_fn)dlsym(h, "mxo_elem_encode_rne");
  o_elem_sr = (esr_fn)dlsym(h, "mxo_elem_encode_sr");
  o_elem_dec = (edec_fn)dlsym(h, "mxo_elem_decode");
  int (*init)(void) = (int (*)(void))dlsym(h, "mxo_init");
  init();
  long count = 0;
  // decoders
  for (uint32_t c = 0; c < 0x7F; ++c)
    if ((double)mxk::e4m3_mag_value(c) != o_e4m3_dec(c)) report("e4m3_value", c, 0, 0, 0);
  for (uint32_t c = 0; c < 16; ++c)
    if ((double)mxk::e2m1_value(c) != o_e2m1_dec(c)) report("e2m1_value", c, 0, 0, 0);
  for (uint32_t c = 0; c < 256; ++c) {
    double w = o_elem_dec(5, c), g = mxk::e5m2_value(c);
    if (!(g == w || (g != g && w != w))) report("e5m2_value", c, 0, 0, 0);
    if ((double)mxk::int8_value(c) != o_elem_dec(4, c)) report("int8_value", c, 0, 0, 0);
  }
  for (uint32_t c = 0; c < 64; ++c) {
    if ((double)mxk::fp6_value<mxk::E3M2>(c) != o_elem_dec(6, c)) report("e3m2_value", c, 0, 0, 0);
    if ((double)mxk::fp6_value<mxk::E2M3>(c) != o_elem_dec(7, c)) report("e2m3_value", c, 0, 0, 0);
  }
  // RNG
  for (uint64_t q = 0; q < 4096; ++q) {
    uint32_t r[8];
    uint64_t seed = q * 0x100000001B3ull, ctr = q * 977;
    mxk::rand16x8(seed, ctr, q, r);
    for (int j = 0; j < 8; ++j)
      if (r[j] != o_rand16(seed, ctr, q * 8 + j)) report("rand16", (uint32_t)q, j, r[j], 0);
  }
  int nt = (int)std::thread::hardware_concurrency();
  if (nt < 1) nt = 1;
  if (nt > 16) nt = 16;
  const uint64_t top = 0x7F800001ull;  // up to and including +Inf
  std::vector<std::thread> th;
  for (int t = 0; t < nt; ++t)
    th.emplace_back([=] { rne_range(top * t / nt, top * (t + 1) / nt); });
  for (auto& x : th) x.join();
  th.clear();
  count += (long)top;
  const long nsr = 1L << 21;
  for (int t = 0; t < nt; ++t) th.emplace_back([=] { sr_range(t + 1, nsr / nt); });
  for (auto& x : th) x.join();
  count += nsr * 6;
  if (bad.load()) { printf("FAIL total %ld\n", bad.load()); return 1; }
  printf("OK %ld\n", count);
  return 0;
}
