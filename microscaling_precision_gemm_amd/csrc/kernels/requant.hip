// requant.hip -- backward-pass requantization: dequantize (NVFP4 or BF16
// source), transpose, and re-quantize to MXFP8 E4M3 with 32-element blocks
// along the former row axis, round-to-nearest-even or stochastic ("Thinking
// Machines ... Inkling 2 Small", section "A precision choice for each stage":
// saved values are de-quantized, transposed at higher precision, then
// stochastically re-quantized to MXFP8).
//
// NVFP4 source (k_requant_nv): a persistent grid of two 512-lane workgroups
// per CU; each walks tiles of 128 source rows x 64 source columns.  Its
// first four waves are producers (global loads, decode, LDS writes) and its
// last four consumers (LDS reads, encode, stores), meeting at one barrier
// per tile over a double-buffered FP32 tile (2 x 32 KB).  On gfx9 loads and
// stores share one wait counter, so a wave that did both would wait for its
// own stores each time it needs a prefetched tile; split by role, the
// producers keep two tiles of loads in flight and the consumers never wait
// on memory.
//   producer lane (r, h): source row r, columns 32h .. 32h+31: one 16-byte
//   code load and two E4M3 scale bytes, decoded by gfx950's FP4 conversion
//   (which applies only the exponent of its scale operand, so it runs with
//   1.0) and one FP32 multiply by the E4M3 scale: the exact product
//   e2m1 * e4m3 (at most 6 significant bits).  The LDS tile holds these FP32
//   values column-major, 128 rows per column, in 4-row groups whose order is
//   XOR-swizzled so that the 32 writes of a producer and the 16-byte reads of
//   a consumer are free of bank conflicts (with 32 and with 64 banks).
//   consumer lane (c, b): output row c (a source column) and the 32 source
//   rows of MXFP8 block b: eight 16-byte LDS reads, the block maximum of
//   |p|, then the tensor scale S (see the consumer code for the exact single
//   product that replaces decode-then-scale), and two 16-byte stores of the
//   block's 32 codes plus its scale byte.
//
// BF16 source (k_requant_bf): one workgroup per tile of 128 source rows x 64
// columns, no persistence (the leg is bound by HBM, not by instructions).
//   phase 1: lane task (m, k) takes source rows 2m and 2m+1, columns
//   8k .. 8k+7 (one 16-byte load per row, so one load instruction reads 8
//   rows x 128 contiguous bytes); for each column the two rows are packed
//   into one 32-bit LDS word (row 2m low), 16 KB column-major.
//   phase 2: lane task (c, j) takes output row c and source rows 8j .. 8j+7
//   (one 16-byte LDS read); a lane quad is one 32-row MXFP8 block (E8M0 scale
//   from the DPP max), and the 16 lanes of an output row store 128
//   contiguous code bytes.
#include "../device/codec.h"
#include "../device/cvt.h"
#include "../device/wave.h"
#include "../launch.h"

namespace mxk {

namespace {

// ---------------------------------------------------------------------------
// BF16 source
// ---------------------------------------------------------------------------
constexpr int kTR = 128;  // source rows per tile (four MXFP8 blocks)
constexpr int kTC = 64;   // source columns per tile
constexpr int kCH = 8;    // columns per phase-1 task (one 16-byte load per row)
constexpr int kChunks = kTC / kCH;          // tasks per row pair
constexpr int kTasks = 64 * kChunks / 256;  // phase-1 tasks per lane

// LDS word of (column c, row pair m).  The row-pair index is XOR-swizzled
// with bits 3..5 of the column, so that the 64 lanes of one phase-1 write
// (8 row pairs x 8 chunks of 8 columns) land in 64 distinct banks, while a
// 16-byte group of 4 row pairs stays contiguous for the phase-2 reads.
__device__ inline uint32_t lds_word(uint32_t c, uint32_t m) { return c * 64u + (m ^ (((c >> 3) & 7u) << 3)); }

template <bool SR>
__global__ __launch_bounds__(256) void k_requant_bf(const uint16_t* __restrict__ xb, int64_t ld_x,
                                                    int64_t rows, int64_t cols,
                                                    uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, uint64_t seed,
                                                    uint64_t counter, uint32_t tiles_x,
                                                    uint32_t tiles_y) {
  __shared__ uint32_t tile[kTC * (kTR / 2)];
  // Workgroup -> tile.  Workgroups are dealt to the 8 XCDs round-robin, so
  // XCD x gets ids x, x + 8, ...; each XCD takes a contiguous run of the
  // column-strip-major tile order (row tile fastest).  An XCD then writes
  // consecutive 128-byte pieces of the same output rows one after another
  // instead of sharing every output row with the seven others.
  uint32_t tx, ty;
  {
    const uint32_t id = blockIdx.x;
    const uint32_t total = tiles_x * tiles_y;
    const uint32_t lin = (total & 7u) == 0 ? (id & 7u) * (total >> 3) + (id >> 3) : id;
    tx = lin / tiles_y;
    ty = lin - tx * tiles_y;
  }
  const int64_t r0 = (int64_t)ty * kTR;
  const int64_t c0 = (int64_t)tx * kTC;
  const uint32_t t = threadIdx.x;
  const int rows_here = (int)((rows - r0) < kTR ? (rows - r0) : kTR);  // multiple of 32
  const int cols_here = (int)((cols - c0) < kTC ? (cols - c0) : kTC);  // multiple of 16

  // phase 1: 64 row pairs x kChunks column chunks; all loads first
  uint4 ha[kTasks], hb[kTasks];
#pragma unroll
  for (int u = 0; u < kTasks; ++u) {
    const uint32_t id = (uint32_t)u * 256u + t;
    const uint32_t m = id / kChunks, k = id % kChunks;
    if ((int)(2 * m) < rows_here && (int)(kCH * k) < cols_here) {  // whole chunks: cols % 16 == 0
      const uint16_t* src = xb + (r0 + 2 * m) * ld_x + c0 + kCH * k;
      ha[u] = *reinterpret_cast<const uint4*>(src);
      hb[u] = *reinterpret_cast<const uint4*>(src + ld_x);
    }
  }
#pragma unroll
  for (int u = 0; u < kTasks; ++u) {
    const uint32_t id = (uint32_t)u * 256u + t;
    const uint32_t m = id / kChunks, k = id % kChunks;
    if ((int)(2 * m) < rows_here && (int)(kCH * k) < cols_here) {
      const uint32_t a4[4] = {ha[u].x, ha[u].y, ha[u].z, ha[u].w};
      const uint32_t b4[4] = {hb[u].x, hb[u].y, hb[u].z, hb[u].w};
#pragma unroll
      for (int d = 0; d < kCH / 2; ++d) {
        // columns kCH k + 2d (low halves) and kCH k + 2d + 1 (high halves)
        tile[lds_word(kCH * k + 2 * d, m)] = (a4[d] & 0xFFFFu) | (b4[d] << 16);
        tile[lds_word(kCH * k + 2 * d + 1, m)] = (a4[d] >> 16) | (b4[d] & 0xFFFF0000u);
      }
    }
  }
  __syncthreads();

  // phase 2: kTC output rows x 16 eight-row chunks, kTC / 16 tasks per lane
#pragma unroll
  for (int u = 0; u < kTC / 16; ++u) {
    const uint32_t id = (uint32_t)u * 256u + t;
    const uint32_t c = id >> 4, j = id & 15u;
    const uint4 w = *reinterpret_cast<const uint4*>(&tile[lds_word(c, 4 * j)]);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
    float v[8];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      v[2 * d] = u2f(ww[d] << 16);
      v[2 * d + 1] = u2f(ww[d] & 0xFFFF0000u);
    }
    // block amax over the bit patterns: NaN and Inf order above every finite value
    uint32_t mx = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bb = f2u(v[i]) & 0x7FFFFFFFu;
      mx = bb > mx ? bb : mx;
    }
    uint32_t o = dpp_xor1(mx);
    mx = o > mx ? o : mx;
    o = dpp_xor2(mx);
    mx = o > mx ? o : mx;
    const uint32_t sc = e8m0_from_amax_bits(mx, 8u);
    const float inv = e8m0_inverse(sc);
    float y[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = v[i] * inv;  // exact scaling by a power of two
    const int64_t oc = c0 + c;         // output row
    const int64_t orow = r0 + 8 * j;   // first output column of this lane
    const int64_t n = oc * rows + orow;
    uint32_t p[2];
    if constexpr (SR) {
      uint32_t rnd[8];
      rand16x8(seed, counter, (uint64_t)(n >> 3), rnd);
      pack_e4m3_sr(y, rnd, p);  // SR on the conversion instruction
    } else {
      pack_e4m3_rne(y, p);
    }
    if (sc == 0xFFu) p[0] = p[1] = 0u;  // NaN / Inf in the block
    if ((int)c < cols_here && (int)(8 * j) < rows_here) {
      store_nt(codes + n, p[0], p[1]);
      if ((t & 3u) == 0) scales[oc * (rows >> 5) + (orow >> 5)] = (uint8_t)sc;
    }
  }
}

// ---------------------------------------------------------------------------
// NVFP4 source
// ---------------------------------------------------------------------------
constexpr int kNvTC = 64;        // source columns per tile
constexpr int kNvProducers = 256;  // lanes of each role
constexpr uint32_t kNvBuf = kNvTC * kTR * 4;  // bytes of one FP32 tile
constexpr uint32_t kNvPerCU = 2;   // resident workgroups per CU (2 x 64 KB of LDS)
constexpr int kNvDepth = 2;        // tiles in flight per producer lane (even)

// 4-row group g (0..31) of column c (0..63) -> its slot in the column (a
// bijection on 0..31 for fixed c).  The XOR of g's bits 3..4 into bits 0..1
// and of the column's low bits (flipped for the upper 32 columns) into bits
// 2..3 spreads the 64 lanes of a producer write (32 rows x 2 column halves,
// one column each) and the 16-byte consumer reads (4 columns x 4 blocks per
// 16 lanes) over distinct banks, with 32 and with 64 banks.
__device__ inline uint32_t nv_slot(uint32_t c, uint32_t g) {
  const uint32_t cc = (c & 3u) ^ (((c >> 5) & 1u) * 3u);
  return g ^ (((g >> 3) & 3u) | (cc << 2));
}
// byte address of element (row r, column c) in the FP32 tile
__device__ inline uint32_t nv_addr(uint32_t c, uint32_t r) {
  return 4u * (c * 128u + 4u * nv_slot(c, r >> 2) + (r & 3u));
}

// 8 FP4 codes (element 2d in the low nibble of byte d) times their E4M3
// block scale: exact FP32 products.  gfx950's FP4 conversion applies only
// the exponent of its scale operand, so it runs with 1.0 and the E4M3 scale
// is one FP32 multiply.
__device__ inline void nv_decode8(uint32_t w, float sb, float* v) {
  const v2f_cvt f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
  const v2f_cvt f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
  const v2f_cvt f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
  const v2f_cvt f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  v[0] = f0[0] * sb; v[1] = f0[1] * sb; v[2] = f1[0] * sb; v[3] = f1[1] * sb;
  v[4] = f2[0] * sb; v[5] = f2[1] * sb; v[6] = f3[0] * sb; v[7] = f3[1] * sb;
}

// One producer lane's share of a tile, as loaded: nothing is computed from
// the loaded registers until the tile is decoded, so a prefetch never waits.
typedef uint32_t nv_u32x4 __attribute__((ext_vector_type(4)));
struct NvTileRegs {
  nv_u32x4 q;        // 32 FP4 codes (16 bytes)
  uint32_t s0, s1;   // the E4M3 scale bytes (both in s0 when the row pitch allows a 2-byte load)
  bool valid, full;  // inside the matrix; all 32 columns inside (else the first 16)
};

// Tile of index L in the tile order: groups of 8 row tiles, row tile
// fastest inside a group, then column tile, then group.
__device__ inline void nv_tile_xy(uint32_t L, uint32_t tiles_x, uint32_t tiles_y, uint32_t* tx,
                                  uint32_t* ty) {
  const uint32_t group = L / (8u * tiles_x);
  const uint32_t first = group * 8u;
  const uint32_t gsize = tiles_y - first < 8u ? tiles_y - first : 8u;
  const uint32_t in = L - group * 8u * tiles_x;
  *ty = first + in % gsize;
  *tx = in / gsize;
}

// Loads of source row r, columns 32h .. 32h+31 of tile L.  Outside the
// matrix the addresses fall back to row 0 / the first 16 columns (always
// inside) and the decode
// discards the values, so every lane issues the same loads.  ALIGNED (cols a
// multiple of 32): 16-byte code rows and 2-byte scale pairs.
template <bool ALIGNED>
__device__ inline void nv_load(const uint8_t* __restrict__ src_codes, const uint8_t* __restrict__ src_scales,
                               int64_t rows, int64_t cols, uint32_t L, uint32_t tiles_x, uint32_t tiles_y,
                               uint32_t r, uint32_t h, NvTileRegs& g) {
  uint32_t tx, ty;
  nv_tile_xy(L, tiles_x, tiles_y, &tx, &ty);
  int64_t gr = (int64_t)ty * kTR + r, gc = (int64_t)tx * kNvTC + 32 * h;
  g.valid = gr < rows && gc < cols;
  if (!g.valid) gr = gc = 0;
  g.full = gc + 32 <= cols;  // cols % 16 == 0: otherwise 16 columns are left
  const uint8_t* pc = src_codes + gr * (cols >> 1) + (gc >> 1);
  const uint8_t* ps = src_scales + gr * (cols >> 4) + (gc >> 4);
  if constexpr (ALIGNED) {
    g.q = *reinterpret_cast<const nv_u32x4*>(pc);
    g.s0 = *reinterpret_cast<const uint16_t*>(ps);
    g.s1 = 0u;
  } else {
    const uint2 a = *reinterpret_cast<const uint2*>(pc);
    const uint2 b = *reinterpret_cast<const uint2*>(pc + (g.full ? 8 : 0));
    g.q = nv_u32x4{a.x, a.y, b.x, b.y};
    g.s0 = ps[0];
    g.s1 = ps[g.full ? 1 : 0];
  }
}

// E4M3 magnitude (code < 0x7F) without a branch: the code shifted into the
// FP32 exponent/mantissa fields is the value times 2^-120, subnormal codes
// included (an FP32 subnormal; FP32 subnormals are not flushed in this
// library's kernels), so one multiply by 2^120 gives it exactly.
__device__ inline float nv_e4m3_mag(uint32_t c) { return u2f(c << 20) * 0x1p+120f; }

// A loaded row piece as 32 FP32 products e2m1 * e4m3 (zeros outside the
// matrix).  The empty asm statement takes the loaded registers as operands:
// nothing that reads them is scheduled before it, so the wait for the loads
// lands here and not earlier in the pipeline.
template <bool ALIGNED>
__device__ inline void nv_decode(NvTileRegs g, float v[32]) {
  asm volatile("" : "+v"(g.q), "+v"(g.s0), "+v"(g.s1));
  uint32_t s0 = ALIGNED ? g.s0 & 0xFFu : g.s0, s1 = ALIGNED ? g.s0 >> 8 : g.s1;
  nv_u32x4 q = g.q;
  const bool keep_hi = g.full && g.valid;
  q.x = g.valid ? q.x : 0u;
  q.y = g.valid ? q.y : 0u;
  q.z = keep_hi ? q.z : 0u;
  q.w = keep_hi ? q.w : 0u;
  s0 = g.valid ? s0 : 0u;
  s1 = keep_hi ? s1 : 0u;
  const float sb0 = nv_e4m3_mag(s0), sb1 = nv_e4m3_mag(s1);
  nv_decode8(q.x, sb0, v);
  nv_decode8(q.y, sb0, v + 8);
  nv_decode8(q.z, sb1, v + 16);
  nv_decode8(q.w, sb1, v + 24);
}

// Tiles of workgroup l of range x: L_i = lo + l + nl * i for L_i < hi (nl
// workgroups per range), so the tiles in flight on one XCD at any time are
// neighbours in the tile order.
struct NvWalk {
  uint32_t first, step, n;
};
__device__ inline NvWalk nv_walk(uint32_t T, uint32_t nranges, uint32_t per_range) {
  const uint32_t x = blockIdx.x % nranges, l = blockIdx.x / nranges, nl = gridDim.x / nranges;
  const uint32_t lo = x * per_range;
  const uint32_t hi = lo + per_range < T ? lo + per_range : T;
  NvWalk w;
  w.first = lo + l;
  w.step = nl;
  w.n = w.first < hi ? (hi - w.first + nl - 1) / nl : 0u;
  return w;
}

template <bool SR, bool ALIGNED>
__global__ __launch_bounds__(2 * kNvProducers) void k_requant_nv(const uint8_t* __restrict__ src_codes,
                                                    const uint8_t* __restrict__ src_scales,
                                                    const float* __restrict__ src_ts, int64_t rows,
                                                    int64_t cols, uint8_t* __restrict__ codes,
                                                    uint8_t* __restrict__ scales, uint64_t seed,
                                                    uint64_t counter, uint32_t tiles_x, uint32_t tiles_y,
                                                    uint32_t nranges, uint32_t per_range) {
  // two FP32 tiles of 128 x 64: the producers fill one while the consumers
  // drain the other
  __shared__ __attribute__((aligned(16))) float nv_tiles[2 * kNvTC * kTR];
  char* lds = reinterpret_cast<char*>(nv_tiles);
  // Workgroup -> run of tiles.  Workgroups are dealt to the XCDs round-robin;
  // range x (= id mod nranges) is a contiguous run of per_range tiles of the
  // tile order, walked by its workgroups in turn, so the tiles in flight on
  // one XCD cover neighbouring row and column tiles.
  const NvWalk walk = nv_walk(tiles_x * tiles_y, nranges, per_range);
  if (walk.n == 0) return;

  if (threadIdx.x < (uint32_t)kNvProducers) {
    // Producers (waves 0..3): global loads, decode, LDS writes.  Their only memory operations are loads, so waiting for a
    // prefetched tile never waits for stores.  Lane: source row r, columns
    // 32h .. 32h+31; its 32 LDS slots are wbase[j & 3] + (j >> 2) * 2048
    // (columns j and j + 4 share the swizzle).
    const uint32_t r = threadIdx.x >> 1, h = threadIdx.x & 1u;
    uint32_t wbase[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wbase[j] = nv_addr(32u * h + (uint32_t)j, r);
    // Prefetch ring of kNvDepth tiles.  Full rounds of kNvDepth steps run
    // without branches around the loads (past the last tile they reload it),
    // so each decode waits only for its own tile; the last partial round
    // follows.
    const uint32_t last = walk.n - 1;
    auto tile_of = [&](uint32_t i) { return walk.first + walk.step * (i < last ? i : last); };
    NvTileRegs pre[kNvDepth];
#pragma unroll
    for (int u = 0; u < kNvDepth; ++u)
      nv_load<ALIGNED>(src_codes, src_scales, rows, cols, tile_of(u), tiles_x, tiles_y, r, h, pre[u]);
    auto put = [&](const float(&v)[32], int u) {
      char* buf = lds + (u & 1) * kNvBuf;  // kNvDepth is even: buffer (s & 1) == (u & 1)
#pragma unroll
      for (int j = 0; j < 32; ++j) *reinterpret_cast<float*>(buf + wbase[j & 3] + (j >> 2) * 2048) = v[j];
      __syncthreads();  // tile s is in LDS
    };
    uint32_t s0 = 0;
    for (; s0 + kNvDepth <= walk.n; s0 += kNvDepth) {
#pragma unroll
      for (int u = 0; u < kNvDepth; ++u) {
        float v[32];
        nv_decode<ALIGNED>(pre[u], v);
        nv_load<ALIGNED>(src_codes, src_scales, rows, cols, tile_of(s0 + kNvDepth + u), tiles_x, tiles_y, r,
                             h, pre[u]);
        put(v, u);
      }
    }
#pragma unroll
    for (int u = 0; u < kNvDepth; ++u) {
      if (s0 + u < walk.n) {
        float v[32];
        nv_decode<ALIGNED>(pre[u], v);
        put(v, u);
      }
    }
  } else {
    // Consumers (waves 4..7): LDS reads, scale, encode, stores.  Lane:
    // output row c of the tile (a source column), block b (source rows
    // 32b .. 32b+31); group i of the block is at rbase ^ (16 i).
    //   The decoded value is fl(p * S) and its MXFP8 element
    //   fl(p * S) * 2^-(code - 127); both roundings are monotone, so the
    //   block's amax is fl(max|p| * S), and where p * S stays a normal FP32
    //   value (|S| >= 2^-116, as |p| >= 2^-10) the element is the single
    //   product fl(p * (S * 2^-(code - 127))), S * 2^-(code - 127) being
    //   exact.
    const uint32_t t = threadIdx.x - (uint32_t)kNvProducers;
    const uint32_t c = t >> 2, b = t & 3u;
    const uint32_t rbase = nv_addr(c, 32u * b);
    const float S = *src_ts;
    const bool fused = __builtin_fabsf(S) >= 0x1p-116f && __builtin_fabsf(S) <= 0x1p+127f;
    for (uint32_t s = 0; s < walk.n; ++s) {
      __syncthreads();  // tile s is in LDS; the producers may now refill the other buffer
      uint32_t tx, ty;
      nv_tile_xy(walk.first + walk.step * s, tiles_x, tiles_y, &tx, &ty);
      const int64_t r0 = (int64_t)ty * kTR, c0 = (int64_t)tx * kNvTC;
      const char* buf = lds + (s & 1u) * kNvBuf;
      float p[32];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 w = *reinterpret_cast<const float4*>(buf + (rbase ^ (16u * i)));
        p[4 * i] = w.x; p[4 * i + 1] = w.y; p[4 * i + 2] = w.z; p[4 * i + 3] = w.w;
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < 32; i += 2)
        m = __builtin_fmaxf(m, __builtin_fmaxf(__builtin_fabsf(p[i]), __builtin_fabsf(p[i + 1])));
      const uint32_t sc = e8m0_from_amax_bits(f2u(m * S) & 0x7FFFFFFFu, 8u);
      const float inv = e8m0_inverse(sc);
      if (fused) {
        // an all-zero block keeps its zeros
        const float k = m == 0.0f ? 0.0f : S * inv;
#pragma unroll
        for (int i = 0; i < 32; ++i) p[i] = __builtin_amdgcn_fmed3f(p[i] * k, -448.0f, 448.0f);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) p[i] = __builtin_amdgcn_fmed3f((p[i] * S) * inv, -448.0f, 448.0f);
      }
      const int64_t oc = c0 + c, orow = r0 + 32 * b;
      const int64_t n = oc * rows + orow;
      uint32_t wq[8];
      if constexpr (SR) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          uint32_t rnd[8];
          rand16x8(seed, counter, (uint64_t)(n >> 3) + (uint64_t)i, rnd);
          pack_e4m3_sr_clamped(p + 8 * i, rnd, wq + 2 * i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pack_e4m3_rne_clamped(p + 8 * i, wq + 2 * i);
      }
      if (sc == 0xFFu) {  // NaN / Inf tensor scale
#pragma unroll
        for (int i = 0; i < 8; ++i) wq[i] = 0u;
      }
      if ((int64_t)c < cols - c0 && (int64_t)(32 * b) < rows - r0) {
        store_nt(codes + n, wq[0], wq[1], wq[2], wq[3]);
        store_nt(codes + n + 16, wq[4], wq[5], wq[6], wq[7]);
        scales[oc * (rows >> 5) + (orow >> 5)] = (uint8_t)sc;
      }
    }
  }
}

// Compute units of the current device (cached per device).
int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

hipError_t launch_requant_transpose(const uint8_t* src_codes, const uint8_t* src_scales,
                                    const float* src_tensor_scale, const uint16_t* x_bf16,
                                    int64_t ld_x, int64_t rows, int64_t cols, uint8_t* codes,
                                    uint8_t* scales, bool sr, uint64_t seed, uint64_t counter,
                                    hipStream_t s) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (src_codes != nullptr) {
    const uint32_t tiles_x = (uint32_t)((cols + kNvTC - 1) / kNvTC), tiles_y = (uint32_t)((rows + kTR - 1) / kTR);
    if ((uint64_t)tiles_x * tiles_y > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const uint32_t T = tiles_x * tiles_y;
    // persistent grid, kNvPerCU workgroups per CU: 8 ranges (one per XCD:
    // workgroups are dealt to the XCDs round-robin) of equal runs of tiles,
    // or one range per tile when there are fewer than 8
    uint32_t nranges, nl;
    if (T < 8) {
      nranges = T;
      nl = 1;
    } else {
      nranges = 8;
      const uint32_t slots = (uint32_t)device_cu_count() * kNvPerCU;
      const uint32_t g = T < slots ? T : slots;
      nl = g / 8 > 0 ? g / 8 : 1;
    }
    const uint32_t per_range = (T + nranges - 1) / nranges;
    const dim3 grid(nranges * nl);
#define MXK_RQNV(SR, AL)                                                                                     \
  hipLaunchKernelGGL((k_requant_nv<SR, AL>), grid, dim3(2 * kNvProducers), 0, s, src_codes, src_scales,      \
                     src_tensor_scale, rows, cols, codes, scales, seed, counter, tiles_x, tiles_y, nranges, per_range)
    const bool aligned = (cols & 31) == 0;
    if (sr) {
      if (aligned) MXK_RQNV(true, true);
      else MXK_RQNV(true, false);
    } else {
      if (aligned) MXK_RQNV(false, true);
      else MXK_RQNV(false, false);
    }
#undef MXK_RQNV
  } else {
    const uint32_t tiles_x = (uint32_t)((cols + kTC - 1) / kTC), tiles_y = (uint32_t)((rows + kTR - 1) / kTR);
    if ((uint64_t)tiles_x * tiles_y > 0x7FFFFFFFull) return hipErrorInvalidValue;
    const dim3 grid(tiles_x * tiles_y);
    if (sr)
      hipLaunchKernelGGL(k_requant_bf<true>, grid, dim3(256), 0, s, x_bf16, ld_x, rows, cols, codes, scales, seed,
                         counter, tiles_x, tiles_y);
    else
      hipLaunchKernelGGL(k_requant_bf<false>, grid, dim3(256), 0, s, x_bf16, ld_x, rows, cols, codes, scales,
                         seed, counter, tiles_x, tiles_y);
  }
  return hipGetLastError();
}

}  // namespace mxk
