// stats.hip -- round-trip error statistics of a decoded tensor against its
// source ("Microscaling (MX) and block-scaled 4-bit formats", section "NVFP4":
// random Hadamard transforms bound block outliers, stochastic rounding keeps
// gradients unbiased; glossary "stochastic rounding": the expected value is
// preserved).  For x (BF16 or FP32) and its decoded y (FP32), both
// [rows, cols], the kernel accumulates in FP64
//   s[0] = sum (y - x)^2,  s[1] = sum x^2,  s[2] = sum (y - x),
//   s[3] = max |y - x|
// from which relative RMSE sqrt(s0 / s1), the mean error (bias) s2 / n and the
// largest error follow.  Memory-bound: one read of x and y.
//
// A workgroup takes whole rows (grid-stride over rows, one workgroup per CU)
// and its lanes take 8 consecutive elements of the row per chunk, two chunks
// in flight; partial
// sums go through a wave reduction and LDS to one FP64 atomic add (and one
// 64-bit atomic max: non-negative doubles order as their bit patterns) per
// workgroup.  The differences are formed in FP64 from the FP32 values.
#include "../device/codec.h"
#include "../launch.h"

namespace mxk {

namespace {

constexpr int kStatThreads = 512;

__global__ void k_stats_clear(double* s) {
  if (threadIdx.x < 4) s[threadIdx.x] = 0.0;
}

template <int XDT>
__device__ inline void load8(const void* __restrict__ x, int64_t off, float (&xv)[8]) {
  if constexpr (XDT == DT_BF16) {
    const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + off);
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xv[2 * i] = u2f(ww[i] << 16);
      xv[2 * i + 1] = u2f(ww[i] & 0xFFFF0000u);
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(static_cast<const float*>(x) + off);
    const float4 a = p[0], b = p[1];
    xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
    xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
  }
}

__device__ inline void accumulate8(const float (&xv)[8], const float (&yv)[8], double& e2, double& x2, double& e1,
                                   double& mx) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double xd = xv[i], d = (double)yv[i] - xd;
    e2 += d * d;
    x2 += xd * xd;
    e1 += d;
    const double ad = __builtin_fabs(d);
    mx = ad > mx ? ad : mx;
  }
}

template <int XDT>
__global__ __launch_bounds__(kStatThreads) void k_error_stats(const void* __restrict__ x, int64_t ld_x,
                                                              const float* __restrict__ y, int64_t ld_y,
                                                              int64_t rows, int64_t cols, double* __restrict__ s) {
  const int64_t cpr = cols >> 3;  // 8-element chunks per row
  double e2 = 0.0, x2 = 0.0, e1 = 0.0, mx = 0.0;
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const int64_t ox = r * ld_x, oy = r * ld_y;
    int64_t c = threadIdx.x;
    for (; c + kStatThreads < cpr; c += 2 * kStatThreads) {  // two chunks in flight
      float xa[8], xb[8], ya[8], yb[8];
      load8<XDT>(x, ox + 8 * c, xa);
      load8<XDT>(x, ox + 8 * (c + kStatThreads), xb);
      load8<DT_F32>(y, oy + 8 * c, ya);
      load8<DT_F32>(y, oy + 8 * (c + kStatThreads), yb);
      accumulate8(xa, ya, e2, x2, e1, mx);
      accumulate8(xb, yb, e2, x2, e1, mx);
    }
    if (c < cpr) {
      float xa[8], ya[8];
      load8<XDT>(x, ox + 8 * c, xa);
      load8<DT_F32>(y, oy + 8 * c, ya);
      accumulate8(xa, ya, e2, x2, e1, mx);
    }
  }
  // wave, then workgroup
  for (int off = 32; off >= 1; off >>= 1) {
    e2 += __shfl_xor(e2, off);
    x2 += __shfl_xor(x2, off);
    e1 += __shfl_xor(e1, off);
    const double o = __shfl_xor(mx, off);
    mx = o > mx ? o : mx;
  }
  __shared__ double red[kStatThreads / 64][4];
  const uint32_t wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63u) == 0) {
    red[wid][0] = e2;
    red[wid][1] = x2;
    red[wid][2] = e1;
    red[wid][3] = mx;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < kStatThreads / 64; ++w) {
      e2 += red[w][0];
      x2 += red[w][1];
      e1 += red[w][2];
      mx = red[w][3] > mx ? red[w][3] : mx;
    }
    atomicAdd(&s[0], e2);
    atomicAdd(&s[1], x2);
    atomicAdd(&s[2], e1);
    atomicMax(reinterpret_cast<unsigned long long*>(&s[3]), (unsigned long long)__double_as_longlong(mx));
  }
}

// C[r, c] = 0 for r < rows, c < cols (row pitch ldc elements, BF16 or FP32):
// the product over an empty K.  Grid-stride over the rows, lanes along a row.
template <typename T>
__global__ __launch_bounds__(256) void k_zero_matrix(T* __restrict__ c, int64_t ldc, int64_t rows, int64_t cols) {
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x)
    for (int64_t j = threadIdx.x; j < cols; j += 256) c[r * ldc + j] = T(0);
}

}  // namespace

hipError_t launch_zero_matrix(void* c, int cdt, int64_t ldc, int64_t rows, int64_t cols, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const int g = (int)(rows < 4096 ? rows : 4096);
  if (cdt == DT_F32)
    hipLaunchKernelGGL(k_zero_matrix<float>, dim3(g), dim3(256), 0, s, static_cast<float*>(c), ldc, rows, cols);
  else
    hipLaunchKernelGGL(k_zero_matrix<uint16_t>, dim3(g), dim3(256), 0, s, static_cast<uint16_t*>(c), ldc, rows,
                       cols);
  return hipGetLastError();
}

hipError_t launch_error_stats(const void* x, int xdt, int64_t ld_x, const float* y, int64_t ld_y, int64_t rows,
                              int64_t cols, double* stats, hipStream_t s) {
  // cleared by a kernel, not a memset: the call stays capturable in a graph
  hipLaunchKernelGGL(k_stats_clear, dim3(1), dim3(64), 0, s, stats);
  if (rows > 0 && cols > 0) {
    // one 512-lane workgroup per CU: the four results live in one cache
    // line, so the per-workgroup atomics serialize there (2048 workgroups of
    // 256 lanes: 125 us at 8192 x 7168; 256 of 256: 82 us; 256 of 512: 65 us,
    // the device-copy rate)
    const int g = (int)(rows < 256 ? rows : 256);
    if (xdt == DT_BF16)
      hipLaunchKernelGGL(k_error_stats<DT_BF16>, dim3(g), dim3(kStatThreads), 0, s, x, ld_x, y, ld_y, rows, cols,
                         stats);
    else
      hipLaunchKernelGGL(k_error_stats<DT_F32>, dim3(g), dim3(kStatThreads), 0, s, x, ld_x, y, ld_y, rows, cols,
                         stats);
  }
  return hipGetLastError();
}

}  // namespace mxk
