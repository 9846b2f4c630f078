// Output similarity for the similarity-based sharing-pattern search
// ([IC-SUMMARY] Appendix C: layer i's attention output with its own index set
// is compared, by cosine similarity, with the output it gets from layer j's
// index set; the matrix entry averages that over the calibration rows).
//
// row_cosine_kernel: one workgroup per row.  The row is streamed once from HBM
// in 16-byte loads, four per input in flight per thread; the three sums
// (a.b, a.a, b.b) are accumulated in float64 (the fp32 products are exact in
// float64) and reduced in a fixed order, so the result repeats bit for bit.
// The work is two reads of 4 bytes per element and six float64 flops: HBM
// bound by a wide margin on gfx950.
// row_mean_kernel: one workgroup sums the per-row values in float64 in a fixed
// order (strided per thread, then a fixed tree).
#include "common.hpp"

namespace {

constexpr int kCosThreads = 256;
constexpr int kMeanThreads = 1024;

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ void acc4(const dsa::f32x4 x, const dsa::f32x4 y, double& d, double& na, double& nb) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const double xc = (double)x[c], yc = (double)y[c];
    d = fma(xc, yc, d);
    na = fma(xc, xc, na);
    nb = fma(yc, yc, nb);
  }
}

__global__ __launch_bounds__(kCosThreads) void row_cosine_kernel(const float* __restrict__ a,
                                                                  const float* __restrict__ b,
                                                                  int64_t width, float* __restrict__ out) {
  __shared__ double red[kCosThreads / 64][3];
  const int64_t r = blockIdx.x;
  const dsa::f32x4* pa = (const dsa::f32x4*)(a + r * width);
  const dsa::f32x4* pb = (const dsa::f32x4*)(b + r * width);
  const int64_t n4 = width >> 2;
  const int t = threadIdx.x;
  double d = 0.0, na = 0.0, nb = 0.0;
  int64_t i = t;
  for (; i + 3 * kCosThreads < n4; i += 4 * kCosThreads) {
    dsa::f32x4 x[4], y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      x[u] = pa[i + u * kCosThreads];
      y[u] = pb[i + u * kCosThreads];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc4(x[u], y[u], d, na, nb);
  }
  for (; i < n4; i += kCosThreads) acc4(pa[i], pb[i], d, na, nb);
  d = wave_sum_f64(d);
  na = wave_sum_f64(na);
  nb = wave_sum_f64(nb);
  const int w = t >> 6;
  if ((t & 63) == 0) {
    red[w][0] = d;
    red[w][1] = na;
    red[w][2] = nb;
  }
  __syncthreads();
  if (t == 0) {
    double sd = 0.0, sa = 0.0, sb = 0.0;
    for (int k = 0; k < kCosThreads / 64; ++k) {
      sd += red[k][0];
      sa += red[k][1];
      sb += red[k][2];
    }
    float c;
    if (sa == 0.0 || sb == 0.0)
      c = (sa == 0.0 && sb == 0.0) ? 1.0f : 0.0f;   // both rows zero agree; one zero row does not
    else
      c = (float)(sd / sqrt(sa * sb));
    out[r] = c;
  }
}

__global__ __launch_bounds__(kMeanThreads) void row_mean_kernel(const float* __restrict__ v, int64_t rows,
                                                                double* __restrict__ mean) {
  __shared__ double red[kMeanThreads / 64];
  double s = 0.0;
  for (int64_t r = threadIdx.x; r < rows; r += kMeanThreads) s += (double)v[r];
  s = wave_sum_f64(s);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
    for (int k = 0; k < kMeanThreads / 64; ++k) tot += red[k];
    *mean = tot / (double)rows;
  }
}

// Fills an n x n float64 matrix with the identity (the diagonal of the
// similarity matrix is 1, the upper triangle 0; the lower one is overwritten).
__global__ __launch_bounds__(256) void identity_f64_kernel(double* m, int64_t n) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e < n * n) m[e] = (e / n == e % n) ? 1.0 : 0.0;
}

}  // namespace

namespace dsa_host {

hipError_t row_cosine_launch(const float* a, const float* b, int64_t rows, int64_t width, float* row_cos,
                             double* mean, hipStream_t s) {
  hipLaunchKernelGGL(row_cosine_kernel, dim3((unsigned)rows), dim3(kCosThreads), 0, s, a, b, width, row_cos);
  if (mean) hipLaunchKernelGGL(row_mean_kernel, dim3(1), dim3(kMeanThreads), 0, s, row_cos, rows, mean);
  return hipGetLastError();
}

hipError_t identity_f64_launch(double* m, int64_t n, hipStream_t s) {
  const int64_t e = n * n;
  hipLaunchKernelGGL(identity_f64_kernel, dim3((unsigned)((e + 255) / 256)), dim3(256), 0, s, m, n);
  return hipGetLastError();
}

}  // namespace dsa_host
