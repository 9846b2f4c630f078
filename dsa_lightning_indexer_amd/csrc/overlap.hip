// Cross-layer overlap |T_a[r] ∩ T_b[r]| per row ([DSA-NOTES] §3.1 overlap
// definition; [IC-SUMMARY] Appendix A).  Rows are ascending with -1 padding,
// so each valid entry of T_a is looked up in T_b (staged in LDS) by binary
// search over T_b's valid prefix.
#include "common.hpp"

namespace {

__global__ __launch_bounds__(256) void overlap_kernel(const int32_t* __restrict__ a,
                                                      const int32_t* __restrict__ b, int32_t k,
                                                      int32_t* row_counts,
                                                      unsigned long long* total) {
  extern __shared__ int32_t rowb[];
  __shared__ uint32_t red[4];
  __shared__ int nb;
  const int64_t r = blockIdx.x;
  const int32_t* ra = a + r * (int64_t)k;
  const int32_t* rb = b + r * (int64_t)k;
  if (threadIdx.x == 0) nb = 0;
  __syncthreads();
  int localn = 0;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const int32_t v = rb[j];
    rowb[j] = v;
    if (v >= 0) ++localn;
  }
  atomicAdd(&nb, localn);
  __syncthreads();
  const int n = nb;
  uint32_t cnt = 0;
  for (int j = threadIdx.x; j < k; j += blockDim.x) {
    const int32_t v = ra[j];
    if (v < 0) continue;
    int lo = 0, hi = n;  // search [lo, hi)
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (rowb[mid] < v) lo = mid + 1; else hi = mid;
    }
    if (lo < n && rowb[lo] == v) ++cnt;
  }
  for (int o = 32; o > 0; o >>= 1) cnt += __shfl_xor(cnt, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = cnt;
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t c = red[0] + red[1] + red[2] + red[3];
    if (row_counts) row_counts[r] = (int32_t)c;
    if (total) atomicAdd(total, (unsigned long long)c);
  }
}

}  // namespace

namespace dsa_host {

hipError_t overlap_launch(const int32_t* a, const int32_t* b, int64_t rows, int32_t k,
                          int32_t* row_counts, unsigned long long* total, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(overlap_kernel, dim3((unsigned)rows), dim3(256), (size_t)k * sizeof(int32_t), s,
                     a, b, k, row_counts, total);
  return hipGetLastError();
}

}  // namespace dsa_host
