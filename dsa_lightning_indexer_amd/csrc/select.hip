// Exact Top-k over materialised fp32 score rows, many workgroups per row.
//
// Selection rule ([IC-SUMMARY] notation, T_t = Top-k(I_t)): the k best
// candidates under the total order (score descending, position ascending);
// a row with no more than k candidates keeps all of them; the output row is
// ascending with -1 padding.
//
// Method: radix select on the order-preserving u32 key of each score, most
// significant digits first (12 + 12 + 8 bits).  Each digit pass builds a
// per-row histogram from many workgroups (LDS histogram, then global atomics);
// the last workgroup of a row to finish (device-scope counter, no spinning)
// picks the digit that holds the k-th key.  After three passes the k-th key T
// and the number r of ties at T that still fit are known, and one workgroup per
// row writes, in position order, every candidate with key > T plus the first r
// candidates with key == T.
#include "common.hpp"

namespace {

constexpr int kMaxChunks = 1024;       // rows up to kMaxChunks * kChunk = 4M scores
constexpr int kH1 = 0, kH2 = 4096, kH3 = 8192, kSt = 8448, kCnt = 8464;
constexpr int kRowWords = kCnt + 2 * kMaxChunks;   // per-row workspace (u32)
// state words
constexpr int kPrefix = 0, kMask = 1, kRem = 2, kDone1 = 4, kDone2 = 5, kDone3 = 6;
constexpr int kChunk = 4096;           // scores per histogram workgroup
constexpr int kHistThreads = 256;

__device__ __forceinline__ int64_t row_len(int64_t r, int32_t n_q, int64_t q_pos0, int32_t n_k) {
  int64_t t = q_pos0 + (r % n_q);
  int64_t n = t + 1;
  return n < n_k ? n : (int64_t)n_k;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += stride) p[i] = 0u;
}

// Block-wide exclusive scan (blockDim.x multiple of 64, <= 1024).
__device__ uint32_t block_excl_scan(uint32_t v, uint32_t* total, uint32_t* sh /*[17]*/) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t wt;
  uint32_t ex = dsa::wave_excl_scan(v, &wt);
  if (lane == 0) sh[wid] = wt;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < nw; ++w) { uint32_t x = sh[w]; sh[w] = acc; acc += x; }
    sh[16] = acc;
  }
  __syncthreads();
  uint32_t res = ex + sh[wid];
  *total = sh[16];
  __syncthreads();
  return res;
}

// Executed by one whole workgroup: find the digit holding the rem-th largest
// key among `nb` histogram bins (scanned from the top) and store the refined
// (prefix, mask, rem) in the row state.
__device__ void find_digit(const uint32_t* hist, int nb, int shift, uint32_t digit_mask,
                           uint32_t rem, uint32_t prefix, uint32_t mask, uint32_t* st,
                           uint32_t* sh) {
  const int per = nb / kHistThreads;
  const int tid = threadIdx.x;
  const int hi = nb - 1 - tid * per;
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) local += ld_agent(&hist[hi - j]);
  uint32_t tot;
  uint32_t ex = block_excl_scan(local, &tot, sh);
  if (ex < rem && rem <= ex + local) {
    uint32_t c = ex;
    for (int j = 0; j < per; ++j) {
      uint32_t h = ld_agent(&hist[hi - j]);
      if (c + h >= rem) {
        uint32_t d = (uint32_t)(hi - j);
        st[kPrefix] = prefix | (d << shift);
        st[kMask] = mask | (digit_mask << shift);
        st[kRem] = rem - c;
        break;
      }
      c += h;
    }
  }
}

// pass: 1, 2 or 3.
template <int PASS>
__global__ __launch_bounds__(kHistThreads) void hist_kernel(const float* __restrict__ scores,
                                                            int64_t row_stride, int32_t n_q,
                                                            int64_t q_pos0, int32_t n_k, int32_t k,
                                                            uint32_t* __restrict__ ws) {
  constexpr int NB = PASS == 3 ? 256 : 4096;
  constexpr int SHIFT = PASS == 1 ? 20 : (PASS == 2 ? 8 : 0);
  constexpr uint32_t DMASK = PASS == 3 ? 0xFFu : 0xFFFu;
  constexpr int HOFF = PASS == 1 ? kH1 : (PASS == 2 ? kH2 : kH3);
  constexpr int DONE = PASS == 1 ? kDone1 : (PASS == 2 ? kDone2 : kDone3);
  __shared__ uint32_t h[NB];
  __shared__ uint32_t sh[17];
  __shared__ uint32_t last;

  const int64_t r = blockIdx.x;
  uint32_t* rw = ws + r * kRowWords;
  uint32_t* st = rw + kSt;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  const bool take_all = len <= k;
  const bool active = !take_all;
  uint32_t prefix = 0, mask = 0;
  if (PASS > 1 && active) {
    prefix = ld_agent(&st[kPrefix]);
    mask = ld_agent(&st[kMask]);
  }
  if (active) {
    for (int i = threadIdx.x; i < NB; i += kHistThreads) h[i] = 0u;
    __syncthreads();
    const float* row = scores + r * row_stride;
    const int64_t b0 = (int64_t)blockIdx.y * kChunk;
    const int64_t b1 = b0 + kChunk < len ? b0 + kChunk : len;
    constexpr int PER = kChunk / kHistThreads;
    float v[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t s = b0 + threadIdx.x + (int64_t)j * kHistThreads;
      v[j] = s < b1 ? row[s] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int64_t s = b0 + threadIdx.x + (int64_t)j * kHistThreads;
      const uint32_t u = dsa::order_key(v[j]);
      if (s < b1 && (u & mask) == prefix) atomicAdd(&h[(u >> SHIFT) & DMASK], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NB; i += kHistThreads) {
      uint32_t c = h[i];
      if (c) atomicAdd(&rw[HOFF + i], c);
    }
  }
  // Last workgroup of this row to arrive picks the digit.
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = (atomicAdd(&st[DONE], 1u) == gridDim.y - 1) ? 1u : 0u;
  __syncthreads();
  if (!last) return;
  __threadfence();
  if (!active) return;
  const uint32_t rem = PASS == 1 ? (uint32_t)k : ld_agent(&st[kRem]);
  find_digit(rw + HOFF, NB, SHIFT, DMASK, rem, prefix, mask, st, sh);
}

// Per chunk: how many entries beat T and how many tie with it.  Each thread
// reads kPerThread consecutive entries (so chunk order = thread order).
constexpr int kPerThread = kChunk / kHistThreads;

__device__ __forceinline__ void load_run(const float* row, int64_t s0, int64_t len, float (&v)[kPerThread]) {
  if (s0 + kPerThread <= len && (((uintptr_t)(row + s0)) & 15) == 0) {
#pragma unroll
    for (int j = 0; j < kPerThread; j += 4) {
      const float4 q = *(const float4*)(row + s0 + j);
      v[j] = q.x; v[j + 1] = q.y; v[j + 2] = q.z; v[j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) v[j] = s0 + j < len ? row[s0 + j] : 0.f;
  }
}

__global__ __launch_bounds__(kHistThreads) void count_kernel(const float* __restrict__ scores,
                                                             int64_t row_stride, int32_t n_q,
                                                             int64_t q_pos0, int32_t n_k, int32_t k,
                                                             uint32_t* __restrict__ ws) {
  __shared__ uint32_t sh[17];
  const int64_t r = blockIdx.x;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  if (len <= k) return;                                   // take-all rows need no counts
  uint32_t* rw = ws + r * kRowWords;
  const uint32_t T = ld_agent(&rw[kSt + kPrefix]);
  const int64_t s0 = (int64_t)blockIdx.y * kChunk + (int64_t)threadIdx.x * kPerThread;
  float v[kPerThread];
  load_run(scores + r * row_stride, s0, len, v);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const uint32_t u = dsa::order_key(v[j]);
    const bool in = s0 + j < len;
    gt += (in && u > T) ? 1u : 0u;
    eq += (in && u == T) ? 1u : 0u;
  }
  uint32_t tg, te;
  block_excl_scan(gt, &tg, sh);
  block_excl_scan(eq, &te, sh);
  if (threadIdx.x == 0) {
    rw[kCnt + 2 * blockIdx.y] = tg;
    rw[kCnt + 2 * blockIdx.y + 1] = te;
  }
}

// Ordered write: chunk p's kept entries start after those of chunks 0..p-1;
// ties at T are kept in position order until the quota is used.
__global__ __launch_bounds__(kHistThreads) void write_kernel(const float* __restrict__ scores,
                                                             int64_t row_stride, int32_t n_q,
                                                             int64_t q_pos0, int32_t n_k, int32_t k,
                                                             const uint32_t* __restrict__ ws,
                                                             int32_t* __restrict__ idx) {
  __shared__ uint32_t sh[17];
  const int64_t r = blockIdx.x;
  const int p = blockIdx.y;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  int32_t* out = idx + r * (int64_t)k;
  const int64_t kept_total = len < k ? len : (int64_t)k;
  if (p == 0) {
    for (int64_t j = kept_total + threadIdx.x; j < k; j += kHistThreads) out[j] = -1;
  }
  const int64_t c0 = (int64_t)p * kChunk;
  if (c0 >= len) return;
  const int64_t s0 = c0 + (int64_t)threadIdx.x * kPerThread;
  if (len <= k) {                                        // take all: position s goes to slot s
    for (int j = 0; j < kPerThread; ++j)
      if (s0 + j < len) out[s0 + j] = (int32_t)(s0 + j);
    return;
  }
  const uint32_t* rw = ws + r * kRowWords;
  const uint32_t T = ld_agent(&rw[kSt + kPrefix]);
  const uint32_t req = ld_agent(&rw[kSt + kRem]);
  // Chunks before this one: sum of their counts.  Ties are kept in position
  // order until the quota req is used, so they contribute min(req, their ties).
  uint32_t gsum = 0, esum = 0;
  for (int q = threadIdx.x; q < p; q += kHistThreads) {
    gsum += ld_agent(&rw[kCnt + 2 * q]);
    esum += ld_agent(&rw[kCnt + 2 * q + 1]);
  }
  uint32_t gtot, etot;
  block_excl_scan(gsum, &gtot, sh);
  block_excl_scan(esum, &etot, sh);
  const uint32_t eq_before = etot;
  const uint32_t base = gtot + (etot < req ? etot : req);
  float v[kPerThread];
  load_run(scores + r * row_stride, s0, len, v);
  uint32_t u[kPerThread];
  uint32_t ne = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    u[j] = dsa::order_key(v[j]);
    ne += (s0 + j < len && u[j] == T) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t tie = block_excl_scan(ne, &tot, sh) + eq_before;
  bool keep[kPerThread];
  uint32_t nk = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    const bool in = s0 + j < len;
    const bool t_ = in && u[j] == T;
    keep[j] = in && (u[j] > T || (t_ && tie < req));
    tie += t_ ? 1u : 0u;
    nk += keep[j] ? 1u : 0u;
  }
  uint32_t pos = block_excl_scan(nk, &tot, sh) + base;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (keep[j]) {
      if (pos < (uint32_t)k) out[pos] = (int32_t)(s0 + j);
      ++pos;
    }
  }
}

inline int64_t max_len(const dsa_host::SelectPlan& p) {
  int64_t n = p.q_pos0 + p.n_q;  // largest t + 1
  return n < p.n_k ? n : (int64_t)p.n_k;
}

}  // namespace

namespace dsa_host {

size_t select_workspace_bytes(int64_t rows) { return (size_t)rows * kRowWords * sizeof(uint32_t); }

hipError_t select_prepare(void* ws, int64_t rows, hipStream_t s) {
  int64_t n = rows * kRowWords;
  int blocks = (int)((n + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, (uint32_t*)ws, n);
  return hipGetLastError();
}

hipError_t select_hist1(const float* scores, const SelectPlan& p, void* ws, hipStream_t s) {
  int64_t P = (max_len(p) + kChunk - 1) / kChunk;
  if (P < 1) P = 1;
  hipLaunchKernelGGL(hist_kernel<1>, dim3((unsigned)p.rows, (unsigned)P), dim3(kHistThreads), 0, s,
                     scores, p.row_stride, p.n_q, p.q_pos0, p.n_k, p.k, (uint32_t*)ws);
  return hipGetLastError();
}

hipError_t select_finish(const float* scores, const SelectPlan& p, void* ws, int32_t* idx,
                         hipStream_t s) {
  int64_t P = (max_len(p) + kChunk - 1) / kChunk;
  if (P < 1) P = 1;
  dim3 g((unsigned)p.rows, (unsigned)P);
  hipLaunchKernelGGL(hist_kernel<2>, g, dim3(kHistThreads), 0, s, scores, p.row_stride, p.n_q,
                     p.q_pos0, p.n_k, p.k, (uint32_t*)ws);
  hipLaunchKernelGGL(hist_kernel<3>, g, dim3(kHistThreads), 0, s, scores, p.row_stride, p.n_q,
                     p.q_pos0, p.n_k, p.k, (uint32_t*)ws);
  hipLaunchKernelGGL(count_kernel, g, dim3(kHistThreads), 0, s, scores, p.row_stride, p.n_q,
                     p.q_pos0, p.n_k, p.k, (uint32_t*)ws);
  hipLaunchKernelGGL(write_kernel, g, dim3(kHistThreads), 0, s, scores, p.row_stride, p.n_q,
                     p.q_pos0, p.n_k, p.k, (const uint32_t*)ws, idx);
  return hipGetLastError();
}

}  // namespace dsa_host
