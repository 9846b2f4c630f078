// Exact Top-k for few long score rows (decode: a handful of query rows, each
// with hundreds of thousands of candidates).
//
// Selection rule ([IC-SUMMARY] notation, T_t = Top-k(I_t)): the k best
// candidates under the total order (score descending, position ascending);
// a row with no more than k candidates keeps all of them; the output row is
// ascending with -1 padding.
//
// Method (exact): a threshold key tau is taken from a strided sample of the row
// so that about 2k keys reach it; the keys >= tau are collected in position
// order (chunk-parallel count, then chunk-parallel ordered write); one
// workgroup per row then radix-selects the k-th key T among these candidates
// in LDS and writes the winners in position order.  Whenever at least k keys
// reach tau, T >= tau, so every key that can be selected -- all keys above T
// and every tie at T -- is a candidate and the result equals a selection over
// the whole row.  If fewer than k keys reach tau, or more than kCandMax do, the
// last kernel selects over the whole row instead (three radix sweeps).
#include "common.hpp"

namespace {

constexpr int kThreads = 1024;          // tau and final kernels
constexpr int kChunk = 4096;            // scores per counting / writing workgroup
constexpr int kChunkThreads = 256;
constexpr int kPerThread = kChunk / kChunkThreads;
constexpr int kMaxChunks = 1024;        // rows up to 4M scores
constexpr int kCandMax = 8192;          // candidates kept per row
constexpr int kSampleMax = 8192;        // sampled keys per row for tau
// per-row workspace (u32 words)
constexpr int kTau = 0, kCnt = 4, kKeys = kCnt + kMaxChunks, kPos = kKeys + kCandMax;
constexpr int kRowWords = kPos + kCandMax;

__device__ __forceinline__ int64_t row_len(int64_t r, int32_t n_q, int64_t q_pos0, int32_t n_k) {
  const int64_t t = q_pos0 + (r % n_q);
  return t + 1 < n_k ? t + 1 : (int64_t)n_k;
}

__device__ __forceinline__ uint32_t ld_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block-wide exclusive scan (blockDim.x a multiple of 64, at most 1024).
__device__ uint32_t block_scan(uint32_t v, uint32_t* total, uint32_t* sh /*[17]*/) {
  const int lane = threadIdx.x & 63, wid = dsa::wave_id(), nw = blockDim.x >> 6;
  uint32_t wt;
  const uint32_t ex = dsa::wave_excl_scan(v, &wt);
  if (lane == 0) sh[wid] = wt;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t acc = 0;
    for (int w = 0; w < nw; ++w) { const uint32_t x = sh[w]; sh[w] = acc; acc += x; }
    sh[16] = acc;
  }
  __syncthreads();
  const uint32_t res = ex + sh[wid];
  *total = sh[16];
  __syncthreads();
  return res;
}

// Add digit d of each lane with `in` set to histogram h.  Keys cluster, so most
// lanes usually share one digit: the first active lane's digit is counted with
// one add and only the other lanes use atomics (same-address LDS atomics
// serialise).
__device__ __forceinline__ void hist_add(uint32_t* h, bool in, uint32_t d) {
  const uint64_t act = dsa::ballot(in);
  if (!act) return;
  const int lead = (int)__builtin_ctzll(act);
  const uint32_t d0 = (uint32_t)__builtin_amdgcn_readlane((int)d, lead);
  const uint64_t same = dsa::ballot(in && d == d0);
  if ((int)(threadIdx.x & 63) == lead) atomicAdd(&h[d0], (uint32_t)__builtin_popcountll(same));
  else if (in && d != d0) atomicAdd(&h[d], 1u);
}

// Whole workgroup: the digit (descending bins) holding the rem-th largest key;
// refines prefix/mask/rem in every thread.  nb <= blockDim.x * per.
__device__ void pick_digit(const uint32_t* h, int nb, int shift, uint32_t dmask, uint32_t& prefix,
                           uint32_t& mask, uint32_t& rem, uint32_t* sh, uint32_t* st) {
  const int per = nb > (int)blockDim.x ? nb / (int)blockDim.x : 1;
  const int hi = nb - 1 - (int)threadIdx.x * per;
  uint32_t local = 0;
  if (hi >= 0)
    for (int j = 0; j < per; ++j) local += h[hi - j];
  uint32_t tot;
  const uint32_t ex = block_scan(local, &tot, sh);
  if (hi >= 0 && ex < rem && rem <= ex + local) {
    uint32_t c = ex;
    for (int j = 0; j < per; ++j) {
      const uint32_t x = h[hi - j];
      if (c + x >= rem) {
        st[0] = prefix | ((uint32_t)(hi - j) << shift);
        st[1] = mask | (dmask << shift);
        st[2] = rem - c;
        break;
      }
      c += x;
    }
  }
  __syncthreads();
  prefix = st[0];
  mask = st[1];
  rem = st[2];
  __syncthreads();
}

// Exact rem-th largest key among n keys in LDS (four 8-bit digits).
__device__ void lds_select(const uint32_t* keys, int n, uint32_t rem, uint32_t* h, uint32_t* sh, uint32_t* st,
                           uint32_t& T, uint32_t& req) {
  uint32_t prefix = 0, mask = 0;
#pragma unroll 1
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) h[i] = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += blockDim.x) {
      const int i = i0 + (int)threadIdx.x;
      const uint32_t u = i < n ? keys[i] : 0u;
      hist_add(h, i < n && (u & mask) == prefix, (u >> shift) & 255u);
    }
    __syncthreads();
    pick_digit(h, 256, shift, 255u, prefix, mask, rem, sh, st);
  }
  T = prefix;
  req = rem;
}

// ---------------------------------------------------------------- tau
__global__ __launch_bounds__(kThreads) void tau_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                       int32_t n_q, int64_t q_pos0, int32_t n_k, int32_t k,
                                                       uint32_t* __restrict__ ws) {
  __shared__ uint32_t skey[kSampleMax];
  __shared__ uint32_t h[256];
  __shared__ uint32_t sh[17];
  __shared__ uint32_t st[4];
  const int64_t r = blockIdx.x;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  uint32_t* rw = ws + r * kRowWords;
  if (len <= k) return;                               // take-all row: no threshold needed
  if (len <= kCandMax) {                              // every key is a candidate
    if (threadIdx.x == 0) rw[kTau] = 0u;
    return;
  }
  const float* row = scores + r * row_stride;
  // the sample: kRuns runs of kRunLen consecutive scores spread evenly over the
  // row (whole 64-byte pieces instead of one score per cache line)
  constexpr int kRunLen = 16, kRuns = kSampleMax / kRunLen;
  const int64_t gap = (len - kRunLen) / (kRuns - 1);        // >= kRunLen since len > kCandMax
  const int ns = kSampleMax;
  {
    const int run = (int)threadIdx.x >> 1, half = (int)threadIdx.x & 1;   // 2 threads per run, 8 scores each
    const float* src = row + (int64_t)run * gap + 8 * half;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = src[j];
#pragma unroll
    for (int j = 0; j < 8; ++j) skey[run * kRunLen + 8 * half + j] = dsa::order_key(v[j]);
  }
  __syncthreads();
  // rank in the sample of a key that about 2k keys of the row reach
  int64_t m = (2 * (int64_t)k * ns + len - 1) / len;
  m = m < 1 ? 1 : (m > ns ? ns : m);
  uint32_t T, req;
  lds_select(skey, ns, (uint32_t)m, h, sh, st, T, req);
  if (threadIdx.x == 0) rw[kTau] = T;
}

// ---------------------------------------------------------------- candidates
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

// Keys >= tau per chunk (each thread reads kPerThread consecutive scores).
__global__ __launch_bounds__(kChunkThreads) void cand_count_kernel(const float* __restrict__ scores,
                                                                   int64_t row_stride, int32_t n_q, int64_t q_pos0,
                                                                   int32_t n_k, int32_t k, uint32_t* __restrict__ ws) {
  __shared__ uint32_t sh[17];
  const int64_t r = blockIdx.x;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  if (len <= k) return;
  uint32_t* rw = ws + r * kRowWords;
  const uint32_t tau = ld_agent(&rw[kTau]);
  const int64_t s0 = (int64_t)blockIdx.y * kChunk + (int64_t)threadIdx.x * kPerThread;
  float v[kPerThread];
  load_run(scores + r * row_stride, s0, len, v);
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) c += (s0 + j < len && dsa::order_key(v[j]) >= tau) ? 1u : 0u;
  uint32_t tot;
  block_scan(c, &tot, sh);
  if (threadIdx.x == 0) rw[kCnt + blockIdx.y] = tot;
}

// Ordered write of (key, position) of every key >= tau: chunk p's entries start
// after those of chunks 0..p-1; entries past kCandMax are dropped (the final
// kernel sees the total and selects over the whole row instead).
__global__ __launch_bounds__(kChunkThreads) void cand_write_kernel(const float* __restrict__ scores,
                                                                   int64_t row_stride, int32_t n_q, int64_t q_pos0,
                                                                   int32_t n_k, int32_t k, uint32_t* __restrict__ ws) {
  __shared__ uint32_t sh[17];
  const int64_t r = blockIdx.x;
  const int p = blockIdx.y;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  if (len <= k || (int64_t)p * kChunk >= len) return;
  uint32_t* rw = ws + r * kRowWords;
  const uint32_t tau = ld_agent(&rw[kTau]);
  uint32_t before = 0;
  for (int q = threadIdx.x; q < p; q += kChunkThreads) before += ld_agent(&rw[kCnt + q]);
  uint32_t base;
  block_scan(before, &base, sh);
  if (base >= (uint32_t)kCandMax) return;
  const int64_t s0 = (int64_t)p * kChunk + (int64_t)threadIdx.x * kPerThread;
  float v[kPerThread];
  load_run(scores + r * row_stride, s0, len, v);
  uint32_t u[kPerThread];
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    u[j] = dsa::order_key(v[j]);
    c += (s0 + j < len && u[j] >= tau) ? 1u : 0u;
  }
  uint32_t tot;
  uint32_t pos = base + block_scan(c, &tot, sh);
#pragma unroll
  for (int j = 0; j < kPerThread; ++j) {
    if (s0 + j < len && u[j] >= tau) {
      if (pos < (uint32_t)kCandMax) {
        rw[kKeys + pos] = u[j];
        rw[kPos + pos] = (uint32_t)(s0 + j);
      }
      ++pos;
    }
  }
}

// ---------------------------------------------------------------- final
// Whole-row exact select (the rare case where the threshold did not work):
// three radix sweeps over the row (12 + 12 + 8 bits), then an ordered write
// over contiguous runs of positions.
__device__ void select_whole_row(const float* row, int64_t len, int32_t k, int32_t* out, uint32_t* h,
                                 uint32_t* sh, uint32_t* st) {
  uint32_t prefix = 0, mask = 0, rem = (uint32_t)k;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 20 : (pass == 1 ? 8 : 0);
    const int nb = pass == 2 ? 256 : 4096;
    const uint32_t dmask = (uint32_t)nb - 1u;
    for (int i = threadIdx.x; i < nb; i += kThreads) h[i] = 0u;
    __syncthreads();
    for (int64_t i0 = 0; i0 < len; i0 += kThreads) {
      const int64_t i = i0 + threadIdx.x;
      const uint32_t u = i < len ? dsa::order_key(row[i]) : 0u;
      hist_add(h, i < len && (u & mask) == prefix, (u >> shift) & dmask);
    }
    __syncthreads();
    pick_digit(h, nb, shift, dmask, prefix, mask, rem, sh, st);
  }
  const uint32_t T = prefix, req = rem;
  const int64_t per = (len + kThreads - 1) / kThreads;
  const int64_t a0 = (int64_t)threadIdx.x * per;
  const int64_t a1 = a0 + per < len ? a0 + per : len;
  uint32_t gt = 0, eq = 0;
  for (int64_t i = a0; i < a1; ++i) {
    const uint32_t u = dsa::order_key(row[i]);
    gt += u > T ? 1u : 0u;
    eq += u == T ? 1u : 0u;
  }
  uint32_t tg, te;
  const uint32_t gt_before = block_scan(gt, &tg, sh);
  const uint32_t eq_before = block_scan(eq, &te, sh);
  uint32_t pos = gt_before + (eq_before < req ? eq_before : req);
  uint32_t tie = eq_before;
  for (int64_t i = a0; i < a1; ++i) {
    const uint32_t u = dsa::order_key(row[i]);
    const bool keep = u > T || (u == T && tie < req);
    tie += u == T ? 1u : 0u;
    if (keep) {
      if (pos < (uint32_t)k) out[pos] = (int32_t)i;
      ++pos;
    }
  }
}

__global__ __launch_bounds__(kThreads) void final_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                         int32_t n_q, int64_t q_pos0, int32_t n_k, int32_t k,
                                                         const uint32_t* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t ckey[kCandMax];
  __shared__ uint32_t cpos[kCandMax];
  __shared__ uint32_t h[256];
  __shared__ uint32_t sh[17];
  __shared__ uint32_t st[4];
  const int64_t r = blockIdx.x;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  int32_t* out = idx + r * (int64_t)k;
  if (len <= k) {                                     // take all, then pad
    for (int64_t j = threadIdx.x; j < k; j += kThreads) out[j] = j < len ? (int32_t)j : -1;
    return;
  }
  const uint32_t* rw = ws + r * kRowWords;
  const int nchunks = (int)((len + kChunk - 1) / kChunk);
  uint32_t c = 0;
  for (int q = threadIdx.x; q < nchunks; q += kThreads) c += ld_agent(&rw[kCnt + q]);
  uint32_t total;
  block_scan(c, &total, sh);
  if (total < (uint32_t)k || total > (uint32_t)kCandMax) {
    // the 4096-bin histogram of the whole-row sweeps reuses the candidate key array
    select_whole_row(scores + r * row_stride, len, k, out, ckey, sh, st);
    return;
  }
  const int n = (int)total;
  {
    // candidates written by the previous kernel: plain loads, all in flight at once
    constexpr int PER = kCandMax / kThreads;
    uint32_t kk[PER], pp[PER];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = (int)threadIdx.x + j * kThreads;
      kk[j] = i < n ? rw[kKeys + i] : 0u;
      pp[j] = i < n ? rw[kPos + i] : 0u;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int i = (int)threadIdx.x + j * kThreads;
      if (i < n) {
        ckey[i] = kk[j];
        cpos[i] = pp[j];
      }
    }
  }
  __syncthreads();
  uint32_t T, req;
  lds_select(ckey, n, (uint32_t)k, h, sh, st, T, req);
  // ordered write: candidates are in position order; thread t owns a contiguous run
  const int per = (n + kThreads - 1) / kThreads;
  const int a0 = (int)threadIdx.x * per;
  const int a1 = a0 + per < n ? a0 + per : n;
  uint32_t gt = 0, eq = 0;
  for (int i = a0; i < a1; ++i) {
    gt += ckey[i] > T ? 1u : 0u;
    eq += ckey[i] == T ? 1u : 0u;
  }
  uint32_t tg, te;
  const uint32_t gt_before = block_scan(gt, &tg, sh);
  const uint32_t eq_before = block_scan(eq, &te, sh);
  uint32_t pos = gt_before + (eq_before < req ? eq_before : req);
  uint32_t tie = eq_before;
  for (int i = a0; i < a1; ++i) {
    const uint32_t u = ckey[i];
    const bool keep = u > T || (u == T && tie < req);
    tie += u == T ? 1u : 0u;
    if (keep) {
      if (pos < (uint32_t)k) out[pos] = (int32_t)cpos[i];
      ++pos;
    }
  }
}

}  // namespace

namespace dsa_host {

size_t select_few_ws_bytes(int64_t rows) { return (size_t)rows * kRowWords * sizeof(uint32_t); }

hipError_t select_few(const float* scores, const SelectPlan& p, void* ws, int32_t* idx, hipStream_t s) {
  const int64_t maxlen = p.q_pos0 + p.n_q < p.n_k ? p.q_pos0 + p.n_q : (int64_t)p.n_k;
  int64_t P = (maxlen + kChunk - 1) / kChunk;
  if (P < 1) P = 1;
  uint32_t* w = (uint32_t*)ws;
  const dim3 rows((unsigned)p.rows), chunks((unsigned)p.rows, (unsigned)P);
  hipLaunchKernelGGL(tau_kernel, rows, dim3(kThreads), 0, s, scores, p.row_stride, p.n_q, p.q_pos0, p.n_k, p.k, w);
  hipLaunchKernelGGL(cand_count_kernel, chunks, dim3(kChunkThreads), 0, s, scores, p.row_stride, p.n_q, p.q_pos0,
                     p.n_k, p.k, w);
  hipLaunchKernelGGL(cand_write_kernel, chunks, dim3(kChunkThreads), 0, s, scores, p.row_stride, p.n_q, p.q_pos0,
                     p.n_k, p.k, w);
  hipLaunchKernelGGL(final_kernel, rows, dim3(kThreads), 0, s, scores, p.row_stride, p.n_q, p.q_pos0, p.n_k, p.k,
                     (const uint32_t*)w, idx);
  return hipGetLastError();
}

}  // namespace dsa_host
