// Exact Top-k for few long score rows (decode: a handful of query rows, each
// with hundreds of thousands of candidates).
//
// Selection rule ([IC-SUMMARY] notation, T_t = Top-k(I_t)): the k best
// candidates under the total order (score descending, position ascending);
// a row with no more than k candidates keeps all of them; the output row is
// ascending with -1 padding.
//
// Method (exact): a histogram of the top 12 bits of every order key of the row
// (built by the decode scan as it writes the scores, or by hist_kernel over
// given scores) names the bin b that holds the k-th key.  Every key that can
// be selected -- all keys above the k-th key T and every tie at T -- lies in a
// bin >= b, so the candidates are the keys of bins >= b, whose number is known
// from the histogram (about k plus one bin).  collect_kernel writes them per
// 16384-score chunk in position order; final_kernel (one workgroup per row)
// gathers the chunks in order into LDS, radix-selects T on the remaining 20 key
// bits and writes the winners in position order.  If the candidates overflow the
// 8192-entry buffer (e.g. a row of equal scores), it selects over the whole row
// instead (three radix sweeps).  The two kernels meet at a kernel boundary: a
// last-workgroup hand-over inside one kernel would need device-scope fences,
// which write back and invalidate the L2 of every workgroup's XCD.
#include "common.hpp"

namespace {

constexpr int kThreads = 1024;
constexpr int kChunk = 16384;                            // scores per workgroup of hist / collect
constexpr int kPer = kChunk / kThreads;                  // consecutive scores per thread
constexpr int kMaxChunks = dsa_host::kSelectMaxRow / kChunk;
constexpr int kBins = dsa_host::kFewHistBins;            // top 12 key bits
constexpr int kBinShift = 32 - 12;
constexpr int kCandMax = 8192;                           // candidates kept per row
// per-row workspace (u32 words): candidate count; the k-th key's bin, the keys
// above that bin and the keys in it; the key histogram; per-chunk (base, count)
// of the candidates; candidate keys; positions
constexpr int kCount = 0, kBin = 1, kAbove = 2, kBinCnt = 3, kHist = dsa_host::kFewHistOffset;
constexpr int kCBase = kHist + kBins, kCCnt = kCBase + kMaxChunks;
constexpr int kKeys = kCCnt + kMaxChunks, kPos = kKeys + kCandMax;
constexpr int kRowWords = kPos + kCandMax;
static_assert(kBins == kThreads * 4, "the bin search gives each thread four bins");
static_assert(kMaxChunks <= kThreads, "one thread per chunk in the gather");

__device__ __forceinline__ int64_t row_len(int64_t r, int32_t n_q, int64_t q_pos0, int32_t n_k) {
  const int64_t t = q_pos0 + (r % n_q);
  return t + 1 < n_k ? t + 1 : (int64_t)n_k;
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

// Exact rem-th largest key among the n keys in LDS that match prefix/mask
// (the candidates' top 12 bits are known): two 10-bit digits.
__device__ void lds_select_low(const uint32_t* keys, int n, uint32_t prefix, uint32_t mask, uint32_t rem, uint32_t* h,
                               uint32_t* sh, uint32_t* st, uint32_t& T, uint32_t& req) {
#pragma unroll 1
  for (int shift = 10; shift >= 0; shift -= 10) {
    for (int i = threadIdx.x; i < 1024; i += blockDim.x) h[i] = 0u;
    __syncthreads();
    for (int i0 = 0; i0 < n; i0 += blockDim.x) {
      const int i = i0 + (int)threadIdx.x;
      const uint32_t u = i < n ? keys[i] : 0u;
      hist_add(h, i < n && (u & mask) == prefix, (u >> shift) & 1023u);
    }
    __syncthreads();
    pick_digit(h, 1024, shift, 1023u, prefix, mask, rem, sh, st);
  }
  T = prefix;
  req = rem;
}

__device__ __forceinline__ void load_run(const float* row, int64_t s0, int64_t len, float (&v)[kPer]) {
  if (s0 + kPer <= len && (((uintptr_t)(row + s0)) & 15) == 0) {
#pragma unroll
    for (int j = 0; j < kPer; j += 4) {
      const float4 q = *(const float4*)(row + s0 + j);
      v[j] = q.x; v[j + 1] = q.y; v[j + 2] = q.z; v[j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kPer; ++j) v[j] = s0 + j < len ? row[s0 + j] : 0.f;
  }
}

// ---------------------------------------------------------------- prepare / histogram
__global__ __launch_bounds__(kThreads) void prepare_kernel(uint32_t* __restrict__ ws) {
  uint32_t* rw = ws + (int64_t)blockIdx.x * kRowWords;
  for (int i = threadIdx.x; i < kHist + kBins; i += kThreads) rw[i] = 0u;   // counters and histogram
}

// Key histogram of given scores, one 16384-score chunk per workgroup.
__global__ __launch_bounds__(kThreads) void hist_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                        int32_t n_q, int64_t q_pos0, int32_t n_k, int32_t k,
                                                        uint32_t* __restrict__ ws) {
  __shared__ uint32_t h[kBins];
  const int64_t r = blockIdx.y;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  const int64_t c0 = (int64_t)blockIdx.x * kChunk;
  if (len <= k || c0 >= len) return;
  for (int i = threadIdx.x; i < kBins; i += kThreads) h[i] = 0u;
  const int64_t s0 = c0 + (int64_t)threadIdx.x * kPer;
  float v[kPer];
  load_run(scores + r * row_stride, s0, len, v);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kPer; ++j) hist_add(h, s0 + j < len, dsa::order_key(v[j]) >> kBinShift);
  __syncthreads();
  uint32_t* gh = ws + r * kRowWords + kHist;
  for (int i = threadIdx.x; i < kBins; i += kThreads)
    if (h[i]) atomicAdd(&gh[i], h[i]);
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

// ---------------------------------------------------------------- collect
// Keys of bins >= b (the bin of the k-th key) of one 16384-score chunk, written
// in position order at a base taken from the row's candidate counter.
__global__ __launch_bounds__(kThreads) void collect_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                           int32_t n_q, int64_t q_pos0, int32_t n_k, int32_t k,
                                                           uint32_t* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t sh[17];
  __shared__ uint32_t s_bin, s_above, s_binc, s_base;
  const int64_t r = blockIdx.y;
  const int chunk = (int)blockIdx.x;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  if (len <= k) {                                     // take all, then pad
    int32_t* out = idx + r * (int64_t)k;
    if (chunk == 0)
      for (int64_t j = threadIdx.x; j < k; j += kThreads) out[j] = j < len ? (int32_t)j : -1;
    return;
  }
  const int nchunks = (int)((len + kChunk - 1) / kChunk);
  if (chunk >= nchunks) return;
  uint32_t* rw = ws + r * kRowWords;
  // this chunk's scores, in flight while the histogram is searched
  const int64_t s0 = (int64_t)chunk * kChunk + (int64_t)threadIdx.x * kPer;
  float v[kPer];
  load_run(scores + r * row_stride, s0, len, v);
  // the bin of the k-th largest key: thread t sums bins kBins-1-4t .. kBins-4-4t
  // (bin 0 if the histogram holds fewer than k keys: then every key is a
  // candidate and the count check sends the row to the whole-row select)
  if (threadIdx.x == 0) { s_bin = 0u; s_above = 0u; s_binc = 0xFFFFFFFFu; }
  {
    const int hi = kBins - 1 - 4 * (int)threadIdx.x;
    const uint32_t* gh = rw + kHist;
    uint32_t hb[4], local = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { hb[j] = gh[hi - j]; local += hb[j]; }
    uint32_t tot;
    const uint32_t ex = block_scan(local, &tot, sh);
    if (ex < (uint32_t)k && (uint32_t)k <= ex + local) {
      uint32_t c = ex;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c + hb[j] >= (uint32_t)k) { s_bin = (uint32_t)(hi - j); s_above = c; s_binc = hb[j]; break; }
        c += hb[j];
      }
    }
    __syncthreads();
  }
  const uint32_t tau = s_bin << kBinShift;
  uint32_t u[kPer];
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    u[j] = dsa::order_key(v[j]);
    c += (s0 + j < len && u[j] >= tau) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t ex = block_scan(c, &tot, sh);
  if (threadIdx.x == 0) {
    const uint32_t base = tot ? atomicAdd(&rw[kCount], tot) : 0u;
    s_base = base;
    rw[kCBase + chunk] = base;
    rw[kCCnt + chunk] = tot;
    if (chunk == 0) {
      rw[kBin] = s_bin;
      rw[kAbove] = s_above;
      rw[kBinCnt] = s_binc;
    }
  }
  __syncthreads();
  uint32_t pos = s_base + ex;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
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
__global__ __launch_bounds__(kThreads) void final_kernel(const float* __restrict__ scores, int64_t row_stride,
                                                         int32_t n_q, int64_t q_pos0, int32_t n_k, int32_t k,
                                                         const uint32_t* __restrict__ ws, int32_t* __restrict__ idx) {
  __shared__ uint32_t ckey[kCandMax];
  __shared__ uint32_t cpos[kCandMax];
  __shared__ uint32_t h[1024];
  __shared__ uint32_t cofs[kMaxChunks + 1];
  __shared__ uint32_t cbase[kMaxChunks];
  __shared__ uint32_t sh[17];
  __shared__ uint32_t st[4];
  const int64_t r = blockIdx.x;
  const int64_t len = row_len(r, n_q, q_pos0, n_k);
  if (len <= k) return;                               // written by collect_kernel
  int32_t* out = idx + r * (int64_t)k;
  const uint32_t* rw = ws + r * kRowWords;
  const int nchunks = (int)((len + kChunk - 1) / kChunk);
  const uint32_t n = rw[kCount];
  const uint32_t tau = rw[kBin] << kBinShift, above = rw[kAbove];
  // the candidates are exactly the keys of bins >= b: any other count means the
  // histogram does not describe these scores, and the whole row is selected
  if (n > (uint32_t)kCandMax || n != above + rw[kBinCnt]) {
    // the 4096-bin histogram of the whole-row sweeps reuses the candidate key array
    select_whole_row(scores + r * row_stride, len, k, out, ckey, sh, st);
    return;
  }
  // chunk order = position order: chunk q's candidates go to [cofs[q], cofs[q+1])
  {
    const uint32_t cc = (int)threadIdx.x < nchunks ? rw[kCCnt + threadIdx.x] : 0u;
    if ((int)threadIdx.x < nchunks) cbase[threadIdx.x] = rw[kCBase + threadIdx.x];
    uint32_t t2;
    const uint32_t o = block_scan(cc, &t2, sh);
    if ((int)threadIdx.x < nchunks) cofs[threadIdx.x] = o;
    if (threadIdx.x == 0) cofs[nchunks] = t2;
    __syncthreads();
  }
  constexpr int PER = kCandMax / kThreads;
  uint32_t kk[PER], pp[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    kk[j] = 0u;
    pp[j] = 0u;
    if (i < (int)n) {
      int lo = 0, hi = nchunks - 1;                  // chunk q with cofs[q] <= i < cofs[q+1]
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (cofs[mid] <= (uint32_t)i) lo = mid; else hi = mid - 1;
      }
      const uint32_t src = cbase[lo] + ((uint32_t)i - cofs[lo]);
      kk[j] = rw[kKeys + src];
      pp[j] = rw[kPos + src];
    }
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    if (i < (int)n) {
      ckey[i] = kk[j];
      cpos[i] = pp[j];
    }
  }
  __syncthreads();
  uint32_t T, req;
  lds_select_low(ckey, (int)n, tau, 0xFFFFFFFFu << kBinShift, (uint32_t)k - above, h, sh, st, T, req);
  // ordered write: candidates are in position order; thread t owns a contiguous run
  const int per = ((int)n + kThreads - 1) / kThreads;
  const int a0 = (int)threadIdx.x * per;
  const int a1 = a0 + per < (int)n ? a0 + per : (int)n;
  uint32_t gt = 0, eq = 0;
  for (int i = a0; i < a1; ++i) {
    gt += ckey[i] > T ? 1u : 0u;
    eq += ckey[i] == T ? 1u : 0u;
  }
  uint32_t tg, te;
  const uint32_t gt_before = block_scan(gt, &tg, sh);
  const uint32_t eq_before = block_scan(eq, &te, sh);
  uint32_t opos = gt_before + (eq_before < req ? eq_before : req);
  uint32_t tie = eq_before;
  for (int i = a0; i < a1; ++i) {
    const uint32_t x = ckey[i];
    const bool keep = x > T || (x == T && tie < req);
    tie += x == T ? 1u : 0u;
    if (keep) {
      if (opos < (uint32_t)k) out[opos] = (int32_t)cpos[i];
      ++opos;
    }
  }
}

}  // namespace

namespace dsa_host {

size_t select_few_ws_bytes(int64_t rows) { return (size_t)rows * kRowWords * sizeof(uint32_t); }

FewHist select_few_hist(void* ws) { return FewHist{(uint32_t*)ws + kHist, (int64_t)kRowWords}; }

hipError_t select_few_prepare(void* ws, int64_t rows, hipStream_t s) {
  hipLaunchKernelGGL(prepare_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, (uint32_t*)ws);
  return hipGetLastError();
}

static dim3 chunk_grid(const SelectPlan& p) {
  const int64_t maxlen = p.q_pos0 + p.n_q < p.n_k ? p.q_pos0 + p.n_q : (int64_t)p.n_k;
  int64_t P = (maxlen + kChunk - 1) / kChunk;
  if (P < 1) P = 1;
  return dim3((unsigned)P, (unsigned)p.rows);
}

hipError_t select_few_hist_scores(const float* scores, const SelectPlan& p, void* ws, hipStream_t s) {
  hipLaunchKernelGGL(hist_kernel, chunk_grid(p), dim3(kThreads), 0, s, scores, p.row_stride, p.n_q, p.q_pos0,
                     p.n_k, p.k, (uint32_t*)ws);
  return hipGetLastError();
}

hipError_t select_few_finish(const float* scores, const SelectPlan& p, void* ws, int32_t* idx, hipStream_t s) {
  hipLaunchKernelGGL(collect_kernel, chunk_grid(p), dim3(kThreads), 0, s, scores, p.row_stride, p.n_q, p.q_pos0,
                     p.n_k, p.k, (uint32_t*)ws, idx);
  hipLaunchKernelGGL(final_kernel, dim3((unsigned)p.rows), dim3(kThreads), 0, s, scores, p.row_stride, p.n_q,
                     p.q_pos0, p.n_k, p.k, (const uint32_t*)ws, idx);
  return hipGetLastError();
}

}  // namespace dsa_host
