// Sparse core attention over selected positions ([DSA-NOTES] §3, equation for o_t):
//     o[h] = sum_{s in T} softmax_s(scale * Q[h] . K[s]) V[s]
//
//  * sa_generic_kernel  any shape, fp32 or bf16, one workgroup per (query row,
//    head): logits in LDS, block max/sum, then P.V with coalesced V reads.
//  * sa_mla4_kernel     bf16 MLA latent layout on MFMA: 16 query heads share one
//    576-wide latent row per position whose first 512 columns are V.  One
//    four-wave workgroup per (query row, split of the index row); per step of
//    16 selected positions:
//      S^T[16 keys x 16 heads] = K_sel . Q^T    (16x16x32 bf16 MFMA; each wave
//                                                contracts its own columns of
//                                                the gathered rows, partials
//                                                are summed through LDS)
//      online softmax per head (the S^T layout gives each lane one head)
//      O^T[128 x 16] += V_sel^T . P^T          (16x16x16 bf16 MFMA per wave on
//                                                its 128 V columns; V^T comes
//                                                from the gathered rows via a
//                                                transposing LDS read)
//    P^T needs no data movement: the S^T accumulator layout (lane = head,
//    registers = 4 consecutive keys) is exactly the B-operand layout of the
//    16x16x16 MFMA.  With several splits per row the partial (max, sum, O) go
//    to the workspace and sa_combine_kernel merges them.
#include "common.hpp"

namespace {

using namespace dsa;

struct SAParams {
  int32_t dtype;
  int32_t batch, n_q, n_k, heads, kv_heads, d_qk, d_v, topk;
  const void* q;
  const void* kv;
  int64_t kv_bs;
  const void* v;
  int64_t v_bs;
  const int32_t* idx;
  float scale;
  float* out;
  int32_t nsplit;
  float* ws_o;    // [rows, nsplit, heads, d_v]
  float* ws_ml;   // [rows, nsplit, heads, 2]
};

__device__ __forceinline__ float ldf(const void* base, int64_t i, bool bf16) {
  if (bf16) return bf16_bits_to_f32(((const uint16_t*)base)[i]);
  return ((const float*)base)[i];
}

__device__ float block_reduce(float v, float* sh, bool is_max) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = blockDim.x >> 6;
  v = is_max ? wave_max(v) : wave_sum(v);
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  float r = sh[0];
  for (int w = 1; w < nw; ++w) r = is_max ? fmaxf(r, sh[w]) : r + sh[w];
  __syncthreads();
  return r;
}

// max / sum over lanes l, l^16, l^32, l^48 (the four lanes holding one head in
// the 16x16 MFMA layouts), with lane swaps instead of LDS permutes
__device__ __forceinline__ float quad_max(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Weights p (4 per lane) as bf16 hi + lo parts: hi = bf16(p), lo = bf16(p - hi),
// converted two at a time.
__device__ __forceinline__ void split_bf16(const float (&pe)[4], bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x2 h = __builtin_convertvector((f32x2){pe[2 * j], pe[2 * j + 1]}, bf16x2);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xffff0000u);
    const bf16x2 l = __builtin_convertvector((f32x2){pe[2 * j] - h0, pe[2 * j + 1] - h1}, bf16x2);
    hi[2 * j] = h[0]; hi[2 * j + 1] = h[1];
    lo[2 * j] = l[0]; lo[2 * j + 1] = l[1];
  }
}

// ---------------------------------------------------------------- generic path
__global__ __launch_bounds__(256) void sa_generic_kernel(SAParams p) {
  extern __shared__ float smem[];
  float* qs = smem;                   // d_qk
  float* z = smem + p.d_qk;           // topk
  __shared__ float red[16];
  const int h = blockIdx.x % p.heads;
  const int64_t gi = blockIdx.x / p.heads;      // flattened (b, i)
  const int b = (int)(gi / p.n_q);
  const bool bf = p.dtype == DSA_BF16;
  const int hk = h * p.kv_heads / p.heads;
  for (int c = threadIdx.x; c < p.d_qk; c += blockDim.x) qs[c] = ldf(p.q, (gi * p.heads + h) * (int64_t)p.d_qk + c, bf);
  __syncthreads();
  const int32_t* ir = p.idx + gi * (int64_t)p.topk;
  float mx = -__builtin_inff();
  for (int e = threadIdx.x; e < p.topk; e += blockDim.x) {
    const int32_t s = ir[e];
    float zz = -__builtin_inff();
    if (s >= 0 && s < p.n_k) {
      const int64_t kb = (int64_t)b * p.kv_bs + ((int64_t)s * p.kv_heads + hk) * p.d_qk;
      float d = 0.f;
      for (int c = 0; c < p.d_qk; ++c) d = fmaf(qs[c], ldf(p.kv, kb + c, bf), d);
      zz = d * p.scale;
    }
    z[e] = zz;
    mx = fmaxf(mx, zz);
  }
  mx = block_reduce(mx, red, true);
  float sum = 0.f;
  for (int e = threadIdx.x; e < p.topk; e += blockDim.x) {
    const float pe = (mx == -__builtin_inff() || z[e] == -__builtin_inff()) ? 0.f : __expf(z[e] - mx);
    z[e] = pe;
    sum += pe;
  }
  sum = block_reduce(sum, red, false);
  __syncthreads();
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
  float* out = p.out + (gi * p.heads + h) * (int64_t)p.d_v;
  const void* vb = p.v ? p.v : p.kv;
  const int64_t vrow = p.v ? (int64_t)p.kv_heads * p.d_v : (int64_t)p.kv_heads * p.d_qk;
  const int64_t vhead = p.v ? p.d_v : p.d_qk;
  const int64_t vbs = p.v ? p.v_bs : p.kv_bs;
  for (int c = threadIdx.x; c < p.d_v; c += blockDim.x) {
    float acc = 0.f;
    for (int e = 0; e < p.topk; ++e) {
      const float pe = z[e];
      if (pe != 0.f) {
        const int32_t s = ir[e];
        acc = fmaf(pe, ldf(vb, (int64_t)b * vbs + (int64_t)s * vrow + hk * vhead + c, bf), acc);
      }
    }
    out[c] = acc * inv;
  }
}

// ---------------------------------------------------------------- MLA MFMA path
constexpr int kH = 16;       // query heads per latent row
constexpr int kTile = 16;    // selected positions per step
constexpr int kMaxTopk = DSA_MAX_TOPK;   // longest index row

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Four waves per (query row, split of its index row).  Wave w owns latent
// columns [128w, 128w + 128): four 32-wide K steps of Q.K and the 128 V columns
// of its slice of the output; waves 0 and 1 also own one of the two rope K
// steps (columns 512 + 32w ..).  Per 16-position step each wave gathers only
// its own columns of the 16 rows (registers, two steps ahead), forms its
// partial S^T, and the four partials meet in LDS (one barrier per step, the
// partial buffer alternates between steps).  Every wave then runs the same
// online softmax on the full S^T and multiplies its own V slice, staged in a
// wave-private LDS tile and read back transposed as in sa_mla_kernel.  The
// output accumulators are a quarter of sa_mla_kernel's, so three workgroups
// fit on a CU.
template <int DQK, int DV>
__global__ __launch_bounds__(256, 3) void sa_mla4_kernel(SAParams p) {
  static_assert(DV % 128 == 0 && DQK - DV == 64, "latent layout: 4 V slices of 128 columns + 64 rope columns");
  constexpr int NW = 4;
  constexpr int CW = DV / NW;            // V columns per wave
  constexpr int KSW = CW / 32;           // K steps inside the wave's V slice
  constexpr int KS = KSW + 1;            // + a rope step (waves 0 and 1)
  constexpr int NDT = CW / 16;           // output tiles of 16 columns per wave
  constexpr int VPITCH = CW * 2 + 32;    // LDS row pitch in bytes (bank spread for the transposed reads)
  __shared__ __attribute__((aligned(16))) uint8_t vt[NW][kTile * VPITCH];
  __shared__ f32x4 spart[2][NW][64];
  __shared__ int32_t sidx[kMaxTopk];      // this split's selected positions

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int g = lane >> 4, col = lane & 15;
  const bool rope = w < 2;
  const int split = (int)(blockIdx.x % p.nsplit);
  const int64_t gi = blockIdx.x / p.nsplit;          // flattened (batch, query row)
  const int b = (int)(gi / p.n_q);
  const int per = (p.topk + p.nsplit - 1) / p.nsplit;
  const int e0 = split * per;
  const int e1 = e0 + per < p.topk ? e0 + per : p.topk;
  // first column (elements) of K step ks of this wave
  auto kcol = [&](int ks) { return ks < KSW ? CW * w + 32 * ks : DV + 32 * w; };

  // Q^T as the B operand: lane holds head `col`, 8 columns of each K step.
  bf16x8 qf[KS];
  const __bf16* qrow = (const __bf16*)p.q + (gi * kH + col) * (int64_t)DQK;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = (ks < KSW || rope) ? *(const bf16x8*)(qrow + kcol(ks) + 8 * g) : bf16x8{};

  f32x4 o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) o[d] = f32x4{};
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float sl2 = p.scale * 1.4426950408889634f;   // scale * log2(e)

  // Gathers are buffer loads over this batch's latent rows: a position that is
  // invalid (or past the split) gets an offset beyond the range and reads
  // zeros, so every fetch is the same straight-line code and the compiler can
  // keep two steps of gathers in flight.  Positions come from LDS, not from
  // vector loads that would have to wait behind the gathers in flight.
  const __amdgpu_buffer_rsrc_t kvr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>((const void*)((const __bf16*)p.kv + (int64_t)b * p.kv_bs)), (short)0,
      (int)((int64_t)p.n_k * DQK * 2), 0x00020000);
  {
    const int32_t* ir = p.idx + gi * (int64_t)p.topk;
    for (int e = e0 + (int)threadIdx.x; e < e1; e += NW * 64) sidx[e - e0] = ir[e];
  }
  __syncthreads();
  uint8_t* wrow = vt[w] + col * VPITCH + 16 * g;
  const uint8_t* rbase = vt[w] + (4 * g + (col >> 2)) * VPITCH + 8 * (col & 3);
  int pbuf = 0;

  auto fetch = [&](int tb, bf16x8 (&kb)[KS], uint64_t& vm) {
    const int e = tb + col;
    const int32_t s = sidx[(e < e1 ? e : e1 - 1) - e0];
    const bool valid = e < e1 && s >= 0 && s < p.n_k;
    vm = ballot(valid);
    const uint32_t base = valid ? (uint32_t)s * (DQK * 2) : 0x80000000u;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t off = (ks < KSW || rope ? base : 0x80000000u) + (uint32_t)(kcol(ks) * 2 + 16 * g);
      kb[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kvr, off, 0, 0));
    }
  };
  auto step = [&](const bf16x8 (&kb)[KS], uint64_t vm) {
    f32x4 acc = f32x4{};
    // (waves 2 and 3 run the rope step on zero operands: same code in every wave)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[ks], qf[ks], acc, 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) *(bf16x8*)(wrow + 64 * ks) = kb[ks];
    spart[pbuf][w][lane] = acc;
    sync_lds_barrier();
    // the same summation order in every wave: identical softmax state everywhere
    const f32x4 sc = ((spart[pbuf][0][lane] + spart[pbuf][1][lane]) + spart[pbuf][2][lane]) + spart[pbuf][3][lane];
    pbuf ^= 1;
    // sc[i]: head `col`, position 4*g + i of this step.  The softmax runs in
    // base 2 (scores times scale * log2 e; the weights are unchanged).
    const uint32_t vb = (uint32_t)(vm >> (4 * g));
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = ((vb >> i) & 1u) ? sc[i] * sl2 : -__builtin_inff();
    const float mx = quad_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    const float m_new = fmaxf(m_run, mx);
    bf16x4 pb_hi = bf16x4{}, pb_lo = bf16x4{};
    float alpha = 1.f;
    if (m_new != -__builtin_inff()) {
      alpha = (m_run == m_new) ? 1.f : ((m_run == -__builtin_inff()) ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new));
      float pe[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) pe[i] = z[i] == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f(z[i] - m_new);
      split_bf16(pe, pb_hi, pb_lo);
      l_run = l_run * alpha + ((pe[0] + pe[1]) + (pe[2] + pe[3]));
      m_run = m_new;
    }
    if (ballot(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rbase + 32 * dt));
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_hi, o[dt], 0, 0, 0);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pb_lo, o[dt], 0, 0, 0);
    }
    // this wave's V tile is rewritten next step only after these reads returned
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  };

  // three register buffers, rotated by unrolling the loop by three steps;
  // fetches past the split read zeros without touching memory
  bf16x8 kbA[KS], kbB[KS], kbC[KS];
  uint64_t vmA = 0, vmB = 0, vmC = 0;
  if (e0 < e1) {
    fetch(e0, kbA, vmA);
    fetch(e0 + kTile, kbB, vmB);
  }
  for (int tb = e0; tb < e1; tb += 3 * kTile) {
    fetch(tb + 2 * kTile, kbC, vmC);
    step(kbA, vmA);
    if (tb + kTile >= e1) break;
    fetch(tb + 3 * kTile, kbA, vmA);
    step(kbB, vmB);
    if (tb + 2 * kTile >= e1) break;
    fetch(tb + 4 * kTile, kbB, vmB);
    step(kbC, vmC);
  }
  l_run = quad_sum(l_run);
  // O^T layout: lane holds head `col`, columns CW*w + 16*dt + 4*g + (0..3)
  if (p.nsplit == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    float* out = p.out + (gi * kH + col) * (int64_t)DV + CW * w + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(out + 16 * dt) = o[dt] * inv;
  } else {
    float* wo = p.ws_o + ((gi * p.nsplit + split) * kH + col) * (int64_t)DV + CW * w + 4 * g;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *(f32x4*)(wo + 16 * dt) = o[dt];
    if (w == 0 && g == 0) {
      // the combine step works in natural-log units
      float* ml = p.ws_ml + ((gi * p.nsplit + split) * kH + col) * 2;
      ml[0] = m_run * 0.6931471805599453f;
      ml[1] = l_run;
    }
  }
}

// Merge the split partials of one (query row, head): thread c loads column c of
// every split's partial output first (all loads in flight at once), while wave
// 0 forms the weights exp(m_s - M) in LDS; then each thread sums its column.
constexpr int kMaxSplit = kMaxTopk / 64;    // splits hold at least 64 positions
__global__ __launch_bounds__(512) void sa_combine_kernel(SAParams p) {
  __shared__ float wsum[2];
  __shared__ float wgt[kMaxSplit];
  const int h = blockIdx.x % p.heads;
  const int64_t gi = blockIdx.x / p.heads;
  const float* ml = p.ws_ml + (gi * p.nsplit * p.heads + h) * 2;   // split stride: heads * 2
  const float* po = p.ws_o + (gi * p.nsplit * p.heads + h) * (int64_t)p.d_v;
  const int64_t sstride = (int64_t)p.heads * p.d_v;
  const int c = threadIdx.x;                 // one output column per thread (d_v = blockDim.x)
  float v[kMaxSplit];
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) v[sp] = sp < p.nsplit ? po[sp * sstride + c] : 0.f;
  if (threadIdx.x < 64) {
    const float ms = (int)threadIdx.x < p.nsplit ? ml[(int64_t)threadIdx.x * p.heads * 2] : -__builtin_inff();
    const float ls = (int)threadIdx.x < p.nsplit ? ml[(int64_t)threadIdx.x * p.heads * 2 + 1] : 0.f;
    const float M = wave_max(ms);
    const float w = (ms == -__builtin_inff()) ? 0.f : __expf(ms - M);
    if ((int)threadIdx.x < kMaxSplit) wgt[threadIdx.x] = w;
    const float L = wave_sum(w * ls);
    if (threadIdx.x == 0) wsum[0] = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp)
    if (sp < p.nsplit) acc = fmaf(wgt[sp], v[sp], acc);
  p.out[(gi * p.heads + h) * (int64_t)p.d_v + c] = acc * wsum[0];
}

bool mla_ok(const dsa_sparse_attn_args& a) {
  // (one batch's latent rows are addressed with 32-bit byte offsets)
  return a.dtype == DSA_BF16 && a.heads == kH && a.kv_heads == 1 && a.d_qk == 576 &&
         a.d_v == 512 && a.v == nullptr && (int64_t)a.n_k * a.d_qk * 2 < ((int64_t)1 << 31);
}

int pick_nsplit(const dsa_sparse_attn_args& a) {
  const int64_t rows = (int64_t)a.batch * a.n_q;
  int64_t ns = (1024 + rows - 1) / rows;
  int64_t maxs = a.topk / 64;
  if (maxs < 1) maxs = 1;
  if (ns > maxs) ns = maxs;
  if (ns < 1) ns = 1;
  return (int)ns;
}

SAParams make(const dsa_sparse_attn_args& a) {
  SAParams p{};
  p.dtype = a.dtype;
  p.batch = a.batch; p.n_q = a.n_q; p.n_k = a.n_k; p.heads = a.heads; p.kv_heads = a.kv_heads;
  p.d_qk = a.d_qk; p.d_v = a.d_v; p.topk = a.topk;
  p.q = a.q; p.kv = a.kv; p.v = a.v; p.idx = a.idx; p.scale = a.scale; p.out = a.out;
  p.kv_bs = a.kv_batch_stride ? a.kv_batch_stride : (int64_t)a.n_k * a.kv_heads * a.d_qk;
  p.v_bs = a.v_batch_stride ? a.v_batch_stride : (int64_t)a.n_k * a.kv_heads * a.d_v;
  p.nsplit = 1;
  return p;
}

}  // namespace

namespace dsa_host {

size_t sparse_attn_ws_bytes(const dsa_sparse_attn_args& a) {
  if (!mla_ok(a)) return 0;
  const int ns = pick_nsplit(a);
  if (ns == 1) return 0;
  const int64_t rows = (int64_t)a.batch * a.n_q;
  return (size_t)rows * ns * a.heads * ((size_t)a.d_v + 2) * sizeof(float);
}

hipError_t sparse_attn_launch(const dsa_sparse_attn_args& a, void* ws, hipStream_t s) {
  SAParams p = make(a);
  if (mla_ok(a)) {
    p.nsplit = pick_nsplit(a);
    const int64_t rows = (int64_t)a.batch * a.n_q;
    if (p.nsplit > 1) {
      p.ws_o = (float*)ws;
      p.ws_ml = p.ws_o + rows * p.nsplit * a.heads * (int64_t)a.d_v;
    }
    dim3 grid((unsigned)(rows * p.nsplit));
    hipLaunchKernelGGL((sa_mla4_kernel<576, 512>), grid, dim3(256), 0, s, p);
    if (p.nsplit > 1) {
      hipLaunchKernelGGL(sa_combine_kernel, dim3((unsigned)(rows * a.heads)), dim3(512), 0, s, p);
    }
    return hipGetLastError();
  }
  const size_t lds = ((size_t)a.d_qk + a.topk) * sizeof(float);
  dim3 grid((unsigned)((int64_t)a.batch * a.n_q * a.heads));
  hipLaunchKernelGGL(sa_generic_kernel, grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace dsa_host
