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
//      O^T[128 x 16] += V_sel^T . P^T          (16x16x32 bf16 MFMA per wave on
//                                                its 128 V columns, P in bf16
//                                                hi and lo parts along K; V^T
//                                                comes from the gathered rows
//                                                via a transposing LDS read)
//    P^T needs no data movement: the S^T accumulator layout (lane = head,
//    registers = 4 consecutive keys) is the B-operand layout of a 16-deep
//    MFMA, and its hi and lo parts side by side that of the 32-deep one.
//    With several splits per row the partial (max, sum, O) go to the
//    workspace and sa_combine_kernel merges them.  Used below 1024 rows
//    (decode), where rows are split to fill the chip.
//  * sa_mla1_kernel     the same arithmetic with one wave per query row (from
//    1024 rows, no splits): the wave gathers whole latent rows straight into
//    LDS, one load instruction per row, which the chip serves faster than four
//    waves each fetching a slice of every row into registers, and needs no
//    partial-score exchange.
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
// converted two at a time.  The P.V products take both parts in one
// v_mfma_f32_16x16x32_bf16 per output tile: a lane's eight K slots hold hi and
// then lo of its four positions, against its V fragment of those positions
// twice.  (Two 16x16x16 products give the same sum, but that form runs at half
// the 16x16x32 form's rate on gfx950.)
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
constexpr uint32_t kInvalid = 0x80000000u;   // byte offset past every latent buffer (n_k * 1152 < 2^31)

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Four waves per (query row, split of its index row).  Wave w owns latent
// columns [128w, 128w + 128): four 32-wide K steps of Q.K and the 128 V columns
// of its slice of the output; waves 0 and 1 also own one of the two rope K
// steps (columns 512 + 32w ..).  Per 16-position step each wave gathers only
// its own columns of the 16 rows (registers, two steps ahead): its 256-byte V
// slice of each row (two whole 128-byte lines) four rows per load instruction,
// sixteen lanes per row, so every instruction fetches whole lines; the slices
// go to a wave-private LDS tile, which serves both the K fragments of Q.K
// (read back row-per-lane) and the transposed V fragments of P.V.  The rope
// slice (64 bytes per row) is loaded straight in the MFMA fragment layout.
// The four partial S^T meet in LDS (one barrier per step, the partial buffer
// alternates between steps).  Every wave then runs the same online softmax on
// the full S^T and multiplies its own V slice.  The output accumulators are a
// quarter of a one-wave-per-query design's, so three workgroups fit on a CU.
template <int DQK, int DV>
__global__ __launch_bounds__(256, 3) void sa_mla4_kernel(SAParams p) {
  static_assert(DV % 128 == 0 && DQK - DV == 64, "latent layout: 4 V slices of 128 columns + 64 rope columns");
  constexpr int NW = 4;
  constexpr int CW = DV / NW;            // V columns per wave
  constexpr int KSW = CW / 32;           // K steps inside the wave's V slice
  constexpr int KS = KSW + 1;            // + a rope step (waves 0 and 1)
  constexpr int NDT = CW / 16;           // output tiles of 16 columns per wave
  constexpr int SLB = CW * 2;            // bytes of the wave's V slice per row
  constexpr int LPR = SLB / 16;          // lanes (16-byte chunks) per row slice: 16
  constexpr int RPL = 64 / LPR;          // rows per load instruction: 4
  static_assert(LPR == 16 && kTile % RPL == 0 && KSW == kTile / RPL, "one V load per K step");
  // LDS row pitch: 76 dwords, so the row-per-lane 16-byte fragment reads (12 r
  // mod 64 banks) and the transposed 8-byte reads (each bank twice per 64
  // lanes) are both conflict-free
  constexpr int VPITCH = SLB + 48;
  __shared__ __attribute__((aligned(16))) uint8_t vt[NW][kTile * VPITCH];
  __shared__ f32x4 spart[2][NW][64];
  // this split's selected rows as byte offsets into the latent rows (kInvalid
  // for entries outside [0, n_k) and for the padding after the split, which
  // the fetches up to four steps past the split's end read)
  __shared__ uint32_t sidx[kMaxTopk + 5 * kTile];

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
    qf[ks] = (ks < KSW || rope) ? __builtin_nontemporal_load((const bf16x8*)(qrow + kcol(ks) + 8 * g)) : bf16x8{};

  f32x4 o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) o[d] = f32x4{};
  // Online softmax in base 2 with a lazily moved reference: scores are scaled
  // by scale * log2 e, and the reference m_run (per head) only moves when a
  // step's maximum exceeds it by more than kLazy, so the weights exp2(z - m_run)
  // stay below 2^kLazy and O and l are rescaled only on those steps (a handful
  // per row instead of every step that raises the maximum).  O / l is the same.
  constexpr float kLazy = 8.f;
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
    for (int e = e0 + (int)threadIdx.x; e < e1 + 5 * kTile; e += NW * 64) {
      const int32_t s = e < e1 ? ir[e] : -1;
      sidx[e - e0] = (s >= 0 && s < p.n_k) ? (uint32_t)s * (DQK * 2) : kInvalid;
    }
  }
  __syncthreads();
  // V slice: load j holds row RPL*j + lane/16, chunk lane%16 of the slice
  uint8_t* wrow = vt[w] + (lane / LPR) * VPITCH + 16 * (lane % LPR);
  // K fragment of step ks: row `col`, 8 columns at 32 ks + 8 g
  const uint8_t* frow = vt[w] + col * VPITCH + 16 * g;
  const uint8_t* rbase = vt[w] + (4 * g + (col >> 2)) * VPITCH + 8 * (col & 3);
  int pbuf = 0;

  // (an invalid entry's offset plus a column offset stays past the buffer range)
  const uint32_t vcol = (uint32_t)(SLB * w + 16 * (lane % LPR));
  const uint32_t rcol = (uint32_t)(kcol(KSW) * 2 + 16 * g);
  auto fetch = [&](int tb, bf16x8 (&kb)[KS], uint64_t& vm) {
    const uint32_t* si = sidx + (tb - e0);
    const uint32_t oc = si[col];
    vm = ballot(oc != kInvalid);
#pragma unroll
    for (int j = 0; j < KSW; ++j) {
      const uint32_t off = si[RPL * j + lane / LPR] + vcol;
      kb[j] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kvr, off, 0, 0));
    }
    // rope step in fragment layout (waves 2 and 3 read zeros without touching memory)
    const uint32_t roff = rope ? oc + rcol : kInvalid;
    kb[KSW] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(kvr, roff, 0, 0));
  };
  auto step = [&](const bf16x8 (&kb)[KS], uint64_t vm) {
#pragma unroll
    for (int j = 0; j < KSW; ++j) *(bf16x8*)(wrow + RPL * VPITCH * j) = kb[j];
    f32x4 acc = f32x4{};
    // (waves 2 and 3 run the rope step on zero operands: same code in every wave)
#pragma unroll
    for (int ks = 0; ks < KSW; ++ks) {
      const bf16x8 kf = *(const bf16x8*)(frow + 64 * ks);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], acc, 0, 0, 0);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb[KSW], qf[KSW], acc, 0, 0, 0);
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
    // (also true on the first valid step, while m_run is still -inf)
    const bool bump = mx > m_run + kLazy;
    if (ballot(bump)) {
      const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;   // 0 on the first step
      m_run = bump ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    // invalid positions have z = -inf and weight exp2(-inf) = 0; before the
    // first valid position the reference is -inf, taken as -FLT_MAX here
    const float mref = fmaxf(m_run, -__FLT_MAX__);
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(z[i] - mref);
    bf16x4 pb_hi, pb_lo;
    split_bf16(pe, pb_hi, pb_lo);
    const bf16x8 pb2 = __builtin_shufflevector(pb_hi, pb_lo, 0, 1, 2, 3, 4, 5, 6, 7);
    l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const bf16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rbase + 32 * dt));
      const bf16x8 v2 = __builtin_shufflevector(va, va, 0, 1, 2, 3, 0, 1, 2, 3);
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, pb2, o[dt], 0, 0, 0);
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
    for (int dt = 0; dt < NDT; ++dt) __builtin_nontemporal_store(o[dt] * inv, (f32x4*)(out + 16 * dt));
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

// One wave per query row; the four waves of a workgroup work on four rows
// independently (no barriers).  Per 16-position step the wave gathers the 16
// selected latent rows whole, straight into LDS (buffer_load ... lds): one load
// instruction per row for its first KiB (the 512 V columns: 64 lanes x 16
// bytes of that row alone) and two for the 16 rope lines (eight rows per
// instruction, eight lanes per 128-byte line).  Each wave has two row tiles,
// the one being consumed and the one being filled two steps ahead.  A tile
// holds the V bytes at a 1040-byte row pitch (260 dwords = 4 mod 64 banks, so
// the row-per-lane K-fragment reads and the transposed V reads are
// conflict-free) and, after them, the rope lines: rope load k (rows 8k..8k+7)
// puts chunk c of row 8k + j in slot 64k + 8j + ((c + j + k) mod 8), which
// spreads the 16 rows' reads of one chunk over 16 distinct bank groups.  The
// tile serves all 18 K steps of S^T = K_sel . Q^T and all 32 output tiles of
// O^T += V_sel^T . P^T, so there is no partial-score exchange and the softmax
// (the same lazily rescaled base-2 online softmax as above) runs once per row.
// The index row goes through a per-wave ring of four 64-entry blocks, also by
// DMA (an LDS copy of the whole row would not fit beside the tiles), converted
// to byte offsets in place.  The output accumulators (16 heads x 512 columns)
// and Q^T take the register file of one wave per SIMD.  The DMAs are invisible to the
// compiler's wait counting: every wait on them is explicit, and a tile is
// refilled only after every read of the step that consumed it returned.
template <int DQK, int DV>
__global__ __launch_bounds__(256, 1) void sa_mla1_kernel(SAParams p, int64_t rows) {
  constexpr int KS = DQK / 32;               // K steps of Q.K (18)
  constexpr int KSV = DV / 32;               // K steps inside V (16)
  constexpr int NDT = DV / 16;               // output tiles of 16 columns (32)
  constexpr int ROWB = DQK * 2;              // bytes per latent row (1152)
  constexpr int VB = DV * 2;                 // V bytes per row: one load instruction
  static_assert(VB == 64 * 16 && ROWB - VB == 128 && KS == KSV + 2 && NDT % 8 == 0,
                "latent layout: 1 KiB of V + one rope line");
  constexpr int VP = VB + 16;                // V row pitch (1040)
  constexpr int ROPE = kTile * VP;           // rope slots start (16640)
  constexpr int TB = ROPE + kTile * 128;     // tile bytes (18688)
  constexpr int NLD = kTile + 2;             // row loads per step
  constexpr int NRING = 4;                   // index blocks of 64 entries
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][2][TB];
  __shared__ __attribute__((aligned(16))) uint32_t ring_all[4][NRING][64];

  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int64_t gi = (int64_t)blockIdx.x * 4 + w;    // flattened (batch, query row)
  if (gi >= rows) return;                              // (no barriers below)
  const int g = lane >> 4, col = lane & 15;
  const int b = (int)(gi / p.n_q);
  uint32_t (*ring)[64] = ring_all[w];
  const int topk = p.topk;

  bf16x8 qf[KS];
  const __bf16* qrow = (const __bf16*)p.q + (gi * kH + col) * (int64_t)DQK;
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qf[ks] = __builtin_nontemporal_load((const bf16x8*)(qrow + 32 * ks + 8 * g));

  f32x4 o[NDT];
#pragma unroll
  for (int d = 0; d < NDT; ++d) o[d] = f32x4{};
  constexpr float kLazy = 8.f;
  float m_run = -__builtin_inff(), l_run = 0.f;
  const float sl2 = p.scale * 1.4426950408889634f;   // scale * log2(e)

  const __amdgpu_buffer_rsrc_t kvr =
      make_rsrc((const __bf16*)p.kv + (int64_t)b * p.kv_bs, (uint32_t)((int64_t)p.n_k * ROWB));
  // the index row (entries past it read zero and are marked invalid below)
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(p.idx + gi * (int64_t)topk, (uint32_t)topk * 4u);
  const int nst = (topk + kTile - 1) / kTile;
  const int nblk = (topk + 63) / 64;

  auto idx_dma = [&](int m) { lds_dma<4>(irs, (const uint8_t*)ring[m % NRING], (uint32_t)(64 * m + lane) * 4u); };
  auto idx_conv = [&](int m) {
    uint32_t* sl = ring[m % NRING];
    const int e = 64 * m + lane;
    const int32_t s = (int32_t)sl[lane];
    sl[lane] = (e < topk && s >= 0 && s < p.n_k) ? (uint32_t)s * ROWB : kInvalid;
  };
  const uint32_t lv = 16u * (uint32_t)lane;
  const int rj = lane >> 3;                                        // rope: row 8k + rj
  // rope: chunk (lane - rj - k) mod 8 of the line, for loads k = 0, 1
  const uint32_t lr0 = (uint32_t)VB + 16u * (uint32_t)((lane - rj) & 7);
  const uint32_t lr1 = (uint32_t)VB + 16u * (uint32_t)((lane - rj - 1) & 7);
  // row DMA of step t into tile `dst` (kInvalid offsets past the last step)
  // (the ring slot is read in any case; past the last step every offset gets the
  // kInvalid bit, so no branch is needed)
  auto row_dma = [&](int t, uint8_t* dst, uint64_t& vm) {
    const uint32_t dead = t < nst ? 0u : kInvalid;
    const uint32_t* si = ring[(t >> 2) % NRING] + 16 * (t & 3);
    u32x4 r4[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) r4[q] = *(const u32x4*)(si + 4 * q);
    const uint32_t o0 = si[rj] | dead, o1 = si[8 + rj] | dead, oc = si[col] | dead;
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma<16>(kvr, dst + (4 * q + i) * VP, (r4[q][i] | dead) + lv);
    lds_dma<16>(kvr, dst + ROPE, o0 + lr0);
    lds_dma<16>(kvr, dst + ROPE + 1024, o1 + lr1);
    vm = ballot(oc != kInvalid);
  };
  // K fragments: V steps at row `col` of the V area; rope steps ks' = 0, 1 read
  // chunk 4 ks' + g of row `col` from its slot
  const int rk = col >> 3, rr = col & 7;
  const uint32_t fv = (uint32_t)(col * VP + 16 * g);
  const uint32_t fr0 = (uint32_t)(ROPE + 16 * (64 * rk + 8 * rr + ((g + rr + rk) & 7)));
  const uint32_t fr1 = (uint32_t)(ROPE + 16 * (64 * rk + 8 * rr + ((4 + g + rr + rk) & 7)));
  const uint32_t fvt = (uint32_t)((4 * g + (col >> 2)) * VP + 8 * (col & 3));

  // Consume the tile of one step; `refill` is called once every read of the
  // tile has returned.  (Refilling earlier -- before the P.V products, or as
  // soon as all fragments are in registers -- measured slower: 25.1 and 29.4 ms
  // against 24.5 ms on the C4 layer.)
  auto step = [&](const uint8_t* tile, uint64_t vm, auto&& refill) {
    // K fragments four ahead of their MFMAs (a ring of four registers sets)
    auto kaddr = [&](int ks) { return ks < KSV ? tile + fv + 64 * ks : tile + (ks == KSV ? fr0 : fr1); };
    f32x4 a0 = f32x4{}, a1 = f32x4{};
    bf16x8 kr[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kr[ks] = *(const bf16x8*)kaddr(ks);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kc = kr[ks & 3];
      if (ks + 4 < KS) kr[ks & 3] = *(const bf16x8*)kaddr(ks + 4);
      if (ks & 1) a1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, qf[ks], a1, 0, 0, 0);
      else a0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kc, qf[ks], a0, 0, 0, 0);
    }
    // keep four K-fragment reads in flight ahead of the MFMAs
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int ks = 0; ks < KS - 4; ++ks) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    // the first eight V fragments are read while the softmax runs
    auto vread = [&](int dt) { return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(tile + fvt + 32 * dt)); };
    bf16x4 va[2][8];
#pragma unroll
    for (int d = 0; d < 8; ++d) va[0][d] = vread(d);
    const f32x4 sc = a0 + a1;
    const uint32_t vb = (uint32_t)(vm >> (4 * g));
    float z[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) z[i] = ((vb >> i) & 1u) ? sc[i] * sl2 : -__builtin_inff();
    const float mx = quad_max(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])));
    const bool bump = mx > m_run + kLazy;
    if (ballot(bump)) {
      const float alpha = bump ? __builtin_amdgcn_exp2f(m_run - mx) : 1.f;
      m_run = bump ? mx : m_run;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[dt] *= alpha;
    }
    const float mref = fmaxf(m_run, -__FLT_MAX__);
    float pe[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(z[i] - mref);
    bf16x4 pb_hi, pb_lo;
    split_bf16(pe, pb_hi, pb_lo);
    const bf16x8 pb2 = __builtin_shufflevector(pb_hi, pb_lo, 0, 1, 2, 3, 4, 5, 6, 7);
    l_run += (pe[0] + pe[1]) + (pe[2] + pe[3]);
    // eight output tiles at a time, the next eight V fragments read before this
    // group's MFMAs
#pragma unroll
    for (int q = 0; q < NDT / 8; ++q) {
      if (q + 1 < NDT / 8) {
#pragma unroll
        for (int d = 0; d < 8; ++d) va[(q + 1) & 1][d] = vread(8 * (q + 1) + d);
      } else {
        // the last group's fragments are the tile's last reads: refill once
        // they have returned, before its MFMAs
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        refill();
      }
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const bf16x8 v2 = __builtin_shufflevector(va[q & 1][d], va[q & 1][d], 0, 1, 2, 3, 0, 1, 2, 3);
        o[8 * q + d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v2, pb2, o[8 * q + d], 0, 0, 0);
      }
    }
  };

  idx_dma(0);
  if (nblk > 1) idx_dma(1);
  vm_wait<0>();
  idx_conv(0);                 // (block 1 is converted at the top of step 0)
  uint64_t vmA = 0, vmB = 0;
  row_dma(0, tiles[w][0], vmA);
  row_dma(1, tiles[w][1], vmB);
  // Per step t: wait for its rows (the next step's NLD loads stay in flight),
  // consume them, then refill the tile with step t + 2 (preceded, every fourth
  // step, by the index block two blocks ahead).  Index block m + 1 is converted
  // at the top of step 4m: its DMA, issued at step 4m - 4, is older than the
  // rows waited for there.
  for (int t = 0; t < nst; t += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tt = t + h;
      if (h == 1 && tt >= nst) break;
      vm_wait<NLD>();
      if ((tt & 3) == 0 && (tt >> 2) + 1 < nblk) idx_conv((tt >> 2) + 1);
      uint64_t& vmr = h == 0 ? vmA : vmB;
      const uint64_t vm = vmr;
      step(tiles[w][h], vm, [&] {
        if ((tt & 3) == 0 && (tt >> 2) + 2 < nblk) idx_dma((tt >> 2) + 2);
        row_dma(tt + 2, tiles[w][h], vmr);
      });
    }
  }
  vm_wait<0>();
  l_run = quad_sum(l_run);
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  float* out = p.out + (gi * kH + col) * (int64_t)DV + 4 * g;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) __builtin_nontemporal_store(o[dt] * inv, (f32x4*)(out + 16 * dt));
}

// Merge the split partials of one (query row, head) over 256 of its output
// columns: one wave, lane c holds columns 4c .. 4c + 3.  Every split's partial
// is loaded first (all loads in flight at once), then the lanes below nsplit
// form the weights exp(m_s - M) and the wave reads them back one split at a
// time.
constexpr int kMaxSplit = kMaxTopk / 64;    // splits hold at least 64 positions
constexpr int kCombineCols = 256;           // output columns per combine wave
__global__ __launch_bounds__(64) void sa_combine_kernel(SAParams p) {
  const int parts = p.d_v / kCombineCols;
  const int part = (int)(blockIdx.x % parts);
  const int64_t rh = blockIdx.x / parts;     // (query row, head)
  const int h = (int)(rh % p.heads);
  const int64_t gi = rh / p.heads;
  const int lane = threadIdx.x;
  const float* ml = p.ws_ml + (gi * p.nsplit * p.heads + h) * 2;   // split stride: heads * 2
  const float* po = p.ws_o + (gi * p.nsplit * p.heads + h) * (int64_t)p.d_v + kCombineCols * part + 4 * lane;
  const int64_t sstride = (int64_t)p.heads * p.d_v;
  f32x4 v[kMaxSplit];
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) v[sp] = sp < p.nsplit ? *(const f32x4*)(po + sp * sstride) : f32x4{};
  const float ms = lane < p.nsplit ? ml[(int64_t)lane * p.heads * 2] : -__builtin_inff();
  const float ls = lane < p.nsplit ? ml[(int64_t)lane * p.heads * 2 + 1] : 0.f;
  const float M = wave_max(ms);
  const float w = (ms == -__builtin_inff()) ? 0.f : __expf(ms - M);
  const float L = wave_sum(w * ls);
  f32x4 acc = f32x4{};
#pragma unroll
  for (int sp = 0; sp < kMaxSplit; ++sp) {
    if (sp < p.nsplit) {
      const float wsp = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(w), sp));
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = fmaf(wsp, v[sp][i], acc[i]);
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  *(f32x4*)(p.out + (gi * p.heads + h) * (int64_t)p.d_v + kCombineCols * part + 4 * lane) = acc * inv;
}

bool mla_ok(const dsa_sparse_attn_args& a) {
  // (one batch's latent rows are addressed with 32-bit byte offsets)
  return a.dtype == DSA_BF16 && a.heads == kH && a.kv_heads == 1 && a.d_qk == 576 &&
         a.d_v == 512 && a.v == nullptr && (int64_t)a.n_k * a.d_qk * 2 < ((int64_t)1 << 31);
}

// Row counts from which the one-wave-per-row kernel runs (one split per row):
// at 1024 rows its 256 workgroups give every CU one.
constexpr int64_t kWaveRows = 1024;

int pick_nsplit(const dsa_sparse_attn_args& a) {
  const int64_t rows = (int64_t)a.batch * a.n_q;
  if (rows >= kWaveRows) return 1;
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
    if (rows >= kWaveRows) {
      hipLaunchKernelGGL((sa_mla1_kernel<576, 512>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p, rows);
      return hipGetLastError();
    }
    if (p.nsplit > 1) {
      p.ws_o = (float*)ws;
      p.ws_ml = p.ws_o + rows * p.nsplit * a.heads * (int64_t)a.d_v;
    }
    dim3 grid((unsigned)(rows * p.nsplit));
    hipLaunchKernelGGL((sa_mla4_kernel<576, 512>), grid, dim3(256), 0, s, p);
    if (p.nsplit > 1) {
      hipLaunchKernelGGL(sa_combine_kernel, dim3((unsigned)(rows * a.heads * (a.d_v / kCombineCols))), dim3(64), 0,
                         s, p);
    }
    return hipGetLastError();
  }
  const size_t lds = ((size_t)a.d_qk + a.topk) * sizeof(float);
  dim3 grid((unsigned)((int64_t)a.batch * a.n_q * a.heads));
  hipLaunchKernelGGL(sa_generic_kernel, grid, dim3(256), lds, s, p);
  return hipGetLastError();
}

}  // namespace dsa_host
