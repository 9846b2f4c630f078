// Training-aware IndexCache: the indexer-side multi-layer distillation loss
// over the selected Top-k and its backward.
//
//   [IC-SUMMARY] §3.2 (the retained layer's indexer is distilled towards every
//   layer that uses its index set; Proposition 1; the KL is taken over the
//   selected top-k tokens in sparse training); [DSA-NOTES] §5.1-5.2 (L_multi =
//   (1/r) sum_j KL(p^(j) || softmax(z)), the average target p_bar), §7.1-7.3
//   (delta = dL/dz = pi - p_bar; dL/dq_j = sum_s delta_s w_j 1[q_j.k_s > 0] k_s;
//   dL/dk_s = delta_s q, summed over heads).
//
// One workgroup of four waves per query row; wave w owns heads [16w, 16w+16).
// Per step of 16 index entries the workgroup gathers the 16 selected key rows
// (256 threads x 16 bytes) into an LDS tile, double-buffered, one barrier per
// step.  Every wave forms, from the same key and q fragments, both
//     D   = q . K^T  (16 heads x 16 keys; lane = key, 4 heads in registers)
//     D^T = K . q^T  (16 keys x 16 heads; lane = head, 4 keys in registers)
// with v_mfma_f32_16x16x32_bf16 over the 128-wide rows (4 K steps).
//   pass 1: z_e = sum_j w_j ReLU(D_je): four in-lane FMAs and a lane-swap sum
//           over the wave's four head groups give each wave's partial; after the
//           next step's barrier wave 0 sums the four partials in a fixed order
//           (loss, delta, dq and dw do not depend on the order the waves run in).
//   softmax over the row's valid entries, the loss against the r teachers and
//           delta_e = pi_e * sum(p_bar) - p_bar_e (LDS, block reductions).
//   pass 2: G_je = delta_e w_j 1[D_je > 0] in both layouts (bf16 hi + lo parts,
//           so the products keep ~2^-17 relative accuracy):
//           dq^T += K^T . G^T  (v_mfma_f32_16x16x16bf16_1k; K^T from a
//                               transposing LDS read of the key tile, G^T is
//                               the D^T accumulator layout as it stands)
//           dk    = G . q      (each wave writes its heads' G, in the D layout,
//                               to an LDS tile of all 64 heads; one step later,
//                               after the next barrier, wave w forms dk for
//                               columns [32w, 32w+32) over every head -- G in
//                               the D layout is the A operand as it stands --
//                               and adds it to dk with one global float atomic
//                               per (key, dim): dk accumulates over query rows
//                               in an order that varies between calls)
//           dw_j += sum_e delta_e ReLU(D_je).
#include "common.hpp"

namespace {

using namespace dsa;

constexpr int kKeys = 16;                   // index entries per step
constexpr int kD = 128;                     // indexer key width (bf16)
constexpr int kPitch = kD * 2 + 32;         // LDS key-row pitch in bytes (bank spread for transposed reads)
constexpr int kMaxTopk = DSA_MAX_TOPK;
constexpr int kMaxTeachers = 8;

struct DistillParams {
  int32_t batch, n_q, n_k, heads, topk, r;
  int64_t q_pos0;
  const __bf16* q;          // [batch, n_q, heads, 128]
  const __bf16* k;          // [batch, n_k, 128], batch stride k_bs
  int64_t k_bs;
  const float* w;           // [batch, n_q, heads]
  const int32_t* idx;       // [batch, n_q, topk]
  const float* teachers;    // [r, batch, n_q, topk]
  float* loss;              // [batch, n_q]
  float* delta;             // [batch, n_q, topk]
  float* dq;                // [batch, n_q, heads, 128]
  float* dw;                // [batch, n_q, heads]
  float* dk;                // [batch, n_k, 128]
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// sum over lanes l, l^16, l^32, l^48 (the four lanes of one column in the
// 16x16 MFMA layouts)
__device__ __forceinline__ float quad_sum(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// four fp32 values as bf16 hi + lo parts (hi = bf16(x), lo = bf16(x - hi))
__device__ __forceinline__ void split4(const float (&x)[4], bf16x4& hi, bf16x4& lo) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const bf16x2v h = __builtin_convertvector((f32x2v){x[2 * j], x[2 * j + 1]}, bf16x2v);
    const uint32_t hb = __builtin_bit_cast(uint32_t, h);
    const float h0 = __uint_as_float(hb << 16), h1 = __uint_as_float(hb & 0xffff0000u);
    const bf16x2v l = __builtin_convertvector((f32x2v){x[2 * j] - h0, x[2 * j + 1] - h1}, bf16x2v);
    hi[2 * j] = h[0]; hi[2 * j + 1] = h[1];
    lo[2 * j] = l[0]; lo[2 * j + 1] = l[1];
  }
}

__device__ float block_sum(float v, float* sh) {
  const int lane = threadIdx.x & 63, wid = wave_id();
  v = wave_sum(v);
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  const float r = (sh[0] + sh[1]) + (sh[2] + sh[3]);
  __syncthreads();
  return r;
}
__device__ float block_max(float v, float* sh) {
  const int lane = threadIdx.x & 63, wid = wave_id();
  v = wave_max(v);
  if (lane == 0) sh[wid] = v;
  __syncthreads();
  const float r = fmaxf(fmaxf(sh[0], sh[1]), fmaxf(sh[2], sh[3]));
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(256, 4) void distill_kernel(DistillParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t tile[2][kKeys * kPitch];
  __shared__ float zpart[2][4][kKeys];        // the waves' partial scores of two steps (pass 1)
  // G of two consecutive steps (pass 2): [2][hi, lo][16 keys][64 heads] bf16
  __shared__ __attribute__((aligned(16))) __bf16 gx[2][2][kKeys * 64];
  __shared__ __attribute__((aligned(16))) float zd[kMaxTopk];   // z, then delta, per index entry
  __shared__ int32_t sidx[kMaxTopk];          // the row's index entries (-1 where nothing is selected)
  __shared__ float red[8];

  const int lane = threadIdx.x & 63, w = wave_id();
  const int g = lane >> 4, col = lane & 15;
  const int64_t gi = blockIdx.x;                         // flattened (batch, query row)
  const int b = (int)(gi / p.n_q);
  const int64_t t = p.q_pos0 + gi % p.n_q;
  const int lim = (int)(t < p.n_k - 1 ? t : p.n_k - 1);  // last candidate position
  const int topk = p.topk;
  const int nsteps = (topk + kKeys - 1) / kKeys;
  const int h0 = 16 * w;                                 // this wave's first head
  const bool hv = h0 + col < p.heads;                    // head of this lane's column valid

  // the row's index entries; entries that select nothing become -1
  for (int e = threadIdx.x; e < nsteps * kKeys; e += 256) {
    int32_t s = e < topk ? p.idx[gi * topk + e] : -1;
    sidx[e] = (s >= 0 && s <= lim) ? s : -1;
  }

  // q fragments: lane holds head h0+col, columns 32 ks + 8 g .. + 8 (A of D, B of D^T)
  bf16x8 qf[4];
  {
    const __bf16* qr = p.q + ((gi * p.heads) + (hv ? h0 + col : 0)) * (int64_t)kD;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = hv ? *(const bf16x8*)(qr + 32 * ks + 8 * g) : bf16x8{};
  }
  // q as the B operand of G . q for this wave's columns: lane holds column
  // 32 w + 16 nt + col, heads 16 kk + 4 g .. + 4
  bf16x4 qb[4][2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 16 * kk + 4 * g + i;
        qb[kk][nt][i] = h < p.heads ? p.q[((gi * p.heads) + h) * (int64_t)kD + 32 * w + 16 * nt + col] : (__bf16)0.f;
      }
    }
  }
  // head weights: wc for the D^T layout (head h0+col), wr[i] for the D layout (heads h0+4g+i)
  const float wc = hv ? p.w[gi * p.heads + h0 + col] : 0.f;
  float wr[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int h = h0 + 4 * g + i;
    wr[i] = h < p.heads ? p.w[gi * p.heads + h] : 0.f;
  }
  __syncthreads();

  // key-tile gather: thread (row = tid / 16, chunk = tid % 16) moves 16 bytes
  const __bf16* kb = p.k + (int64_t)b * p.k_bs;
  const int trow = threadIdx.x >> 4, tch = threadIdx.x & 15;
  auto gload = [&](int st) -> i32x4 {
    const int e = st * kKeys + trow;
    const int32_t s = e < nsteps * kKeys ? sidx[e] : -1;
    return s >= 0 ? *(const i32x4*)(kb + (int64_t)s * kD + 8 * tch) : i32x4{};
  };
  auto gstore = [&](int buf, const i32x4& v) { *(i32x4*)(tile[buf] + trow * kPitch + 16 * tch) = v; };
  auto kfrag = [&](int buf, int ks) -> bf16x8 {
    return *(const bf16x8*)(tile[buf] + col * kPitch + (32 * ks + 8 * g) * 2);
  };

  // ---------------- pass 1: z
  {
    i32x4 nxt = gload(0);
    gstore(0, nxt);
    nxt = gload(1);
    // z of step st from the four partials (fixed order), after the next barrier
    auto zsum = [&](int st) {
      if (w == 0 && lane < kKeys) {
        const float* zp = &zpart[st & 1][0][0];
        zd[st * kKeys + lane] = ((zp[lane] + zp[kKeys + lane]) + zp[2 * kKeys + lane]) + zp[3 * kKeys + lane];
      }
    };
    for (int st = 0; st < nsteps; ++st) {
      sync_lds_barrier();
      const int buf = st & 1;
      if (st > 0) zsum(st - 1);
      if (st + 1 < nsteps) gstore(buf ^ 1, nxt);
      if (st + 2 < nsteps) nxt = gload(st + 2);
      f32x4 d = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kfrag(buf, ks), d, 0, 0, 0);
      // lane (g, col): key col, heads h0 + 4g + i
      float zp = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) zp = fmaf(wr[i], fmaxf(d[i], 0.f), zp);
      zp = quad_sum(zp);
      if (g == 0) zpart[st & 1][w][col] = zp;
    }
    sync_lds_barrier();
    zsum(nsteps - 1);
  }
  __syncthreads();

  // ---------------- softmax, loss, delta
  constexpr int PER = kMaxTopk / 256;
  float zv[PER];
  float mx = -__builtin_inff();
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x + 256 * j;
    zv[j] = (e < topk && sidx[e] >= 0) ? zd[e] : -__builtin_inff();
    mx = fmaxf(mx, zv[j]);
  }
  mx = block_max(mx, red);
  float se = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) se += zv[j] == -__builtin_inff() ? 0.f : __expf(zv[j] - mx);
  se = block_sum(se, red);
  const float lse = mx + __logf(se);
  const int r = p.r;
  const float inv_r = 1.f / (float)r;
  float pbar[PER], lossp = 0.f, psum = 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x + 256 * j;
    pbar[j] = 0.f;
    if (zv[j] == -__builtin_inff()) continue;
    const float logpi = zv[j] - lse;
    for (int l = 0; l < r; ++l) {
      const float pl = p.teachers[((int64_t)l * p.batch * p.n_q + gi) * topk + e];
      pbar[j] += pl;
      if (pl > 0.f) lossp += pl * (__logf(pl) - logpi);
    }
    pbar[j] *= inv_r;
    psum += pbar[j];
  }
  lossp = block_sum(lossp, red) * inv_r;
  psum = block_sum(psum, red);
  if (threadIdx.x == 0) p.loss[gi] = mx == -__builtin_inff() ? 0.f : lossp;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int e = threadIdx.x + 256 * j;
    const float dl = zv[j] == -__builtin_inff() ? 0.f : __expf(zv[j] - lse) * psum - pbar[j];
    if (e < nsteps * kKeys) zd[e] = dl;
    if (e < topk) p.delta[gi * topk + e] = dl;
  }
  __syncthreads();

  // ---------------- pass 2: dq, dw, dk
  f32x4 dqa[8];
#pragma unroll
  for (int nt = 0; nt < 8; ++nt) dqa[nt] = f32x4{};
  float dwa = 0.f;
  float* dkb = p.dk + (int64_t)b * p.n_k * kD;
  const uint8_t* rb = nullptr;
  // dk rows of step st from the G tile in gx[st & 1]: wave w, columns 32 w ..;
  // lane (g, col): column 32 w + 16 nt + col, keys 4 g .. 4 g + 3
  auto dk_step = [&](int st) {
    const __bf16* gh = gx[st & 1][0];
    const __bf16* gl = gx[st & 1][1];
    f32x4 o[2] = {f32x4{}, f32x4{}};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x4 ah = *(const bf16x4*)(gh + col * 64 + 16 * kk + 4 * g);
      const bf16x4 al = *(const bf16x4*)(gl + col * 64 + 16 * kk + 4 * g);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ah, qb[kk][nt], o[nt], 0, 0, 0);
        o[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(al, qb[kk][nt], o[nt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int s = sidx[st * kKeys + 4 * g + i];
      if (s < 0) continue;
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        if (o[nt][i] != 0.f) atomicAdd(&dkb[(int64_t)s * kD + 32 * w + 16 * nt + col], o[nt][i]);
    }
  };
  {
    i32x4 nxt = gload(0);
    gstore(0, nxt);
    nxt = gload(1);
    for (int st = 0; st < nsteps; ++st) {
      sync_lds_barrier();
      const int buf = st & 1;
      // every wave's G of the previous step is in LDS now
      if (st > 0) dk_step(st - 1);
      if (st + 1 < nsteps) gstore(buf ^ 1, nxt);
      if (st + 2 < nsteps) nxt = gload(st + 2);
      f32x4 d = f32x4{}, dt = f32x4{};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 kf = kfrag(buf, ks);
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qf[ks], kf, d, 0, 0, 0);    // lane = key col, heads 4g+i
        dt = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], dt, 0, 0, 0);  // lane = head col, keys 4g+i
      }
      const int e0 = st * kKeys;
      const f32x4 dl4 = *(const f32x4*)&zd[e0 + 4 * g];   // delta of keys 4g .. 4g+3
      const float dlc = zd[e0 + col];                      // delta of key col
      // G^T (lane = head col) and G (lane = key col): delta_key * w_head * 1[D > 0]; dw partial
      float gt[4], gk[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        gt[i] = dt[i] > 0.f ? dl4[i] * wc : 0.f;
        dwa = fmaf(dl4[i], fmaxf(dt[i], 0.f), dwa);
        gk[i] = d[i] > 0.f ? dlc * wr[i] : 0.f;
      }
      bf16x4 gth, gtl, gkh, gkl;
      split4(gt, gth, gtl);
      split4(gk, gkh, gkl);
      // G rows for the dk step: key col, heads h0 + 4 g .. + 4
      *(bf16x4*)(gx[buf][0] + col * 64 + h0 + 4 * g) = gkh;
      *(bf16x4*)(gx[buf][1] + col * 64 + h0 + 4 * g) = gkl;
      // dq^T[16 nt + col-row][head] += K^T . G^T
      rb = tile[buf] + (4 * g + (col >> 2)) * kPitch + 8 * (col & 3);
#pragma unroll
      for (int nt = 0; nt < 8; ++nt) {
        const bf16x4 ka = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(rb + 32 * nt));
        dqa[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, gth, dqa[nt], 0, 0, 0);
        dqa[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ka, gtl, dqa[nt], 0, 0, 0);
      }
    }
    sync_lds_barrier();
    dk_step(nsteps - 1);
  }
  // dq^T layout: lane (g, col): head h0 + col, dims 16 nt + 4 g + i
  if (hv) {
    float* dqr = p.dq + ((gi * p.heads) + h0 + col) * (int64_t)kD;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) *(f32x4*)(dqr + 16 * nt + 4 * g) = dqa[nt];
  }
  dwa = quad_sum(dwa);
  if (hv && g == 0) p.dw[gi * p.heads + h0 + col] = dwa;
}

__global__ void zero_f32_kernel(float* p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

}  // namespace

namespace dsa_host {

bool distill_supported(const dsa_indexer_args& a, int32_t topk, int32_t r) {
  return a.dtype == DSA_BF16 && a.dim == kD && a.heads >= 1 && a.heads <= 64 && topk >= 1 && topk <= kMaxTopk &&
         r >= 1 && r <= kMaxTeachers;
}

hipError_t distill_launch(const dsa_indexer_args& a, int32_t topk, int32_t r, const int32_t* idx,
                          const float* teachers, float* loss, float* delta, float* dq, float* dw, float* dk,
                          hipStream_t s) {
  DistillParams p{};
  p.batch = a.batch; p.n_q = a.n_q; p.n_k = a.n_k; p.heads = a.heads; p.topk = topk; p.r = r;
  p.q_pos0 = a.q_pos0;
  p.q = (const __bf16*)a.q;
  p.k = (const __bf16*)a.k;
  p.k_bs = a.k_batch_stride ? a.k_batch_stride : (int64_t)a.n_k * a.dim;
  p.w = a.w;
  p.idx = idx; p.teachers = teachers;
  p.loss = loss; p.delta = delta; p.dq = dq; p.dw = dw; p.dk = dk;
  const int64_t ndk = (int64_t)a.batch * a.n_k * kD;
  hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)((ndk + 255) / 256)), dim3(256), 0, s, dk, ndk);
  // rows with fewer heads than 64 still run four waves (the spare waves hold zero heads)
  hipLaunchKernelGGL(distill_kernel, dim3((unsigned)((int64_t)a.batch * a.n_q)), dim3(256), 0, s, p);
  return hipGetLastError();
}

}  // namespace dsa_host
