// Lightning-indexer kernels for gfx950 ([DSA-NOTES] §2.1 score equation):
//     I[t, s] = sum_j w[t, j] * ReLU(q[t, j, :] . k[s, :]),  s = 0..t
//
//  * indexer_f32_kernel   fp32 inputs, plain VALU dot products (small/debug shapes).
//  * ix_tile_kernel       bf16 / fp8-e4m3 inputs on MFMA.  One wave owns one query
//    row: its q (heads x dim) stays in registers as the MFMA A operand (heads are
//    the M dimension, 32 per tile), 64-key tiles of k are staged once per
//    workgroup in LDS and read as the B operand.  The epilogue applies ReLU and
//    the head weights in registers and reduces over heads inside each lane (the
//    32x32 MFMA output puts 16 head rows of one key column in each lane), then
//    across the two half-waves, leaving one score per lane per 64-key tile.
//      MODE_SCORES writes the scores (debug / inspection path).
//      MODE_TOPK never writes them: each wave keeps a candidate buffer in LDS,
//      filtered by the running k-th key, compacted by a wave-level radix select
//      when full.  Candidates arrive in position order and compaction is
//      stable, so the kept set stays in ascending position order and ties are
//      broken toward the lower position with no extra sort.
//  * ix_scan_kernel       decode shape (few query rows, long key range): keys are
//    split over many workgroups, B operands come straight from HBM in 128-byte
//    rows, fp32 scores go to a workspace row for the multi-workgroup select.
//
// fp8: q = q_scale[t, j] * code, k = k_scale[s] * code with positive scales, so
// w_j * ReLU(q_j . k) = k_scale[s] * (w_j * q_scale[t, j]) * ReLU(code_q . code_k):
// the MFMA runs on raw e4m3 codes and both scales are applied in the epilogue.
#include "common.hpp"

namespace {

using namespace dsa;

enum { DT_BF16 = 1, DT_FP8 = 2 };
enum { MODE_SCORES = 0, MODE_TOPK = 1 };

constexpr int kTileKeys = 64;
constexpr int kRowsPerBlock = 4;       // scores kernel: one query row per wave
// fused kernel: one query row per wave, kTopkWaves rows per workgroup
constexpr int kTopkWaves = 4;
constexpr int kTopkThreads = 64 * kTopkWaves;
constexpr int kTopkBlocksPerCu = 8 / kTopkWaves;   // two waves per SIMD

struct IxParams {
  const void* q;
  const float* q_scale;
  const void* k;
  int64_t k_bs;          // elements between batches of k
  const float* k_scale;
  int64_t ks_bs;
  const float* w;
  int32_t batch, n_q, n_k, heads;
  int64_t q_pos0;
  int64_t row0, rows;    // query rows handled (scores mode: a window)
  float* out;            // scores [batch, rows, n_k]
  int32_t* idx;          // [batch, n_q, topk]
  int32_t topk;
  uint32_t* hist;        // decode scan: per-row key histograms (or null)
  int64_t hist_rw;       // u32 words between the histograms of consecutive rows
};

// ---------------------------------------------------------------- fp32 path
__global__ __launch_bounds__(256) void indexer_f32_kernel(IxParams p, int dim, int64_t out_rs) {
  extern __shared__ float qs[];                 // heads * dim (+ heads weights)
  const int64_t rr = blockIdx.y;                // row within the window
  const int b = blockIdx.z;
  const int64_t i = p.row0 + rr;
  const int64_t t = p.q_pos0 + i;
  const float* q = (const float*)p.q + ((int64_t)b * p.n_q + i) * p.heads * dim;
  const float* w = p.w + ((int64_t)b * p.n_q + i) * p.heads;
  float* wsh = qs + p.heads * dim;
  for (int x = threadIdx.x; x < p.heads * dim; x += blockDim.x) qs[x] = q[x];
  for (int x = threadIdx.x; x < p.heads; x += blockDim.x) wsh[x] = w[x];
  __syncthreads();
  const int64_t s = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= p.n_k) return;
  float* out = p.out + ((int64_t)b * p.rows + rr) * out_rs;
  if (s > t) { out[s] = -__builtin_inff(); return; }
  const float* kr = (const float*)p.k + b * p.k_bs + s * dim;
  float acc = 0.f;
  for (int j = 0; j < p.heads; ++j) {
    float d = 0.f;
    for (int c = 0; c < dim; ++c) d = fmaf(qs[j * dim + c], kr[c], d);
    acc = fmaf(wsh[j], fmaxf(d, 0.f), acc);
  }
  out[s] = acc + 0.0f;
}

// ---------------------------------------------------------------- MFMA tiles
template <int DT, int D, int TK = kTileKeys>
struct Cfg {
  static constexpr int ES = DT == DT_BF16 ? 2 : 1;          // element size
  static constexpr int ROWB = D * ES;                        // bytes per key row
  static constexpr int PITCH = ROWB + 16;                    // LDS row pitch (bank spread)
  static constexpr int KSTEP = DT == DT_BF16 ? 16 : 64;      // MFMA K per instruction
  static constexpr int NKS = D / KSTEP;
  static constexpr int CPR = ROWB / 16;                      // 16-byte chunks per row
  static constexpr int TILE_CHUNKS = TK * CPR;
  static constexpr int NCH = TILE_CHUNKS / 256;              // chunks per thread
  static constexpr int TILE_BYTES = TK * PITCH;
  // staged tile of the fused kernel: the rows, then (fp8) the TK key scales
  static constexpr int BUF_BYTES = TILE_BYTES + (DT == DT_FP8 ? TK * 4 : 0);
};

template <int DT>
struct AFrag;
template <>
struct AFrag<DT_BF16> { typedef bf16x8 T; };
template <>
struct AFrag<DT_FP8> { typedef i32x8 T; };

template <int DT>
__device__ __forceinline__ f32x16 mfma(const typename AFrag<DT>::T& a, const typename AFrag<DT>::T& b,
                                       f32x16 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
  }
}

// Load this lane's K-slice of one operand row: for bf16, 8 elements starting at
// element 16*ks + 8*(lane/32); for fp8, 32 bytes starting at 64*ks + 32*(lane/32).
// The same slice map is used for q (A) and k (B), so each dot product covers
// every element of the row exactly once.
template <int DT>
__device__ __forceinline__ typename AFrag<DT>::T load_frag(const uint8_t* rowp, int ks, int lane) {
  if constexpr (DT == DT_BF16) {
    return *(const bf16x8*)(rowp + (16 * ks + 8 * (lane >> 5)) * 2);
  } else {
    const i32x4* p = (const i32x4*)(rowp + 64 * ks + 32 * (lane >> 5));
    i32x4 lo = p[0], hi = p[1];
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
}

template <int DT, int D, int HT>
struct RowState {
  typename AFrag<DT>::T a[HT][Cfg<DT, D>::NKS];
  float c[HT][16];
};

// q fragments and per-(row, head) epilogue weights of query row `gi` (flattened
// batch*n_q index).  Heads >= H are zero rows with zero weight.  FLAT issues
// every load unconditionally (heads past H read head 0 and are zeroed
// afterwards), so they are all in flight together and waited for once: the
// decode scan, whose workgroups score only a few thousand keys per row, cannot
// afford one memory latency per weight.  The fused kernel, at its register limit,
// keeps the conditional loads (one row per few hundred thousand MFMAs).
template <int DT, int D, int HT, bool FLAT = false>
__device__ __forceinline__ void load_row(const IxParams& p, int64_t gi, int lane,
                                         RowState<DT, D, HT>& rs) {
  typedef Cfg<DT, D> C;
  typedef typename AFrag<DT>::T F;
  const uint8_t* qb = (const uint8_t*)p.q;
  if constexpr (FLAT) {
    float wv[HT][16], sv[HT][16];
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      const int head = 32 * h + (lane & 31);
      const uint8_t* rowp = qb + ((gi * p.heads + (head < p.heads ? head : 0)) * (int64_t)D) * C::ES;
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) rs.a[h][ks] = load_frag<DT>(rowp, ks, lane);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = 32 * h + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        const int64_t o = gi * p.heads + (hh < p.heads ? hh : 0);
        wv[h][i] = p.w[o];
        if constexpr (DT == DT_FP8) sv[h][i] = p.q_scale[o];
      }
    }
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      if (32 * h + (lane & 31) >= p.heads) {
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) rs.a[h][ks] = F{};
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = 32 * h + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        float cv = wv[h][i];
        if constexpr (DT == DT_FP8) cv *= sv[h][i];
        rs.c[h][i] = hh < p.heads ? cv : 0.f;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < HT; ++h) {
      const int head = 32 * h + (lane & 31);
      if (head < p.heads) {
        const uint8_t* rowp = qb + ((gi * p.heads + head) * (int64_t)D) * C::ES;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) rs.a[h][ks] = load_frag<DT>(rowp, ks, lane);
      } else {
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) rs.a[h][ks] = F{};
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = 32 * h + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        float cv = 0.f;
        if (hh < p.heads) {
          cv = p.w[gi * p.heads + hh];
          if constexpr (DT == DT_FP8) cv *= p.q_scale[gi * p.heads + hh];
        }
        rs.c[h][i] = cv;
      }
    }
  }
}

// Consume the row's q fragments and weights in an empty asm statement so their
// loads are waited for once here; otherwise the wait-count pass treats them as
// possibly in flight on every iteration of the tile loop and drains the tile
// prefetch along with them.
template <int DT, int D, int HT>
__device__ __forceinline__ void settle_row(RowState<DT, D, HT>& rs) {
#pragma unroll
  for (int h = 0; h < HT; ++h) {
#pragma unroll
    for (int ks = 0; ks < Cfg<DT, D>::NKS; ++ks) asm volatile("" : "+v"(rs.a[h][ks]));
#pragma unroll
    for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(rs.c[h][i]));
  }
}

// Scores of keys [s0, s0+64) for the wave's row; lane l gets key s0 + l.
// kt: LDS tile (PITCH-byte rows) or, when kt_global, the k row of key s0.
template <int DT, int D, int HT>
__device__ __forceinline__ float tile_scores(const RowState<DT, D, HT>& rs, const uint8_t* kt,
                                             int pitch, int lane) {
  typedef Cfg<DT, D> C;
  // Two 32-key subtiles, one after the other: the head-sum epilogue of the
  // first overlaps the MFMAs of the second and only 16*HT accumulators live.
  float part[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    f32x16 acc[HT];
#pragma unroll
    for (int h = 0; h < HT; ++h) acc[h] = f32x16{};
    const uint8_t* rowp = kt + (32 * n + (lane & 31)) * pitch;
    // B fragments are read one K step ahead of the MFMAs that consume them.
    typename AFrag<DT>::T bf = load_frag<DT>(rowp, 0, lane);
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      typename AFrag<DT>::T nxt = bf;
      if (ks + 1 < C::NKS) nxt = load_frag<DT>(rowp, ks + 1, lane);
#pragma unroll
      for (int h = 0; h < HT; ++h) acc[h] = mfma<DT>(rs.a[h][ks], bf, acc[h]);
      bf = nxt;
    }
    // 32x32 output: lane l holds column (key) l%32 and rows 8*(i/4) + 4*(l/32) + i%4.
    float pp = 0.f;
#pragma unroll
    for (int h = 0; h < HT; ++h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pp = fmaf(rs.c[h][i], fmaxf(acc[h][i], 0.f), pp);
    }
    part[n] = pp;
  }
  // lanes l and l^32 hold complementary head rows of the same key column:
  // lanes 0-31 finish keys 0-31 (subtile 0), lanes 32-63 keys 32-63 (subtile 1).
  // v_permlane32_swap(x = part[0], y = part[1]) exchanges the upper half of x
  // with the lower half of y: afterwards x holds subtile 0's partials of lanes
  // 0-31 in both halves, y subtile 1's partials of lanes 32-63 in both halves.
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[1]),
                                                   false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Scores of NG consecutive 64-key groups of an LDS tile (PITCH-byte rows):
// sc[g] of lane l is key 64 g + l.  The 32-key subtiles run one after the
// other, so each subtile's head-sum epilogue can overlap the next one's MFMAs
// (only the last subtile's epilogue is left without MFMAs to hide under).
template <int DT, int D, int HT, int NG>
__device__ __forceinline__ void tile_scores_multi(const RowState<DT, D, HT>& rs, const uint8_t* kt, int lane,
                                                  float (&sc)[NG]) {
  typedef Cfg<DT, D> C;
  float part[2 * NG];
#pragma unroll
  for (int n = 0; n < 2 * NG; ++n) {
    f32x16 acc[HT];
#pragma unroll
    for (int h = 0; h < HT; ++h) acc[h] = f32x16{};
    const uint8_t* rowp = kt + (32 * n + (lane & 31)) * C::PITCH;
    typename AFrag<DT>::T bf = load_frag<DT>(rowp, 0, lane);
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      typename AFrag<DT>::T nxt = bf;
      if (ks + 1 < C::NKS) nxt = load_frag<DT>(rowp, ks + 1, lane);
#pragma unroll
      for (int h = 0; h < HT; ++h) acc[h] = mfma<DT>(rs.a[h][ks], bf, acc[h]);
      bf = nxt;
    }
    float pp = 0.f;
#pragma unroll
    for (int h = 0; h < HT; ++h) {
#pragma unroll
      for (int i = 0; i < 16; ++i) pp = fmaf(rs.c[h][i], fmaxf(acc[h][i], 0.f), pp);
    }
    part[n] = pp;
  }
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[2 * g]), __float_as_uint(part[2 * g + 1]),
                                                     false, false);
    sc[g] = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
}

// Half-wave combine of the two 32-key subtiles' partials (lanes l and l^32
// hold complementary head rows of the same key column): lane l ends with key l.
__device__ __forceinline__ float combine_halves(float p0, float p1) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Cooperative 256-thread copy of the 64-key tile `tile` into registers, then LDS
// (rows of PITCH bytes).  Keys at or past n_k read as zero.
template <int DT, int D>
__device__ __forceinline__ void load_ktile(const uint8_t* kbase, int64_t n_k, int tile,
                                           i32x4 (&pre)[Cfg<DT, D>::NCH]) {
  typedef Cfg<DT, D> C;
#pragma unroll
  for (int j = 0; j < C::NCH; ++j) {
    const int c = threadIdx.x + 256 * j;
    const int key = c / C::CPR, part = c % C::CPR;
    const int64_t s = (int64_t)tile * kTileKeys + key;
    pre[j] = s < n_k ? *(const i32x4*)(kbase + s * C::ROWB + part * 16) : i32x4{};
  }
}
template <int DT, int D>
__device__ __forceinline__ void store_ktile(uint8_t* dst, const i32x4 (&pre)[Cfg<DT, D>::NCH]) {
  typedef Cfg<DT, D> C;
#pragma unroll
  for (int j = 0; j < C::NCH; ++j) {
    const int c = threadIdx.x + 256 * j;
    const int key = c / C::CPR, part = c % C::CPR;
    *(i32x4*)(&dst[key * C::PITCH + part * 16]) = pre[j];
  }
}


// Workgroup barrier without the fence of __syncthreads (whose release would
// wait for every load in flight, including the next tiles' staging): LDS
// accesses before it have completed (lgkmcnt), the asm keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct HBM -> LDS staging of TK-key tiles (buffer_load ... lds).  Lane l of
// one such load writes LDS bytes [base + 16 l, base + 16 l + 16), so 64 rows of
// PITCH bytes (ROWB data bytes + 16 pad bytes) are SPR = CPR + 1 loads of 64
// 16-byte slots: slot q holds part q % SPR of row q / SPR, and pad slots read
// past the buffer's end (zeros).  Load j of a tile is issued by wave j % W.
// Offsets go in the per-lane offset so that the buffer's range check covers
// them: keys at or past the end of the range read as zero.
template <int DT, int D, int W, int TK>
struct TileDma {
  typedef Cfg<DT, D, TK> C;
  static constexpr int SPR = C::CPR + 1;
  static constexpr int NG = TK / 64;                       // 64-row groups per tile
  static constexpr int NR = NG * SPR;                      // loads of rows and pads
  static constexpr int NI = NR + (DT == DT_FP8 ? NG : 0);  // + 4-byte-per-lane loads of the key scales
  static constexpr int NPW = (NI + W - 1) / W;       // loads per wave and tile, at most (W waves)
  uint32_t goff[NPW];
  int nload;                                          // loads this wave issues per tile
  int wid;
  __device__ __forceinline__ TileDma(int wid_, int lane) : wid(wid_) {
    nload = (NI - wid_ + W - 1) / W;
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
      const int q = 64 * (wid_ + W * m) + lane;
      const int row = q / SPR, part = q % SPR;
      goff[m] = part < C::CPR ? (uint32_t)(row * C::ROWB + part * 16) : 0x80000000u;
    }
  }
  // sr: the key scales (fp8), as a buffer of floats
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, __amdgpu_buffer_rsrc_t sr, int tile,
                                       uint8_t* dst, int lane) const {
    const uint32_t toff = (uint32_t)tile * (TK * C::ROWB);
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
      const int j = wid + W * m;
      if (j < NR) {
        lds_dma<16>(r, dst + j * 1024, goff[m] + toff);
      } else if (DT == DT_FP8 && j < NI) {
        const int g = j - NR;
        lds_dma<4>(sr, dst + C::TILE_BYTES + 256 * g, (uint32_t)(tile * TK + 64 * g + lane) * 4u);
      }
    }
  }
  // Wait until this wave's loads of the oldest tile in flight are done while
  // those of `younger` later tiles may still run (loads complete in issue
  // order; the wave issues NPW or NPW-1 loads per tile).
  __device__ __forceinline__ void wait_oldest(int younger) const {
    const int n = younger * (nload == NPW ? NPW : NPW - 1);
    // s_waitcnt encoding (gfx9): vmcnt in bits 3:0; expcnt and lgkmcnt at their maxima
    switch (n) {
#define DSA_VMW(c) case c: __builtin_amdgcn_s_waitcnt(0x0F70 | c); break;
      DSA_VMW(1) DSA_VMW(2) DSA_VMW(3) DSA_VMW(4) DSA_VMW(5) DSA_VMW(6) DSA_VMW(7)
      DSA_VMW(8) DSA_VMW(9) DSA_VMW(10) DSA_VMW(11) DSA_VMW(12) DSA_VMW(13) DSA_VMW(14) DSA_VMW(15)
#undef DSA_VMW
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  }
};

// ---------------------------------------------------------------- wave select
// A wave owns one query row's candidate buffer (order keys cu[], positions ci[])
// in a private slice of the workspace.  Entries are appended in position order.
__device__ __forceinline__ void lds_sync() { __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup"); }

constexpr int kCandCap = 16384;        // candidates per row before a compaction
// Rows shorter than kShortRow keys compact first at kShortFirstCap entries: their
// final select then runs over a few thousand entries instead of up to 16384.
// Longer rows keep the full first buffer (an early threshold is too loose there
// and costs extra compactions later).
constexpr int kShortRow = 32768;
constexpr int kShortFirstCap = 8192;

// Entries [j, j+4) of a candidate array in one 16-byte load.  The arrays are
// 16-byte aligned and their capacity is a multiple of 4, so a load that starts
// below n stays inside the slice (entries at or past n are ignored).
__device__ __forceinline__ u32x4 ld4(const uint32_t* p, int j) { return *(const u32x4*)(p + j); }

// The select passes stream the candidate buffer from L2 with kSelVec 16-byte
// loads in flight per lane (1024-2048 entries per wave step).  They are kept out
// of line: a call returns with its memory operations complete, whereas inlined,
// the compaction's stores would still be counted as outstanding at the top of
// the tile loop, where the compiler would then wait for every vector memory
// operation -- the tile loads in flight included -- on every tile.
constexpr int kSelVec = 8;

// Result of a radix pass: the digit holding the rem-th largest key, the rank
// of that key inside the digit's bucket and the bucket's size.  (The select
// helpers take and return values only: a reference or pointer to a local
// would put it in scratch memory, and the tile loop would then reload the
// threshold from there, behind waits for every vector memory operation.)
struct RadixPick {
  uint32_t digit, rem, bucket;
};
// One radix pass: histogram of the 8-bit digit at SHIFT among entries whose
// masked key equals `prefix`; then pick the digit holding the rem-th largest.  Full steps load without bounds checks.  The top
// byte (sign and high exponent bits) is nearly the same for every key of a row:
// that pass counts the entries whose top byte equals the first entry's in a
// register, four entries per compare, and sends only the others to LDS atomics
// (same-address LDS atomics serialise, and this code shares its SIMD with the
// MFMA stream of the other workgroup, where every instruction counts).
template <int SHIFT>
__device__ __attribute__((noinline)) RadixPick wave_radix_pass(const uint32_t* cu, int n, uint32_t prefix,
                                                               uint32_t mask, uint32_t rem, uint32_t* hist, int lane) {
  constexpr int STEP = 64 * 4 * kSelVec;
#pragma unroll
  for (int j = 0; j < 4; ++j) hist[lane * 4 + j] = 0u;
  lds_sync();
  const uint32_t d0 = SHIFT == 24 ? (uint32_t)__builtin_amdgcn_readfirstlane((int)cu[0]) >> 24 : 0u;
  const uint32_t base = d0 << 24;
  uint32_t same = 0;
  auto count = [&](const u32x4& v, int jb) {
    if constexpr (SHIFT == 24) {
      const uint32_t x = (v[0] ^ base) | (v[1] ^ base) | (v[2] ^ base) | (v[3] ^ base);
      if ((x >> 24) == 0u && jb + 4 <= n) {
        same += 4u;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (jb + e < n) {
            const uint32_t d = v[e] >> 24;
            if (d == d0) ++same;
            else atomicAdd(&hist[d], 1u);
          }
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (jb + e < n && (v[e] & mask) == prefix) atomicAdd(&hist[(v[e] >> SHIFT) & 255u], 1u);
    }
  };
  int j0 = 0;
  for (; j0 + STEP <= n; j0 += STEP) {
    u32x4 u[kSelVec];
#pragma unroll
    for (int r = 0; r < kSelVec; ++r) u[r] = ld4(cu, j0 + 4 * (r * 64 + lane));
#pragma unroll
    for (int r = 0; r < kSelVec; ++r) count(u[r], j0 + 4 * (r * 64 + lane));
  }
  if (j0 < n) {
    u32x4 u[kSelVec];
#pragma unroll
    for (int r = 0; r < kSelVec; ++r) {
      const int j = j0 + 4 * (r * 64 + lane);
      u[r] = j < n ? ld4(cu, j) : u32x4{};
    }
#pragma unroll
    for (int r = 0; r < kSelVec; ++r) count(u[r], j0 + 4 * (r * 64 + lane));
  }
  if constexpr (SHIFT == 24) {
    uint32_t tot;
    wave_excl_scan(same, &tot);
    if (lane == 0 && tot) atomicAdd(&hist[d0], tot);
  }
  lds_sync();
  // lane owns bins 255-4*lane .. 252-4*lane (descending)
  const uint32_t c0 = hist[255 - 4 * lane], c1 = hist[254 - 4 * lane];
  const uint32_t c2 = hist[253 - 4 * lane], c3 = hist[252 - 4 * lane];
  const uint32_t local = c0 + c1 + c2 + c3;
  uint32_t tot;
  const uint32_t ex = wave_excl_scan(local, &tot);
  const bool mine = ex < rem && rem <= ex + local;
  uint32_t digit = 0, nrem = 0, bsz = 0;
  if (mine) {
    uint32_t cc = ex;
    const uint32_t cs[4] = {c0, c1, c2, c3};
    for (int j = 0; j < 4; ++j) {
      if (cc + cs[j] >= rem) { digit = 255u - 4u * lane - j; nrem = rem - cc; bsz = cs[j]; break; }
      cc += cs[j];
    }
  }
  const int src = __builtin_ctzll(ballot(mine));
  RadixPick r;
  r.digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, src);
  r.rem = (uint32_t)__builtin_amdgcn_readlane((int)nrem, src);
  r.bucket = (uint32_t)__builtin_amdgcn_readlane((int)bsz, src);
  lds_sync();
  return r;
}

// Stable in-place compaction of cu/ci[0..n) keeping every entry with key >= T
// (a shrink).  Each lane takes 4 consecutive entries per block; ranks in buffer
// order come from one ballot per entry slot.  A step loads all its blocks
// before it writes, and an entry is never written past its own slot, so in
// place is safe.  Returns the number kept.
__device__ __attribute__((noinline)) int wave_keep_ge(uint32_t* cu, uint32_t* ci, int n, uint32_t T, int lane) {
  constexpr int R = kSelVec;
  int out = 0;
  for (int j0 = 0; j0 < n; j0 += 64 * 4 * R) {
    const bool full = j0 + 64 * 4 * R <= n;
    u32x4 u[R], id[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = j0 + 4 * (r * 64 + lane);
      const bool ok = full || j < n;
      u[r] = ok ? ld4(cu, j) : u32x4{};
      id[r] = ok ? ld4(ci, j) : u32x4{};
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int jb = j0 + 4 * (r * 64 + lane);
      bool keep[4];
      uint64_t km[4];
      uint32_t kb = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = (full || jb + e < n) && u[r][e] >= T;
        km[e] = ballot(keep[e]);
        kb += lanes_below(km[e]);
      }
      int d = out + (int)kb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keep[e]) {
          cu[d] = u[r][e];
          ci[d] = id[r][e];
          ++d;
        }
        out += __builtin_popcountll(km[e]);
      }
    }
  }
  lds_sync();
  return out;
}

// Stable in-place compaction of cu/ci[0..n): keeps entries with key > T plus the
// first tie_limit entries with key == T.  With out_idx set, the kept positions
// go there instead (at most `limit`).  Returns the number kept.  Same blocking
// as wave_keep_ge.
__device__ __attribute__((noinline)) int wave_keep(uint32_t* cu, uint32_t* ci, int n, uint32_t T, int64_t tie_limit, int lane,
                         int32_t* out_idx, int limit) {
  constexpr int R = kSelVec;
  int out = 0;
  int64_t eqseen = 0;
  for (int j0 = 0; j0 < n; j0 += 64 * 4 * R) {
    u32x4 u[R], id[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int j = j0 + 4 * (r * 64 + lane);
      u[r] = j < n ? ld4(cu, j) : u32x4{};
      id[r] = j < n ? ld4(ci, j) : u32x4{};
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int jb = j0 + 4 * (r * 64 + lane);
      bool tie[4], keep[4];
      uint64_t tm[4], km[4];
      uint32_t tb = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        tie[e] = jb + e < n && u[r][e] == T;
        tm[e] = ballot(tie[e]);
        tb += lanes_below(tm[e]);
      }
      int64_t trank = eqseen + tb;
      uint32_t kb = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        keep[e] = jb + e < n && (u[r][e] > T || (tie[e] && trank < tie_limit));
        trank += tie[e] ? 1 : 0;
        km[e] = ballot(keep[e]);
        kb += lanes_below(km[e]);
      }
      int d = out + (int)kb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (keep[e]) {
          if (d < limit) {
            if (out_idx) {
              out_idx[d] = (int32_t)id[r][e];
            } else {
              cu[d] = u[r][e];
              ci[d] = id[r][e];
            }
          }
          ++d;
        }
        eqseen += __builtin_popcountll(tm[e]);
        out += __builtin_popcountll(km[e]);
      }
    }
  }
  lds_sync();
  return out;
}

// Exact k-th largest key T among cu[0..n) and how many entries equal to T fit
// (T and that count in `rem`).
struct ExactPick {
  uint32_t T, req;
};
__device__ __attribute__((noinline)) ExactPick wave_select_exact(const uint32_t* cu, int n, int k, uint32_t* hist,
                                                                 int lane) {
  const RadixPick a = wave_radix_pass<24>(cu, n, 0u, 0u, (uint32_t)k, hist, lane);
  const uint32_t p1 = a.digit << 24;
  const RadixPick b = wave_radix_pass<16>(cu, n, p1, 0xFF000000u, a.rem, hist, lane);
  const uint32_t p2 = p1 | (b.digit << 16);
  const RadixPick c = wave_radix_pass<8>(cu, n, p2, 0xFFFF0000u, b.rem, hist, lane);
  const uint32_t p3 = p2 | (c.digit << 8);
  const RadixPick d = wave_radix_pass<0>(cu, n, p3, 0xFFFFFF00u, c.rem, hist, lane);
  return ExactPick{p3 | d.digit, d.rem};
}

// Shrink a full buffer while keeping every entry that can still be in the row's
// Top-k.  First try the 16-bit prefix of the k-th key (two passes): keep every
// entry at or above it; new arrivals must then be >= that prefix.  If ties or a
// crowded bucket leave the buffer too full, select exactly (k entries kept,
// arrivals must beat T strictly: a later position loses a tie).  Returns the
// entries kept, the new threshold and whether arrivals must beat it strictly.
struct Shrunk {
  int n;
  uint32_t thr;
  bool strict;
};
__device__ __forceinline__ Shrunk wave_shrink(uint32_t* cu, uint32_t* ci, int n, int k, uint32_t* hist, int lane) {
  const RadixPick a = wave_radix_pass<24>(cu, n, 0u, 0u, (uint32_t)k, hist, lane);
  const RadixPick b = wave_radix_pass<16>(cu, n, a.digit << 24, 0xFF000000u, a.rem, hist, lane);
  const uint32_t P = (a.digit << 24) | (b.digit << 16);
  const int kept = (k - (int)b.rem) + (int)b.bucket;          // entries with key >= P
  if (kept <= n - n / 4) return Shrunk{wave_keep_ge(cu, ci, n, P, lane), P, false};
  const ExactPick e = wave_select_exact(cu, n, k, hist, lane);
  return Shrunk{wave_keep(cu, ci, n, e.T, (int64_t)e.req, lane, nullptr, n), e.T, true};
}

// ---------------------------------------------------------------- prefill kernels
// Scores mode: materialise I for a window of query rows (-inf where s > t).
template <int DT, int D, int HT>
__global__ __launch_bounds__(256, 2) void ix_scores_kernel(IxParams p) {
  typedef Cfg<DT, D> C;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[2][C::TILE_BYTES];
  const int wid = wave_id(), lane = threadIdx.x & 63;
  const int b = (int)(blockIdx.x % p.batch);
  const int64_t rloc = (int64_t)(blockIdx.x / p.batch) * kRowsPerBlock + wid;
  const bool vrow = rloc < p.rows;
  const int64_t i = p.row0 + rloc;
  const int64_t t = p.q_pos0 + i;
  const int ntiles = (int)((p.n_k + kTileKeys - 1) / kTileKeys);
  const int64_t gi = (int64_t)b * p.n_q + i;
  RowState<DT, D, HT> rs;
  if (vrow) load_row<DT, D, HT>(p, gi, lane, rs);
  const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)b * p.k_bs * C::ES;
  const float* ksc = (DT == DT_FP8) ? p.k_scale + (int64_t)b * p.ks_bs : nullptr;
  i32x4 pre[C::NCH];
  load_ktile<DT, D>(kbase, p.n_k, 0, pre);
  store_ktile<DT, D>(ktile[0], pre);
  for (int it = 0; it < ntiles; ++it) {
    __syncthreads();
    if (it + 1 < ntiles) load_ktile<DT, D>(kbase, p.n_k, it + 1, pre);
    if (vrow) {
      float sc = tile_scores<DT, D, HT>(rs, &ktile[it & 1][0], C::PITCH, lane);
      const int64_t s = (int64_t)it * kTileKeys + lane;
      if (s < p.n_k) {
        if constexpr (DT == DT_FP8) sc *= ksc[s];
        float* out = p.out + ((int64_t)b * p.rows + rloc) * p.n_k;
        out[s] = s <= t ? sc + 0.0f : -__builtin_inff();
      }
    }
    if (it + 1 < ntiles) store_ktile<DT, D>(ktile[(it + 1) & 1], pre);
  }
}

// Fused INDEXER + Top-k.  Persistent: each workgroup repeatedly takes the next
// block of 4 query rows (heaviest rows first) from a device counter; blockIdx.x
// names its private candidate slice in the workspace.
template <int DT, int D, int HT>
__global__ __launch_bounds__(kTopkThreads, kTopkBlocksPerCu) void ix_topk_kernel(IxParams p, uint32_t* work,
                                                                                    uint32_t* cand) {
  // 128-key tiles where two buffers of three fit two workgroups per CU in LDS
  // (fp8 and the narrower bf16 rows); 64-key tiles for bf16 d = 128
  constexpr int TK = Cfg<DT, D, 128>::BUF_BYTES <= 24576 ? 128 : 64;
  constexpr int NG = TK / 64;
  typedef Cfg<DT, D, TK> C;
  // staging buffers (as many as fit two workgroups per CU, at most 3): tiles
  // it+1 .. it+STAGES-1 load while tile it is scored
  constexpr int STAGES = C::BUF_BYTES > 24576 ? 2 : 3;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[STAGES][C::BUF_BYTES];
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ int64_t s_item;

  const int wid = wave_id(), lane = threadIdx.x & 63;
  uint32_t* cu = cand + ((size_t)blockIdx.x * kTopkWaves + wid) * 2 * kCandCap;
  uint32_t* ci = cu + kCandCap;
  // candidate slice as a buffer: appends are 32-bit offsets (keys at [0, cap),
  // positions at [cap, 2 cap))
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(cu, 2u * kCandCap * 4u);
  const int64_t nrb = (p.rows + kTopkWaves - 1) / kTopkWaves;
  const int64_t total = nrb * p.batch;
  const int k = p.topk;
  const TileDma<DT, D, kTopkWaves, TK> td(wid, lane);

  for (;;) {
    if (threadIdx.x == 0) s_item = (int64_t)atomicAdd(work, 1u);
    __syncthreads();
    const int64_t item = s_item;
    __syncthreads();
    if (item >= total) break;
    const int b = (int)(item % p.batch);
    const int64_t rb = nrb - 1 - item / p.batch;                 // heaviest rows first
    const int64_t rloc0 = rb * kTopkWaves;
    const int64_t rloc = rloc0 + wid;
    const bool vrow = rloc < p.rows;
    const int64_t i = p.row0 + rloc;
    // positions fit in 32 bits (n_k < 2^31)
    const int t = vrow ? (int)(p.q_pos0 + i) : -1;
    const int64_t rlast = rloc0 + kTopkWaves - 1 < p.rows ? rloc0 + kTopkWaves - 1 : p.rows - 1;
    const int64_t t_last = p.q_pos0 + p.row0 + rlast;
    const int nkeys = (int)(t_last + 1 < p.n_k ? t_last + 1 : p.n_k);
    // every row of the item selects all its positions: no scores needed (the
    // item's key count is the same for all waves, so the barriers still match)
    const int ntiles = nkeys <= k ? 0 : (nkeys + TK - 1) / TK;
    const int tlim = t < p.n_k - 1 ? t : p.n_k - 1;             // last candidate position
    const int first_cap = tlim < kShortRow ? kShortFirstCap : kCandCap;
    const int64_t gi = (int64_t)b * p.n_q + i;

    RowState<DT, D, HT> rs;
    if (vrow) load_row<DT, D, HT>(p, gi, lane, rs);
    settle_row(rs);
    const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)b * p.k_bs * C::ES;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)nkeys * C::ROWB);
    // fp8 key scales (unused for bf16: an empty range)
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(DT == DT_FP8 ? (const void*)(p.k_scale + (int64_t)b * p.ks_bs) : (const void*)kbase,
                  DT == DT_FP8 ? (uint32_t)nkeys * 4u : 0u);

    int cnt = 0;
    bool full = false, strict = false;
    uint32_t thr = 0;
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
      if (i < ntiles) td.load(krs, srs, i, ktile[i], lane);
    for (int it = 0; it < ntiles; ++it) {
      // tiles it .. it+younger are in flight; this wave's loads of tile it must be done
      const int ahead = ntiles - 1 - it;
      td.wait_oldest(ahead < STAGES - 2 ? ahead : STAGES - 2);
      tile_barrier();
      // buffer (it-1) % STAGES was last read in iteration it-1, which every wave has left
      if (it + STAGES - 1 < ntiles) td.load(krs, srs, it + STAGES - 1, ktile[(it + STAGES - 1) % STAGES], lane);
      const uint8_t* kt = ktile[it % STAGES];
      if (it * TK <= tlim) {
        float sc[NG];
        tile_scores_multi<DT, D, HT, NG>(rs, kt, lane, sc);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const int s0 = it * TK + 64 * g;
          if (s0 > tlim) break;
          const int s = s0 + lane;
          float v = sc[g];
          if constexpr (DT == DT_FP8) v *= *(const float*)(kt + C::TILE_BYTES + (64 * g + lane) * 4);
          const uint32_t u = order_key(v);
          if (cnt + 64 > (full ? kCandCap : first_cap)) {
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            const Shrunk sh = wave_shrink(cu, ci, cnt, k, hist[wid], lane);
            cnt = sh.n;
            thr = sh.thr;
            strict = sh.strict;
            full = true;
            __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
          }
          const bool pr = s <= tlim && (!full || (strict ? u > thr : u >= thr));
          const uint64_t m = ballot(pr);
          if (pr) {
            const uint32_t d = (uint32_t)cnt + lanes_below(m);
            __builtin_amdgcn_raw_buffer_store_b32(u, crs, d * 4u, 0, 0);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)s, crs, d * 4u, kCandCap * 4, 0);
          }
          cnt += __builtin_popcountll(m);
        }
      }
    }
    if (vrow) {
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      int32_t* out = p.idx + gi * (int64_t)k;
      int nout;
      if (tlim < k) {                                            // all of 0..t
        for (int j = lane; j <= tlim; j += 64) out[j] = j;
        nout = tlim + 1;
      } else if (cnt > k) {
        const ExactPick e = wave_select_exact(cu, cnt, k, hist[wid], lane);
        nout = wave_keep(cu, ci, cnt, e.T, (int64_t)e.req, lane, out, k);
        nout = nout < k ? nout : k;
      } else {
        for (int j = lane; j < cnt; j += 64) out[j] = (int32_t)ci[j];
        nout = cnt;
      }
      for (int j = nout + lane; j < k; j += 64) out[j] = -1;
      lds_sync();
    }
  }
}

// ---------------------------------------------------------------- fused, two rows per wave (d = 128)
// 16x16 MFMA tiles: A = 16 heads of one query row, B = 16 keys (K^T), both with
// lane (g = lane >> 4, c = lane & 15) holding row/column c and a quarter of the
// K slice (bf16 v_mfma_f32_16x16x32_bf16: elements 8g..8g+7 of each 32-wide
// step; fp8 v_mfma_scale_f32_16x16x128_f8f6f4: bytes 32g..32g+31 of the whole
// 128-byte row); D lane (g, c) holds key c, heads 4g..4g+3 of the tile.  A wave
// owns two adjacent query rows, so every key fragment read from LDS feeds both
// rows' MFMAs and a workgroup's staged tiles serve eight rows.
template <int DT>
struct Frag2;
template <>
struct Frag2<DT_BF16> {
  typedef bf16x8 T;
  static constexpr int NKS = 4;          // 32-element K steps per 128-element row
};
template <>
struct Frag2<DT_FP8> {
  typedef i32x8 T;
  static constexpr int NKS = 1;          // one 128-byte step
};

template <int DT>
__device__ __forceinline__ f32x4 mfma16(const typename Frag2<DT>::T& a, const typename Frag2<DT>::T& b, f32x4 c) {
  if constexpr (DT == DT_BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// This lane's K slice of step ks of one 128-element row at rowp (bytes).
template <int DT>
__device__ __forceinline__ typename Frag2<DT>::T load_frag2(const uint8_t* rowp, int ks, int g) {
  if constexpr (DT == DT_BF16) {
    return *(const bf16x8*)(rowp + 64 * ks + 16 * g);
  } else {
    const i32x4* q = (const i32x4*)(rowp + 32 * g);
    const i32x4 lo = q[0], hi = q[1];
    i32x8 r;
    r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
    r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
    return r;
  }
}

template <int DT>
struct Row2 {
  typename Frag2<DT>::T a[2][4][Frag2<DT>::NKS];   // [row][head tile][K step]
};

// q fragments of row j into registers; its epilogue weights (w, times the
// query scale for fp8) into the wave's LDS table w2[j][0..64) (zero for heads
// >= H), read back by the epilogue with broadcast loads (the lanes of one
// 16-lane group read the same 4 weights).
template <int DT>
__device__ __forceinline__ void load_row2(const IxParams& p, int64_t gi, bool valid, int j, int lane, Row2<DT>& rs,
                                          float (*w2)[64]) {
  typedef Cfg<DT, 128> C;
  const int g = lane >> 4, col = lane & 15;
  float cw = 0.f;
  if (valid && lane < p.heads) {
    cw = p.w[gi * p.heads + lane];
    if constexpr (DT == DT_FP8) cw *= p.q_scale[gi * p.heads + lane];
  }
  w2[j][lane] = cw;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int head = 16 * h + col;
    if (valid && head < p.heads) {
      const uint8_t* rowp = (const uint8_t*)p.q + (gi * p.heads + head) * (int64_t)C::ROWB;
#pragma unroll
      for (int ks = 0; ks < Frag2<DT>::NKS; ++ks) rs.a[j][h][ks] = load_frag2<DT>(rowp, ks, g);
    } else {
#pragma unroll
      for (int ks = 0; ks < Frag2<DT>::NKS; ++ks) rs.a[j][h][ks] = typename Frag2<DT>::T{};
    }
  }
}

template <int DT>
__device__ __forceinline__ void settle_row2(Row2<DT>& rs) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int h = 0; h < 4; ++h)
#pragma unroll
      for (int ks = 0; ks < Frag2<DT>::NKS; ++ks) asm volatile("" : "+v"(rs.a[j][h][ks]));
}

// Scores of an LDS tile's keys for both rows: group q of 64 keys, lane l gets
// key 64 q + l.  The rows are staggered by half a 16-key step so that each
// row's ReLU-w epilogue runs under the other row's MFMAs: row 0 of step t+1 is
// multiplied while row 1 of step t is summed, with one row's accumulators in
// flight at a time.
template <int DT>
__device__ __forceinline__ void mfma_row2(const typename Frag2<DT>::T (&a)[4][Frag2<DT>::NKS],
                                          const typename Frag2<DT>::T (&bf)[Frag2<DT>::NKS], f32x4 (&acc)[4]) {
#pragma unroll
  for (int h = 0; h < 4; ++h) acc[h] = f32x4{};
#pragma unroll
  for (int ks = 0; ks < Frag2<DT>::NKS; ++ks)
#pragma unroll
    for (int h = 0; h < 4; ++h) acc[h] = mfma16<DT>(a[h][ks], bf[ks], acc[h]);
}
// This lane's part of the head sum (its 16 heads) for key c of one step.
__device__ __forceinline__ float epi_row2(const f32x4 (&acc)[4], const float* w, int g) {
  float pp = 0.f;
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const f32x4 cw = *(const f32x4*)&w[16 * h + 4 * g];
#pragma unroll
    for (int i = 0; i < 4; ++i) pp = fmaf(cw[i], fmaxf(acc[h][i], 0.f), pp);
  }
  return pp;
}
// Reduce-scatter of four steps' parts over the four 16-lane groups: lane
// (g, c) ends with the full sum of step g, key 16 g + c, i.e. key `lane`.
// v_permlane16_swap(x, y) swaps x's odd 16-lane rows with y's even rows, so
// x + y then holds x's step in the even rows and y's in the odd rows, each
// summed over the row pair; v_permlane32_swap does the same across halves.
__device__ __forceinline__ float scatter4(float p0, float p1, float p2, float p3) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(p0), __float_as_uint(p1), false, false);
  const float sa = __uint_as_float(a[0]) + __uint_as_float(a[1]);       // row r: step r & 1, rows {r, r ^ 1}
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(p2), __float_as_uint(p3), false, false);
  const float sb = __uint_as_float(b[0]) + __uint_as_float(b[1]);       // row r: step 2 + (r & 1)
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(sa), __float_as_uint(sb), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);                 // row r: step r, all four rows
}
template <int DT>
__device__ __forceinline__ void load_bf2(const uint8_t* kt, int t, int g, int col,
                                         typename Frag2<DT>::T (&bf)[Frag2<DT>::NKS]) {
  typedef Cfg<DT, 128> C;
  const uint8_t* rowp = kt + (16 * t + col) * C::PITCH;
#pragma unroll
  for (int ks = 0; ks < Frag2<DT>::NKS; ++ks) bf[ks] = load_frag2<DT>(rowp, ks, g);
}
template <int DT, int NG>
__device__ __forceinline__ void tile_scores2(const Row2<DT>& rs, const uint8_t* kt, const float (*w2)[64], int lane,
                                             float (&sc)[NG][2]) {
  constexpr int NS = 4 * NG;                       // 16-key steps per tile
  const int g = lane >> 4, col = lane & 15;
  typename Frag2<DT>::T bf[Frag2<DT>::NKS];
  f32x4 acc0[4], acc1[4];
  float p0[NS], p1[NS];                            // per-step parts of rows 0 and 1
  load_bf2<DT>(kt, 0, g, col, bf);
  mfma_row2<DT>(rs.a[0], bf, acc0);
#pragma unroll
  for (int t = 0; t < NS - 1; ++t) {
    mfma_row2<DT>(rs.a[1], bf, acc1);              // row 1, step t
    load_bf2<DT>(kt, t + 1, g, col, bf);           // (its latency hidden by row 0's sum)
    p0[t] = epi_row2(acc0, w2[0], g);              // row 0, step t (under row 1's MFMAs)
    mfma_row2<DT>(rs.a[0], bf, acc0);              // row 0, step t + 1
    p1[t] = epi_row2(acc1, w2[1], g);              // row 1, step t (under row 0's MFMAs)
  }
  mfma_row2<DT>(rs.a[1], bf, acc1);                // row 1, last step
  p0[NS - 1] = epi_row2(acc0, w2[0], g);
  p1[NS - 1] = epi_row2(acc1, w2[1], g);
#pragma unroll
  for (int q = 0; q < NG; ++q) {
    sc[q][0] = scatter4(p0[4 * q], p0[4 * q + 1], p0[4 * q + 2], p0[4 * q + 3]);
    sc[q][1] = scatter4(p1[4 * q], p1[4 * q + 1], p1[4 * q + 2], p1[4 * q + 3]);
  }
}

// Tile staging of the two-row kernel: the TileDma loads without per-lane offset
// registers (each load's offset is recomputed when it is issued, a few VALU ops):
// a spilled offset reloaded inside the tile loop would wait for every load in
// flight, the staged tiles included.
template <int DT, int TK>
struct TileDma2 {
  typedef Cfg<DT, 128, TK> C;
  static constexpr int SPR = C::CPR + 1;                 // data slots + 1 pad slot per row
  static constexpr int NGR = TK / 64;
  static constexpr int NR = NGR * SPR;                   // row loads per tile
  static constexpr int NI = NR + (DT == DT_FP8 ? NGR : 0);   // + key-scale loads
  static constexpr int NPW = (NI + kTopkWaves - 1) / kTopkWaves;
  int wid, nload;
  __device__ __forceinline__ explicit TileDma2(int wid_) : wid(wid_), nload((NI - wid_ + kTopkWaves - 1) / kTopkWaves) {}
  __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, __amdgpu_buffer_rsrc_t sr, int tile, uint8_t* dst,
                                       int lane) const {
    const uint32_t toff = (uint32_t)tile * (TK * C::ROWB);
#pragma unroll
    for (int m = 0; m < NPW; ++m) {
      const int j = wid + kTopkWaves * m;
      if (j < NR) {
        const int q = 64 * j + lane;
        const int row = q / SPR, part = q - row * SPR;
        const uint32_t off = part < C::CPR ? (uint32_t)(row * C::ROWB + part * 16) : 0x80000000u;
        lds_dma<16>(r, dst + j * 1024, off + toff);
      } else if (DT == DT_FP8 && j < NI) {
        const int q = j - NR;
        lds_dma<4>(sr, dst + C::TILE_BYTES + 256 * q, (uint32_t)(tile * TK + 64 * q + lane) * 4u);
      }
    }
  }
  __device__ __forceinline__ void wait_oldest(int younger) const {
    const int n = younger * (nload == NPW ? NPW : NPW - 1);
    switch (n) {
#define DSA_VMW(c) case c: __builtin_amdgcn_s_waitcnt(0x0F70 | c); break;
      DSA_VMW(1) DSA_VMW(2) DSA_VMW(3) DSA_VMW(4) DSA_VMW(5) DSA_VMW(6) DSA_VMW(7)
      DSA_VMW(8) DSA_VMW(9) DSA_VMW(10) DSA_VMW(11) DSA_VMW(12) DSA_VMW(13) DSA_VMW(14) DSA_VMW(15)
#undef DSA_VMW
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  }
};

constexpr int kRowsPerWave2 = 2;
constexpr int kRowsPerItem2 = kTopkWaves * kRowsPerWave2;

template <int DT>
__global__ __launch_bounds__(kTopkThreads, kTopkBlocksPerCu) void ix_topk2_kernel(IxParams p, uint32_t* work,
                                                                                     uint32_t* cand) {
  // 128-key tiles where three buffers fit two workgroups per CU (fp8), else 64
  constexpr int TK = Cfg<DT, 128, 128>::BUF_BYTES <= 24576 ? 128 : 64;
  constexpr int NG = TK / 64;
  typedef Cfg<DT, 128, TK> C;
  constexpr int STAGES = 3;
  __shared__ __attribute__((aligned(16))) uint8_t ktile[STAGES][C::BUF_BYTES];
  __shared__ uint32_t hist[kTopkWaves][256];
  __shared__ __attribute__((aligned(16))) float w2s[kTopkWaves][2][64];
  __shared__ int64_t s_item;

  const int wid = wave_id(), lane = threadIdx.x & 63;
  uint32_t* cu0 = cand + (((size_t)blockIdx.x * kTopkWaves + wid) * 2) * 2 * kCandCap;
  uint32_t* cu1 = cu0 + 2 * kCandCap;
  uint32_t* const cus[2] = {cu0, cu1};
  const __amdgpu_buffer_rsrc_t crs0 = make_rsrc(cu0, 2u * kCandCap * 4u);
  const __amdgpu_buffer_rsrc_t crs1 = make_rsrc(cu1, 2u * kCandCap * 4u);
  const int64_t nrb = (p.rows + kRowsPerItem2 - 1) / kRowsPerItem2;
  const int64_t total = nrb * p.batch;
  const int k = p.topk;
  const TileDma2<DT, TK> td(wid);

  for (;;) {
    if (threadIdx.x == 0) s_item = (int64_t)atomicAdd(work, 1u);
    __syncthreads();
    const int64_t item = s_item;
    __syncthreads();
    if (item >= total) break;
    const int b = (int)(item % p.batch);
    const int64_t rb = nrb - 1 - item / p.batch;                 // heaviest rows first
    const int64_t rloc0 = rb * kRowsPerItem2;
    const int64_t rlast = rloc0 + kRowsPerItem2 - 1 < p.rows ? rloc0 + kRowsPerItem2 - 1 : p.rows - 1;
    const int64_t t_last = p.q_pos0 + p.row0 + rlast;
    const int nkeys = (int)(t_last + 1 < p.n_k ? t_last + 1 : p.n_k);
    const int ntiles = nkeys <= k ? 0 : (nkeys + TK - 1) / TK;   // as in ix_topk_kernel

    bool vrow[2];
    int tlim[2], first_cap[2];
    int64_t gi[2];
    Row2<DT> rs;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t rloc = rloc0 + 2 * wid + j;
      vrow[j] = rloc < p.rows;
      const int64_t i = p.row0 + rloc;
      const int t = vrow[j] ? (int)(p.q_pos0 + i) : -1;
      tlim[j] = t < p.n_k - 1 ? t : p.n_k - 1;
      first_cap[j] = tlim[j] < kShortRow ? kShortFirstCap : kCandCap;
      gi[j] = (int64_t)b * p.n_q + i;
      load_row2<DT>(p, gi[j], vrow[j], j, lane, rs, w2s[wid]);
    }
    settle_row2<DT>(rs);
    const int tmax = tlim[0] > tlim[1] ? tlim[0] : tlim[1];
    const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)b * p.k_bs * C::ES;
    const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, (uint32_t)nkeys * C::ROWB);
    // fp8 key scales (unused for bf16: an empty range)
    const __amdgpu_buffer_rsrc_t srs =
        make_rsrc(DT == DT_FP8 ? (const void*)(p.k_scale + (int64_t)b * p.ks_bs) : (const void*)kbase,
                  DT == DT_FP8 ? (uint32_t)nkeys * 4u : 0u);

    int cnt[2] = {0, 0};
    bool full[2] = {false, false}, strict[2] = {false, false};
    uint32_t thr[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < STAGES - 1; ++i)
      if (i < ntiles) td.load(krs, srs, i, ktile[i], lane);
    for (int it = 0; it < ntiles; ++it) {
      const int ahead = ntiles - 1 - it;
      td.wait_oldest(ahead < STAGES - 2 ? ahead : STAGES - 2);
      tile_barrier();
      if (it + STAGES - 1 < ntiles) td.load(krs, srs, it + STAGES - 1, ktile[(it + STAGES - 1) % STAGES], lane);
      const uint8_t* kt = ktile[it % STAGES];
      if (it * TK <= tmax) {
        // Scores at normal wave priority, everything else (appends, compactions, the
        // next tile's wait, barrier and DMA issue, the final select, the next row
        // block's set-up) raised: the SIMD's other wave is then mostly issuing MFMAs,
        // each of which keeps the matrix core busy for 16 (bf16) or 32 (fp8) cycles.
        // Measured 0.5-2% faster; the order of the work itself is unchanged.
        __builtin_amdgcn_s_setprio(0);
        float sc[NG][2];
        tile_scores2<DT, NG>(rs, kt, w2s[wid], lane, sc);
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          const int s0 = it * TK + 64 * q;
          if (s0 > tmax) break;
          const int s = s0 + lane;
          float kscale = 1.f;
          if constexpr (DT == DT_FP8) kscale = *(const float*)(kt + C::TILE_BYTES + (64 * q + lane) * 4);
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            if (s0 > tlim[j]) continue;
            float v = sc[q][j];
            if constexpr (DT == DT_FP8) v *= kscale;
            const uint32_t u = order_key(v);
            if (cnt[j] + 64 > (full[j] ? kCandCap : first_cap[j])) {
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
              const Shrunk sh = wave_shrink(cus[j], cus[j] + kCandCap, cnt[j], k, hist[wid], lane);
              cnt[j] = sh.n;
              thr[j] = sh.thr;
              strict[j] = sh.strict;
              full[j] = true;
              __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
            }
            const bool pr = s <= tlim[j] && (!full[j] || (strict[j] ? u > thr[j] : u >= thr[j]));
            const uint64_t m = ballot(pr);
            if (pr) {
              const uint32_t d = (uint32_t)cnt[j] + lanes_below(m);
              const __amdgpu_buffer_rsrc_t crs = j == 0 ? crs0 : crs1;
              __builtin_amdgcn_raw_buffer_store_b32(u, crs, d * 4u, 0, 0);
              __builtin_amdgcn_raw_buffer_store_b32((uint32_t)s, crs, d * 4u, kCandCap * 4, 0);
            }
            cnt[j] += __builtin_popcountll(m);
          }
        }
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (!vrow[j]) continue;
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
      uint32_t* cu = cus[j];
      uint32_t* ci = cu + kCandCap;
      int32_t* out = p.idx + gi[j] * (int64_t)k;
      int nout;
      if (tlim[j] < k) {
        for (int x = lane; x <= tlim[j]; x += 64) out[x] = x;
        nout = tlim[j] + 1;
      } else if (cnt[j] > k) {
        const ExactPick e = wave_select_exact(cu, cnt[j], k, hist[wid], lane);
        nout = wave_keep(cu, ci, cnt[j], e.T, (int64_t)e.req, lane, out, k);
        nout = nout < k ? nout : k;
      } else {
        for (int x = lane; x < cnt[j]; x += 64) out[x] = (int32_t)ci[x];
        nout = cnt[j];
      }
      for (int x = nout + lane; x < k; x += 64) out[x] = -1;
      lds_sync();
    }
  }
}

// ---------------------------------------------------------------- decode scan
// The grid holds about two workgroups per CU (one round, no tail).  The G
// workgroups of a row sweep its keys together in 256-key blocks: workgroup x
// takes blocks x, x + G, x + 2G, ... (its wave w the 64 keys w of each block), so
// at any time the row's reads fall in one contiguous window of the cache.

template <int DT, int D, int HT>
__global__ __launch_bounds__(256, 2) void ix_scan_kernel(IxParams p) {
  typedef Cfg<DT, D> C;
  // histogram of the top 12 bits of the scores' order keys (for the few-row select)
  __shared__ uint32_t khist[dsa_host::kFewHistBins];
  const int wid = wave_id(), lane = threadIdx.x & 63;
  const int64_t gi = blockIdx.y;                  // flattened (batch, query row)
  const int b = (int)(gi / p.n_q);
  const int64_t i = gi % p.n_q;
  const int64_t t = p.q_pos0 + i;
  const int64_t len = t + 1 < p.n_k ? t + 1 : p.n_k;
  const int64_t nblk = (len + 4 * kTileKeys - 1) / (4 * kTileKeys);
  if ((int64_t)blockIdx.x >= nblk) return;
  const int nstages = (int)((nblk - blockIdx.x + gridDim.x - 1) / gridDim.x);
  const bool hist = p.hist != nullptr;
  if (hist) {
    for (int i = threadIdx.x; i < dsa_host::kFewHistBins; i += 256) khist[i] = 0u;
    __syncthreads();
  }
  const uint8_t* kbase = (const uint8_t*)p.k + (int64_t)b * p.k_bs * C::ES;
  const float* ksc = (DT == DT_FP8) ? p.k_scale + (int64_t)b * p.ks_bs : nullptr;
  float* out = p.out + gi * (int64_t)p.n_k;
  // B operands and (fp8) key scales straight from HBM, one stage (64 keys) ahead
  // of the MFMAs.  The next stage is loaded unconditionally (rows past the end
  // read key len-1 and are masked on output): under a condition, the wait before
  // the MFMAs would have to assume the younger loads absent and drain them along
  // with the current stage.
  typedef typename AFrag<DT>::T F;
  auto stage_key0 = [&](int st) {
    return ((int64_t)st * gridDim.x + blockIdx.x) * (4 * kTileKeys) + (int64_t)wid * kTileKeys;
  };
  auto load_stage = [&](int st, F (&bf)[2][C::NKS], float& kscale) {
    const int64_t s0 = stage_key0(st);
    const int64_t srow = s0 + (lane & 31);
    const int64_t s_a = srow < len ? srow : len - 1;
    const int64_t s_b = srow + 32 < len ? srow + 32 : len - 1;
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
      bf[0][ks] = load_frag<DT>(kbase + s_a * C::ROWB, ks, lane);
      bf[1][ks] = load_frag<DT>(kbase + s_b * C::ROWB, ks, lane);
    }
    if constexpr (DT == DT_FP8) {
      const int64_t sk = s0 + lane;
      kscale = ksc[sk < len ? sk : len - 1];
    }
  };
  RowState<DT, D, HT> rs;
  // scores of stage st from its operands bf (key scales kscale)
  // (the two 32-key halves one after the other: half the accumulators live, and
  // the first half's head-sum epilogue overlaps the second half's MFMAs)
  auto score_stage = [&](int st, const F (&bf)[2][C::NKS], float kscale) {
    float pp[2];
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      f32x16 acc[HT];
#pragma unroll
      for (int h = 0; h < HT; ++h) acc[h] = f32x16{};
#pragma unroll
      for (int ks = 0; ks < C::NKS; ++ks) {
#pragma unroll
        for (int h = 0; h < HT; ++h) acc[h] = mfma<DT>(rs.a[h][ks], bf[n][ks], acc[h]);
      }
      float q = 0.f;
#pragma unroll
      for (int h = 0; h < HT; ++h) {
#pragma unroll
        for (int ii = 0; ii < 16; ++ii) q = fmaf(rs.c[h][ii], fmaxf(acc[h][ii], 0.f), q);
      }
      pp[n] = q;
    }
    float sc = combine_halves(pp[0], pp[1]);
    const int64_t s = stage_key0(st) + lane;
    if (s < len) {
      if constexpr (DT == DT_FP8) sc *= kscale;
      const float o = sc + 0.0f;
      out[s] = o;
      if (hist) atomicAdd(&khist[order_key(o) >> 20], 1u);
    }
  };
  // Three operand buffers used in turn, two stages in flight while one is scored
  // (the loop body is unrolled by three, so all three are live at once and the
  // loads go out ahead of the MFMAs); only where they fit the register budget
  // (64 heads of bf16 d = 128 would spill: that case loads and scores one stage
  // at a time).
  constexpr bool kPrefetch = 2 * C::NKS * sizeof(F) <= 128;
  F ba[2][C::NKS], bb[2][C::NKS], bc[2][C::NKS];
  float sa = 1.f, sb = 1.f, sc3 = 1.f;
  auto valid = [&](int st) { return st < nstages && stage_key0(st) < len; };
  if constexpr (kPrefetch) {
    load_stage(0, ba, sa);
    load_stage(1, bb, sb);
  }
  load_row<DT, D, HT, true>(p, gi, lane, rs);
  settle_row(rs);
  if constexpr (kPrefetch) {
#pragma unroll 1
    for (int st = 0; valid(st); st += 3) {
      load_stage(st + 2, bc, sc3);
      score_stage(st, ba, sa);
      if (!valid(st + 1)) break;
      load_stage(st + 3, ba, sa);
      score_stage(st + 1, bb, sb);
      if (!valid(st + 2)) break;
      load_stage(st + 4, bb, sb);
      score_stage(st + 2, bc, sc3);
    }
  } else {
#pragma unroll 1
    for (int st = 0; valid(st); ++st) {
      load_stage(st, ba, sa);
      score_stage(st, ba, sa);
    }
  }
  if (hist) {
    __syncthreads();
    uint32_t* gh = p.hist + gi * p.hist_rw;
    for (int i = threadIdx.x; i < dsa_host::kFewHistBins; i += 256)
      if (khist[i]) atomicAdd(&gh[i], khist[i]);
  }
}

// ---------------------------------------------------------------- dispatch
IxParams make_params(const dsa_indexer_args& a) {
  IxParams p{};
  p.q = a.q;
  p.q_scale = a.q_scale;
  p.k = a.k;
  p.k_bs = a.k_batch_stride ? a.k_batch_stride : (int64_t)a.n_k * a.dim;
  p.k_scale = a.k_scale;
  p.ks_bs = a.k_scale_batch_stride ? a.k_scale_batch_stride : (int64_t)a.n_k;
  p.w = a.w;
  p.batch = a.batch;
  p.n_q = a.n_q;
  p.n_k = a.n_k;
  p.heads = a.heads;
  p.q_pos0 = a.q_pos0;
  p.row0 = 0;
  p.rows = a.n_q;
  return p;
}

template <int DT, int D>
hipError_t launch_scores_dt(const IxParams& p, hipStream_t s) {
  const int64_t nrb = (p.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  dim3 grid((unsigned)(nrb * p.batch));
  if (p.heads > 32) {
    hipLaunchKernelGGL((ix_scores_kernel<DT, D, 2>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((ix_scores_kernel<DT, D, 1>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

int persistent_blocks() {
  static int cached = 0;
  if (cached) return cached;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  int nb = kTopkBlocksPerCu * cus;
  if (nb > dsa_host::kTopkWaveSlots / kTopkWaves) nb = dsa_host::kTopkWaveSlots / kTopkWaves;
  cached = nb;
  return nb;
}

template <int DT, int D>
hipError_t launch_topk_dt(const IxParams& p, void* ws, hipStream_t s) {
  uint32_t* work = (uint32_t*)ws;
  uint32_t* cand = (uint32_t*)((char*)ws + 256);
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, s, work, 64);
  const int64_t nrb = (p.rows + kTopkWaves - 1) / kTopkWaves;
  int64_t items = nrb * p.batch;
  int64_t nb = persistent_blocks();
  if (nb > items) nb = items;
  dim3 grid((unsigned)nb);
  if constexpr (D == 128) {
    if (p.heads > 32) {
      const int64_t items2 = ((p.rows + kRowsPerItem2 - 1) / kRowsPerItem2) * p.batch;
      int64_t nb2 = persistent_blocks();
      if (nb2 > dsa_host::kTopkWaveSlots / kRowsPerItem2) nb2 = dsa_host::kTopkWaveSlots / kRowsPerItem2;
      if (nb2 > items2) nb2 = items2;
      hipLaunchKernelGGL(ix_topk2_kernel<DT>, dim3((unsigned)nb2), dim3(kTopkThreads), 0, s, p, work, cand);
      return hipGetLastError();
    }
  }
  if (p.heads > 32) {
    hipLaunchKernelGGL((ix_topk_kernel<DT, D, 2>), grid, dim3(kTopkThreads), 0, s, p, work, cand);
  } else {
    hipLaunchKernelGGL((ix_topk_kernel<DT, D, 1>), grid, dim3(kTopkThreads), 0, s, p, work, cand);
  }
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_scan_dt(const IxParams& p0, hipStream_t s) {
  IxParams p = p0;
  const int64_t len = p.q_pos0 + p.n_q < p.n_k ? p.q_pos0 + p.n_q : p.n_k;
  const int64_t rows = (int64_t)p.batch * p.n_q;
  // about two workgroups per CU over all rows (at most one per 256-key block)
  int64_t per_row = (persistent_blocks() + rows - 1) / rows;
  const int64_t nblk = (len + 4 * kTileKeys - 1) / (4 * kTileKeys);
  if (per_row > nblk) per_row = nblk;
  if (per_row < 1) per_row = 1;
  dim3 grid((unsigned)per_row, (unsigned)rows);
  if (p.heads > 32) {
    hipLaunchKernelGGL((ix_scan_kernel<DT, D, 2>), grid, dim3(256), 0, s, p);
  } else {
    hipLaunchKernelGGL((ix_scan_kernel<DT, D, 1>), grid, dim3(256), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

namespace dsa_host {

bool indexer_mfma_supported(const dsa_indexer_args& a) {
  if (a.heads < 1 || a.heads > 64) return false;
  if (a.dtype == DSA_BF16) return a.dim == 32 || a.dim == 64 || a.dim == 128;
  if (a.dtype == DSA_FP8_E4M3) return a.dim == 64 || a.dim == 128;
  return false;
}

hipError_t indexer_scores_f32(const dsa_indexer_args& a, int64_t row0, int64_t rows, float* out,
                              int64_t out_row_stride, hipStream_t s) {
  IxParams p = make_params(a);
  p.row0 = row0;
  p.rows = rows;
  p.out = out;
  dim3 grid((unsigned)((a.n_k + 255) / 256), (unsigned)rows, (unsigned)a.batch);
  size_t lds = (size_t)(a.heads * a.dim + a.heads) * sizeof(float);
  hipLaunchKernelGGL(indexer_f32_kernel, grid, dim3(256), lds, s, p, a.dim, out_row_stride);
  return hipGetLastError();
}

hipError_t indexer_scores_mfma(const dsa_indexer_args& a, int64_t row0, int64_t rows, float* out,
                               hipStream_t s) {
  IxParams p = make_params(a);
  p.row0 = row0;
  p.rows = rows;
  p.out = out;
  if (a.dtype == DSA_BF16) {
    if (a.dim == 128) return launch_scores_dt<DT_BF16, 128>(p, s);
    if (a.dim == 64) return launch_scores_dt<DT_BF16, 64>(p, s);
    if (a.dim == 32) return launch_scores_dt<DT_BF16, 32>(p, s);
  } else if (a.dtype == DSA_FP8_E4M3) {
    if (a.dim == 128) return launch_scores_dt<DT_FP8, 128>(p, s);
    if (a.dim == 64) return launch_scores_dt<DT_FP8, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

size_t topk_fused_ws_bytes() {
  return 256 + (size_t)kTopkWaveSlots * 2 * kCandCap * sizeof(uint32_t);
}

hipError_t indexer_topk_fused(const dsa_indexer_args& a, int32_t k, int32_t* idx, void* ws, hipStream_t s) {
  IxParams p = make_params(a);
  p.idx = idx;
  p.topk = k;
  if (a.dtype == DSA_BF16) {
    if (a.dim == 128) return launch_topk_dt<DT_BF16, 128>(p, ws, s);
    if (a.dim == 64) return launch_topk_dt<DT_BF16, 64>(p, ws, s);
    if (a.dim == 32) return launch_topk_dt<DT_BF16, 32>(p, ws, s);
  } else if (a.dtype == DSA_FP8_E4M3) {
    if (a.dim == 128) return launch_topk_dt<DT_FP8, 128>(p, ws, s);
    if (a.dim == 64) return launch_topk_dt<DT_FP8, 64>(p, ws, s);
  }
  return hipErrorInvalidValue;
}

hipError_t indexer_scan(const dsa_indexer_args& a, float* scores, const FewHist* hist, hipStream_t s) {
  IxParams p = make_params(a);
  p.out = scores;
  if (hist) {
    p.hist = hist->base;
    p.hist_rw = hist->row_words;
  }
  if (a.dtype == DSA_BF16) {
    if (a.dim == 128) return launch_scan_dt<DT_BF16, 128>(p, s);
    if (a.dim == 64) return launch_scan_dt<DT_BF16, 64>(p, s);
    if (a.dim == 32) return launch_scan_dt<DT_BF16, 32>(p, s);
  } else if (a.dtype == DSA_FP8_E4M3) {
    if (a.dim == 128) return launch_scan_dt<DT_FP8, 128>(p, s);
    if (a.dim == 64) return launch_scan_dt<DT_FP8, 64>(p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa_host
