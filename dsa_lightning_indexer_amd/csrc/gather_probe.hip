// Gather-bandwidth probe (a measurement helper, not a step of the method): reads
// the selected 1152-byte latent rows of every query's index row, as a sparse
// attention pass must ([DSA-NOTES] §3: each query reads the k rows its index
// set names), with no arithmetic beyond an XOR checksum that keeps every load
// alive.  Its rate is the ceiling the sparse-attention kernel's gathers are
// measured against.  Access patterns (16 selected positions per step, DEPTH
// steps in flight, positions staged in LDS, invalid entries read as zeros):
//   mode 0  quarter rows: one query per four-wave workgroup; wave w reads the
//           bytes the attention kernel's wave w reads (V columns 128w..128w+127
//           and, for w < 2, rope columns 512 + 32w..), 64 bytes of 16 rows per
//           load instruction
//   mode 1  whole rows, strided: one query per wave (four per workgroup); each
//           load instruction covers 64 bytes of each of 16 rows
//   mode 2  whole rows, contiguous: one query per wave; load j of a step covers
//           the j-th KiB of the step's 16 rows laid end to end (eight lanes per
//           128-byte line)
// mode + 3: the same pattern with deeper prefetch: four steps in flight for
//           quarter rows, three for whole rows (four would not fit the
//           register file).
//   mode 6  the attention kernel's own pattern: one query per four-wave
//           workgroup; wave w reads its 256-byte V slice of four rows per load
//           instruction (whole lines) and, for w < 2, the 64-byte rope slice of
//           16 rows (two steps in flight)
//   mode 7  mode 6 with the rope line split by rows instead of columns: wave w
//           reads the whole 128-byte rope line of rows 4w..4w+3 (one request per
//           line instead of two)
//   mode 8  one query per four-wave workgroup, whole rows end to end: wave w
//           reads rows 4w..4w+3 of each step (4.5 KiB, the last load half
//           full), as mode 2 does for all 16 rows
//   mode 9  the one-wave-per-query attention kernel's pattern: one query per
//           wave; per step one load instruction per row for its first KiB (64
//           lanes, that row alone) and two for the 16 rope lines (eight rows
//           per instruction, eight lanes per line), two steps in flight
//   mode 10 the same instructions landing in LDS (buffer_load ... lds) with the
//           DMA attention kernel's schedule: two row tiles per wave (one being
//           read, one being filled), the index row through a four-block ring,
//           each step's tile read back whole once
#include "common.hpp"

namespace {

using namespace dsa;

constexpr int kRowB = 1152;            // 576 bf16 latent columns
constexpr int kChunks = kRowB / 16;    // 16-byte chunks per row
constexpr int kStep = 16;              // positions per step
constexpr int kMaxK = DSA_MAX_TOPK;

struct ProbeParams {
  const void* table;
  uint32_t table_bytes;
  const int32_t* idx;
  int64_t n_q;
  int32_t n_rows, topk;
  uint32_t* out;
};

__device__ __forceinline__ uint32_t xor4(u32x4 v) { return v[0] ^ v[1] ^ v[2] ^ v[3]; }

template <int MODE>
struct Pattern;

// quarter rows: lane (g, col) reads chunks of row `col` of the step
template <>
struct Pattern<0> {
  static constexpr int kLoads = 5;
  static constexpr int kQueriesPerWg = 1;
  __device__ static uint32_t offset(int w, int lane, int j, uint32_t rowbase) {
    const int g = lane >> 4;
    if (j < 4) return rowbase + 256 * w + 64 * j + 16 * g;
    return w < 2 ? rowbase + 1024 + 64 * w + 16 * g : 0x80000000u;
  }
  __device__ static int row_of(int, int lane, int) { return lane & 15; }
};

// whole rows, 64 bytes of 16 rows per instruction
template <>
struct Pattern<1> {
  static constexpr int kLoads = kChunks / 4;     // 18
  static constexpr int kQueriesPerWg = 4;
  __device__ static uint32_t offset(int, int lane, int j, uint32_t rowbase) {
    return rowbase + 64 * j + 16 * (lane >> 4);
  }
  __device__ static int row_of(int, int lane, int) { return lane & 15; }
};

// whole rows end to end: chunk c = 64 j + lane of the step's 16 x 72 chunks
template <>
struct Pattern<2> {
  static constexpr int kLoads = kStep * kChunks / 64;   // 18
  static constexpr int kQueriesPerWg = 4;
  __device__ static uint32_t offset(int, int lane, int j, uint32_t rowbase) {
    return rowbase + 16 * ((64 * j + lane) % kChunks);
  }
  __device__ static int row_of(int, int lane, int j) { return (64 * j + lane) / kChunks; }
};

// the attention kernel's own pattern: per wave, its 256-byte V slice of four rows
// per load instruction (16 lanes per row, whole lines), then (waves 0 and 1) the
// 64-byte rope slice of 16 rows in the MFMA fragment layout
template <>
struct Pattern<3> {
  static constexpr int kLoads = 5;
  static constexpr int kQueriesPerWg = 1;
  __device__ static uint32_t offset(int w, int lane, int j, uint32_t rowbase) {
    if (j < 4) return rowbase + 256 * w + 16 * (lane & 15);
    return w < 2 ? rowbase + 1024 + 64 * w + 16 * (lane >> 4) : 0x80000000u;
  }
  __device__ static int row_of(int, int lane, int j) { return j < 4 ? 4 * j + (lane >> 4) : (lane & 15); }
};

// the attention pattern with each row's rope line read whole, by one wave: wave w
// reads the 128-byte rope lines of rows 4w..4w+3 (lanes 0..31, eight per line)
template <>
struct Pattern<4> {
  static constexpr int kLoads = 5;
  static constexpr int kQueriesPerWg = 1;
  __device__ static uint32_t offset(int w, int lane, int j, uint32_t rowbase) {
    if (j < 4) return rowbase + 256 * w + 16 * (lane & 15);
    return lane < 32 ? rowbase + 1024 + 16 * (lane & 7) : 0x80000000u;
  }
  __device__ static int row_of(int w, int lane, int j) { return j < 4 ? 4 * j + (lane >> 4) : 4 * w + ((lane >> 3) & 3); }
};

// whole rows end to end, four waves per query: chunk c = 64 j + lane of wave w's
// 4 x 72 chunks (rows 4w..4w+3); lanes past the 288th chunk read nothing
template <>
struct Pattern<5> {
  static constexpr int kLoads = 5;
  static constexpr int kQueriesPerWg = 1;
  __device__ static uint32_t offset(int, int lane, int j, uint32_t rowbase) {
    const int c = 64 * j + lane;
    return c < 4 * kChunks ? rowbase + 16 * (c % kChunks) : 0x80000000u;
  }
  __device__ static int row_of(int w, int lane, int j) {
    const int c = 64 * j + lane;
    return 4 * w + (c < 4 * kChunks ? c / kChunks : 3);
  }
};

// one query per wave; per step: load r < 16 is row r's first KiB (one row per
// instruction), loads 16 and 17 the 128-byte rope lines of rows 8k + lane/8
template <>
struct Pattern<6> {
  static constexpr int kLoads = kStep + 2;
  static constexpr int kQueriesPerWg = 4;
  __device__ static uint32_t offset(int, int lane, int j, uint32_t rowbase) {
    return j < kStep ? rowbase + 16 * lane : rowbase + 1024 + 16 * (lane & 7);
  }
  __device__ static int row_of(int, int lane, int j) { return j < kStep ? j : 8 * (j - kStep) + (lane >> 3); }
};

template <int MODE, int DEPTH>
__global__ __launch_bounds__(256) void gather_probe_kernel(ProbeParams p) {
  using P = Pattern<MODE>;
  constexpr int QW = P::kQueriesPerWg;
  __shared__ int32_t sidx[QW][kMaxK];
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int64_t q0 = (int64_t)blockIdx.x * QW;
  for (int qq = 0; qq < QW; ++qq) {
    const int64_t q = q0 + qq;
    for (int e = threadIdx.x; e < p.topk; e += 256) sidx[qq][e] = q < p.n_q ? p.idx[q * p.topk + e] : -1;
  }
  __syncthreads();
  const int qq = QW == 1 ? 0 : w;
  const int64_t q = q0 + qq;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p.table), (short)0, (int)p.table_bytes, 0x00020000);
  const int nsteps = (p.topk + kStep - 1) / kStep;

  auto issue = [&](int step, u32x4 (&buf)[P::kLoads]) {
#pragma unroll
    for (int j = 0; j < P::kLoads; ++j) {
      const int e = step * kStep + P::row_of(w, lane, j);
      const int32_t s = (step < nsteps && e < p.topk) ? sidx[qq][e] : -1;
      const bool valid = s >= 0 && s < p.n_rows;
      const uint32_t base = valid ? (uint32_t)s * kRowB : 0x80000000u;
      const uint32_t off = P::offset(w, lane, j, base);
      buf[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  };
  u32x4 buf[DEPTH][P::kLoads];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(d, buf[d]);
  uint32_t acc = 0;
  for (int step = 0; step < nsteps; step += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
#pragma unroll
      for (int j = 0; j < P::kLoads; ++j) acc ^= xor4(buf[d][j]);
      issue(step + DEPTH + d, buf[d]);
    }
  }
  // fold the wave's checksum into lane 0 and store one word per wave
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0 && q < p.n_q) p.out[(int64_t)blockIdx.x * 4 + w] = acc;
}

template <int MODE, int DEPTH>
void launch(const ProbeParams& p, hipStream_t s) {
  const int64_t wgs = (p.n_q + Pattern<MODE>::kQueriesPerWg - 1) / Pattern<MODE>::kQueriesPerWg;
  hipLaunchKernelGGL((gather_probe_kernel<MODE, DEPTH>), dim3((unsigned)wgs), dim3(256), 0, s, p);
}

// mode 10: the schedule of the DMA attention kernel without its arithmetic
constexpr int kDmaVP = 1040;                       // V row pitch in a tile
constexpr int kDmaRope = kStep * kDmaVP;           // rope lines after the V rows
constexpr int kDmaTB = kDmaRope + kStep * 128;     // tile bytes
__global__ __launch_bounds__(256, 1) void gather_dma_kernel(ProbeParams p) {
  constexpr int NRING = 4;
  constexpr uint32_t kInv = 0x80000000u;
  __shared__ __attribute__((aligned(16))) uint8_t tiles[4][2][kDmaTB];
  __shared__ __attribute__((aligned(16))) uint32_t ring_all[4][NRING][64];
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const int64_t q = (int64_t)blockIdx.x * 4 + w;
  if (q >= p.n_q) return;                          // (no barriers below)
  uint32_t (*ring)[64] = ring_all[w];
  const int topk = p.topk;
  const __amdgpu_buffer_rsrc_t kvr = make_rsrc(p.table, p.table_bytes);
  const __amdgpu_buffer_rsrc_t irs = make_rsrc(p.idx + q * topk, (uint32_t)topk * 4u);
  const int nst = (topk + kStep - 1) / kStep;
  const int nblk = (topk + 63) / 64;
  auto idx_dma = [&](int m) { lds_dma<4>(irs, (const uint8_t*)ring[m % NRING], (uint32_t)(64 * m + lane) * 4u); };
  auto idx_conv = [&](int m) {
    uint32_t* sl = ring[m % NRING];
    const int e = 64 * m + lane;
    const int32_t s = (int32_t)sl[lane];
    sl[lane] = (e < topk && s >= 0 && s < p.n_rows) ? (uint32_t)s * kRowB : kInv;
  };
  const uint32_t lv = 16u * (uint32_t)lane;
  const int rj = lane >> 3;
  const uint32_t lr0 = 1024u + 16u * (uint32_t)((lane - rj) & 7);
  const uint32_t lr1 = 1024u + 16u * (uint32_t)((lane - rj - 1) & 7);
  auto row_dma = [&](int t, uint8_t* dst) {
    const uint32_t dead = t < nst ? 0u : kInv;
    const uint32_t* si = ring[(t >> 2) % NRING] + 16 * (t & 3);
    u32x4 r4[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) r4[qq] = *(const u32x4*)(si + 4 * qq);
    const uint32_t o0 = si[rj] | dead, o1 = si[8 + rj] | dead;
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
#pragma unroll
      for (int i = 0; i < 4; ++i) lds_dma<16>(kvr, dst + (4 * qq + i) * kDmaVP, (r4[qq][i] | dead) + lv);
    lds_dma<16>(kvr, dst + kDmaRope, o0 + lr0);
    lds_dma<16>(kvr, dst + kDmaRope + 1024, o1 + lr1);
  };
  uint32_t acc = 0;
  auto consume = [&](const uint8_t* tile) {
#pragma unroll
    for (int r = 0; r < kStep; ++r) acc ^= xor4(*(const u32x4*)(tile + r * kDmaVP + 16 * lane));
#pragma unroll
    for (int k = 0; k < 2; ++k) acc ^= xor4(*(const u32x4*)(tile + kDmaRope + 1024 * k + 16 * lane));
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  };
  idx_dma(0);
  if (nblk > 1) idx_dma(1);
  vm_wait<0>();
  idx_conv(0);
  row_dma(0, tiles[w][0]);
  row_dma(1, tiles[w][1]);
  for (int t = 0; t < nst; t += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int tt = t + h;
      if (h == 1 && tt >= nst) break;
      vm_wait<kStep + 2>();
      if ((tt & 3) == 0 && (tt >> 2) + 1 < nblk) idx_conv((tt >> 2) + 1);
      consume(tiles[w][h]);
      if ((tt & 3) == 0 && (tt >> 2) + 2 < nblk) idx_dma((tt >> 2) + 2);
      row_dma(tt + 2, tiles[w][h]);
    }
  }
  vm_wait<0>();
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0) p.out[(int64_t)blockIdx.x * 4 + w] = acc;
}

}  // namespace

namespace dsa_host {

int64_t gather_probe_out_words(int64_t n_q, int32_t mode) {
  // queries per workgroup: one in modes 0, 3, 6, 7, 8; four in the others
  const int qw = (mode == 0 || mode == 3 || (mode >= 6 && mode <= 8)) ? 1 : 4;
  return (n_q + qw - 1) / qw * 4;
}

hipError_t gather_probe_launch(const void* table, int32_t n_rows, const int32_t* idx, int64_t n_q, int32_t topk,
                               int32_t mode, uint32_t* out, hipStream_t s) {
  ProbeParams p{table, (uint32_t)((int64_t)n_rows * kRowB), idx, n_q, n_rows, topk, out};
  switch (mode) {
    case 0: launch<0, 2>(p, s); break;
    case 1: launch<1, 2>(p, s); break;
    case 2: launch<2, 2>(p, s); break;
    case 3: launch<0, 4>(p, s); break;
    case 4: launch<1, 3>(p, s); break;
    case 5: launch<2, 3>(p, s); break;
    case 6: launch<3, 2>(p, s); break;
    case 7: launch<4, 2>(p, s); break;
    case 8: launch<5, 2>(p, s); break;
    case 9: launch<6, 2>(p, s); break;
    case 10: hipLaunchKernelGGL(gather_dma_kernel, dim3((unsigned)((p.n_q + 3) / 4)), dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa_host

// ---------------------------------------------------------------- streaming read probe
// Reads a contiguous buffer once, in order, with no arithmetic beyond an XOR
// checksum per wave: the rate bounds what a scan over the same bytes (the decode
// indexer's K cache) can reach.  Workgroup x reads 16-KiB chunks x, x + G,
// x + 2G, ... (G workgroups); each lane issues four 16-byte loads per chunk, and
// UNROLL chunks are in flight per wave.
namespace {

constexpr int kStreamChunk = 256 * 64;      // bytes per workgroup per chunk: 256 lanes x 4 x 16 B

template <int UNROLL>
__global__ __launch_bounds__(256) void stream_probe_kernel(const uint8_t* buf, uint32_t nchunks, uint32_t* out) {
  const int lane = threadIdx.x & 63;
  const int w = wave_id();
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(buf), (short)0, (int)(nchunks * (uint32_t)kStreamChunk),
                                        0x00020000);
  uint32_t acc = 0;
  // within a chunk: wave w reads its 4 KiB (4 loads of 64 lanes x 16 B, 1 KiB each)
  const uint32_t lofs = (uint32_t)(w * 4096 + 16 * lane);
  for (uint32_t c0 = blockIdx.x; c0 < nchunks; c0 += gridDim.x * UNROLL) {
    u32x4 v[UNROLL][4];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const uint32_t c = c0 + (uint32_t)u * gridDim.x;
      // past the end: an offset beyond the range reads zeros without touching memory
      const uint32_t base = c < nchunks ? c * (uint32_t)kStreamChunk + lofs : 0x80000000u;
#pragma unroll
      for (int j = 0; j < 4; ++j)
        v[u][j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, base + 1024u * j, 0, 0));
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc ^= xor4(v[u][j]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0) out[blockIdx.x * 4 + w] = acc;
}

}  // namespace

namespace dsa_host {

int64_t stream_probe_chunk_bytes() { return kStreamChunk; }

hipError_t stream_probe_launch(const void* buf, int64_t nchunks, int32_t wgs, int32_t unroll, uint32_t* out,
                               hipStream_t s) {
  const uint8_t* b = (const uint8_t*)buf;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(stream_probe_kernel<1>, dim3((unsigned)wgs), dim3(256), 0, s, b, (uint32_t)nchunks, out); break;
    case 2: hipLaunchKernelGGL(stream_probe_kernel<2>, dim3((unsigned)wgs), dim3(256), 0, s, b, (uint32_t)nchunks, out); break;
    case 4: hipLaunchKernelGGL(stream_probe_kernel<4>, dim3((unsigned)wgs), dim3(256), 0, s, b, (uint32_t)nchunks, out); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dsa_host
