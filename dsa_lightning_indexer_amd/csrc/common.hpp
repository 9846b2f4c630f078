// Shared device/host helpers for the gfx950 kernels (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/dsa.h"

namespace dsa {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// Monotone map fp32 -> u32: a > b (as reals) iff key(a) > key(b).  Both zeros
// map to the key of +0.0 so that -0.0 and +0.0 tie (and the lower position wins).
__device__ __forceinline__ uint32_t order_key(float x) {
  uint32_t b = __float_as_uint(x);
  b = (x == 0.0f) ? 0u : b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar) value:
// derived from it, buffer resources and per-wave bases stay in SGPRs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// Workgroup barrier for LDS data only: waits for this wave's LDS accesses
// (lgkmcnt) but not for global loads in flight, unlike __syncthreads, whose
// release fence drains every outstanding vector-memory operation.  The asm
// keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void sync_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Buffer-resource view of a byte range (gfx9 family resource word: raw buffer,
// out-of-range reads return zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// One buffer_load ... lds of `bytes` (4 or 16) per lane at byte offset voff,
// landing at LDS address lds + bytes * lane.  Issued from inline asm so that
// the compiler's wait-count tracking, which would otherwise wait for the load
// before every later LDS read of the same array, leaves it alone; callers wait
// for it explicitly (vmcnt) before the barrier that publishes the data.  The
// load takes its LDS base from M0, which the compiler reserves: the asm saves
// M0, sets it (one wait state before the load reads it) and restores it.  Its
// only register output is that saved copy.
template <int BYTES>
__device__ __forceinline__ void lds_dma(__amdgpu_buffer_rsrc_t r, const uint8_t* lds, uint32_t voff) {
  const uint32_t a = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint8_t*)lds;
  uint32_t saved;
  if constexpr (BYTES == 16)
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(a), "v"(voff), "s"(r) : "memory");
  else
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %2, %3, 0 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(a), "v"(voff), "s"(r) : "memory");
}

// vmcnt(N) wait (N < 64), leaving lgkmcnt and expcnt alone.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Lane-mask helpers (wave64).
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}
__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Exclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
  const int lane = threadIdx.x & 63;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  *total = __shfl(x, 63, 64);
  return x - v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace dsa

// Host-side launch helpers (defined in the kernel translation units).
namespace dsa_host {

struct SelectPlan {
  // rows are flattened (batch, n_q); row r has query position q_pos0 + r % n_q and
  // candidates s = 0..min(t, n_k-1).
  int64_t rows;
  int32_t n_q;
  int64_t q_pos0;
  int32_t n_k;
  int32_t k;
  int64_t row_stride;  // elements between score rows
};

constexpr int kSelectMaxRow = 1024 * 4096;   // longest score row the select handles
size_t select_workspace_bytes(int64_t rows);
// Zero the select state (fill kernel; safe under stream capture).
hipError_t select_prepare(void* ws, int64_t rows, hipStream_t s);
// First histogram pass over materialised scores (skip if the producer fused it).
hipError_t select_hist1(const float* scores, const SelectPlan& p, void* ws, hipStream_t s);
// Remaining passes and the ordered write of idx [rows, k].
hipError_t select_finish(const float* scores, const SelectPlan& p, void* ws, int32_t* idx,
                         hipStream_t s);

// Few long rows (at most kSelectFewRows), select_few.hip: a histogram of the top
// 12 bits of each row's order keys (kFewHistBins u32 counters per row, rows
// FewHist::row_words apart) names the bin of the k-th key; the keys of that bin
// and above are collected and selected exactly.  Sequence: select_few_prepare
// (zero the counters), the histogram (fused into the decode scan, or
// select_few_hist_scores over given scores), select_few_finish.
constexpr int64_t kSelectFewRows = 256;
constexpr int kFewHistBins = 4096;
constexpr int kFewHistOffset = 4;            // u32 words before a row's histogram
struct FewHist {
  uint32_t* base;                            // histogram of row 0
  int64_t row_words;                         // u32 words between rows
};
size_t select_few_ws_bytes(int64_t rows);
FewHist select_few_hist(void* ws);
hipError_t select_few_prepare(void* ws, int64_t rows, hipStream_t s);
hipError_t select_few_hist_scores(const float* scores, const SelectPlan& p, void* ws, hipStream_t s);
hipError_t select_few_finish(const float* scores, const SelectPlan& p, void* ws, int32_t* idx, hipStream_t s);

hipError_t indexer_scores_f32(const dsa_indexer_args& a, int64_t row0, int64_t rows, float* out,
                              int64_t out_row_stride, hipStream_t s);
hipError_t indexer_scores_mfma(const dsa_indexer_args& a, int64_t row0, int64_t rows, float* out,
                               hipStream_t s);
// Fused prefill INDEXER + Top-k: persistent grid, one or two query rows per
// wave; each query row in flight owns one of kTopkWaveSlots candidate slices in
// the workspace (topk_fused_ws_bytes()).
constexpr int kTopkWaveSlots = 4096;
size_t topk_fused_ws_bytes();
hipError_t indexer_topk_fused(const dsa_indexer_args& a, int32_t k, int32_t* idx, void* ws, hipStream_t s);
// Decode-shaped scan: fp32 scores of every (row, s) into `scores` [batch*n_q, n_k],
// plus each row's key histogram into `hist` (zeroed beforehand) when given.
hipError_t indexer_scan(const dsa_indexer_args& a, float* scores, const FewHist* hist, hipStream_t s);
bool indexer_mfma_supported(const dsa_indexer_args& a);

// Distillation loss over the selected Top-k and its backward (distill.hip).
bool distill_supported(const dsa_indexer_args& a, int32_t topk, int32_t r);
hipError_t distill_launch(const dsa_indexer_args& a, int32_t topk, int32_t r, const int32_t* idx,
                          const float* teachers, float* loss, float* delta, float* dq, float* dw, float* dk,
                          hipStream_t s);

size_t sparse_attn_ws_bytes(const dsa_sparse_attn_args& a);
hipError_t sparse_attn_launch(const dsa_sparse_attn_args& a, void* ws, hipStream_t s);

hipError_t overlap_launch(const int32_t* a, const int32_t* b, int64_t rows, int32_t k,
                          int32_t* row_counts, unsigned long long* total, hipStream_t s);

// Output similarity for the pattern search (similarity.hip).
hipError_t row_cosine_launch(const float* a, const float* b, int64_t rows, int64_t width, float* row_cos,
                             double* mean, hipStream_t s);
hipError_t identity_f64_launch(double* m, int64_t n, hipStream_t s);
// Gather-bandwidth probe over 1152-byte latent rows (gather_probe.hip).
int64_t gather_probe_out_words(int64_t n_q, int32_t mode);
hipError_t gather_probe_launch(const void* table, int32_t n_rows, const int32_t* idx, int64_t n_q, int32_t topk,
                               int32_t mode, uint32_t* out, hipStream_t s);

// Streaming read probe over a contiguous buffer of 16-KiB chunks (gather_probe.hip).
int64_t stream_probe_chunk_bytes();
hipError_t stream_probe_launch(const void* buf, int64_t nchunks, int32_t wgs, int32_t unroll, uint32_t* out,
                               hipStream_t s);

// indexcache_forward's validation and workspace need (api.cpp).
dsa_status forward_workspace_need(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k, size_t* need);
// Sets the thread-local text dsa_last_error() returns (api.cpp) and returns st.
dsa_status set_error(dsa_status st, const char* msg);

// Sharing-pattern dynamic program, host code (pattern_search.cpp).  False if no
// admissible pattern exists.
bool pattern_search_dp(const double* S, int n, int M, char* pattern, double* score);

}  // namespace dsa_host
