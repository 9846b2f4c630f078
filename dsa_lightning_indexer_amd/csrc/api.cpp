// C ABI: argument validation, workspace sizing, kernel dispatch and the
// IndexCache F/S layer loop ([IC-SUMMARY] Algorithm (b); [DSA-NOTES] §2.2).
// Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <climits>
#include <cstring>
#include <string>

#include "common.hpp"

namespace {

thread_local std::string g_last_error;

dsa_status fail(dsa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

dsa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return DSA_OK;
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// ------------------------------------------------------------------ indexer args
dsa_status check_indexer_shape(const dsa_indexer_args* a) {
  if (!a) return fail(DSA_ERR_INVALID, "indexer args is NULL");
  if (a->dtype != DSA_F32 && a->dtype != DSA_BF16 && a->dtype != DSA_FP8_E4M3)
    return fail(DSA_ERR_INVALID, "unknown indexer dtype %d", a->dtype);
  if (a->batch < 1 || a->n_q < 1 || a->n_k < 1)
    return fail(DSA_ERR_INVALID, "batch, n_q and n_k must be >= 1 (got %d, %d, %d)", a->batch,
                a->n_q, a->n_k);
  if (a->q_pos0 < 0) return fail(DSA_ERR_INVALID, "q_pos0 must be >= 0");
  if (a->heads < 1 || a->heads > DSA_MAX_INDEXER_HEADS)
    return fail(DSA_ERR_UNSUPPORTED, "indexer heads must be 1..%d (got %d)", DSA_MAX_INDEXER_HEADS,
                a->heads);
  if (a->dtype == DSA_F32) {
    if (a->dim < 1 || a->dim > 256 || a->heads * a->dim > 8192)
      return fail(DSA_ERR_UNSUPPORTED, "F32 indexer needs dim 1..256 and heads*dim <= 8192");
    if (a->n_q > 65535 || a->batch > 65535)
      return fail(DSA_ERR_UNSUPPORTED, "F32 indexer needs n_q and batch <= 65535");
  } else if (!dsa_host::indexer_mfma_supported(*a)) {
    return fail(DSA_ERR_UNSUPPORTED, "indexer dim %d unsupported for dtype %d (bf16: 32/64/128, fp8: 64/128)",
                a->dim, a->dtype);
  }
  if (a->k_batch_stride != 0 && a->k_batch_stride < (int64_t)a->n_k * a->dim)
    return fail(DSA_ERR_INVALID, "k_batch_stride smaller than n_k*dim");
  if (a->k_scale_batch_stride != 0 && a->k_scale_batch_stride < a->n_k)
    return fail(DSA_ERR_INVALID, "k_scale_batch_stride smaller than n_k");
  return DSA_OK;
}

dsa_status check_indexer_data(const dsa_indexer_args* a) {
  if (!a->q || !a->k || !a->w) return fail(DSA_ERR_INVALID, "indexer q, k and w must be non-NULL");
  if (a->dtype == DSA_FP8_E4M3 && (!a->q_scale || !a->k_scale))
    return fail(DSA_ERR_INVALID, "fp8 indexer needs q_scale and k_scale");
  const size_t al = a->dtype == DSA_F32 ? 4 : 16;
  if (!aligned(a->q, al) || !aligned(a->k, al) || !aligned(a->w, 4))
    return fail(DSA_ERR_INVALID, "indexer q/k must be %zu-byte aligned, w 4-byte aligned", al);
  if (a->dtype != DSA_F32 && a->k_batch_stride != 0 &&
      (a->k_batch_stride * (a->dtype == DSA_BF16 ? 2 : 1)) % 16 != 0)
    return fail(DSA_ERR_INVALID, "k batch stride must keep 16-byte row alignment");
  return DSA_OK;
}

bool decode_shaped(const dsa_indexer_args* a) {
  return (int64_t)a->batch * a->n_q <= 256 && a->n_k > 2048;
}

enum TopkPath { PATH_SELECT, PATH_F32, PATH_FUSED, PATH_SCAN };

TopkPath topk_path(const dsa_indexer_args* a, const float* scores) {
  if (scores) return PATH_SELECT;
  if (a->dtype == DSA_F32) return PATH_F32;
  return decode_shaped(a) ? PATH_SCAN : PATH_FUSED;
}

size_t topk_ws(const dsa_indexer_args* a, const float* scores) {
  const int64_t rows = (int64_t)a->batch * a->n_q;
  const size_t sel = rows <= dsa_host::kSelectFewRows ? dsa_host::select_few_ws_bytes(rows)
                                                       : dsa_host::select_workspace_bytes(rows);
  switch (topk_path(a, scores)) {
    case PATH_SELECT: return align_up(sel);
    case PATH_F32:
    case PATH_SCAN:
      return align_up((size_t)rows * a->n_k * sizeof(float)) + align_up(sel);
    case PATH_FUSED: return align_up(dsa_host::topk_fused_ws_bytes());
  }
  return 0;
}

// Limits of the kernels the chosen Top-k path launches.  Every caller that
// scores an F layer (dsa_topk, indexcache_forward, dsa_similarity_matrix) runs
// this before enqueueing anything.
dsa_status check_topk_path(const dsa_indexer_args* a, const float* scores) {
  const TopkPath path = topk_path(a, scores);
  if (path != PATH_FUSED) {
    // the materialised-score selects keep per-chunk state for at most this many scores per row
    if (a->n_k > (int32_t)dsa_host::kSelectMaxRow)
      return fail(DSA_ERR_UNSUPPORTED, "this Top-k path handles rows of at most %d scores", dsa_host::kSelectMaxRow);
    return DSA_OK;
  }
  // the fused kernels address one batch's keys with 32-bit byte offsets and
  // hold query positions in 32-bit integers
  if ((int64_t)a->n_k * a->dim * (a->dtype == DSA_BF16 ? 2 : 1) >= (int64_t)1 << 31)
    return fail(DSA_ERR_UNSUPPORTED, "fused indexer+Top-k needs n_k * dim * element size < 2^31 bytes");
  if (a->q_pos0 + a->n_q > (int64_t)INT32_MAX)
    return fail(DSA_ERR_UNSUPPORTED, "fused indexer+Top-k needs q_pos0 + n_q <= 2^31 - 1");
  return DSA_OK;
}

dsa_status check_topk(const dsa_indexer_args* a, const float* scores, int32_t k, const int32_t* idx,
                      const void* ws, size_t ws_bytes) {
  dsa_status st = check_indexer_shape(a);
  if (st != DSA_OK) return st;
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "k must be 1..%d (got %d)", DSA_MAX_TOPK, k);
  if (!idx) return fail(DSA_ERR_INVALID, "idx is NULL");
  if (!aligned(idx, 4)) return fail(DSA_ERR_INVALID, "idx must be 4-byte aligned");
  if (scores) {
    if (!aligned(scores, 4)) return fail(DSA_ERR_INVALID, "scores must be 4-byte aligned");
  } else {
    st = check_indexer_data(a);
    if (st != DSA_OK) return st;
  }
  st = check_topk_path(a, scores);
  if (st != DSA_OK) return st;
  const size_t need = topk_ws(a, scores);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (ws && !aligned(ws, kAlign)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  return DSA_OK;
}

dsa_status run_topk(const dsa_indexer_args* a, const float* scores, int32_t k, int32_t* idx, void* ws,
                    hipStream_t s) {
  const int64_t rows = (int64_t)a->batch * a->n_q;
  dsa_host::SelectPlan plan{rows, a->n_q, a->q_pos0, a->n_k, k, (int64_t)a->n_k};
  const TopkPath path = topk_path(a, scores);
  hipError_t e = hipSuccess;
  if (path == PATH_FUSED) {
    e = dsa_host::indexer_topk_fused(*a, k, idx, ws, s);
    return hip_status(e, "fused indexer+topk launch");
  }
  const float* sc = scores;
  void* sel_ws = ws;
  const bool few = rows <= dsa_host::kSelectFewRows;
  if (path == PATH_F32 || path == PATH_SCAN) {
    float* buf = (float*)ws;
    sel_ws = (char*)ws + align_up((size_t)rows * a->n_k * sizeof(float));
    sc = buf;
  }
  if (few) {
    e = dsa_host::select_few_prepare(sel_ws, rows, s);
    if (e != hipSuccess) return hip_status(e, "top-k select launch");
  }
  if (path == PATH_F32) {
    e = dsa_host::indexer_scores_f32(*a, 0, a->n_q, (float*)sc, a->n_k, s);
  } else if (path == PATH_SCAN) {
    // the scan builds the few-row select's key histograms as it writes the scores
    const dsa_host::FewHist h = dsa_host::select_few_hist(sel_ws);
    e = dsa_host::indexer_scan(*a, (float*)sc, few ? &h : nullptr, s);
  }
  if (e != hipSuccess) return hip_status(e, "indexer scoring launch");
  if (few) {
    if (path != PATH_SCAN) e = dsa_host::select_few_hist_scores(sc, plan, sel_ws, s);
    if (e == hipSuccess) e = dsa_host::select_few_finish(sc, plan, sel_ws, idx, s);
  } else {
    e = dsa_host::select_prepare(sel_ws, rows, s);
    if (e == hipSuccess) e = dsa_host::select_hist1(sc, plan, sel_ws, s);
    if (e == hipSuccess) e = dsa_host::select_finish(sc, plan, sel_ws, idx, s);
  }
  return hip_status(e, "top-k select launch");
}

// ------------------------------------------------------------------ attention args
dsa_status check_sa(const dsa_sparse_attn_args* a, bool need_idx, bool need_out = true) {
  if (!a) return fail(DSA_ERR_INVALID, "sparse attention args is NULL");
  if (a->dtype != DSA_F32 && a->dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "sparse attention dtype must be F32 or BF16 (got %d)", a->dtype);
  if (a->batch < 1 || a->n_q < 1 || a->n_k < 1 || a->heads < 1 || a->kv_heads < 1)
    return fail(DSA_ERR_INVALID, "sparse attention sizes must be >= 1");
  if (a->heads % a->kv_heads) return fail(DSA_ERR_INVALID, "heads must be a multiple of kv_heads");
  if (a->d_qk < 1 || a->d_qk > 1024 || a->d_v < 1 || a->d_v > 1024)
    return fail(DSA_ERR_UNSUPPORTED, "d_qk and d_v must be 1..1024");
  if (!a->v && a->d_v > a->d_qk) return fail(DSA_ERR_INVALID, "latent V needs d_v <= d_qk");
  if (a->topk < 1 || a->topk > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "topk must be 1..%d", DSA_MAX_TOPK);
  if (!a->q || !a->kv || (need_out && !a->out) || (need_idx && !a->idx))
    return fail(DSA_ERR_INVALID, "sparse attention q, kv, idx and out must be non-NULL");
  if (!(a->scale == a->scale)) return fail(DSA_ERR_INVALID, "scale is NaN");
  const int64_t row = (int64_t)a->kv_heads * a->d_qk;
  if (a->kv_batch_stride != 0 && a->kv_batch_stride < (int64_t)a->n_k * row)
    return fail(DSA_ERR_INVALID, "kv_batch_stride too small");
  if (a->v && a->v_batch_stride != 0 && a->v_batch_stride < (int64_t)a->n_k * a->kv_heads * a->d_v)
    return fail(DSA_ERR_INVALID, "v_batch_stride too small");
  const size_t al = a->dtype == DSA_BF16 ? 16 : 4;
  if (!aligned(a->q, al) || !aligned(a->kv, al) || (a->out && !aligned(a->out, 4)) ||
      (a->idx && !aligned(a->idx, 4)) || (a->v && !aligned(a->v, 4)))
    return fail(DSA_ERR_INVALID, "sparse attention pointers misaligned");
  if (a->dtype == DSA_BF16 && a->kv_batch_stride % 8 != 0)
    return fail(DSA_ERR_INVALID, "bf16 kv batch stride must keep 16-byte alignment");
  return DSA_OK;
}

}  // namespace

namespace dsa_host {
// Error text for callers in other translation units (same thread-local buffer).
dsa_status set_error(dsa_status st, const char* msg) { return fail(st, "%s", msg); }
}  // namespace dsa_host

extern "C" {

int32_t dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_string(int32_t st) {
  switch (st) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported configuration";
    case DSA_ERR_WORKSPACE: return "workspace missing or too small";
    case DSA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* dsa_last_error(void) { return g_last_error.c_str(); }

dsa_status dsa_indexer_scores(const dsa_indexer_args* a, int64_t row0, int64_t rows, float* scores,
                              hipStream_t stream) {
  g_last_error.clear();
  dsa_status st = check_indexer_shape(a);
  if (st != DSA_OK) return st;
  st = check_indexer_data(a);
  if (st != DSA_OK) return st;
  if (!scores || !aligned(scores, 4)) return fail(DSA_ERR_INVALID, "scores must be non-NULL and 4-byte aligned");
  if (row0 < 0 || rows < 1 || row0 + rows > a->n_q)
    return fail(DSA_ERR_INVALID, "row window [%lld, %lld) outside [0, %d)", (long long)row0,
                (long long)(row0 + rows), a->n_q);
  hipError_t e = a->dtype == DSA_F32
                     ? dsa_host::indexer_scores_f32(*a, row0, rows, scores, a->n_k, stream)
                     : dsa_host::indexer_scores_mfma(*a, row0, rows, scores, stream);
  return hip_status(e, "indexer scores launch");
}

size_t dsa_topk_workspace_size(const dsa_indexer_args* a, const float* scores, int32_t k) {
  (void)k;
  if (!a || check_indexer_shape(a) != DSA_OK) return 0;
  return topk_ws(a, scores);
}

dsa_status dsa_topk(const dsa_indexer_args* a, const float* scores, int32_t k, int32_t* idx, void* ws,
                    size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  dsa_status st = check_topk(a, scores, k, idx, ws, ws_bytes);
  if (st != DSA_OK) return st;
  return run_topk(a, scores, k, idx, ws, stream);
}

size_t dsa_sparse_attn_workspace_size(const dsa_sparse_attn_args* a) {
  // (the size depends on the shapes only: idx and out may still be NULL)
  if (!a || check_sa(a, false, false) != DSA_OK) return 0;
  return align_up(dsa_host::sparse_attn_ws_bytes(*a));
}

dsa_status dsa_sparse_attn(const dsa_sparse_attn_args* a, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  dsa_status st = check_sa(a, true);
  if (st != DSA_OK) return st;
  const size_t need = dsa_host::sparse_attn_ws_bytes(*a);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (ws && !aligned(ws, kAlign)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  return hip_status(dsa_host::sparse_attn_launch(*a, ws, stream), "sparse attention launch");
}

// ws_topk / ws_attn (optional): the largest Top-k and attention workspace needs
// on their own (the overlapped loop gives each its own region).
static dsa_status check_forward(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k,
                                size_t* ws_need, size_t* ws_topk = nullptr, size_t* ws_attn = nullptr) {
  if (!pattern) return fail(DSA_ERR_INVALID, "pattern is NULL");
  if (n < 1) return fail(DSA_ERR_INVALID, "n_layers must be >= 1");
  if ((int64_t)strnlen(pattern, (size_t)n + 1) != n)
    return fail(DSA_ERR_INVALID, "pattern length differs from n_layers=%d", n);
  for (int32_t l = 0; l < n; ++l)
    if (pattern[l] != 'F' && pattern[l] != 'S')
      return fail(DSA_ERR_INVALID, "pattern[%d]='%c' is neither F nor S", l, pattern[l]);
  if (pattern[0] != 'F') return fail(DSA_ERR_INVALID, "the first layer must be F");
  if (!layers) return fail(DSA_ERR_INVALID, "layers is NULL");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "k must be 1..%d", DSA_MAX_TOPK);
  size_t need = 0, need_topk = 0, need_attn = 0;
  int32_t src = -1;
  for (int32_t l = 0; l < n; ++l) {
    const dsa_layer& L = layers[l];
    if (pattern[l] == 'F') {
      src = l;
      dsa_status st = check_indexer_shape(&L.ix);
      if (st == DSA_OK) st = check_indexer_data(&L.ix);
      if (st == DSA_OK) st = check_topk_path(&L.ix, nullptr);
      if (st != DSA_OK) return fail(st, "layer %d (F): %s", l, g_last_error.c_str());
      if (!L.idx_out || !aligned(L.idx_out, 4)) return fail(DSA_ERR_INVALID, "layer %d (F): idx_out NULL/misaligned", l);
      const size_t w = topk_ws(&L.ix, nullptr);
      if (w > need_topk) need_topk = w;
    }
    dsa_status st = check_sa(&L.sa, false);
    if (st != DSA_OK) return fail(st, "layer %d: %s", l, g_last_error.c_str());
    const dsa_indexer_args& S = layers[src].ix;
    if (L.sa.batch != S.batch || L.sa.n_q != S.n_q || L.sa.topk != k)
      return fail(DSA_ERR_INVALID, "layer %d: attention batch/n_q/topk (%d,%d,%d) must match the cached "
                  "index tensor (%d,%d,%d)", l, L.sa.batch, L.sa.n_q, L.sa.topk, S.batch, S.n_q, k);
    const size_t w = align_up(dsa_host::sparse_attn_ws_bytes(L.sa));
    if (w > need_attn) need_attn = w;
  }
  need = need_topk > need_attn ? need_topk : need_attn;
  *ws_need = need;
  if (ws_topk) *ws_topk = need_topk;
  if (ws_attn) *ws_attn = need_attn;
  return DSA_OK;
}

// The overlapped loop's extra conditions: an F layer l > first attends with the
// previous F layer's tensor while its own indexer writes idx_out, so the
// shapes must agree and the two buffers must differ.
static dsa_status check_forward_mli(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k,
                                    size_t* ws_need, size_t* ws_topk) {
  size_t need = 0, need_topk = 0, need_attn = 0;
  dsa_status st = check_forward(pattern, n, layers, k, &need, &need_topk, &need_attn);
  if (st != DSA_OK) return st;
  int32_t prev = -1;
  for (int32_t l = 0; l < n; ++l) {
    if (pattern[l] != 'F') continue;
    if (prev >= 0) {
      const dsa_layer& L = layers[l];
      const dsa_indexer_args& P = layers[prev].ix;
      if (L.sa.batch != P.batch || L.sa.n_q != P.n_q)
        return fail(DSA_ERR_INVALID, "layer %d: attention batch/n_q (%d,%d) must match the index tensor of F "
                    "layer %d (%d,%d) it attends with", l, L.sa.batch, L.sa.n_q, prev, P.batch, P.n_q);
      if (L.idx_out == layers[prev].idx_out)
        return fail(DSA_ERR_INVALID, "layers %d and %d (consecutive F layers) share idx_out: the overlapped loop "
                    "writes one while attention reads the other", prev, l);
    }
    prev = l;
  }
  // the indexer stream and the attention stream each get their own region
  *ws_topk = need_topk;
  *ws_need = need_topk + need_attn;
  return DSA_OK;
}

}  // extern "C"

namespace dsa_host {
dsa_status forward_workspace_need(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k, size_t* need) {
  g_last_error.clear();
  *need = 0;
  return check_forward(pattern, n, layers, k, need);
}
}  // namespace dsa_host

extern "C" {

size_t indexcache_forward_workspace_size(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k) {
  size_t need = 0;
  if (check_forward(pattern, n, layers, k, &need) != DSA_OK) return 0;
  return need;
}

dsa_status indexcache_forward(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k,
                              int32_t* src_layer, void* ws, size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  size_t need = 0;
  dsa_status st = check_forward(pattern, n, layers, k, &need);
  if (st != DSA_OK) return st;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (ws && !aligned(ws, kAlign)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  const int32_t* cache = nullptr;   // the current index tensor (T_cache)
  int32_t src = -1;
  for (int32_t l = 0; l < n; ++l) {
    const dsa_layer& L = layers[l];
    if (pattern[l] == 'F') {
      // F: INDEXER + Top-k; the result replaces the cached tensor.
      st = run_topk(&L.ix, nullptr, k, L.idx_out, ws, stream);
      if (st != DSA_OK) return st;
      cache = L.idx_out;
      src = l;
    }
    // S: reuse the cached tensor; no indexer launch, L.ix and L.idx_out untouched.
    if (src_layer) src_layer[l] = src;
    dsa_sparse_attn_args sa = L.sa;
    sa.idx = cache;
    st = hip_status(dsa_host::sparse_attn_launch(sa, ws, stream), "sparse attention launch");
    if (st != DSA_OK) return st;
  }
  return DSA_OK;
}

size_t indexcache_forward_mli_workspace_size(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k) {
  size_t need = 0, need_topk = 0;
  if (check_forward_mli(pattern, n, layers, k, &need, &need_topk) != DSA_OK) return 0;
  return need;
}

dsa_status indexcache_forward_mli(const char* pattern, int32_t n, const dsa_layer* layers, int32_t k,
                                  int32_t* src_layer, void* ws, size_t ws_bytes, hipStream_t stream,
                                  hipStream_t index_stream) {
  g_last_error.clear();
  size_t need = 0, need_topk = 0;
  dsa_status st = check_forward_mli(pattern, n, layers, k, &need, &need_topk);
  if (st != DSA_OK) return st;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws ? ws_bytes : 0);
  if (ws && !aligned(ws, kAlign)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  void* ws_index = ws;
  void* ws_attn = need > need_topk ? (void*)((uint8_t*)ws + need_topk) : nullptr;
  const bool two = index_stream != stream;
  // One event per F layer marks its index tensor done (on the indexer stream);
  // one marks where the attention stream stands when layer l starts (the
  // layer's input is ready): layer l's indexer waits for it.
  int32_t n_f = 0;
  for (int32_t l = 0; l < n; ++l) n_f += pattern[l] == 'F';
  hipEvent_t* ev = nullptr;
  int32_t n_ev = 0;
  auto cleanup = [&]() {
    for (int32_t i = 0; i < n_ev; ++i) (void)hipEventDestroy(ev[i]);
    delete[] ev;
  };
  if (two) {
    ev = new hipEvent_t[2 * (size_t)n_f];
    for (; n_ev < 2 * n_f; ++n_ev) {
      hipError_t e = hipEventCreateWithFlags(&ev[n_ev], hipEventDisableTiming);
      if (e != hipSuccess) {
        cleanup();
        return hip_status(e, "event create");
      }
    }
  }
  int32_t prev = -1;        // latest F layer whose indexer was enqueued
  int32_t fi = 0;           // F layers seen so far
  int32_t waited = -1;      // latest F layer the attention stream has waited for
  hipError_t e = hipSuccess;
  for (int32_t l = 0; l < n && e == hipSuccess && st == DSA_OK; ++l) {
    const dsa_layer& L = layers[l];
    int32_t done_ev = -1;
    if (pattern[l] == 'F') {
      if (two) {
        e = hipEventRecord(ev[2 * fi], stream);                       // layer l's input is ready
        if (e == hipSuccess) e = hipStreamWaitEvent(index_stream, ev[2 * fi], 0);
        if (e != hipSuccess) break;
      }
      st = run_topk(&L.ix, nullptr, k, L.idx_out, ws_index, two ? index_stream : stream);
      if (st != DSA_OK) break;
      if (two) e = hipEventRecord(ev[2 * fi + 1], index_stream);
      done_ev = 2 * fi + 1;
      ++fi;
    }
    // attend with the previous F layer's tensor; the first layer with its own
    const int32_t src = prev >= 0 ? prev : l;
    if (src_layer) src_layer[l] = src;
    if (two && src > waited && e == hipSuccess) {
      // the event of F layer src: its own (first layer) or the one recorded when it ran
      int32_t src_ev = done_ev;
      if (src != l) {
        int32_t f = 0;
        for (int32_t j = 0; j < src; ++j) f += pattern[j] == 'F';
        src_ev = 2 * f + 1;
      }
      e = hipStreamWaitEvent(stream, ev[src_ev], 0);
      waited = src;
    }
    if (e != hipSuccess) break;
    dsa_sparse_attn_args sa = L.sa;
    sa.idx = layers[src].idx_out;
    st = hip_status(dsa_host::sparse_attn_launch(sa, ws_attn, stream), "sparse attention launch");
    if (pattern[l] == 'F') prev = l;
  }
  // join: later work on `stream` is ordered after every indexer of this call
  if (two && e == hipSuccess && st == DSA_OK && fi > 0) e = hipStreamWaitEvent(stream, ev[2 * (fi - 1) + 1], 0);
  cleanup();
  if (st != DSA_OK) return st;
  return hip_status(e, "stream ordering");
}

dsa_status dsa_indexer_distill(const dsa_distill_args* a, hipStream_t stream) {
  g_last_error.clear();
  if (!a) return fail(DSA_ERR_INVALID, "distillation args is NULL");
  dsa_status st = check_indexer_shape(&a->ix);
  if (st == DSA_OK) st = check_indexer_data(&a->ix);
  if (st != DSA_OK) return st;
  if (a->topk < 1 || a->topk > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "topk must be 1..%d", DSA_MAX_TOPK);
  if (a->n_teachers < 1 || a->n_teachers > 8) return fail(DSA_ERR_INVALID, "n_teachers must be 1..8");
  if (!dsa_host::distill_supported(a->ix, a->topk, a->n_teachers))
    return fail(DSA_ERR_UNSUPPORTED, "distillation needs BF16 indexer inputs with dim 128 and at most 64 heads");
  if (!a->idx || !a->teachers || !a->loss || !a->delta || !a->dq || !a->dw || !a->dk)
    return fail(DSA_ERR_INVALID, "idx, teachers, loss, delta, dq, dw and dk are required");
  if (!aligned(a->idx, 4) || !aligned(a->teachers, 4) || !aligned(a->loss, 4) || !aligned(a->delta, 4) ||
      !aligned(a->dw, 4) || !aligned(a->dk, 4) || !aligned(a->dq, 16))
    return fail(DSA_ERR_INVALID, "misaligned pointer (dq needs 16 bytes, the others 4)");
  return hip_status(dsa_host::distill_launch(a->ix, a->topk, a->n_teachers, a->idx, a->teachers, a->loss,
                                             a->delta, a->dq, a->dw, a->dk, stream),
                    "distillation launch");
}

dsa_status dsa_index_overlap(const int32_t* a, const int32_t* b, int64_t rows, int32_t k,
                             int32_t* row_counts, unsigned long long* total, hipStream_t stream) {
  g_last_error.clear();
  if (rows < 0) return fail(DSA_ERR_INVALID, "rows must be >= 0");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "k must be 1..%d", DSA_MAX_TOPK);
  if (rows > 0 && (!a || !b)) return fail(DSA_ERR_INVALID, "index tensors must be non-NULL");
  if (!row_counts && !total) return fail(DSA_ERR_INVALID, "need row_counts and/or total");
  return hip_status(dsa_host::overlap_launch(a, b, rows, k, row_counts, total, stream), "overlap launch");
}

dsa_status dsa_row_cosine(const float* a, const float* b, int64_t rows, int64_t width, float* row_cos,
                          double* mean, hipStream_t stream) {
  g_last_error.clear();
  if (rows < 1 || rows > INT32_MAX) return fail(DSA_ERR_INVALID, "rows must be 1..2^31-1");
  if (width < 4 || width > ((int64_t)1 << 26) || width % 4 != 0)
    return fail(DSA_ERR_INVALID, "width must be a multiple of 4 in [4, 2^26]");
  if (!a || !b || !row_cos) return fail(DSA_ERR_INVALID, "a, b and row_cos are required");
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(row_cos, 4) || (mean && !aligned(mean, 8)))
    return fail(DSA_ERR_INVALID, "a and b must be 16-byte aligned, row_cos 4, mean 8");
  return hip_status(dsa_host::row_cosine_launch(a, b, rows, width, row_cos, mean, stream), "cosine launch");
}

// Workspace: O_own and O_other (fp32 [rows, heads * d_v] each, sized for the
// widest layer), the per-row cosines, then the Top-k / attention workspace
// (the calls run one after another on the stream and share it).
struct SimLayout {
  size_t out_bytes, cos_bytes, tail_bytes, total;
};

// sizing: only shapes matter (the index tensors need not exist yet).
static dsa_status check_similarity(int32_t n, const dsa_layer* layers, int32_t k, SimLayout* lay, bool sizing) {
  if (n < 1 || n > 1024) return fail(DSA_ERR_INVALID, "n_layers must be 1..1024");
  if (!layers) return fail(DSA_ERR_INVALID, "layers is NULL");
  if (k < 1 || k > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "k must be 1..%d", DSA_MAX_TOPK);
  size_t width = 0, tail = 0;
  const int64_t rows = (int64_t)layers[0].ix.batch * layers[0].ix.n_q;
  for (int32_t l = 0; l < n; ++l) {
    const dsa_layer& L = layers[l];
    dsa_status st = check_indexer_shape(&L.ix);
    if (st == DSA_OK) st = check_indexer_data(&L.ix);
    if (st == DSA_OK) st = check_topk_path(&L.ix, nullptr);
    if (st != DSA_OK) return fail(st, "layer %d: %s", l, g_last_error.c_str());
    if (!sizing && (!L.idx_out || !aligned(L.idx_out, 4)))
      return fail(DSA_ERR_INVALID, "layer %d: idx_out NULL/misaligned", l);
    st = check_sa(&L.sa, false, false);   // sa.idx and sa.out are not used
    if (st != DSA_OK) return fail(st, "layer %d: %s", l, g_last_error.c_str());
    if (L.ix.batch != layers[0].ix.batch || L.ix.n_q != layers[0].ix.n_q || L.sa.batch != L.ix.batch ||
        L.sa.n_q != L.ix.n_q || L.sa.topk != k)
      return fail(DSA_ERR_INVALID, "layer %d: indexer and attention batch/n_q must match layer 0's and "
                  "sa.topk must equal k", l);
    const int64_t w = (int64_t)L.sa.heads * L.sa.d_v;
    if (w % 4 != 0) return fail(DSA_ERR_UNSUPPORTED, "layer %d: heads * d_v must be a multiple of 4", l);
    if ((size_t)w > width) width = (size_t)w;
    const size_t t1 = topk_ws(&L.ix, nullptr);
    const size_t t2 = align_up(dsa_host::sparse_attn_ws_bytes(L.sa));
    if (t1 > tail) tail = t1;
    if (t2 > tail) tail = t2;
  }
  lay->out_bytes = align_up((size_t)rows * width * sizeof(float));
  lay->cos_bytes = align_up((size_t)rows * sizeof(float));
  lay->tail_bytes = tail;
  lay->total = 2 * lay->out_bytes + lay->cos_bytes + tail;
  return DSA_OK;
}

size_t dsa_similarity_matrix_workspace_size(int32_t n, const dsa_layer* layers, int32_t k) {
  SimLayout lay{};
  if (check_similarity(n, layers, k, &lay, true) != DSA_OK) return 0;
  return lay.total;
}

dsa_status dsa_similarity_matrix(int32_t n, const dsa_layer* layers, int32_t k, double* S, void* ws,
                                 size_t ws_bytes, hipStream_t stream) {
  g_last_error.clear();
  SimLayout lay{};
  dsa_status st = check_similarity(n, layers, k, &lay, false);
  if (st != DSA_OK) return st;
  if (!S || !aligned(S, 8)) return fail(DSA_ERR_INVALID, "S must be non-NULL and 8-byte aligned");
  if (!ws || ws_bytes < lay.total)
    return fail(DSA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", lay.total, ws ? ws_bytes : 0);
  if (!aligned(ws, kAlign)) return fail(DSA_ERR_INVALID, "workspace must be 256-byte aligned");
  uint8_t* base = (uint8_t*)ws;
  float* o_own = (float*)base;
  float* o_other = (float*)(base + lay.out_bytes);
  float* row_cos = (float*)(base + 2 * lay.out_bytes);
  void* tail = lay.tail_bytes ? (void*)(base + 2 * lay.out_bytes + lay.cos_bytes) : nullptr;
  const int64_t rows = (int64_t)layers[0].ix.batch * layers[0].ix.n_q;
  st = hip_status(dsa_host::identity_f64_launch(S, n, stream), "matrix fill launch");
  if (st != DSA_OK) return st;
  // every layer F: T_l = Top-k of its own indexer
  for (int32_t l = 0; l < n; ++l) {
    st = run_topk(&layers[l].ix, nullptr, k, layers[l].idx_out, tail, stream);
    if (st != DSA_OK) return st;
  }
  for (int32_t i = 1; i < n; ++i) {
    dsa_sparse_attn_args sa = layers[i].sa;
    const int64_t width = (int64_t)sa.heads * sa.d_v;
    sa.idx = layers[i].idx_out;
    sa.out = o_own;
    st = hip_status(dsa_host::sparse_attn_launch(sa, tail, stream), "sparse attention launch");
    if (st != DSA_OK) return st;
    for (int32_t j = 0; j < i; ++j) {
      sa.idx = layers[j].idx_out;
      sa.out = o_other;
      st = hip_status(dsa_host::sparse_attn_launch(sa, tail, stream), "sparse attention launch");
      if (st != DSA_OK) return st;
      st = hip_status(dsa_host::row_cosine_launch(o_own, o_other, rows, width, row_cos, S + (int64_t)i * n + j,
                                                  stream),
                      "cosine launch");
      if (st != DSA_OK) return st;
    }
  }
  return DSA_OK;
}

int64_t dsa_gather_probe_out_words(int64_t n_q, int32_t mode) {
  if (n_q < 1 || mode < 0 || mode > 10) return 0;
  return dsa_host::gather_probe_out_words(n_q, mode);
}

dsa_status dsa_gather_probe(const void* table, int32_t n_rows, const int32_t* idx, int64_t n_q, int32_t topk,
                            int32_t mode, uint32_t* out, hipStream_t stream) {
  g_last_error.clear();
  if (mode < 0 || mode > 10) return fail(DSA_ERR_INVALID, "mode must be 0..10");
  if (n_rows < 1 || (int64_t)n_rows * 1152 >= ((int64_t)1 << 31))
    return fail(DSA_ERR_UNSUPPORTED, "n_rows must be 1..%lld (1152-byte rows, 32-bit offsets)",
                (long long)((((int64_t)1 << 31) - 1) / 1152));
  if (n_q < 1 || n_q > (int64_t)INT32_MAX) return fail(DSA_ERR_INVALID, "n_q must be 1..2^31 - 1");
  if (topk < 1 || topk > DSA_MAX_TOPK) return fail(DSA_ERR_INVALID, "topk must be 1..%d", DSA_MAX_TOPK);
  if (!table || !idx || !out) return fail(DSA_ERR_INVALID, "table, idx and out are required");
  if (!aligned(table, 16) || !aligned(idx, 4) || !aligned(out, 4))
    return fail(DSA_ERR_INVALID, "table must be 16-byte aligned, idx and out 4-byte aligned");
  return hip_status(dsa_host::gather_probe_launch(table, n_rows, idx, n_q, topk, mode, out, stream), "probe launch");
}

dsa_status dsa_stream_probe(const void* buf, int64_t bytes, int32_t workgroups, int32_t unroll, uint32_t* out,
                            hipStream_t stream) {
  g_last_error.clear();
  const int64_t chunk = dsa_host::stream_probe_chunk_bytes();
  if (!buf || !out) return fail(DSA_ERR_INVALID, "buf and out are required");
  if (!aligned(buf, 16) || !aligned(out, 4)) return fail(DSA_ERR_INVALID, "buf must be 16-byte aligned, out 4-byte");
  if (bytes < chunk || bytes % chunk != 0 || bytes >= ((int64_t)1 << 31))
    return fail(DSA_ERR_INVALID, "bytes must be a positive multiple of %lld below 2^31", (long long)chunk);
  if (workgroups < 1 || workgroups > 65536) return fail(DSA_ERR_INVALID, "workgroups must be 1..65536");
  if (unroll != 1 && unroll != 2 && unroll != 4) return fail(DSA_ERR_INVALID, "unroll must be 1, 2 or 4");
  return hip_status(dsa_host::stream_probe_launch(buf, bytes / chunk, workgroups, unroll, out, stream), "probe launch");
}

dsa_status dsa_pattern_search(const double* S, int32_t n, int32_t n_full, char* pattern, double* score) {
  g_last_error.clear();
  if (n < 1 || n > 1024) return fail(DSA_ERR_INVALID, "n_layers must be 1..1024");
  if (n_full < 1 || n_full > n) return fail(DSA_ERR_INVALID, "n_full must be 1..n_layers");
  if (!S || !pattern) return fail(DSA_ERR_INVALID, "S and pattern are required");
  for (int32_t i = 1; i < n; ++i)
    for (int32_t j = 0; j < i; ++j)
      if (!std::isfinite(S[(int64_t)i * n + j])) return fail(DSA_ERR_INVALID, "S[%d, %d] is not finite", i, j);
  if (!dsa_host::pattern_search_dp(S, n, n_full, pattern, score))
    return fail(DSA_ERR_INVALID, "no admissible pattern");
  return DSA_OK;
}

}  // extern "C"
