/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek-Sparse-Attention step with
 * IndexCache cross-layer index reuse.
 *
 * Sources (web pages, cited by title and section):
 *   [DSA-NOTES]  "IndexCache：跨层复用稀疏索引，以及它为什么能被训练"
 *                (reading notes on IndexCache, notes.kuangjux.top)
 *   [IC-SUMMARY] "IndexCache: Accelerating Sparse Attention via Cross-Layer
 *                Index Reuse" (section-by-section summary, papercache.org)
 *
 * Conventions shared by every call
 *   - Every tensor pointer is a DEVICE pointer unless marked "host".  The
 *     caller owns every buffer, including the workspace; the library
 *     allocates no device memory and keeps no state between calls.
 *   - Layouts are row-major and dense unless a batch stride is given.
 *     Strides are in elements of the tensor's own type.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream); no
 *     call synchronises the host with the device.
 *   - Arguments are validated on the host before anything is enqueued; on a
 *     non-OK status nothing was enqueued (except DSA_ERR_HIP, which reports
 *     a launch failure of already-enqueued work).  dsa_last_error() gives a
 *     thread-local description of the last failure.
 *   - Query row i of batch b sits at absolute position t = q_pos0 + i.  Its
 *     indexer candidates are the positions s = 0..min(t, n_k-1) (causal,
 *     inclusive of s = t).
 *   - Index tensors hold, per query row, the selected positions in ascending
 *     order followed by -1 padding.  Rows with fewer than k candidates select
 *     all of them.  Ties in score go to the lower position; -0.0 equals +0.0.
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 1
#define DSA_MAX_TOPK 2048
#define DSA_MAX_INDEXER_HEADS 64

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID = 1,      /* a required pointer is NULL, a size is out of range, bad pattern */
  DSA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (dtype/shape combination) */
  DSA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than the *_workspace_size() result */
  DSA_ERR_HIP = 4           /* a HIP launch or runtime call failed */
} dsa_status;

typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2          /* OCP fp8 e4m3fn (max 448, no infinities) */
} dsa_dtype;

/*
 * Inputs of one F layer's lightning indexer ([DSA-NOTES] §2.1, score equation;
 * [IC-SUMMARY] §2.1):
 *     I[t, s] = sum_{j < heads} w[t, j] * ReLU(q[t, j, :] . k[s, :])
 * The key has no head index: one key per token serves every head.
 *
 *   q       [batch, n_q, heads, dim]   dtype
 *   q_scale [batch, n_q, heads] fp32   FP8 only (NULL otherwise): q = q_scale * code
 *   k       [batch, n_k, dim] dtype, batch stride k_batch_stride (0 = n_k*dim)
 *   k_scale [batch, n_k] fp32, batch stride k_scale_batch_stride (0 = n_k); FP8 only
 *   w       [batch, n_q, heads] fp32   dynamic per-token head weights (any sign)
 * Limits: 1 <= heads <= 64; dim in {32, 64, 128} (F32 accepts 1..256).
 */
typedef struct dsa_indexer_args {
  int32_t dtype;
  int32_t batch, n_q, n_k, heads, dim;
  int64_t q_pos0;
  const void* q;
  const float* q_scale;
  const void* k;
  int64_t k_batch_stride;
  const float* k_scale;
  int64_t k_scale_batch_stride;
  const float* w;
} dsa_indexer_args;

/*
 * Inputs of one layer's sparse core attention ([DSA-NOTES] §3, equation for
 * o_t): for query row (b, i) and head h,
 *     o = sum_{s in T} softmax_{s in T}(scale * Q[b,i,h,:] . K[b,s,g,:]) V[b,s,g,:]
 * with T the row's index set and g = h * kv_heads / heads.
 *
 *   q   [batch, n_q, heads, d_qk]      dtype (F32 or BF16)
 *   kv  [batch, n_k, kv_heads, d_qk]   dtype, batch stride kv_batch_stride (0 = dense)
 *   v   NULL: V is the first d_v columns of each kv row (MLA latent layout);
 *       else [batch, n_k, kv_heads, d_v], batch stride v_batch_stride (0 = dense)
 *   idx [batch, n_q, topk] int32; entries outside [0, n_k) (e.g. -1) select
 *       nothing; a row selecting nothing yields zeros
 *   out [batch, n_q, heads, d_v] fp32
 * Limits: d_qk, d_v <= 1024; heads % kv_heads == 0; 1 <= topk <= 2048.
 */
typedef struct dsa_sparse_attn_args {
  int32_t dtype;
  int32_t batch, n_q, n_k, heads, kv_heads, d_qk, d_v, topk;
  const void* q;
  const void* kv;
  int64_t kv_batch_stride;
  const void* v;
  int64_t v_batch_stride;
  const int32_t* idx;
  float scale;
  float* out;
} dsa_sparse_attn_args;

/* Library version of this header (DSA_ABI_VERSION). */
int32_t dsa_abi_version(void);
/* Static text for a status code. */
const char* dsa_status_string(int32_t status);
/* Thread-local text of the last failure of a call made on this thread ("" if none). */
const char* dsa_last_error(void);

/*
 * INDEXER, materialised ([DSA-NOTES] §2.1).  Writes the scores of query rows
 * [row0, row0 + rows) of every batch into scores[b][r][s] (fp32, dense
 * [batch, rows, n_k]); positions s > t are written as -inf.  For inspection and
 * for callers that want the scores; the Top-k path below never materialises them.
 */
dsa_status dsa_indexer_scores(const dsa_indexer_args* args, int64_t row0, int64_t rows,
                              float* scores, hipStream_t stream);

/*
 * Top-k ([IC-SUMMARY] notation: T_t = Top-k(I_t); Algorithm (b) steps 3-4).
 *   scores == NULL: score and select in one pass (INDEXER + Top-k).  bf16/fp8
 *     prefill never writes the score matrix; decode-shaped calls (few query
 *     rows, long n_k) and F32 inputs stage fp32 scores in the workspace.
 *   scores != NULL: select from caller scores laid out [batch, n_q, n_k]
 *     (the dsa_indexer_scores() layout with row0 = 0, rows = n_q); only
 *     positions s <= t are candidates.  args->q/k/w are then not read.
 *   k: 1..2048.  idx: [batch, n_q, k] int32 output.
 *   ws/ws_bytes: workspace of at least dsa_topk_workspace_size() bytes
 *     (may be NULL when that size is 0).
 */
size_t dsa_topk_workspace_size(const dsa_indexer_args* args, const float* scores, int32_t k);
dsa_status dsa_topk(const dsa_indexer_args* args, const float* scores, int32_t k,
                    int32_t* idx, void* ws, size_t ws_bytes, hipStream_t stream);

/* SPARSEATTN ([IC-SUMMARY] Algorithm (b) step 9; [DSA-NOTES] §3). */
size_t dsa_sparse_attn_workspace_size(const dsa_sparse_attn_args* args);
dsa_status dsa_sparse_attn(const dsa_sparse_attn_args* args, void* ws, size_t ws_bytes,
                           hipStream_t stream);

/*
 * One layer of the IndexCache loop.
 *   ix      F layers: the layer's indexer inputs.  S layers: never read (may be
 *           all zero / NULL pointers) -- an S layer has no indexer and no
 *           indexer K cache ([DSA-NOTES] §11.1-11.2).
 *   sa      the layer's own attention inputs; sa.idx is ignored and replaced
 *           by the cached index tensor.
 *   idx_out F layers: [batch, n_q, k] int32 output (becomes the cached index
 *           tensor).  S layers: never read or written.
 */
typedef struct dsa_layer {
  dsa_indexer_args ix;
  dsa_sparse_attn_args sa;
  int32_t* idx_out;
} dsa_layer;

/*
 * IndexCache inference loop ([IC-SUMMARY] Algorithm (b) and §3 core
 * mechanism; [DSA-NOTES] §2.2 FSSS FSSS trace).  pattern (host) is n_layers
 * characters of 'F'/'S' with pattern[0] == 'F'.  For l = 1..N: an F layer runs
 * INDEXER + Top-k into its idx_out, which becomes the cached index tensor
 * (overwriting the previous one); an S layer reuses the cached tensor with no
 * launch and no copy.  Every layer then runs its own sparse attention on that
 * tensor.  src_layer (host, optional) receives f(l), the 0-based layer whose
 * index tensor layer l used.  layers[] is a host array.
 */
size_t indexcache_forward_workspace_size(const char* pattern, int32_t n_layers,
                                         const dsa_layer* layers, int32_t k);
dsa_status indexcache_forward(const char* pattern, int32_t n_layers, const dsa_layer* layers,
                              int32_t k, int32_t* src_layer, void* ws, size_t ws_bytes,
                              hipStream_t stream);

/*
 * IndexCache loop with the multi-layer-indexer shift ([MLI] "核心思路" and
 * "与 IndexCache／IndexShare 的组合"; [MLI] is the page "MLI重构DeepSeek稀疏注意力：
 * 跨层复用索引免训提速", zicq.com): layer l attends with the index tensor of the
 * nearest F layer before it (layer 0 with its own), so an F layer's indexer no
 * longer precedes its own attention and can run beside it.
 *   Same pattern, layers, k and src_layer as indexcache_forward; src_layer[l]
 *   receives the shifted source.  Consecutive F layers need distinct idx_out
 *   buffers (one is written while attention reads the other), and an F layer's
 *   attention shape must match the previous F layer's index tensor.
 *   stream        sparse attention of every layer, in layer order
 *   index_stream  every F layer's INDEXER + Top-k; layer l's indexer waits until
 *                 the attention of layer l - 1 is done (layer l's input is
 *                 ready), and the first attention that uses its tensor waits
 *                 for it.  index_stream == stream runs everything in order on
 *                 one stream (the same results).  Both streams on one device.
 *   On return, later work enqueued on `stream` is ordered after every indexer of
 *   the call.  The call creates and releases 2 events per F layer (host-side
 *   runtime objects; no device memory).
 *   ws >= indexcache_forward_mli_workspace_size(): separate regions for the
 *   indexer stream and the attention stream.
 */
size_t indexcache_forward_mli_workspace_size(const char* pattern, int32_t n_layers,
                                             const dsa_layer* layers, int32_t k);
dsa_status indexcache_forward_mli(const char* pattern, int32_t n_layers, const dsa_layer* layers,
                                  int32_t k, int32_t* src_layer, void* ws, size_t ws_bytes,
                                  hipStream_t stream, hipStream_t index_stream);

/*
 * indexcache_forward without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops and
 * harnesses that forbid hipMalloc.  The call allocates nothing; the kernels'
 * scratch memory (decode scores and select state, attention split partials)
 * is one static device array of DSA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends.
 *   Arguments, outputs and results are those of indexcache_forward.
 *   The first call on a device looks up that device's array (make it before
 *   capturing a graph); the stream must belong to the current device.
 *   Layers whose workspace need (indexcache_forward_workspace_size) exceeds
 *   DSA_NOALLOC_SCRATCH_BYTES are rejected with DSA_ERR_WORKSPACE before
 *   anything is enqueued: decode stacks fit (8 x 204800 keys need about
 *   8.5 MB), prefill F layers on the fused path (537 MB of candidate slices)
 *   do not.
 *   Every call on one GPU shares that GPU's array: calls that overlap in time
 *   on one GPU (two streams, two threads) race and must be serialised by the
 *   caller.  Each call clears the state it needs before using it.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
dsa_status indexcache_forward_noalloc(const char* pattern, int32_t n_layers, const dsa_layer* layers,
                                      int32_t k, int32_t* src_layer, hipStream_t stream);

/*
 * Cross-layer overlap ([DSA-NOTES] §3.1; [IC-SUMMARY] Appendix A):
 * |T_a[r] ∩ T_b[r]| for rows r = 0..rows-1 of two index tensors with k columns
 * (each row ascending with -1 padding, as produced above).  row_counts
 * (device int32 [rows], optional) receives each row's count; *total (device
 * uint64, optional) is incremented by the sum.  overlap = sum / (rows * k).
 */
dsa_status dsa_index_overlap(const int32_t* idx_a, const int32_t* idx_b, int64_t rows,
                             int32_t k, int32_t* row_counts, unsigned long long* total,
                             hipStream_t stream);

/*
 * Training-aware IndexCache: the indexer-side multi-layer distillation loss over
 * the selected Top-k and its backward ([IC-SUMMARY] §3.2 and Proposition 1;
 * [DSA-NOTES] §5.1-5.2, §7.1-7.3).  An F layer's indexer is distilled towards
 * the attention distributions p^(1..r) of the r layers that use its index set.
 * For query row (b, i) at position t with index row T (entries outside
 * [0, min(t, n_k - 1)], e.g. the -1 padding, take no part):
 *     z_e     = sum_j w[j] ReLU(q[j] . k[T_e])                 (indexer scores)
 *     pi      = softmax(z)
 *     loss    = (1/r) sum_l sum_e p_l[e] (log p_l[e] - log pi_e)   (0 log 0 = 0)
 *     delta_e = dloss/dz_e = pi_e * sum(p_bar) - p_bar_e,  p_bar = (1/r) sum_l p_l
 *               (= pi_e - p_bar_e when the teachers are distributions)
 *     dw[j]   = sum_e delta_e ReLU(q[j] . k[T_e])
 *     dq[j]   = sum_e delta_e w[j] 1[q[j] . k[T_e] > 0] k[T_e]
 *     dk[s]  += sum over rows and entries e with T_e = s of
 *               delta_e sum_j w[j] 1[q[j] . k[s] > 0] q[j]
 *
 *   ix        the F layer's indexer inputs: BF16, dim 128, 1 <= heads <= 64
 *             (q_scale / k_scale unused)
 *   topk      index row length (1..2048); n_teachers = r (1..8)
 *   idx       [batch, n_q, topk] int32 (the F layer's index tensor)
 *   teachers  [r, batch, n_q, topk] fp32: each serving layer's teacher weight of
 *             every index entry (0 on the padding)
 *   loss      [batch, n_q] fp32 out (per query row)
 *   delta     [batch, n_q, topk] fp32 out (0 on entries that take no part)
 *   dq        [batch, n_q, heads, 128] fp32 out (16-byte aligned)
 *   dw        [batch, n_q, heads] fp32 out
 *   dk        [batch, n_k, 128] fp32 out (dense): overwritten -- cleared, then
 *             accumulated with float atomics, so its summation order (and its
 *             last bits) varies from call to call
 * No workspace.
 */
typedef struct dsa_distill_args {
  dsa_indexer_args ix;
  int32_t topk, n_teachers;
  const int32_t* idx;
  const float* teachers;
  float* loss;
  float* delta;
  float* dq;
  float* dw;
  float* dk;
} dsa_distill_args;

dsa_status dsa_indexer_distill(const dsa_distill_args* args, hipStream_t stream);

/*
 * Per-row cosine similarity of two outputs ([IC-SUMMARY] Appendix C: the
 * similarity-based pattern search compares attention outputs by cosine
 * similarity):
 *     row_cos[r] = <a_r, b_r> / (|a_r| |b_r|)
 * over the width values of row r (for an attention output [rows, heads, d_v]:
 * every head and value column of one query row).  A row pair where both rows
 * are zero gives 1, exactly one zero row gives 0.  The three sums are taken in
 * float64 in a fixed order (the result repeats bit for bit).
 *   a, b     device fp32 [rows, width], row-major and dense, 16-byte aligned
 *   rows     1 .. 2^31 - 1;  width: a multiple of 4, 4 .. 2^26
 *   row_cos  device fp32 [rows] out (required)
 *   mean     device float64 [1] out, optional: the mean of row_cos over the
 *            rows, summed in float64 in a fixed order
 */
dsa_status dsa_row_cosine(const float* a, const float* b, int64_t rows, int64_t width,
                          float* row_cos, double* mean, hipStream_t stream);

/*
 * Similarity matrix of the pattern search ([IC-SUMMARY] Appendix C,
 * construction of S).  Every layer runs INDEXER + Top-k (all layers F) into
 * layers[l].idx_out; then for each layer i its attention output with its own
 * index tensor, O_i, is compared with its output under every earlier layer j's
 * index tensor:
 *     S[i*N + j] = mean over the rows of row_cos(O_i, attention_i(T_j))  (i > j)
 *     S[i*N + i] = 1,  S[i*N + j] = 0 for j > i            (N = n_layers)
 *   layers[]  host array: ix and idx_out ([batch, n_q, k] int32) required for
 *             every layer; sa as in indexcache_forward (sa.idx and sa.out are
 *             ignored: the outputs go to the workspace).  Every layer has the
 *             same batch and n_q; heads * d_v is a multiple of 4.
 *   S         device float64 [N * N] out
 *   ws        >= dsa_similarity_matrix_workspace_size bytes, 256-byte aligned
 *             (the size depends on the shapes only; idx_out may be NULL when
 *             sizing)
 * Work on stream: N Top-k calls, N - 1 + N(N-1)/2 attention calls, N(N-1)/2 cosine
 * calls.  n_layers 1..1024.
 */
size_t dsa_similarity_matrix_workspace_size(int32_t n_layers, const dsa_layer* layers, int32_t k);
dsa_status dsa_similarity_matrix(int32_t n_layers, const dsa_layer* layers, int32_t k, double* S,
                                 void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Sharing-pattern search by dynamic programming ([IC-SUMMARY] Appendix C):
 * the pattern of n_layers layers, layer 0 F and exactly n_full F layers, that
 * maximises the total similarity
 *     sum over the S layers l of S[l, src(l)],  src(l) = the nearest F layer before l
 * (F layers add nothing).  dp[i][m] is the best total of layers 0..i with m F
 * layers and layer i F: dp[i][m] = max_{j<i} dp[j][m-1] + sum_{j<l<i} S[l, j];
 * the answer is max_i dp[i][n_full] + sum_{l>i} S[l, i], and backtracking the
 * choices gives the pattern.  Host code, no GPU work, O(n_layers^2 n_full).
 *   S        host float64 [n_layers * n_layers]; only S[i*N + j] with i > j is
 *            read, and must be finite
 *   n_layers 1..1024;  n_full 1..n_layers
 *   pattern  host char [n_layers + 1] out: 'F'/'S', NUL-terminated
 *   score    host float64 out, optional: the pattern's total
 * Ties: each dp step keeps the earliest predecessor, the last step the earliest
 * final F layer.
 */
dsa_status dsa_pattern_search(const double* S, int32_t n_layers, int32_t n_full, char* pattern,
                              double* score);

/*
 * Measurement helper, not a step of the method: gather-bandwidth probe.  Reads
 * every selected 1152-byte row (576 bf16 latent columns, the MLA layout the
 * sparse attention gathers; [DSA-NOTES] §3) of every query's index row, as a
 * sparse-attention pass must, with no arithmetic beyond an XOR checksum per
 * wave.  Its rate bounds what the attention kernel's gathers can reach.
 *   table   device [n_rows, 1152 bytes], 16-byte aligned; n_rows * 1152 < 2^31
 *   idx     device int32 [n_q, topk]; entries outside [0, n_rows) read nothing
 *   mode    0: four waves per query, each reading the quarter of every row the
 *              attention kernel's wave reads (two steps of 16 rows in flight)
 *           1: one wave per query, whole rows, 64 bytes of 16 rows per load
 *           2: one wave per query, whole rows, the 16 rows of a step read end
 *              to end (eight lanes per 128-byte line)
 *           3, 4, 5: modes 0, 1, 2 with deeper prefetch (4, 3, 3 steps in flight)
 *           6: four waves per query reading as the attention kernel does: a
 *              wave's 256-byte V slice of four rows per load (whole lines),
 *              then the 64-byte rope slice of 16 rows (two steps in flight)
 *           7: mode 6 with the rope line split by rows: wave w reads the whole
 *              128-byte rope line of rows 4w..4w+3
 *           8: four waves per query, wave w reading rows 4w..4w+3 of each step
 *              whole, end to end (mode 2's pattern split over four waves)
 *           9: one wave per query reading as the one-wave-per-row attention
 *              kernel does: one load instruction per selected row for its first
 *              KiB, two for the 16 rope lines (eight rows each), two steps in
 *              flight
 *           10: mode 9's load instructions landing in LDS (buffer_load ... lds)
 *              with the prefill attention kernel's schedule: two row tiles per
 *              wave, the index row through a four-block LDS ring
 *   out     device uint32 [dsa_gather_probe_out_words(n_q, mode)] checksums
 */
int64_t dsa_gather_probe_out_words(int64_t n_q, int32_t mode);
dsa_status dsa_gather_probe(const void* table, int32_t n_rows, const int32_t* idx, int64_t n_q,
                            int32_t topk, int32_t mode, uint32_t* out, hipStream_t stream);

/*
 * Measurement helper, not a step of the method: streaming read probe.  Reads
 * `bytes` of a contiguous device buffer once, in order, with no arithmetic
 * beyond an XOR checksum per wave; its rate bounds what a scan of the same
 * bytes (the decode indexer's K cache) can reach.  Workgroup x (of
 * `workgroups`, 256 threads each) reads 16-KiB chunks x, x + G, x + 2G, ...,
 * with `unroll` (1, 2 or 4) chunks in flight per wave.
 *   buf    device, 16-byte aligned; bytes a multiple of 16384, below 2^31
 *   out    device uint32 [4 * workgroups] checksums
 */
dsa_status dsa_stream_probe(const void* buf, int64_t bytes, int32_t workgroups, int32_t unroll,
                            uint32_t* out, hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
