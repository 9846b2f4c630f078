/* Host-side checks of the C ABI under AddressSanitizer and UndefinedBehaviorSanitizer.
 * Built by tests/test_host_sanitizers.py with the library's host code
 * instrumented; needs no GPU: every call below either fails validation before
 * anything is enqueued or only sizes a workspace, so the fake device pointers
 * are never dereferenced.  Also compiles include/dsa.h as C11 with -Werror. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "dsa.h"

#define FAKE ((void*)(uintptr_t)0x7F0000000000ull)
static int failures = 0;

#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__, __LINE__, \
              #cond, dsa_last_error());                                         \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

static dsa_indexer_args ix(int dtype, int batch, int n_q, int n_k, int heads, int dim, int64_t q_pos0) {
  dsa_indexer_args a;
  memset(&a, 0, sizeof a);
  a.dtype = dtype; a.batch = batch; a.n_q = n_q; a.n_k = n_k; a.heads = heads; a.dim = dim;
  a.q_pos0 = q_pos0;
  a.q = FAKE; a.k = FAKE; a.w = (const float*)FAKE;
  if (dtype == DSA_FP8_E4M3) { a.q_scale = (const float*)FAKE; a.k_scale = (const float*)FAKE; }
  return a;
}

static dsa_sparse_attn_args sa(int batch, int n_q, int n_k, int topk) {
  dsa_sparse_attn_args a;
  memset(&a, 0, sizeof a);
  a.dtype = DSA_BF16; a.batch = batch; a.n_q = n_q; a.n_k = n_k; a.heads = 16; a.kv_heads = 1;
  a.d_qk = 576; a.d_v = 512; a.topk = topk; a.scale = 1.0f / 24.0f;
  a.q = FAKE; a.kv = FAKE; a.idx = (const int32_t*)FAKE; a.out = (float*)FAKE;
  return a;
}

static void check_indexer_and_topk(void) {
  dsa_indexer_args a = ix(DSA_BF16, 1, 64, 64, 64, 128, 0);
  EXPECT(dsa_topk(&a, NULL, 16, NULL, NULL, 0, NULL) == DSA_ERR_INVALID);
  EXPECT(strlen(dsa_last_error()) > 0);
  EXPECT(dsa_topk(&a, NULL, 0, (int32_t*)FAKE, NULL, 0, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_topk(&a, NULL, 2049, (int32_t*)FAKE, NULL, 0, NULL) == DSA_ERR_INVALID);
  a.heads = 65;
  EXPECT(dsa_topk(&a, NULL, 16, (int32_t*)FAKE, NULL, 0, NULL) == DSA_ERR_UNSUPPORTED);
  a = ix(DSA_BF16, 1, 64, 64, 64, 96, 0);
  EXPECT(dsa_topk(&a, NULL, 16, (int32_t*)FAKE, NULL, 0, NULL) == DSA_ERR_UNSUPPORTED);
  a = ix(DSA_BF16, 1, 16384, 16384, 64, 128, 0);
  const size_t fused = dsa_topk_workspace_size(&a, NULL, 2048);
  EXPECT(fused > 0);
  EXPECT(dsa_topk(&a, NULL, 2048, (int32_t*)FAKE, FAKE, fused - 1, NULL) == DSA_ERR_WORKSPACE);
  /* the fused path's 2^31-byte key range and 32-bit positions */
  a = ix(DSA_BF16, 1, 4096, 1 << 23, 64, 128, 0);
  EXPECT(dsa_topk(&a, NULL, 16, (int32_t*)FAKE, FAKE, (size_t)1 << 40, NULL) == DSA_ERR_UNSUPPORTED);
  a = ix(DSA_BF16, 1, 4096, 4096, 64, 128, ((int64_t)1 << 31) - 100);
  EXPECT(dsa_topk(&a, NULL, 16, (int32_t*)FAKE, FAKE, (size_t)1 << 40, NULL) == DSA_ERR_UNSUPPORTED);
  /* decode-shaped rows past the select's limit */
  a = ix(DSA_FP8_E4M3, 8, 1, 4 * 1024 * 1024 + 1, 64, 128, 4 * 1024 * 1024);
  EXPECT(dsa_topk(&a, NULL, 16, (int32_t*)FAKE, FAKE, (size_t)1 << 40, NULL) == DSA_ERR_UNSUPPORTED);
  a = ix(DSA_FP8_E4M3, 8, 1, 204800, 64, 128, 204799);
  EXPECT(dsa_topk_workspace_size(&a, NULL, 2048) >= (size_t)8 * 204800 * 4);
  a = ix(DSA_BF16, 1, 64, 64, 64, 128, 0);
  EXPECT(dsa_indexer_scores(&a, 60, 10, (float*)FAKE, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_indexer_scores(&a, 0, 4, NULL, NULL) == DSA_ERR_INVALID);
}

static void check_attention(void) {
  dsa_sparse_attn_args a = sa(8, 1, 204800, 2048);
  EXPECT(dsa_sparse_attn_workspace_size(&a) > 0);
  EXPECT(dsa_sparse_attn(&a, NULL, 0, NULL) == DSA_ERR_WORKSPACE);
  {
    /* the size query reads the shapes only */
    dsa_sparse_attn_args b = a;
    b.idx = NULL;
    b.out = NULL;
    EXPECT(dsa_sparse_attn_workspace_size(&b) == dsa_sparse_attn_workspace_size(&a));
  }
  a.topk = 0;
  EXPECT(dsa_sparse_attn(&a, NULL, 0, NULL) == DSA_ERR_INVALID);
  a = sa(1, 4, 100, 16);
  a.heads = 15; a.kv_heads = 2;
  EXPECT(dsa_sparse_attn(&a, NULL, 0, NULL) == DSA_ERR_INVALID);
  a = sa(1, 4, 100, 16);
  a.idx = NULL;
  EXPECT(dsa_sparse_attn(&a, NULL, 0, NULL) == DSA_ERR_INVALID);
}

static void check_drivers(void) {
  dsa_layer layers[8];
  memset(layers, 0, sizeof layers);
  const char* pattern = "FSSSFSSS";
  for (int l = 0; l < 8; ++l) {
    if (pattern[l] == 'F') {
      layers[l].ix = ix(DSA_BF16, 1, 4, 4, 64, 128, 0);
      layers[l].idx_out = (int32_t*)((uintptr_t)FAKE + 4096u * (unsigned)l);
    }
    layers[l].sa = sa(1, 4, 4, 16);
  }
  const size_t need = indexcache_forward_workspace_size(pattern, 8, layers, 16);
  EXPECT(need > 0);
  int32_t src[8];
  EXPECT(indexcache_forward(pattern, 8, layers, 16, src, NULL, 0, NULL) == DSA_ERR_WORKSPACE);
  EXPECT(indexcache_forward("SFFF", 4, layers, 16, src, FAKE, need, NULL) == DSA_ERR_INVALID);
  EXPECT(indexcache_forward("FSX", 3, layers, 16, src, FAKE, need, NULL) == DSA_ERR_INVALID);
  EXPECT(indexcache_forward(pattern, 9, layers, 16, src, FAKE, need, NULL) == DSA_ERR_INVALID);
  EXPECT(indexcache_forward_mli_workspace_size(pattern, 8, layers, 16) >= need);
  EXPECT(indexcache_forward_mli(pattern, 8, layers, 16, src, NULL, 0, NULL, NULL) == DSA_ERR_WORKSPACE);
  /* the allocation-free driver refuses before touching a device */
  EXPECT(indexcache_forward_noalloc("SFFF", 4, layers, 16, src, NULL) == DSA_ERR_INVALID);
  layers[0].ix = ix(DSA_BF16, 1, 16384, 16384, 64, 128, 0);
  layers[0].sa = sa(1, 16384, 16384, 16);
  EXPECT(indexcache_forward_noalloc("F", 1, layers, 16, src, NULL) == DSA_ERR_WORKSPACE);
  /* an F layer over the fused path's key range, through every driver */
  layers[0].ix = ix(DSA_BF16, 1, 4096, 1 << 23, 64, 128, 0);
  layers[0].sa = sa(1, 4096, 1 << 23, 16);
  EXPECT(indexcache_forward("F", 1, layers, 16, src, FAKE, (size_t)1 << 40, NULL) == DSA_ERR_UNSUPPORTED);
  EXPECT(dsa_similarity_matrix(1, layers, 16, (double*)FAKE, FAKE, (size_t)1 << 40, NULL) == DSA_ERR_UNSUPPORTED);
  EXPECT(indexcache_forward_mli("F", 1, layers, 16, src, FAKE, (size_t)1 << 40, NULL, NULL) == DSA_ERR_UNSUPPORTED);
}

static void check_helpers(void) {
  EXPECT(dsa_abi_version() == DSA_ABI_VERSION);
  EXPECT(strcmp(dsa_status_string(DSA_OK), "ok") == 0);
  EXPECT(dsa_index_overlap((const int32_t*)FAKE, (const int32_t*)FAKE, 4, 0, (int32_t*)FAKE, NULL, NULL) ==
         DSA_ERR_INVALID);
  EXPECT(dsa_row_cosine((const float*)FAKE, (const float*)FAKE, 4, 6, (float*)FAKE, NULL, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_gather_probe(FAKE, 100, (const int32_t*)FAKE, 4, 16, 11, (uint32_t*)FAKE, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_gather_probe_out_words(5, 1) == 8 && dsa_gather_probe_out_words(5, 0) == 20 &&
         dsa_gather_probe_out_words(5, 6) == 20 &&
         dsa_gather_probe_out_words(5, 7) == 20 && dsa_gather_probe_out_words(5, 8) == 20 && dsa_gather_probe_out_words(5, 9) == 8 && dsa_gather_probe_out_words(5, 10) == 8 && dsa_gather_probe_out_words(5, 11) == 0);
  EXPECT(dsa_stream_probe(FAKE, 16384 * 3 + 4, 8, 2, (uint32_t*)FAKE, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_stream_probe(FAKE, 16384, 8, 3, (uint32_t*)FAKE, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_stream_probe(FAKE, (int64_t)1 << 31, 8, 2, (uint32_t*)FAKE, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_stream_probe(FAKE, 16384, 0, 2, (uint32_t*)FAKE, NULL) == DSA_ERR_INVALID);
  dsa_distill_args d;
  memset(&d, 0, sizeof d);
  d.ix = ix(DSA_BF16, 1, 4, 4, 64, 128, 0);
  d.topk = 0;
  EXPECT(dsa_indexer_distill(&d, NULL) == DSA_ERR_INVALID);
  EXPECT(dsa_indexer_distill(NULL, NULL) == DSA_ERR_INVALID);
}

/* The sharing-pattern dynamic program on sizes up to 1024 layers. */
static void check_pattern_search(void) {
  const int sizes[] = {1, 2, 4, 47, 78, 1024};
  for (size_t t = 0; t < sizeof sizes / sizeof sizes[0]; ++t) {
    const int n = sizes[t];
    double* S = (double*)malloc(sizeof(double) * (size_t)n * (size_t)n);
    char* pat = (char*)malloc((size_t)n + 1);
    unsigned x = 12345u;
    for (int i = 0; i < n * n; ++i) {
      x = x * 1103515245u + 12345u;
      S[i] = (double)(x >> 8) / (double)(1u << 24);
    }
    const int m = n < 8 ? 1 : n / 4;
    double score = -1.0;
    EXPECT(dsa_pattern_search(S, n, m, pat, &score) == DSA_OK);
    int f = 0;
    for (int i = 0; i < n; ++i) f += pat[i] == 'F';
    EXPECT((int)strlen(pat) == n && pat[0] == 'F' && f == m && score >= 0.0);
    EXPECT(dsa_pattern_search(S, n, n + 1, pat, &score) == DSA_ERR_INVALID);
    free(S);
    free(pat);
  }
}

int main(void) {
  check_indexer_and_topk();
  check_attention();
  check_drivers();
  check_helpers();
  check_pattern_search();
  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("ALL OK\n");
  return 0;
}
