"""CPU oracle for the DSA step with IndexCache cross-layer index reuse.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this package: only the test suite, the smoke check and
the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library and never reads a value that the HIP library produced as an input.

Plain, slow, float64 NumPy.  Sources (web pages, cited by title and section):
  [DSA-NOTES]  "IndexCache：跨层复用稀疏索引，以及它为什么能被训练"
               (reading notes on IndexCache, notes.kuangjux.top)
  [IC-SUMMARY] "IndexCache: Accelerating Sparse Attention via Cross-Layer Index
               Reuse" (section-by-section summary, papercache.org)
  [MLI]        "MLI重构DeepSeek稀疏注意力：跨层复用索引免训提速" (zicq.com)

Parity pins: every function here is pinned by the CPU test suite against
worked examples printed on those pages, closed forms, library routines or
invariants -- see tests/test_oracle_pins.py, tests/test_oracle_distill_pins.py and
tests/test_oracle_pattern_pins.py.
No function is unpinned.
"""
from .numerics import bf16_bits_to_f64, e4m3fn_codes_to_f64, dequantize  # noqa: F401
from .dsa import (  # noqa: F401
    indexer_scores, topk_row, indexer_topk, sparse_attn, source_layers,
    indexcache_forward, mli_source_layers, mli_forward, overlap, overlap_matrix, amdahl_speedup,
)
from .distill import kl_multi, kl_average, indexer_distill  # noqa: F401
from .pattern_search import (  # noqa: F401
    row_cosine, output_similarity, similarity_matrix, pattern_objective, pattern_search_brute,
)
