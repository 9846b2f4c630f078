"""Thin Python binding over libdsa.so (the C ABI declared in include/dsa.h).

Argument marshalling only: every step of the DSA / IndexCache path runs in the
HIP kernels of libdsa.so.  torch provides device memory and the current HIP
stream.  Importing fails loudly when the library has not been built.
"""
from ._lib import (  # noqa: F401
    LIB, LIB_PATH, DsaError, IndexerArgs, SparseAttnArgs, Layer, DistillArgs, dtype_code, abi_version,
    indexer_args, sparse_attn_args,
)
from .api import (  # noqa: F401
    indexer_scores, topk, topk_workspace_size, sparse_attn, sparse_attn_workspace_size,
    indexcache_forward, indexcache_forward_workspace_size, indexcache_forward_mli,
    indexcache_forward_mli_workspace_size, indexcache_forward_noalloc, index_overlap, indexer_distill,
    row_cosine, similarity_matrix, similarity_matrix_workspace_size, pattern_search, gather_probe, stream_probe,
)
