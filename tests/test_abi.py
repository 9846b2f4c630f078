"""C-ABI tests that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before anything is enqueued.

Every call here fails validation (or only sizes a workspace), so no kernel is
ever launched with the fake pointers used below."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

L = pytest.importorskip("dsa_lightning_indexer_amd._lib")

FAKE = 0x7F0000000000   # 256-byte aligned non-NULL value; never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


def test_header_and_exports_agree():
    decl = declared_functions()
    assert set(decl) == set(L.EXPORTS), decl
    for name in decl:
        assert hasattr(L.LIB, name), name


def test_version_and_status_strings():
    assert L.abi_version() == 1
    assert L.dsa_status_string(0) == b"ok"
    assert b"workspace" in L.dsa_status_string(3)


def ix(**kw):
    a = L.IndexerArgs()
    a.dtype, a.batch, a.n_q, a.n_k, a.heads, a.dim = L.DSA_BF16, 1, 64, 64, 64, 128
    a.q = a.k = a.w = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def topk_status(a, k=16, idx=FAKE, scores=None, ws=None, ws_bytes=0):
    return L.dsa_topk(ctypes.byref(a), scores, k, idx, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,k,expect", [
    (dict(), 0, 1), (dict(), 2049, 1),
    (dict(dtype=7), 16, 1), (dict(batch=0), 16, 1), (dict(n_k=0), 16, 1), (dict(q_pos0=-1), 16, 1),
    (dict(heads=65), 16, 2), (dict(heads=0), 16, 2), (dict(dim=96), 16, 2),
    (dict(dtype=L.DSA_FP8_E4M3, dim=32), 16, 2),
    (dict(q=None), 16, 1), (dict(w=None), 16, 1),
    (dict(dtype=L.DSA_FP8_E4M3), 16, 1),                   # fp8 without scales
    (dict(q=FAKE + 4), 16, 1),                            # misaligned
    (dict(k_batch_stride=5), 16, 1),
    (dict(dtype=L.DSA_F32, dim=300), 16, 2),
])
def test_topk_rejects(kw, k, expect):
    assert topk_status(ix(**kw), k=k) == expect
    assert L.dsa_last_error() != b""


def test_topk_null_idx():
    assert topk_status(ix(), idx=None) == 1


def test_workspace_sizes_and_errors():
    a = ix(batch=8, n_q=1, n_k=204800, q_pos0=204799, dtype=L.DSA_FP8_E4M3, q_scale=FAKE, k_scale=FAKE)
    need = L.dsa_topk_workspace_size(ctypes.byref(a), None, 2048)
    assert need >= 8 * 204800 * 4
    assert topk_status(a, k=2048, ws=None, ws_bytes=0) == 3
    assert topk_status(a, k=2048, ws=FAKE, ws_bytes=need - 1) == 3
    # prefill-shaped bf16 fused path: candidate slices for the persistent grid
    b = ix(n_q=16384, n_k=16384)
    fused = L.dsa_topk_workspace_size(ctypes.byref(b), None, 2048)
    assert fused >= 512 * 4 * 2 * 16384 * 4
    assert topk_status(b, k=2048, ws=FAKE, ws_bytes=fused - 1) == 3
    # materialised-scores path needs the select state
    assert L.dsa_topk_workspace_size(ctypes.byref(b), FAKE, 2048) > 0
    assert topk_status(b, k=2048, scores=FAKE) == 3


def test_indexer_scores_rejects_bad_window():
    a = ix()
    assert L.dsa_indexer_scores(ctypes.byref(a), 60, 10, FAKE, None) == 1
    assert L.dsa_indexer_scores(ctypes.byref(a), -1, 10, FAKE, None) == 1
    assert L.dsa_indexer_scores(ctypes.byref(a), 0, 0, FAKE, None) == 1
    assert L.dsa_indexer_scores(ctypes.byref(a), 0, 4, None, None) == 1


def sa(**kw):
    a = L.SparseAttnArgs()
    a.dtype, a.batch, a.n_q, a.n_k, a.heads, a.kv_heads = L.DSA_BF16, 1, 4, 100, 16, 1
    a.d_qk, a.d_v, a.topk, a.scale = 576, 512, 2048, 1 / 24
    a.q = a.kv = a.idx = a.out = FAKE
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@pytest.mark.parametrize("kw,expect", [
    (dict(dtype=L.DSA_FP8_E4M3), 2), (dict(heads=15, kv_heads=2), 1), (dict(d_v=600), 1),
    (dict(d_qk=2000), 2), (dict(topk=0), 1), (dict(topk=4096), 1), (dict(idx=None), 1),
    (dict(out=None), 1), (dict(scale=float("nan")), 1), (dict(kv_batch_stride=10), 1),
])
def test_sparse_attn_rejects(kw, expect):
    assert L.dsa_sparse_attn(ctypes.byref(sa(**kw)), None, 0, None) == expect


def test_sparse_attn_decode_needs_workspace():
    a = sa(batch=8, n_q=1, n_k=204800)
    need = L.dsa_sparse_attn_workspace_size(ctypes.byref(a))
    assert need > 0
    assert L.dsa_sparse_attn(ctypes.byref(a), None, 0, None) == 3
    # the size query needs only the shapes: no idx or output yet
    assert L.dsa_sparse_attn_workspace_size(ctypes.byref(sa(batch=8, n_q=1, n_k=204800, idx=None, out=None))) == need


def test_sparse_attn_workspace_size_binding():
    # the Python query (no output tensor) agrees with what the launch asks for
    import torch
    from dsa_lightning_indexer_amd import api
    q = torch.empty((8, 1, 16, 576), dtype=torch.bfloat16)
    kv = torch.empty((8, 204800, 1, 576), dtype=torch.bfloat16)
    idx = torch.empty((8, 1, 2048), dtype=torch.int32)
    need = L.dsa_sparse_attn_workspace_size(ctypes.byref(sa(batch=8, n_q=1, n_k=204800)))
    assert api.sparse_attn_workspace_size(q, kv, idx, 512) == need > 0


def layers(pattern, null_s=True):
    arr = (L.Layer * len(pattern))()
    for i, c in enumerate(pattern):
        if c == "F" or not null_s:
            arr[i].ix = ix(n_q=4, n_k=4)
            arr[i].idx_out = FAKE
        arr[i].sa = sa(n_q=4, n_k=4, topk=16)
    return arr


def fwd_status(pattern, arr, n=None, k=16):
    n = len(pattern) if n is None else n
    return L.indexcache_forward_c(pattern.encode(), n, arr, k, None, None, 0, None)


def test_forward_pattern_validation():
    assert fwd_status("SFFF", layers("FFFF")) == 1            # first layer must be F
    assert fwd_status("FXSS", layers("FFFF")) == 1
    assert fwd_status("FSS", layers("FSS"), n=4) == 1         # length mismatch
    assert fwd_status("FSS", layers("FSS"), k=0) == 1
    assert L.indexcache_forward_c(None, 3, layers("FSS"), 16, None, None, 0, None) == 1
    assert L.indexcache_forward_c(b"FSS", 3, None, 16, None, None, 0, None) == 1


def test_forward_s_layers_need_no_indexer_inputs():
    """An S layer's indexer arguments are never read: validation (and workspace
    sizing) succeeds with every S-layer indexer pointer NULL."""
    arr = layers("FSSSFSSS", null_s=True)
    assert L.indexcache_forward_workspace_size(b"FSSSFSSS", 8, arr, 16) > 0
    # the same NULL indexer on an F layer is rejected
    arr[0].ix = L.IndexerArgs()
    assert fwd_status("FSSSFSSS", arr) == 1


def test_forward_attention_shape_must_match_cached_tensor():
    arr = layers("FS")
    arr[1].sa.n_q = 5
    assert fwd_status("FS", arr) == 1
    arr = layers("FS")
    arr[1].sa.topk = 8
    assert fwd_status("FS", arr) == 1


def test_overlap_rejects():
    assert L.dsa_index_overlap(FAKE, FAKE, 4, 0, FAKE, None, None) == 1
    assert L.dsa_index_overlap(None, FAKE, 4, 16, FAKE, None, None) == 1
    assert L.dsa_index_overlap(FAKE, FAKE, 4, 16, None, None, None) == 1
    assert L.dsa_index_overlap(FAKE, FAKE, -1, 16, FAKE, None, None) == 1


def distill_status(**kw):
    d = L.DistillArgs()
    d.ix = ix(**{k: v for k, v in kw.items() if k in ("dtype", "dim", "heads", "q", "w")})
    d.topk, d.n_teachers = kw.get("topk", 64), kw.get("n_teachers", 2)
    for name in ("idx", "teachers", "loss", "delta", "dq", "dw", "dk"):
        setattr(d, name, kw.get(name, FAKE))
    return L.dsa_indexer_distill(ctypes.byref(d), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(topk=0), 1), (dict(topk=2049), 1), (dict(n_teachers=0), 1), (dict(n_teachers=9), 1),
    (dict(teachers=None), 1), (dict(dk=None), 1), (dict(delta=None), 1),
    (dict(dq=FAKE + 4), 1),                                # dq needs 16-byte alignment
    (dict(dim=64), 2), (dict(dtype=L.DSA_FP8_E4M3), 1),    # fp8 without scales fails data checks first
    (dict(dtype=L.DSA_F32, dim=128), 2),
])
def test_distill_rejects(kw, expect):
    assert distill_status(**kw) == expect
    assert L.dsa_last_error() != b""


def test_distill_null_args():
    assert L.dsa_indexer_distill(None, None) == 1


def test_row_cosine_rejects():
    ok = dict(a=FAKE, b=FAKE, rows=4, width=8192, row_cos=FAKE, mean=None)

    def st(**kw):
        a = dict(ok, **kw)
        return L.dsa_row_cosine(a["a"], a["b"], a["rows"], a["width"], a["row_cos"], a["mean"], None)
    for kw in (dict(rows=0), dict(rows=1 << 31), dict(width=6), dict(width=0), dict(width=(1 << 26) + 4),
               dict(a=None), dict(b=None), dict(row_cos=None), dict(a=FAKE + 8), dict(mean=FAKE + 4)):
        assert st(**kw) == 1, kw
        assert L.dsa_last_error() != b""


def test_similarity_matrix_validation_and_workspace():
    arr = layers("FFF", null_s=False)
    need = L.dsa_similarity_matrix_workspace_size(3, arr, 16)
    # two outputs of 4 rows x 16 heads x 512 fp32 and the row cosines at least
    assert need >= 2 * 4 * 16 * 512 * 4
    assert L.dsa_similarity_matrix(3, arr, 16, FAKE, None, 0, None) == 3       # workspace missing
    assert L.dsa_similarity_matrix(3, arr, 16, FAKE, FAKE, need - 1, None) == 3
    assert L.dsa_similarity_matrix(3, arr, 16, None, FAKE, need, None) == 1    # S missing
    assert L.dsa_similarity_matrix(0, arr, 16, FAKE, FAKE, need, None) == 1
    assert L.dsa_similarity_matrix(3, arr, 0, FAKE, FAKE, need, None) == 1
    bad = layers("FFF", null_s=False)
    bad[2].idx_out = None                                   # every layer needs its T (not to size the workspace)
    assert L.dsa_similarity_matrix_workspace_size(3, bad, 16) == need
    assert L.dsa_similarity_matrix(3, bad, 16, FAKE, FAKE, need, None) == 1
    bad = layers("FFF", null_s=False)
    bad[1].sa.n_q = 5                                                          # rows must agree
    assert L.dsa_similarity_matrix(3, bad, 16, FAKE, FAKE, need, None) == 1
    assert L.dsa_similarity_matrix(3, None, 16, FAKE, FAKE, need, None) == 1
    free = layers("FFF", null_s=False)
    for a in free:
        a.sa.out = None                                     # attention outputs live in the workspace
        a.sa.idx = None
    assert L.dsa_similarity_matrix_workspace_size(3, free, 16) == need


def one_f_layer(ixa, sa_rows=None):
    """A one-layer pattern "F" whose attention matches the indexer's rows."""
    arr = (L.Layer * 1)()
    arr[0].ix = ixa
    arr[0].idx_out = FAKE
    arr[0].sa = sa(batch=ixa.batch, n_q=ixa.n_q, n_k=ixa.n_k, topk=16)
    return arr


@pytest.mark.parametrize("kw", [
    # decode-shaped layer (scan + few-row select) longer than the select's row limit
    dict(batch=8, n_q=1, n_k=4 * 1024 * 1024 + 1, q_pos0=4 * 1024 * 1024, dtype=L.DSA_FP8_E4M3, q_scale=FAKE,
         k_scale=FAKE),
    # fused prefill layer whose keys span 2^31 bytes (32-bit buffer offsets)
    dict(n_q=4096, n_k=1 << 23),
    # fused prefill layer whose last query position does not fit an int32
    dict(n_q=4096, n_k=4096, q_pos0=(1 << 31) - 100),
])
def test_driver_applies_the_topk_path_limits(kw):
    """Every F layer of indexcache_forward and dsa_similarity_matrix goes through
    the same path limits as dsa_topk, before anything is enqueued."""
    a = ix(**kw)
    assert topk_status(a, k=16, ws=FAKE, ws_bytes=1 << 40) == 2
    arr = one_f_layer(a)
    assert L.indexcache_forward_c(b"F", 1, arr, 16, None, FAKE, 1 << 40, None) == 2
    assert b"layer 0" in L.dsa_last_error()
    assert L.indexcache_forward_workspace_size(b"F", 1, arr, 16) == 0
    assert L.dsa_similarity_matrix(1, arr, 16, FAKE, FAKE, 1 << 40, None) == 2
    assert L.dsa_similarity_matrix_workspace_size(1, arr, 16) == 0


def test_driver_accepts_the_largest_fused_layer():
    """Just inside the limits: validation passes and only the workspace is missing."""
    arr = one_f_layer(ix(n_q=4096, n_k=(1 << 23) - 8, q_pos0=0))
    assert L.indexcache_forward_c(b"F", 1, arr, 16, None, None, 0, None) == 3


def test_binding_rejects_non_dense_layouts():
    """The kernels read q, w, idx and out densely and k/kv rows back to back;
    the binding refuses views with other strides instead of passing a base
    pointer that would be read with the wrong layout."""
    import torch
    q = torch.zeros(1, 8, 4, 32)
    k = torch.zeros(1, 8, 32)
    w = torch.zeros(1, 8, 4)
    L.indexer_args(q, k, w)                                           # dense: fine
    L.indexer_args(q, torch.zeros(2, 20, 32)[:, :8], torch.zeros(2, 8, 4).contiguous()[:1])  # batch stride: fine
    with pytest.raises(ValueError):
        L.indexer_args(q.transpose(1, 2).contiguous().transpose(1, 2), k, w)   # head/row transposed q
    with pytest.raises(ValueError):
        L.indexer_args(q, torch.zeros(1, 8, 64)[..., :32], w)                  # k rows with stride 64
    with pytest.raises(ValueError):
        L.indexer_args(q, k, torch.zeros(1, 4, 8).transpose(1, 2))             # transposed w
    Q = torch.zeros(1, 4, 16, 576)
    kv = torch.zeros(1, 10, 1, 576)
    idx = torch.zeros(1, 4, 16, dtype=torch.int32)
    out = torch.zeros(1, 4, 16, 512)
    L.sparse_attn_args(Q, kv, idx, 1.0, out)                          # dense: fine
    L.sparse_attn_args(Q, torch.zeros(2, 30, 1, 576)[:, :10], idx, 1.0, out)   # batch stride: fine
    with pytest.raises(ValueError):
        L.sparse_attn_args(torch.zeros(1, 4, 32, 576)[:, :, :16], kv, idx, 1.0, out)   # head slice of Q
    with pytest.raises(ValueError):
        L.sparse_attn_args(Q, torch.zeros(1, 10, 1, 640)[..., :576], idx, 1.0, out)    # strided kv rows
    with pytest.raises(ValueError):
        L.sparse_attn_args(Q, kv, torch.zeros(1, 16, 4, dtype=torch.int32).transpose(1, 2), 1.0, out)
    with pytest.raises(ValueError):
        L.sparse_attn_args(Q, kv, idx, 1.0, torch.zeros(1, 4, 16, 1024)[..., :512])


def test_noalloc_rejects_before_touching_the_device():
    """The allocation-free driver validates like indexcache_forward and refuses
    layers whose scratch need exceeds its static array, before any device call
    (these run on a machine without a GPU)."""
    st = lambda pat, arr, k=16: L.indexcache_forward_noalloc_c(pat.encode(), len(pat), arr, k, None, None)
    assert st("SFFF", layers("FFFF")) == 1
    assert st("FSS", layers("FSS"), k=0) == 1
    # a prefill F layer takes the fused path: 537 MB of candidate slices > 64 MiB
    arr = one_f_layer(ix(n_q=16384, n_k=16384))
    assert L.indexcache_forward_workspace_size(b"F", 1, arr, 16) > L.NOALLOC_SCRATCH_BYTES
    assert st("F", arr) == 3
    assert b"scratch" in L.dsa_last_error()
    # a decode layer just over the limit: 8 rows x n_k fp32 scores alone exceed it
    big = one_f_layer(ix(batch=8, n_q=1, n_k=(1 << 21) + 1024, q_pos0=(1 << 21) + 1023, dtype=L.DSA_FP8_E4M3,
                         q_scale=FAKE, k_scale=FAKE))
    assert L.indexcache_forward_workspace_size(b"F", 1, big, 16) > L.NOALLOC_SCRATCH_BYTES
    assert st("F", big) == 3


def mli_status(pattern, arr, k=16, ws=None, ws_bytes=0):
    return L.indexcache_forward_mli_c(pattern.encode(), len(pattern), arr, k, None, ws, ws_bytes, None, None)


def test_mli_forward_validation():
    """The overlapped loop validates like indexcache_forward, and also refuses
    consecutive F layers that share idx_out (one is written while attention
    reads the other); its workspace holds separate indexer and attention
    regions."""
    assert mli_status("SFFF", layers("FFFF")) == 1
    arr = layers("FSFS")
    arr[2].idx_out = FAKE + 4096
    need = L.indexcache_forward_mli_workspace_size(b"FSFS", 4, arr, 16)
    assert need >= L.indexcache_forward_workspace_size(b"FSFS", 4, arr, 16) > 0
    assert mli_status("FSFS", arr) == 3                         # workspace missing
    assert mli_status("FSFS", arr, ws=FAKE + 8, ws_bytes=need) == 1   # misaligned workspace
    arr[2].idx_out = arr[0].idx_out                            # consecutive F layers share a buffer
    assert mli_status("FSFS", arr, ws=FAKE, ws_bytes=need) == 1
    assert b"share idx_out" in L.dsa_last_error()
    assert L.indexcache_forward_mli_workspace_size(b"FSFS", 4, arr, 16) == 0
    arr = layers("FSFS")
    arr[2].idx_out = FAKE + 4096
    arr[2].sa.n_q = 5                                          # does not match layer 0's tensor
    arr[2].ix.n_q = 5
    arr[3].sa.n_q = 5
    assert mli_status("FSFS", arr, ws=FAKE, ws_bytes=need) == 1
