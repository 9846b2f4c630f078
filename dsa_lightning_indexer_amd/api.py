"""Torch-tensor wrappers of the C ABI.  Marshalling only: shapes and pointers in,
status codes checked; outputs and workspaces are allocated with torch when the
caller does not pass them."""
import ctypes

import torch

from . import _lib as L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ws(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is not None:
        return ws, ws.numel() * ws.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def indexer_scores(q, k, w, *, q_scale=None, k_scale=None, q_pos0=0, row0=0, rows=None, out=None):
    """Materialised indexer scores [B, rows, n_k] fp32 (-inf where s > t)."""
    B, n_q = q.shape[:2]
    rows = n_q - row0 if rows is None else rows
    if out is None:
        out = torch.empty((B, rows, k.shape[1]), dtype=torch.float32, device=q.device)
    a = L.indexer_args(q, k, w, q_scale, k_scale, q_pos0)
    L.check(L.dsa_indexer_scores(ctypes.byref(a), row0, rows, out.data_ptr(), _stream()))
    return out


def topk_workspace_size(q, k, w, topk, *, q_scale=None, k_scale=None, q_pos0=0, scores=None):
    a = L.indexer_args(q, k, w, q_scale, k_scale, q_pos0)
    return L.dsa_topk_workspace_size(ctypes.byref(a), None if scores is None else scores.data_ptr(), topk)


def topk(q, k, w, topk, *, q_scale=None, k_scale=None, q_pos0=0, scores=None, out=None, ws=None):
    """INDEXER + Top-k (scores=None) or Top-k over given scores [B, n_q, n_k].
    Returns int32 [B, n_q, topk], ascending rows with -1 padding."""
    B, n_q = q.shape[:2]
    if out is None:
        out = torch.empty((B, n_q, topk), dtype=torch.int32, device=q.device)
    a = L.indexer_args(q, k, w, q_scale, k_scale, q_pos0)
    sp = None if scores is None else scores.data_ptr()
    need = L.dsa_topk_workspace_size(ctypes.byref(a), sp, topk)
    wbuf, wbytes = _ws(need, q.device, ws)
    L.check(L.dsa_topk(ctypes.byref(a), sp, topk, out.data_ptr(), None if wbuf is None else wbuf.data_ptr(),
                       wbytes, _stream()))
    return out


def sparse_attn_workspace_size(q, kv, idx, d_v, *, v=None):
    dummy = torch.empty(0)
    a = L.sparse_attn_args(q, kv, idx, 1.0, dummy, v=v, d_v=d_v)
    return L.dsa_sparse_attn_workspace_size(ctypes.byref(a))


def sparse_attn(q, kv, idx, scale, *, d_v=None, v=None, out=None, ws=None):
    """Sparse attention; returns fp32 [B, n_q, H, d_v]."""
    B, n_q, H, _ = q.shape
    if d_v is None:
        d_v = v.shape[-1] if v is not None else kv.shape[-1]
    if out is None:
        out = torch.empty((B, n_q, H, d_v), dtype=torch.float32, device=q.device)
    a = L.sparse_attn_args(q, kv, idx, scale, out, v=v, d_v=d_v)
    need = L.dsa_sparse_attn_workspace_size(ctypes.byref(a))
    wbuf, wbytes = _ws(need, q.device, ws)
    L.check(L.dsa_sparse_attn(ctypes.byref(a), None if wbuf is None else wbuf.data_ptr(), wbytes, _stream()))
    return out


def _layers(specs, k):
    arr = (L.Layer * len(specs))()
    for i, s in enumerate(specs):
        ix = s.get("ix")
        if ix is not None:
            arr[i].ix = L.indexer_args(ix["q"], ix["k"], ix["w"], ix.get("q_scale"), ix.get("k_scale"),
                                       ix.get("q_pos0", 0))
        sa = s["sa"]
        arr[i].sa = L.sparse_attn_args(sa["q"], sa["kv"], None, sa["scale"], sa["out"], v=sa.get("v"),
                                       d_v=sa.get("d_v"))
        arr[i].sa.topk = k
        io = s.get("idx_out")
        arr[i].idx_out = None if io is None else io.data_ptr()
    return arr


def indexcache_forward_workspace_size(pattern, specs, k):
    arr = _layers(specs, k)
    return L.indexcache_forward_workspace_size(pattern.encode(), len(specs), arr, k)


def indexcache_forward(pattern, specs, k, *, ws=None):
    """IndexCache loop.  specs[l] = {"ix": {...} (F layers only), "sa": {"q", "kv", "scale", "out",
    optional "v", "d_v"}, "idx_out": int32 tensor (F layers only)}.  Returns the 0-based source layer
    of every layer's index tensor."""
    arr = _layers(specs, k)
    n = len(specs)
    need = L.indexcache_forward_workspace_size(pattern.encode(), n, arr, k)
    dev = specs[0]["sa"]["q"].device
    wbuf, wbytes = _ws(need, dev, ws)
    src = (ctypes.c_int32 * n)()
    L.check(L.indexcache_forward_c(pattern.encode(), n, arr, k, src,
                                   None if wbuf is None else wbuf.data_ptr(), wbytes, _stream()))
    return list(src)


def indexcache_forward_mli_workspace_size(pattern, specs, k):
    arr = _layers(specs, k)
    return L.indexcache_forward_mli_workspace_size(pattern.encode(), len(specs), arr, k)


def indexcache_forward_mli(pattern, specs, k, *, index_stream=None, ws=None):
    """IndexCache loop with the multi-layer-indexer shift: layer l attends with
    the nearest earlier F layer's index tensor (layer 0 with its own); F-layer
    indexers run on `index_stream` (a torch.cuda.Stream; None = the current
    stream, i.e. in order), attention on the current stream.  Same specs as
    indexcache_forward; returns the 0-based source layer of every layer."""
    arr = _layers(specs, k)
    n = len(specs)
    need = L.indexcache_forward_mli_workspace_size(pattern.encode(), n, arr, k)
    dev = specs[0]["sa"]["q"].device
    wbuf, wbytes = _ws(need, dev, ws)
    src = (ctypes.c_int32 * n)()
    main = _stream()
    side = main if index_stream is None else ctypes.c_void_p(index_stream.cuda_stream)
    L.check(L.indexcache_forward_mli_c(pattern.encode(), n, arr, k, src,
                                       None if wbuf is None else wbuf.data_ptr(), wbytes, main, side))
    if index_stream is not None and ws is None and wbuf is not None:
        wbuf.record_stream(index_stream)
    return list(src)


def indexcache_forward_noalloc(pattern, specs, k):
    """indexcache_forward with the library's static per-GPU scratch instead of a
    workspace: nothing is allocated.  Same specs and result."""
    arr = _layers(specs, k)
    n = len(specs)
    src = (ctypes.c_int32 * n)()
    L.check(L.indexcache_forward_noalloc_c(pattern.encode(), n, arr, k, src, _stream()))
    return list(src)


def index_overlap(a, b, k, *, rows=None, row_counts=None, total=None):
    """Adds sum_r |a[r] ∩ b[r]| to `total` (uint64 stored in an int64 tensor of one element);
    optionally writes per-row counts.  a, b: int32 [rows, k] (any leading dims flattened)."""
    a2 = a.reshape(-1, k)
    b2 = b.reshape(-1, k)
    rows = a2.shape[0] if rows is None else rows
    if total is None:
        total = torch.zeros(1, dtype=torch.int64, device=a.device)
    L.check(L.dsa_index_overlap(a2.data_ptr(), b2.data_ptr(), rows, k,
                                None if row_counts is None else row_counts.data_ptr(),
                                total.data_ptr(), _stream()))
    return total


def indexer_distill(q, k, w, idx, teachers, *, q_pos0=0):
    """Distillation loss over the selected Top-k and its backward.
    q [B, n_q, H, 128] bf16, k [B, n_k, 128] bf16, w [B, n_q, H] fp32,
    idx [B, n_q, topk] int32, teachers [r, B, n_q, topk] fp32.
    Returns dict(loss [B, n_q], delta [B, n_q, topk], dq [B, n_q, H, 128],
    dw [B, n_q, H], dk [B, n_k, 128]), all fp32."""
    B, n_q, H, d = q.shape
    n_k = k.shape[1]
    r, topk = teachers.shape[0], idx.shape[2]
    L._dense("idx", idx)
    L._dense("teachers", teachers)
    dev = q.device
    out = dict(loss=torch.empty((B, n_q), dtype=torch.float32, device=dev),
               delta=torch.empty((B, n_q, topk), dtype=torch.float32, device=dev),
               dq=torch.empty((B, n_q, H, d), dtype=torch.float32, device=dev),
               dw=torch.empty((B, n_q, H), dtype=torch.float32, device=dev),
               dk=torch.empty((B, n_k, d), dtype=torch.float32, device=dev))
    a = L.DistillArgs()
    a.ix = L.indexer_args(q, k, w, None, None, q_pos0)
    a.topk, a.n_teachers = topk, r
    a.idx, a.teachers = idx.data_ptr(), teachers.data_ptr()
    for name in ("loss", "delta", "dq", "dw", "dk"):
        setattr(a, name, out[name].data_ptr())
    L.check(L.dsa_indexer_distill(ctypes.byref(a), _stream()))
    return out


def row_cosine(a, b, *, row_cos=None, mean=None):
    """Per-row cosine similarity of two fp32 tensors (leading dim = rows, the rest
    flattened).  Returns (row_cos fp32 [rows], mean float64 [1])."""
    rows = a.shape[0]
    width = a[0].numel() if rows else 0
    L._dense("a", a)
    L._dense("b", b)
    if row_cos is None:
        row_cos = torch.empty(rows, dtype=torch.float32, device=a.device)
    if mean is None:
        mean = torch.empty(1, dtype=torch.float64, device=a.device)
    L.check(L.dsa_row_cosine(a.data_ptr(), b.data_ptr(), rows, width, row_cos.data_ptr(), mean.data_ptr(),
                             _stream()))
    return row_cos, mean


def _all_f_layers(ix_list, sa_list, k, idx_out):
    specs = [{"ix": ix, "sa": sa, "idx_out": io} for ix, sa, io in zip(ix_list, sa_list, idx_out)]
    return _layers(specs, k)


def _sim_layers(ix_list, sa_list, k, idx_out):
    dev = sa_list[0]["q"].device
    if any(sa.get("d_v") is None and sa.get("v") is None for sa in sa_list):
        raise ValueError("each attention spec needs d_v (or a separate v)")
    dummy = torch.empty(0, device=dev)
    sas = [dict(sa, out=dummy, d_v=sa.get("d_v") or sa["v"].shape[-1]) for sa in sa_list]
    return _all_f_layers(ix_list, sas, k, idx_out)


def similarity_matrix_workspace_size(ix_list, sa_list, k):
    arr = _sim_layers(ix_list, sa_list, k, [None] * len(ix_list))
    return L.dsa_similarity_matrix_workspace_size(len(ix_list), arr, k)


def similarity_matrix(ix_list, sa_list, k, *, idx_out=None, ws=None):
    """Similarity matrix of the pattern search: every layer's own Top-k, then
    S[i, j] = mean row cosine of layer i's attention output under T_i and under T_j.
    ix_list[l]: {"q", "k", "w", optional "q_scale", "k_scale", "q_pos0"};
    sa_list[l]: {"q", "kv", "scale", optional "v", "d_v"} ("out" is not used).
    Returns (S float64 [N, N] on the device, [T_l int32 [B, n_q, k]])."""
    n = len(ix_list)
    dev = sa_list[0]["q"].device
    B, n_q = ix_list[0]["q"].shape[:2]
    if idx_out is None:
        idx_out = [torch.empty((B, n_q, k), dtype=torch.int32, device=dev) for _ in range(n)]
    arr = _sim_layers(ix_list, sa_list, k, idx_out)
    need = L.dsa_similarity_matrix_workspace_size(n, arr, k)
    if need == 0:
        L.check(L.dsa_similarity_matrix(n, arr, k, None, None, 0, _stream()))   # raises with the reason
    wbuf, wbytes = _ws(need, dev, ws)
    S = torch.empty((n, n), dtype=torch.float64, device=dev)
    L.check(L.dsa_similarity_matrix(n, arr, k, S.data_ptr(), wbuf.data_ptr(), wbytes, _stream()))
    return S, idx_out


def pattern_search(S, n_full):
    """Sharing pattern with layer 0 F and n_full F layers maximising the total
    similarity (host dynamic program).  S: [N, N] (numpy or torch, any device).
    Returns (pattern str, score)."""
    if isinstance(S, torch.Tensor):
        S = S.detach().to("cpu", torch.float64).numpy()
    import numpy as np
    S = np.ascontiguousarray(S, dtype=np.float64)
    n = S.shape[0]
    buf = ctypes.create_string_buffer(n + 1)
    score = ctypes.c_double()
    L.check(L.dsa_pattern_search(S.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), n, int(n_full), buf,
                                 ctypes.byref(score)))
    return buf.value.decode(), score.value


def gather_probe(kv, idx, mode, *, out=None):
    """Measurement helper: read every selected 1152-byte latent row (kv
    [n_rows, 576] bf16 or [n_rows, 1, 576]) of idx [n_q, topk] with access
    pattern `mode` (0..10); returns the uint32 checksums (as int32)."""
    n_rows = kv.shape[0]
    L._dense("kv", kv)
    L._dense("idx", idx)
    idx2 = idx.reshape(-1, idx.shape[-1])
    n_q, topk = idx2.shape
    words = L.dsa_gather_probe_out_words(n_q, mode)
    if out is None:
        out = torch.empty(max(words, 1), dtype=torch.int32, device=kv.device)
    L.check(L.dsa_gather_probe(kv.data_ptr(), n_rows, idx2.data_ptr(), n_q, topk, mode, out.data_ptr(), _stream()))
    return out


def stream_probe(buf, workgroups, unroll, *, out=None):
    """Measurement helper: read the contiguous device buffer `buf` (its bytes a
    multiple of 16384) once in order with `workgroups` workgroups and `unroll`
    16-KiB chunks in flight per wave; returns the uint32 checksums (as int32)."""
    L._dense("buf", buf)
    nbytes = buf.numel() * buf.element_size()
    if out is None:
        out = torch.empty(4 * workgroups, dtype=torch.int32, device=buf.device)
    L.check(L.dsa_stream_probe(buf.data_ptr(), nbytes, workgroups, unroll, out.data_ptr(), _stream()))
    return out
