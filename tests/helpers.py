"""Test-side glue: raw tensor bytes -> oracle inputs, and the parity rules.

Parity rules (floating point):
  * indexer scores: |I_gpu - I_ref| <= 1e-3 * A_ref, with A = sum_j |w| ReLU(q.k)
  * index sets on float inputs: equal sizes, and every position in the
    symmetric difference has |I_ref(s) - I_ref(kth)| <= 1e-3 * |I_ref(kth)|
  * sparse attention: per (row, head) max_c |o_gpu - o_ref| <= 2e-3 * max_c |o_ref|
Integer-valued inputs: indices bit-exact and scores exactly equal.
"""
import numpy as np
import torch

import oracle

SCORE_RTOL = 1e-3
ATTN_RTOL = 2e-3


def raw(t: torch.Tensor):
    """torch tensor -> (numpy raw storage, dtype string) for oracle.dequantize."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy(), "f32"
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16), "bf16"
    if t.dtype == torch.float8_e4m3fn:
        return t.view(torch.uint8).numpy(), "fp8"
    raise TypeError(t.dtype)


def deq(t: torch.Tensor, scale: torch.Tensor = None):
    r, dt = raw(t)
    s = None if scale is None else scale.detach().cpu().float().numpy()
    return oracle.dequantize(r, dt, s)


def indexer_f64(ix, b=0, q_rows=None, k_rows=None):
    """Dequantised float64 (q [n_q,H,d], k [n_k,d], w [n_q,H]) for batch b."""
    q = ix.q[b] if q_rows is None else ix.q[b, q_rows]
    qs = None if ix.q_scale is None else (ix.q_scale[b] if q_rows is None else ix.q_scale[b, q_rows])
    k = ix.k[b] if k_rows is None else ix.k[b, k_rows]
    ks = None if ix.k_scale is None else (ix.k_scale[b] if k_rows is None else ix.k_scale[b, k_rows])
    w = ix.w[b] if q_rows is None else ix.w[b, q_rows]
    return deq(q, qs), deq(k, ks), w.detach().cpu().double().numpy()


def sa_f64(sa, b=0, q_rows=None):
    Q = deq(sa.q[b] if q_rows is None else sa.q[b, q_rows])
    KV = deq(sa.kv[b])
    V = KV[..., :sa.d_v] if sa.v is None else deq(sa.v[b])
    return Q, KV, V


def check_index_set(gpu_row, ref_row, ref_scores, k):
    """Float-input index-set rule; returns None if fine, else a message."""
    g = set(int(x) for x in gpu_row if x >= 0)
    r = set(int(x) for x in ref_row if x >= 0)
    if len(g) != len(r):
        return f"set sizes differ: gpu {len(g)} ref {len(r)}"
    diff = g ^ r
    if not diff:
        return None
    sc = np.asarray(ref_scores, dtype=np.float64)
    order = np.lexsort((np.arange(sc.size), -sc))
    kth = sc[order[min(k, sc.size) - 1]]
    bad = [s for s in diff if abs(sc[s] - kth) > SCORE_RTOL * abs(kth)]
    if bad:
        return f"{len(bad)} positions outside the tie window, e.g. s={bad[0]} score={sc[bad[0]]} kth={kth}"
    return None


def check_ascending_padded(row, t, k):
    row = np.asarray(row)
    n = int((row >= 0).sum())
    assert n == min(k, t + 1), (n, t, k)
    assert (row[n:] == -1).all()
    v = row[:n]
    assert (np.diff(v) > 0).all() if n > 1 else True
    assert (v >= 0).all() and (v <= t).all()


def attn_close(gpu, ref):
    """max over rows/heads of  max_c|diff| / max_c|ref|  (<= ATTN_RTOL passes)."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    num = np.abs(gpu - ref).max(axis=-1)
    den = np.maximum(np.abs(ref).max(axis=-1), 1e-30)
    return float((num / den).max())
