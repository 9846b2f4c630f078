"""Oracle for the DSA indexer, Top-k, sparse attention and IndexCache's F/S
layer loop.  Float64, one batch element at a time, no blocking or fusion.

Readings taken where the pages leave a step open (each also listed in the
design notes of the repository):
  * causal candidates for query position t are s = 0..t inclusive;
  * the indexer key carries no head index (one key per token for all heads);
  * no extra scale factor inside the score beyond w;
  * Top-k is taken under the total order (score descending, position
    ascending) -- ties go to the lower position; -0.0 equals +0.0;
  * a row with fewer than k candidates selects all of them;
  * an index row is returned in ascending position order, padded with -1;
  * an index entry outside [0, n_k) (e.g. the -1 padding) selects nothing;
  * attention over an empty selection returns zeros.
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def indexer_scores(q, k, w, q_pos0=0, rows=None):
    """Lightning-indexer scores ([DSA-NOTES] §2.1, score equation; candidates are
    all previous tokens, [IC-SUMMARY] §2.1):

        I[t, s] = sum_j w[t, j] * ReLU(q[t, j, :] . k[s, :]),   s <= t

    q: [n_q, H, d], k: [n_k, d], w: [n_q, H]   (float64, already dequantised)
    rows: query rows to evaluate (default all).  Query row i sits at absolute
    position t = q_pos0 + i.
    Returns (I, A): both [len(rows), n_k]; I is -inf where s > t.  A is the
    error scale sum_j |w[t, j]| * ReLU(q . k) used by the parity tolerance.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    n_q = q.shape[0]
    n_k = k.shape[0]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    I = np.full((len(rows), n_k), NEG_INF)
    A = np.zeros((len(rows), n_k))
    for r, i in enumerate(rows):
        t = int(q_pos0) + int(i)
        n = min(t + 1, n_k)
        if n <= 0:
            continue
        D = q[i] @ k[:n].T                     # [H, n]: per-head dot products
        R = np.maximum(D, 0.0)
        I[r, :n] = w[i] @ R + 0.0              # + 0.0 turns -0.0 into +0.0
        A[r, :n] = np.abs(w[i]) @ R
    return I, A


def topk_row(scores, k):
    """Top-k of one row ([IC-SUMMARY] notation: T_t = Top-k(I_t), k = 2048).

    scores: the row's candidate scores, position s at scores[s].
    Returns int64 [k]: the selected positions ascending, then -1 padding."""
    scores = np.asarray(scores, dtype=np.float64) + 0.0
    n = scores.shape[0]
    pos = np.arange(n)
    order = np.lexsort((pos, -scores))        # primary: score desc; secondary: pos asc
    sel = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:sel.shape[0]] = sel
    return out


def indexer_topk(q, k, w, topk, q_pos0=0, rows=None):
    """INDEXER then Top-k for the given query rows ([IC-SUMMARY] Algorithm (b),
    steps 3-4).  Returns (idx [len(rows), topk], I, A)."""
    I, A = indexer_scores(q, k, w, q_pos0, rows)
    n_k = np.asarray(k).shape[0]
    rows_ = np.arange(np.asarray(q).shape[0]) if rows is None else np.asarray(rows)
    idx = np.empty((len(rows_), topk), dtype=np.int64)
    for r, i in enumerate(rows_):
        n = min(int(q_pos0) + int(i) + 1, n_k)
        idx[r] = topk_row(I[r, :max(n, 0)], topk)
    return idx, I, A


def sparse_attn(Q, K, V, idx, scale, rows=None):
    """Sparse core attention over selected positions ([DSA-NOTES] §3, equation
    for o_t: softmax over s in T_t of Q_t.K_s / sqrt(d), weighting V_s).

    Q: [n_q, heads, d_qk]; K: [n_k, kv_heads, d_qk]; V: [n_k, kv_heads, d_v];
    idx: [n_q, topk] (entries outside [0, n_k) are ignored); scale replaces
    1/sqrt(d).  Query head h reads kv head h * kv_heads // heads.
    Returns [len(rows), heads, d_v] float64."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    n_q, heads, _ = Q.shape
    n_k, kv_heads, _ = K.shape
    d_v = V.shape[-1]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    out = np.zeros((len(rows), heads, d_v))
    for r, i in enumerate(rows):
        sel = np.asarray(idx[i])
        sel = sel[(sel >= 0) & (sel < n_k)]
        if sel.size == 0:
            continue
        for h in range(heads):
            hk = h * kv_heads // heads
            z = scale * (K[sel, hk, :] @ Q[i, h, :])
            p = np.exp(z - z.max())
            p /= p.sum()
            out[r, h] = p @ V[sel, hk, :]
    return out


def source_layers(pattern: str):
    """f(l) = max{j <= l : c_j = F} for every layer (1-based), per [IC-SUMMARY]
    §3 (IndexCache core mechanism): an S layer inherits the nearest preceding F
    layer's index set; layer 1 is always F.  An F layer is its own source."""
    if not pattern or any(c not in "FS" for c in pattern):
        raise ValueError("pattern must be a non-empty string over {F, S}")
    if pattern[0] != "F":
        raise ValueError("the first layer must be F")
    src, last = [], None
    for l, c in enumerate(pattern, start=1):
        if c == "F":
            last = l
        src.append(last)
    return src


def indexcache_forward(pattern, indexer_fn, attn_fn):
    """IndexCache inference loop ([IC-SUMMARY] Algorithm (b); [DSA-NOTES] §2.2,
    FSSS FSSS trace): for l = 1..N, an F layer runs its indexer and Top-k and
    replaces the cached index tensor; an S layer reuses the cached tensor.
    Every layer then runs its own sparse attention on the layer's index tensor.

    indexer_fn(l) -> index tensor of F layer l (1-based; called for F layers only)
    attn_fn(l, T) -> that layer's attention output given index tensor T
    Returns (src, T_per_layer, outputs, indexer_calls)."""
    src = source_layers(pattern)
    T_cache = None
    Ts, outs, calls = [], [], []
    for l, c in enumerate(pattern, start=1):
        if c == "F":
            T_cache = indexer_fn(l)
            calls.append(l)
        Ts.append(T_cache)
        outs.append(attn_fn(l, T_cache))
    return src, Ts, outs, calls


def mli_source_layers(pattern: str):
    """Sources under the multi-layer-indexer shift ([MLI] "核心思路": a layer
    reuses the index set the previous indexer already produced, which frees its
    own indexer to run beside its attention), combined with IndexCache's F/S
    pattern ([MLI] "与 IndexCache／IndexShare 的组合"): layer l attends with the
    index tensor of the nearest F layer j < l; layer 1 has no earlier indexer
    and uses its own.  An S layer's source is the one IndexCache gives it; an F
    layer l > 1 takes the source IndexCache gives layer l - 1.  1-based."""
    source_layers(pattern)                       # same validation
    src, last = [], None
    for l, c in enumerate(pattern, start=1):
        src.append(l if last is None else last)
        if c == "F":
            last = l
    return src


def mli_forward(pattern, indexer_fn, attn_fn):
    """IndexCache loop with the multi-layer-indexer shift ([MLI] "核心思路"):
    for l = 1..N, an F layer runs its indexer (beside its attention, on
    hardware that overlaps them); layer l's attention uses the cached index
    tensor as it stood before layer l's indexer, except on layer 1, which has
    none and waits for its own; then an F layer's new tensor replaces the cache.
    Same arguments and returns as indexcache_forward."""
    src = mli_source_layers(pattern)
    T_cache = None
    Ts, outs, calls = [], [], []
    for l, c in enumerate(pattern, start=1):
        T_new = None
        if c == "F":
            T_new = indexer_fn(l)
            calls.append(l)
        T_use = T_cache if T_cache is not None else T_new
        Ts.append(T_use)
        outs.append(attn_fn(l, T_use))
        if T_new is not None:
            T_cache = T_new
    return src, Ts, outs, calls


def overlap(Ta, Tb, k, rows=None):
    """overlap(i, j) = |T^(i) ∩ T^(j)| / k ([DSA-NOTES] §3.1; [IC-SUMMARY]
    Appendix A), averaged over the given rows (default: every row).  Entries
    equal to -1 are padding and belong to no set."""
    Ta = np.asarray(Ta)
    Tb = np.asarray(Tb)
    rows = np.arange(Ta.shape[0]) if rows is None else np.asarray(rows)
    if len(rows) == 0:
        return float("nan")
    tot = 0.0
    for r in rows:
        a = set(int(x) for x in Ta[r] if x >= 0)
        b = set(int(x) for x in Tb[r] if x >= 0)
        tot += len(a & b) / k
    return tot / len(rows)


def overlap_matrix(T_layers, k, rows=None):
    n = len(T_layers)
    M = np.eye(n)
    for i in range(n):
        for j in range(i + 1, n):
            M[i, j] = M[j, i] = overlap(T_layers[i], T_layers[j], k, rows)
    return M


def amdahl_speedup(indexer_fraction, retained_fraction):
    """Speedup when only a fraction of indexer work is kept and the rest of the
    time is unchanged ([DSA-NOTES] §10.2): 1 / ((1 - f) + f * r)."""
    f = float(indexer_fraction)
    return 1.0 / ((1.0 - f) + f * float(retained_fraction))
