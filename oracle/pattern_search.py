"""Oracle for the similarity-based sharing-pattern search.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Float64 NumPy; the
search is a brute-force enumeration of every admissible pattern (the plain
definition of the optimum), usable for small layer counts only.

Source: [IC-SUMMARY] Appendix C ("基于相似度的模式搜索", similarity-based
pattern search): for every layer pair (i, j) with i > j, S[i, j] is the cosine
similarity between layer i's core attention output computed with its own index
set and the same output computed with layer j's index set; given S and a target
number M of F layers, the pattern c* maximising the total similarity is sought,
where an S layer l takes its index set from src(l) = max{j < l : c_j = F}.  The
page solves it with a dynamic program over dp[i][k] (best total for layers
1..i with exactly k F layers, layer i itself F); its objective and transition
equations are not legible on the page.

Readings (also listed in the design notes):
  * the cosine similarity of two attention outputs is taken per query row over
    the row's whole output (every head, every value column) and averaged over the
    calibration rows; a row where both outputs are zero counts 1 (they agree),
    a row where exactly one is zero counts 0;
  * the objective is the sum over the S layers l of S[l, src(l)]; F layers add
    nothing (their own index set; adding a constant per F layer would not move
    the argmax at a fixed M);
  * the first layer is always F (every S layer needs a preceding F layer), as
    in every pattern the pages print;
  * layers are numbered from 0 here: S[i, j] is row i (the layer that reuses),
    column j (the layer whose index set it reuses), i > j.
"""
from __future__ import annotations

import itertools

import numpy as np


def row_cosine(a, b):
    """Per-row cosine similarity of two equally shaped outputs, each row
    flattened ([IC-SUMMARY] Appendix C; the zero-row convention is a reading).
    Returns float64 [rows]."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    a = a.reshape(a.shape[0], -1)
    b = b.reshape(b.shape[0], -1)
    out = np.empty(a.shape[0])
    for r in range(a.shape[0]):
        na = np.sqrt(np.dot(a[r], a[r]))
        nb = np.sqrt(np.dot(b[r], b[r]))
        if na == 0.0 or nb == 0.0:
            out[r] = 1.0 if (na == 0.0 and nb == 0.0) else 0.0
        else:
            out[r] = np.dot(a[r], b[r]) / (na * nb)
    return out


def output_similarity(own, reused):
    """One entry S[i, j]: mean over rows of the per-row cosine between layer i's
    output with its own index set (`own`) and with layer j's (`reused`)."""
    c = row_cosine(own, reused)
    return float(c.mean()) if c.size else float("nan")


def similarity_matrix(attn_fn, T_layers):
    """S for N layers ([IC-SUMMARY] Appendix C, construction of the matrix):
    attn_fn(i, T) -> layer i's attention output given index tensor T;
    T_layers[j] -> layer j's own index tensor.  Returns [N, N] with S[i, j] for
    i > j, 1 on the diagonal and 0 above it."""
    n = len(T_layers)
    S = np.eye(n)
    for i in range(n):
        own = attn_fn(i, T_layers[i])
        for j in range(i):
            S[i, j] = output_similarity(own, attn_fn(i, T_layers[j]))
    return S


def sources(pattern: str):
    """src(l) for every layer (0-based): l itself for an F layer, else the
    nearest preceding F layer."""
    if not pattern or any(c not in "FS" for c in pattern) or pattern[0] != "F":
        raise ValueError("a pattern is a string over {F, S} that starts with F")
    out, last = [], 0
    for l, c in enumerate(pattern):
        if c == "F":
            last = l
        out.append(last)
    return out


def pattern_objective(S, pattern: str) -> float:
    """Total similarity of a pattern: sum over its S layers l of S[l, src(l)]."""
    S = np.asarray(S, dtype=np.float64)
    src = sources(pattern)
    return float(sum(S[l, src[l]] for l, c in enumerate(pattern) if c == "S"))


def pattern_search_brute(S, n_full: int):
    """Every pattern of len(S) layers with layer 0 F and exactly n_full F layers,
    scored by pattern_objective.  Returns (best score, [optimal patterns]) where a
    pattern is optimal when its score is within 1e-12 * (1 + |best|) of the best."""
    S = np.asarray(S, dtype=np.float64)
    n = S.shape[0]
    if not 1 <= n_full <= n:
        raise ValueError("n_full must lie in [1, number of layers]")
    scored = []
    for rest in itertools.combinations(range(1, n), n_full - 1):
        c = ["S"] * n
        c[0] = "F"
        for l in rest:
            c[l] = "F"
        p = "".join(c)
        scored.append((pattern_objective(S, p), p))
    best = max(s for s, _ in scored)
    tol = 1e-12 * (1.0 + abs(best))
    return best, [p for s, p in scored if s >= best - tol]
