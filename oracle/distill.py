"""Oracle for training-aware IndexCache: the indexer-side multi-layer
distillation loss over the selected Top-k positions and its backward.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Float64 NumPy, one
query row at a time, no blocking or fusion.

Sources:
  [IC-SUMMARY] §3.2 "training-aware IndexCache with layer-wise distillation":
      a retained (F) layer's indexer is distilled towards the attention
      distributions of every layer that uses its index set; Proposition 1: the
      gradient of the summed KL terms equals that of a single KL to the average
      target; in the sparse-training stage the KL is taken over the selected
      top-k tokens only.
  [DSA-NOTES] §5.1 (L_multi = (1/r) sum_j KL(p^(j) || pi_theta), pi = softmax(z)),
      §5.2 (the average teacher p_bar and the gradient identity),
      §7.1 (delta_s = dL/dz_s = pi_s - p_s; dL/dq = sum_s delta_s k_s;
      dL/dk_s = delta_s q; dL/dW_q = (dL/dq) x^T),
      §7.2 (worked example: pi = (0.7, 0.3), p = (0.2, 0.8) -> delta = (0.5, -0.5),
      dL/dW_q = [[0.5, 0], [-0.5, 0]]),
      §7.3 (multi-head ReLU scores: dL/dq_j = sum_s delta_s w_j 1[q_j.k_s > 0] k_s).

Readings (also listed in the design notes):
  * z_t(s) is the lightning-indexer score I[t, s] of the selected position s;
    pi_t = softmax over the valid entries of the row's index set (the -1
    padding and positions outside [0, min(t, n_k - 1)] take no part);
  * the loss carries the 1/r normalisation of [DSA-NOTES] §5.1 (the form for
    which Proposition 1 holds as an equality); 0 * log 0 = 0 for teacher zeros;
  * teachers are given per selected entry; they need not sum to 1, so the exact
    derivative dL/dz_e = pi_e * sum(p_bar) - p_bar_e is used (it is the pages'
    pi_e - p_bar_e when the teachers are distributions);
  * ReLU's derivative is 1[q_j . k_s > 0] ([DSA-NOTES] §7.3), 0 at 0;
  * the key-side gradient accumulates, for every key s, the contributions of
    every (query row, head) pair whose index set holds s: dL/dk_s =
    sum_t delta_t(s) sum_j w_tj 1[q_tj . k_s > 0] q_tj (the single-head form
    dL/dk_s = delta_s q of §7.1, summed over heads and query rows).
"""
from __future__ import annotations

import numpy as np


def kl_multi(z, teachers):
    """Multi-layer distillation loss of one row and its gradient w.r.t. the
    scores ([DSA-NOTES] §5.1-5.2, §7.1).

    z: [n] indexer scores of the row's valid selected entries.
    teachers: [r, n] teacher weights p^(j) over the same entries.
    Returns (loss, pi, delta): loss = (1/r) sum_j sum_e p_je (log p_je - log pi_e)
    with 0 log 0 = 0; pi = softmax(z); delta = dloss/dz = pi * sum(p_bar) - p_bar.
    """
    z = np.asarray(z, dtype=np.float64)
    P = np.atleast_2d(np.asarray(teachers, dtype=np.float64))
    r = P.shape[0]
    if z.size == 0:
        return 0.0, z.copy(), z.copy()
    m = z.max()
    lse = m + np.log(np.exp(z - m).sum())
    log_pi = z - lse
    pi = np.exp(log_pi)
    loss = 0.0
    for j in range(r):
        p = P[j]
        nz = p > 0
        loss += float((p[nz] * (np.log(p[nz]) - log_pi[nz])).sum())
    loss /= r
    p_bar = P.mean(axis=0)
    delta = pi * p_bar.sum() - p_bar
    return loss, pi, delta


def kl_average(z, teachers):
    """The single-target loss of Proposition 1 ([DSA-NOTES] §5.2):
    KL(p_bar || softmax(z)) with p_bar the mean teacher.  Returns (loss, delta)."""
    P = np.atleast_2d(np.asarray(teachers, dtype=np.float64))
    loss, pi, delta = kl_multi(z, P.mean(axis=0, keepdims=True))
    return loss, delta


def selected_valid(idx_row, t, n_k):
    """Entries of one index row that select a candidate: positions in
    [0, min(t, n_k - 1)] (causal), the -1 padding excluded."""
    idx_row = np.asarray(idx_row, dtype=np.int64)
    lim = min(int(t), n_k - 1)
    return (idx_row >= 0) & (idx_row <= lim)


def indexer_distill(q, k, w, idx, teachers, q_pos0=0, rows=None):
    """Forward and backward of the distillation loss for one batch element.

    q: [n_q, H, d], k: [n_k, d], w: [n_q, H] (float64, dequantised);
    idx: [n_q, topk] index rows (ascending, -1 padded);
    teachers: [r, n_q, topk] teacher weights per index entry (0 on padding);
    rows: query rows to evaluate (default all).  Row i sits at t = q_pos0 + i.

    Per row: z_e = sum_j w_j ReLU(q_j . k_{idx_e}) over the valid entries,
    (loss, pi, delta) = kl_multi(z, teachers); then
      dw_j = sum_e delta_e ReLU(D_je),
      dq_j = sum_e delta_e w_j 1[D_je > 0] k_{idx_e},
      dk_s += sum_{e: idx_e = s} delta_e sum_j w_j 1[D_je > 0] q_j,
    with D_je = q_j . k_{idx_e}.
    Returns dict(loss [R], delta [R, topk] (0 on invalid entries), dq [R, H, d],
    dw [R, H], dk [n_k, d] (summed over the evaluated rows), dq_scale,
    dw_scale, dk_scale): the *_scale arrays hold the same sums with every term
    taken in absolute value (the error scale of the parity tolerance).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    idx = np.asarray(idx, dtype=np.int64)
    T = np.asarray(teachers, dtype=np.float64)
    n_q, H, d = q.shape
    n_k = k.shape[0]
    topk = idx.shape[1]
    rows = np.arange(n_q) if rows is None else np.asarray(rows)
    R = len(rows)
    out = dict(loss=np.zeros(R), delta=np.zeros((R, topk)), dq=np.zeros((R, H, d)), dw=np.zeros((R, H)),
               dk=np.zeros((n_k, d)), dq_scale=np.zeros((R, H, d)), dw_scale=np.zeros((R, H)),
               dk_scale=np.zeros((n_k, d)))
    for r, i in enumerate(rows):
        t = int(q_pos0) + int(i)
        valid = selected_valid(idx[i], t, n_k)
        e = np.nonzero(valid)[0]
        if e.size == 0:
            continue
        s = idx[i, e]
        Ks = k[s]                                   # [n, d]
        D = q[i] @ Ks.T                             # [H, n]
        M = (D > 0).astype(np.float64)
        Rl = D * M                                  # ReLU(D)
        z = w[i] @ Rl
        loss, pi, delta = kl_multi(z, T[:, i, e])
        out['loss'][r] = loss
        out['delta'][r, e] = delta
        out['dw'][r] = Rl @ delta
        out['dw_scale'][r] = Rl @ np.abs(delta)
        G = (w[i][:, None] * M) * delta[None, :]    # [H, n]: dz_e/dD_je * delta_e
        out['dq'][r] = G @ Ks
        out['dq_scale'][r] = np.abs(G) @ np.abs(Ks)
        Y = G.T @ q[i]                              # [n, d]: per-entry key gradients
        Ys = np.abs(G).T @ np.abs(q[i])
        np.add.at(out['dk'], s, Y)
        np.add.at(out['dk_scale'], s, Ys)
    return out
