"""GPU parity of the similarity-based pattern search's device steps
([IC-SUMMARY] Appendix C): the per-row cosine kernel and the similarity matrix
(every layer's own Top-k, attention under its own and every earlier layer's
index tensor, row cosines, row mean) against the float64 oracle.

Tolerances:
  * row cosine on the same fp32 inputs: |c_gpu - c_ref| <= 2e-7 (the kernel sums
    in float64; only the final rounding to fp32 remains); mean within 2e-7
  * index tensors (integer-valued inputs): bit-exact
  * S entries: |S_gpu - S_ref| <= 1e-4 (attention outputs agree to ~1e-5
    relative; a cosine moves by less)
  * the searched pattern: its objective under S_ref within N * 1e-4 of the
    brute-force optimum of S_ref
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import pattern_search as ps
from synth import inputs as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import dsa_lightning_indexer_amd as m
    return m


def _rows(dev, rows, width, seed):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    a = torch.randn((rows, width), generator=g, device=dev)
    b = 0.7 * a + 0.5 * torch.randn((rows, width), generator=g, device=dev)
    return a, b


@pytest.mark.parametrize("rows,width", [(37, 8192), (5, 4), (9, 1028), (3, 12292)])
def test_row_cosine_matches_oracle(dsa, dev, rows, width):
    """Widths that run the unrolled loop, only the tail loop, and both."""
    a, b = _rows(dev, rows, width, seed=rows + width)
    b[1] = -3.0 * a[1]                      # antiparallel -> -1
    b[2] = 0.0
    a[2] = 0.0                              # both zero -> 1
    if rows > 3:
        b[3] = 0.0                          # one zero row -> 0
    c, m = dsa.row_cosine(a, b)
    torch.cuda.synchronize()
    ref = ps.row_cosine(a.cpu().numpy(), b.cpu().numpy())
    got = c.cpu().double().numpy()
    assert np.abs(got - ref).max() <= 2e-7, float(np.abs(got - ref).max())
    assert got[1] == pytest.approx(-1.0, abs=2e-7) and got[2] == 1.0
    if rows > 3:
        assert got[3] == 0.0
    assert abs(float(m.item()) - ref.mean()) <= 2e-7
    c2, m2 = dsa.row_cosine(a, b)
    assert torch.equal(c, c2) and torch.equal(m, m2)


def test_row_cosine_full_size_sampled(dsa, dev):
    """Attention-output shape of a 16384-row calibration layer (16 heads x 512)."""
    rows, width = 16384, 16 * 512
    a, b = _rows(dev, rows, width, seed=7)
    c, m = dsa.row_cosine(a, b)
    torch.cuda.synchronize()
    sample = np.array([0, 1, 4095, 4096, 9999, rows - 1])
    ref = ps.row_cosine(a[sample].cpu().numpy(), b[sample].cpu().numpy())
    assert np.abs(c[sample].cpu().double().numpy() - ref).max() <= 2e-7
    # mean in float64 of the fp32 row values
    assert abs(float(m.item()) - c.double().mean().item()) <= 1e-12


def _specs(layers):
    ixs = [dict(q=ix.q, k=ix.k, w=ix.w, q_scale=ix.q_scale, k_scale=ix.k_scale, q_pos0=ix.q_pos0) for ix, _ in layers]
    sas = [dict(q=sa.q, kv=sa.kv, scale=sa.scale, d_v=sa.d_v) for _, sa in layers]
    return ixs, sas


def _oracle_matrix(layers, k, b_rows):
    """Oracle S from the oracle's own Top-k: rows of every batch element stacked."""
    n = len(layers)
    T = []
    for ix, _ in layers:
        per_b = []
        for b in range(ix.q.shape[0]):
            q, kk, w = H.indexer_f64(ix, b)
            idx, _, _ = oracle.indexer_topk(q, kk, w, k, q_pos0=ix.q_pos0)
            per_b.append(idx)
        T.append(per_b)

    def attn(i, Ti):
        sa = layers[i][1]
        outs = []
        for b in range(b_rows):
            Q, KV, V = H.sa_f64(sa, b)
            outs.append(oracle.sparse_attn(Q, KV, V, Ti[b], sa.scale))
        return np.concatenate(outs, axis=0)
    return ps.similarity_matrix(attn, T), T


@pytest.mark.parametrize("case", ["prefill_bf16", "decode_fp8"])
def test_similarity_matrix_matches_oracle(dsa, dev, case):
    if case == "prefill_bf16":
        layers, _ = syn.drift_stack(n_layers=5, n_q=160, values="int", seed=11, device=dev, p_jump=0.3)
        k = 64
    else:   # decode rows: one query per sequence at the end of a 3000-key cache
        layers, _ = syn.drift_stack(n_layers=4, B=2, n_q=1, n_k=3000, q_pos0=2999, dtype=syn.FP8, values="int",
                                    seed=12, device=dev)
        k = 256
    ixs, sas = _specs(layers)
    S, T = dsa.similarity_matrix(ixs, sas, k)
    torch.cuda.synchronize()
    S_ref, T_ref = _oracle_matrix(layers, k, layers[0][0].q.shape[0])
    for l in range(len(layers)):
        for b in range(len(T_ref[l])):
            assert np.array_equal(T[l][b].cpu().numpy(), T_ref[l][b]), (l, b)
    S = S.cpu().numpy()
    assert np.abs(S - S_ref).max() <= 1e-4, float(np.abs(S - S_ref).max())
    n = len(layers)
    for m in range(1, n + 1):
        pat, score = dsa.pattern_search(S, m)
        best, _ = ps.pattern_search_brute(S_ref, m)
        assert ps.pattern_objective(S_ref, pat) >= best - n * 1e-4


def test_similarity_matrix_full_size_properties(dsa, dev):
    """Calibration prefill at L = 16384 (float inputs, 4 layers): each T_l equals
    the layer's own Top-k call, each S entry equals the row-cosine mean of two
    separate attention calls (the same kernels), the diagonal is 1, the upper
    triangle 0 and every entry lies in [-1, 1]; rows t < k select every causal
    position under any layer's index tensor, so their cosine is exactly 1."""
    L_, k = 16384, 2048
    layers, _ = syn.drift_stack(n_layers=4, n_q=L_, seed=13, device=dev)
    ixs, sas = _specs(layers)
    S, T = dsa.similarity_matrix(ixs, sas, k)
    torch.cuda.synchronize()
    n = len(layers)
    Sc = S.cpu().numpy()
    assert np.array_equal(np.diag(Sc), np.ones(n)) and np.all(np.triu(Sc, 1) == 0)
    assert np.all(np.abs(Sc) <= 1.0 + 1e-6)
    for l, (ix, _) in enumerate(layers):
        assert torch.equal(T[l], dsa.topk(ix.q, ix.k, ix.w, k))
    for i, j in [(1, 0), (3, 1), (3, 2)]:
        sa = layers[i][1]
        o_own = dsa.sparse_attn(sa.q, sa.kv, T[i], sa.scale, d_v=sa.d_v)
        o_re = dsa.sparse_attn(sa.q, sa.kv, T[j], sa.scale, d_v=sa.d_v)
        c, m = dsa.row_cosine(o_own.reshape(L_, -1), o_re.reshape(L_, -1))
        assert float(m.item()) == Sc[i, j]
        assert torch.all(c[:k] == 1.0)
