"""Pins of the similarity-based pattern-search oracle ([IC-SUMMARY] Appendix C)
against closed forms: cosines of vectors at known angles, single-position
attention (whose output is the selected value row), and objective/search cases
whose optimum follows from the structure of S."""
import math

import numpy as np
import pytest

import oracle
from oracle import pattern_search as ps


def test_row_cosine_known_angles():
    """Row r holds 3 (cos t_r, sin t_r, 0) against 2 (1, 0, 0): the cosine is
    cos t_r whatever the lengths; a dropped square root or a missing norm
    changes it."""
    t = np.array([0.0, 0.3, 1.1, math.pi / 2, 2.5, math.pi])
    a = 3.0 * np.stack([np.cos(t), np.sin(t), np.zeros_like(t)], axis=1)
    b = np.tile(np.array([2.0, 0.0, 0.0]), (len(t), 1))
    assert np.allclose(ps.row_cosine(a, b), np.cos(t), atol=1e-15)
    assert np.allclose(ps.row_cosine(b, a), np.cos(t), atol=1e-15)


def test_row_cosine_flattens_each_row_and_zero_rows():
    """A row is compared as one vector over all its heads and columns: two heads
    (1, 0) and (0, 1) against (1, 0) and (0, 0) -> cos = 1/sqrt(2).  Both rows zero
    -> 1; one zero row -> 0."""
    a = np.array([[[1.0, 0.0], [0.0, 1.0]], [[0.0, 0.0], [0.0, 0.0]], [[0.0, 0.0], [0.0, 0.0]]])
    b = np.array([[[1.0, 0.0], [0.0, 0.0]], [[0.0, 0.0], [0.0, 0.0]], [[5.0, 0.0], [0.0, 0.0]]])
    assert np.allclose(ps.row_cosine(a, b), [1 / math.sqrt(2), 1.0, 0.0], atol=1e-15)
    assert ps.output_similarity(a, b) == pytest.approx((1 / math.sqrt(2) + 1.0) / 3, abs=1e-15)


def _single_position_layers(phis, picks):
    """Layers whose attention selects one position per row (k = 1): the output is
    that position's value row exactly.  Layer i's values are unit 2-D vectors at
    angles phis[i][s]; picks[j] is layer j's index tensor [n_q, 1]."""
    n_q = picks[0].shape[0]

    def attn(i, T):
        V = np.stack([np.cos(phis[i]), np.sin(phis[i])], axis=1)[:, None, :]   # [n_k, 1, 2]
        K = np.zeros((len(phis[i]), 1, 4))
        Q = np.zeros((n_q, 1, 4))
        return oracle.sparse_attn(Q, K, V, T, scale=1.0)
    return attn


def test_similarity_matrix_single_position_closed_form():
    """S[i, j] = mean over rows of cos(phi_i[T_i(r)] - phi_i[T_j(r)]): layer i's own
    values, layer j's picks.  Using layer j's values, or the wrong triangle,
    changes the result."""
    rng = np.random.default_rng(3)
    n, n_k, n_q = 4, 9, 5
    phis = [rng.uniform(0, 2 * math.pi, n_k) for _ in range(n)]
    picks = [rng.integers(0, n_k, (n_q, 1)) for _ in range(n)]
    S = ps.similarity_matrix(_single_position_layers(phis, picks), picks)
    for i in range(n):
        assert S[i, i] == 1.0
        for j in range(n):
            if j > i:
                assert S[i, j] == 0.0
            elif j < i:
                want = np.mean(np.cos(phis[i][picks[i][:, 0]] - phis[i][picks[j][:, 0]]))
                assert S[i, j] == pytest.approx(want, abs=1e-14)


def test_similarity_matrix_identical_index_sets():
    """A layer whose reused index set equals its own scores exactly 1."""
    rng = np.random.default_rng(4)
    n_q, n_k, H, d = 6, 30, 2, 8
    Q = rng.standard_normal((n_q, H, d))
    K = rng.standard_normal((n_k, 1, d))
    V = rng.standard_normal((n_k, 1, d))
    T = np.sort(rng.choice(n_k, (n_q, 7)), axis=1)
    S = ps.similarity_matrix(lambda i, t: oracle.sparse_attn(Q, K, V, t, 0.3), [T, T.copy(), T.copy()])
    assert np.allclose(S[np.tril_indices(3, -1)], 1.0, atol=1e-14)


S4 = np.array([[1.0, 0.0, 0.0, 0.0],
               [0.9, 1.0, 0.0, 0.0],
               [0.5, 0.8, 1.0, 0.0],
               [0.2, 0.6, 0.7, 1.0]])


def test_objective_by_hand():
    """Sum over S layers of S[l, src(l)], worked by hand on a 4-layer matrix."""
    assert ps.sources("FSSFS") == [0, 0, 0, 3, 3]
    assert ps.pattern_objective(S4, "FSFS") == pytest.approx(0.9 + 0.7)
    assert ps.pattern_objective(S4, "FSSF") == pytest.approx(0.9 + 0.5)
    assert ps.pattern_objective(S4, "FFSS") == pytest.approx(0.8 + 0.6)
    assert ps.pattern_objective(S4, "FSSS") == pytest.approx(0.9 + 0.5 + 0.2)
    assert ps.pattern_objective(S4, "FFFF") == 0.0
    best, pats = ps.pattern_search_brute(S4, 2)
    assert best == pytest.approx(1.6) and pats == ["FSFS"]
    with pytest.raises(ValueError):
        ps.pattern_objective(S4, "SFSF")


@pytest.mark.parametrize("n", [2, 5, 8, 10])
def test_search_previous_layer_only(n):
    """S[i, j] = 1 when j = i - 1, else 0: an S layer scores only right after an F
    layer, so the optimum is min(M, N - M)."""
    S = np.eye(n) + np.eye(n, k=-1)
    for m in range(1, n + 1):
        best, pats = ps.pattern_search_brute(S, m)
        assert best == min(m, n - m)
        assert all(p.count("F") == m and p[0] == "F" for p in pats)


def test_search_row_constant():
    """S[i, j] = a_i for every j < i: the optimum makes F the M - 1 layers (after
    layer 0) with the smallest a, scoring sum(a[1:]) minus those."""
    rng = np.random.default_rng(5)
    n = 9
    a = rng.permutation(np.arange(1, n + 1, dtype=np.float64)) / 10
    S = np.tril(np.tile(a[:, None], (1, n)), -1) + np.eye(n)
    for m in range(1, n + 1):
        best, pats = ps.pattern_search_brute(S, m)
        small = np.sort(a[1:])[: m - 1]
        assert best == pytest.approx(a[1:].sum() - small.sum(), abs=1e-12)
        want = ["F"] + ["F" if a[l] in small else "S" for l in range(1, n)]
        assert pats == ["".join(want)]


@pytest.mark.parametrize("n,m", [(9, 3), (12, 4), (12, 3), (10, 5)])
def test_search_distance_penalty(n, m):
    """S[i, j] = -(i - j): a block of one F layer and b - 1 S layers costs
    b(b - 1)/2, so equal blocks of N/M layers are the unique optimum."""
    i, j = np.indices((n, n))
    S = np.where(i > j, -(i - j).astype(np.float64), np.eye(n))
    b = n // m
    best, pats = ps.pattern_search_brute(S, m)
    assert best == -m * b * (b - 1) / 2
    assert pats == [("F" + "S" * (b - 1)) * m]


def test_search_extremes():
    """M = N: every layer F, score 0.  M = 1: only layer 0 F, score sum_l S[l, 0]."""
    rng = np.random.default_rng(6)
    S = np.tril(rng.uniform(-1, 1, (7, 7)), -1) + np.eye(7)
    assert ps.pattern_search_brute(S, 7) == (0.0, ["F" * 7])
    best, pats = ps.pattern_search_brute(S, 1)
    assert pats == ["F" + "S" * 6] and best == pytest.approx(S[1:, 0].sum(), abs=1e-14)
    with pytest.raises(ValueError):
        ps.pattern_search_brute(S, 0)
