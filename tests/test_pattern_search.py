"""The library's sharing-pattern search (host dynamic program behind
dsa_pattern_search, [IC-SUMMARY] Appendix C) against the oracle's brute-force
optimum on every size it can enumerate, and through properties of an optimum at
the sizes of the pages' models (47 and 78 layers).  Host code: no GPU needed."""
import json
import os

import numpy as np
import pytest

from oracle import pattern_search as ps

dsa = pytest.importorskip("dsa_lightning_indexer_amd")

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def lower(rng, n, kind):
    if kind == "uniform":
        A = rng.uniform(-1.0, 1.0, (n, n))
    elif kind == "int":          # many exact ties
        A = rng.integers(0, 3, (n, n)).astype(np.float64)
    elif kind == "decay":        # similarity falling with depth distance, with jumps
        i, j = np.indices((n, n))
        A = np.exp(-0.15 * (i - j)) + 0.05 * rng.standard_normal((n, n))
    else:
        raise ValueError(kind)
    return np.tril(A, -1) + np.eye(n)


@pytest.mark.parametrize("kind", ["uniform", "int", "decay"])
@pytest.mark.parametrize("n", [1, 2, 3, 5, 8, 11, 13])
def test_dp_matches_brute_force(n, kind):
    rng = np.random.default_rng(100 * n + len(kind))
    S = lower(rng, n, kind)
    for m in range(1, n + 1):
        best, optimal = ps.pattern_search_brute(S, m)
        pat, score = dsa.pattern_search(S, m)
        assert len(pat) == n and pat[0] == "F" and pat.count("F") == m
        assert abs(score - best) <= 1e-12 * n * (1 + abs(best)), (m, score, best)
        assert abs(ps.pattern_objective(S, pat) - score) <= 1e-12 * n * (1 + abs(best))
        assert pat in optimal, (m, pat, optimal[:3])


def _neighbours(pat):
    """Patterns one move away: one F layer other than layer 0 moved to an S slot."""
    f = [i for i, c in enumerate(pat) if c == "F" and i > 0]
    s = [i for i, c in enumerate(pat) if c == "S"]
    for a in f:
        for b in s:
            c = list(pat)
            c[a], c[b] = "S", "F"
            yield "".join(c)


@pytest.mark.parametrize("n,counts", [(47, (24, 12, 7)), (78, (40, 22))])
@pytest.mark.parametrize("kind", ["uniform", "decay"])
def test_dp_optimal_at_model_sizes(n, counts, kind):
    """Where enumeration is out of reach: the pattern's reported score is its
    objective, and no uniform pattern, printed searched pattern, random pattern
    or single-move neighbour does better."""
    rng = np.random.default_rng(n + len(kind))
    S = lower(rng, n, kind)
    printed = json.load(open(os.path.join(GOLD, "searched_patterns.json")))["patterns_as_printed"]
    for m in counts:
        pat, score = dsa.pattern_search(S, m)
        assert pat[0] == "F" and pat.count("F") == m
        assert abs(ps.pattern_objective(S, pat) - score) <= 1e-9
        rivals = []
        for r in (2, 4, 8):
            u = "".join("F" if i % r == 0 else "S" for i in range(n))
            if u.count("F") == m:
                rivals.append(u)
        if n == 47:
            rivals += [p[:47] for p in printed.values() if p[:47].count("F") == m]
        for _ in range(500):
            c = ["S"] * n
            c[0] = "F"
            for l in rng.choice(np.arange(1, n), m - 1, replace=False):
                c[l] = "F"
            rivals.append("".join(c))
        rivals += list(_neighbours(pat))
        worst_gap = max(ps.pattern_objective(S, p) - score for p in rivals)
        assert worst_gap <= 1e-9, worst_gap


def test_rejects_bad_arguments():
    S = np.eye(4)
    for m in (0, 5, -1):
        with pytest.raises(dsa.DsaError):
            dsa.pattern_search(S, m)
    bad = S.copy()
    bad[2, 1] = np.nan
    with pytest.raises(dsa.DsaError, match="finite"):
        dsa.pattern_search(bad, 2)
    with pytest.raises(dsa.DsaError):
        dsa.pattern_search(np.eye(1025), 3)
    # entries on and above the diagonal are never read
    up = np.tril(np.random.default_rng(1).uniform(size=(6, 6)), -1)
    junk = up + np.triu(np.full((6, 6), np.inf))
    assert dsa.pattern_search(junk, 3) == dsa.pattern_search(up, 3)
