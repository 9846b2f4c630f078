"""Pins for the CPU oracle (no GPU): worked examples printed on the pages,
closed forms, library routines and invariants.  Each pin is chosen so that a
plausible slip in the oracle (dropped ReLU, wrong sign or weight, transposed
operand, off-by-one causal bound, reversed tie-break, missing scale, wrong
kv-head map, wrong overlap denominator, off-by-one source layer) fails it."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def gold(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def rng(seed):
    return np.random.default_rng(seed)


# --- storage formats --------------------------------------------------------------

def test_e4m3fn_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = oracle.e4m3fn_codes_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert (np.isnan(mine) == nan).all()
    assert np.array_equal(mine[~nan], ref[~nan])
    assert set(np.flatnonzero(nan)) == {0x7F, 0xFF}
    assert np.nanmax(mine) == 448.0 and np.nanmin(np.abs(mine[mine != 0])) == 2.0 ** -9


def test_bf16_decode_matches_torch():
    bits = rng(0).integers(0, 65536, 4096).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # drop inf/nan patterns
    mine = oracle.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(mine, ref)


def test_dequantize_applies_vector_scale():
    codes = np.array([[0x38, 0x40], [0xB8, 0x00]], dtype=np.uint8)  # 1.0, 2.0 ; -1.0, 0
    x = oracle.dequantize(codes, "fp8", np.array([0.5, 3.0], dtype=np.float32))
    assert np.array_equal(x, [[0.5, 1.0], [-3.0, 0.0]])


# --- indexer scores ---------------------------------------------------------------

def _rand_indexer(seed, n=37, H=5, d=7, ints=False):
    r = rng(seed)
    if ints:
        q = r.integers(-3, 4, (n, H, d)).astype(np.float64)
        k = r.integers(-3, 4, (n, d)).astype(np.float64)
        w = 2.0 ** r.integers(-2, 2, (n, H))
    else:
        q = r.standard_normal((n, H, d))
        k = r.standard_normal((n, d))
        w = r.uniform(0, 1, (n, H))
    return q, k, w


def test_scores_single_head_nonnegative_is_matmul():
    r = rng(1)
    q = r.uniform(0, 1, (20, 1, 6))
    k = r.uniform(0, 1, (20, 6))
    I, _ = oracle.indexer_scores(q, k, np.ones((20, 1)))
    ref = torch.matmul(torch.from_numpy(q[:, 0]), torch.from_numpy(k).T).numpy()
    tri = np.tril(np.ones((20, 20), bool))
    assert np.allclose(I[tri], ref[tri], rtol=1e-14, atol=0)
    assert np.isneginf(I[~tri]).all()


def test_scores_relu_odd_part_is_linear():
    """ReLU(x) - ReLU(-x) = x, so I(q,k) - I(q,-k) = (sum_j w_j q_j) . k."""
    q, k, w = _rand_indexer(2)
    Ip, _ = oracle.indexer_scores(q, k, w)
    Im, _ = oracle.indexer_scores(q, -k, w)
    lin = torch.matmul(torch.from_numpy((w[:, :, None] * q).sum(1)), torch.from_numpy(k).T).numpy()
    tri = np.tril(np.ones(Ip.shape, bool))
    with np.errstate(invalid="ignore"):
        diff = Ip - Im
    assert np.allclose(diff[tri], lin[tri], rtol=1e-12, atol=1e-12)


def test_scores_relu_even_part_is_abs():
    """ReLU(x) + ReLU(-x) = |x|, so I(q,k) + I(q,-k) = sum_j w_j |q_j . k|."""
    q, k, w = _rand_indexer(3)
    Ip, Ap = oracle.indexer_scores(q, k, w)
    Im, _ = oracle.indexer_scores(q, -k, w)
    D = torch.einsum("thd,sd->ths", torch.from_numpy(q), torch.from_numpy(k)).abs()
    ev = (torch.from_numpy(w)[:, :, None] * D).sum(1).numpy()
    tri = np.tril(np.ones(Ip.shape, bool))
    assert np.allclose((Ip + Im)[tri], ev[tri], rtol=1e-12, atol=1e-12)
    assert np.allclose(Ap[tri], Ip[tri])               # w >= 0  =>  A == I


def test_scores_one_hot_weight_selects_one_head():
    q, k, _ = _rand_indexer(4)
    for j in range(q.shape[1]):
        w = np.zeros((q.shape[0], q.shape[1]))
        w[:, j] = 1.0
        I, _ = oracle.indexer_scores(q, k, w)
        ref = np.maximum(torch.matmul(torch.from_numpy(q[:, j]), torch.from_numpy(k).T).numpy(), 0)
        tri = np.tril(np.ones(I.shape, bool))
        assert np.allclose(I[tri], ref[tri], rtol=1e-14, atol=0)


def test_scores_causal_bound_is_inclusive_and_prefix_only():
    q, k, w = _rand_indexer(5, ints=True)
    I, _ = oracle.indexer_scores(q, k, w)
    n = q.shape[0]
    for t in range(n):
        assert np.isfinite(I[t, : t + 1]).all() and np.isneginf(I[t, t + 1:]).all()
    # a row only depends on keys 0..t: perturbing later keys changes nothing
    k2 = k.copy()
    k2[20:] += 5
    I2, _ = oracle.indexer_scores(q, k2, w)
    assert np.array_equal(I[:20], I2[:20])
    # row offsets: the decode form (one query at q_pos0) equals the prefill row
    Id, _ = oracle.indexer_scores(q[n - 1:], k, w[n - 1:], q_pos0=n - 1)
    assert np.array_equal(Id[0], I[n - 1])


def test_scores_scale_folding_invariant():
    q, k, w = _rand_indexer(6, ints=True)
    e = rng(6).integers(-3, 4, q.shape[1])
    I, _ = oracle.indexer_scores(q, k, w)
    I2, _ = oracle.indexer_scores(q * 2.0 ** e[None, :, None], k, w * 2.0 ** -e[None, :])
    assert np.array_equal(I, I2)


def test_scores_signed_weights_error_scale():
    q, k, w = _rand_indexer(7)
    w = w - 0.5
    I, A = oracle.indexer_scores(q, k, w)
    tri = np.tril(np.ones(I.shape, bool))
    assert (A[tri] >= np.abs(I[tri]) - 1e-12).all()


def test_scores_integer_exact_small_config():
    """Integer-valued inputs give exactly representable scores: the oracle's
    float64 result equals an int64 evaluation of the same definition."""
    q, k, w = _rand_indexer(8, ints=True)
    I, _ = oracle.indexer_scores(q, k, w)
    D = torch.einsum("thd,sd->ths", torch.from_numpy(q).long(), torch.from_numpy(k).long())
    w4 = torch.from_numpy(w * 4).long()                    # w in {1/4..2} -> integer quarters
    ref = (w4[:, :, None] * D.clamp(min=0)).sum(1).double().numpy() / 4
    tri = np.tril(np.ones(I.shape, bool))
    assert np.array_equal(I[tri], ref[tri])


# --- Top-k --------------------------------------------------------------------------

def test_topk_worked_example_shared_budget():
    g = gold("topk_shared_budget_example.json")
    names = g["candidates"]
    avg = np.array(g["average"])
    assert np.allclose((np.array(g["layer1"]) + np.array(g["layer2"])) / 2, avg)
    for kk, key in ((1, "top1"), (2, "top2")):
        sel = oracle.topk_row(avg, kk)
        assert [names[s] for s in sel if s >= 0] == sorted(g[key], key=names.index)


def test_topk_matches_torch_topk_on_distinct_scores():
    for seed in range(5):
        s = rng(seed).permutation(500).astype(np.float64) * 0.37 - 40
        for kk in (1, 7, 64, 499, 500):
            mine = oracle.topk_row(s, kk)
            ref = torch.topk(torch.from_numpy(s), kk).indices.sort().values.numpy()
            assert np.array_equal(mine, ref)


def test_topk_ties_go_to_lower_position():
    assert np.array_equal(oracle.topk_row(np.zeros(10), 4), [0, 1, 2, 3])
    s = np.array([1.0, 3.0, 1.0, 3.0, 2.0, 1.0])
    assert np.array_equal(oracle.topk_row(s, 4), [0, 1, 3, 4])
    assert np.array_equal(oracle.topk_row(np.array([-0.0, 0.0, -1.0]), 1), [0])
    assert np.array_equal(oracle.topk_row(np.array([0.0, -0.0, -1.0]), 1), [0])


def test_topk_total_order_invariant_integer_ties():
    for seed in range(20):
        r = rng(100 + seed)
        s = r.integers(-4, 5, r.integers(1, 200)).astype(np.float64)
        kk = int(r.integers(1, 80))
        sel = oracle.topk_row(s, kk)
        chosen = sel[sel >= 0]
        assert len(chosen) == min(kk, len(s))
        rest = np.setdiff1d(np.arange(len(s)), chosen)
        if len(rest) and len(chosen):
            worst_in = min(chosen, key=lambda p: (s[p], -p))
            best_out = max(rest, key=lambda p: (s[p], -p))
            assert (s[worst_in], -worst_in) > (s[best_out], -best_out)


def test_topk_short_row_selects_all_and_pads():
    assert np.array_equal(oracle.topk_row(np.array([5.0, 1.0, 3.0]), 5), [0, 1, 2, -1, -1])
    assert np.array_equal(oracle.topk_row(np.array([]), 3), [-1, -1, -1])


def test_indexer_topk_rows_below_k_take_all_predecessors():
    q, k, w = _rand_indexer(9, n=40, ints=True)
    idx, _, _ = oracle.indexer_topk(q, k, w, topk=16)
    for t in range(40):
        n = min(16, t + 1)
        assert (idx[t, n:] == -1).all()
        if t < 16:
            assert np.array_equal(idx[t, :t + 1], np.arange(t + 1))
        assert idx[t, :n].max() <= t


# --- sparse attention ---------------------------------------------------------------

def test_sparse_attn_full_selection_is_causal_sdpa():
    r = rng(10)
    n, H, d = 24, 3, 8
    Q = r.standard_normal((n, H, d))
    K = r.standard_normal((n, H, d))
    V = r.standard_normal((n, H, d))
    idx = np.array([[s if s <= t else -1 for s in range(n)] for t in range(n)])
    mine = oracle.sparse_attn(Q, K, V, idx, 1 / np.sqrt(d))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).transpose(0, 1), torch.from_numpy(K).transpose(0, 1),
        torch.from_numpy(V).transpose(0, 1), is_causal=True).transpose(0, 1).numpy()
    assert np.allclose(mine, ref, rtol=1e-12, atol=1e-12)


def test_sparse_attn_scale_and_subset_match_sdpa_with_mask():
    r = rng(11)
    n, H, d = 30, 2, 5
    Q, K, V = (r.standard_normal((n, H, d)) for _ in range(3))
    idx = syn.random_sorted_indices(n_q=n, topk=6, seed=3)[0].numpy()
    mask = np.zeros((n, n), bool)
    for t in range(n):
        mask[t, idx[t][idx[t] >= 0]] = True
    mine = oracle.sparse_attn(Q, K, V, idx, 0.3)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).transpose(0, 1), torch.from_numpy(K).transpose(0, 1),
        torch.from_numpy(V).transpose(0, 1), attn_mask=torch.from_numpy(mask),
        scale=0.3).transpose(0, 1).numpy()
    assert np.allclose(mine, ref, rtol=1e-12, atol=1e-12)


def test_sparse_attn_single_position_returns_value_row():
    r = rng(12)
    Q, K = r.standard_normal((4, 2, 3)), r.standard_normal((9, 1, 3))
    V = r.standard_normal((9, 1, 5))
    idx = np.array([[7, -1], [0, -1], [3, -1], [-1, -1]])
    out = oracle.sparse_attn(Q, K, V, idx, 1.0)
    assert np.allclose(out[0], V[7, 0]) and np.allclose(out[1], V[0, 0])
    assert np.allclose(out[2], V[3, 0]) and (out[3] == 0).all()


def test_sparse_attn_mqa_equals_repeated_kv_heads():
    r = rng(13)
    Q = r.standard_normal((6, 4, 8))
    K = r.standard_normal((6, 1, 8))
    V = r.standard_normal((6, 1, 3))
    idx = syn.random_sorted_indices(n_q=6, topk=3, seed=1)[0].numpy()
    a = oracle.sparse_attn(Q, K, V, idx, 0.5)
    b = oracle.sparse_attn(Q, np.repeat(K, 4, 1), np.repeat(V, 4, 1), idx, 0.5)
    assert np.allclose(a, b, rtol=1e-14)
    # grouped heads: query heads 0,1 -> kv head 0; 2,3 -> kv head 1
    K2 = r.standard_normal((6, 2, 8))
    V2 = r.standard_normal((6, 2, 3))
    g = oracle.sparse_attn(Q, K2, V2, idx, 0.5)
    h0 = oracle.sparse_attn(Q[:, :2], K2[:, :1], V2[:, :1], idx, 0.5)
    h1 = oracle.sparse_attn(Q[:, 2:], K2[:, 1:], V2[:, 1:], idx, 0.5)
    assert np.allclose(g, np.concatenate([h0, h1], 1), rtol=1e-14)


def test_sparse_attn_order_of_indices_irrelevant():
    r = rng(14)
    Q, K, V = r.standard_normal((5, 2, 4)), r.standard_normal((20, 1, 4)), r.standard_normal((20, 1, 6))
    idx = np.array([[3, 9, 1, 15]] * 5)
    a = oracle.sparse_attn(Q, K, V, idx, 0.7)
    b = oracle.sparse_attn(Q, K, V, idx[:, ::-1].copy(), 0.7)
    assert np.allclose(a, b, rtol=1e-14)


# --- IndexCache layer loop ------------------------------------------------------------

def test_fsss_trace_from_the_page():
    g = gold("fsss_trace.json")
    src = oracle.source_layers(g["pattern"])
    assert src == g["source_layer_1based"]
    seen = []

    def indexer_fn(l):
        seen.append(l)
        return np.full((2, 3), l)

    src2, Ts, outs, calls = oracle.indexcache_forward(g["pattern"], indexer_fn, lambda l, T: (l, int(T[0, 0])))
    assert calls == g["indexer_layers_1based"] == seen
    for l, T in enumerate(Ts, start=1):
        assert int(T[0, 0]) == src[l - 1]
        assert T is Ts[src[l - 1] - 1]                  # S layers reuse the F layer's tensor
    assert [o[0] for o in outs] == list(range(1, 9))  # every layer runs its own attention


def test_pattern_rules():
    with pytest.raises(ValueError):
        oracle.source_layers("SFFF")
    with pytest.raises(ValueError):
        oracle.source_layers("FXF")
    assert oracle.source_layers("F") == [1]
    assert oracle.source_layers("FFSF") == [1, 2, 2, 4]
    assert oracle.source_layers(syn.DECODE_PATTERN).count(None) == 0
    assert syn.DECODE_PATTERN.count("F") == 12 and len(syn.DECODE_PATTERN) == 47
    assert [i + 1 for i, c in enumerate(syn.DECODE_PATTERN) if c == "F"] == list(range(1, 46, 4))


def test_searched_patterns_from_the_page():
    """[IC-SUMMARY] Appendix B: the searched 47-layer patterns keep 24, 12 and 7 F
    layers; the driver inputs are the printed strings, 47 characters each, and
    every one starts with an F layer.  The 1/8 pattern has its F layers at
    1, 5, 14, 18, 24, 29 and 38 (1-based), as printed."""
    g = gold("searched_patterns.json")
    assert [i + 1 for i, c in enumerate(g["patterns_as_printed"]["1/8"]) if c == "F"] == \
        g["f_positions_1based"]["1/8"] == [1, 5, 14, 18, 24, 29, 38]
    for r, text in g["patterns_as_printed"].items():
        used = syn.SEARCHED_PATTERNS_47[r]
        assert len(text) == len(used) == g["n_layers"] == 47
        assert used == text
        assert used.count("F") == g["f_counts"][r]
        src = oracle.source_layers(used)
        assert src[0] == 1 and None not in src
        # an S layer's source is the nearest F layer before it
        for l, c in enumerate(used, start=1):
            if c == "F":
                assert src[l - 1] == l
            else:
                assert used[src[l - 1] - 1] == "F" and "F" not in used[src[l - 1]:l - 1]


# --- overlap and report arithmetic ---------------------------------------------------------

def test_overlap_worked_example():
    g = gold("overlap_example.json")
    names = sorted(set(g["original"]) | set(g["reused"]))
    a = np.array([[names.index(x) for x in g["original"]]])
    b = np.array([[names.index(x) for x in g["reused"]]])
    assert oracle.overlap(a, b, g["k"]) == pytest.approx(g["overlap"])


def test_overlap_invariants():
    T = syn.random_sorted_indices(n_q=50, topk=8, seed=5)[0].numpy()
    assert oracle.overlap(T[10:], T[10:], 8) == 1.0
    U = syn.random_sorted_indices(n_q=50, topk=8, seed=6)[0].numpy()
    assert oracle.overlap(T, U, 8) == pytest.approx(oracle.overlap(U, T, 8))
    assert oracle.overlap(np.array([[0, 1, -1]]), np.array([[2, 3, -1]]), 3) == 0.0
    assert oracle.overlap(np.array([[0, 1, -1]]), np.array([[1, 0, -1]]), 3) == pytest.approx(2 / 3)
    M = oracle.overlap_matrix([T, T, U], 8, rows=np.arange(7, 50))
    assert M[0, 1] == 1.0 and M[0, 2] == M[2, 0] and M[2, 2] == 1.0


def test_amdahl_example():
    g = gold("amdahl_example.json")
    total = g["indexer_ms"] + g["other_ms"]
    f = g["indexer_ms"] / total
    s = oracle.amdahl_speedup(f, g["retained"])
    assert total / s == pytest.approx(g["after_ms"])
    assert round(s, 2) == g["speedup_printed"]


def test_mli_shift_from_the_page():
    """[MLI] 核心思路: with an indexer on every layer, layer L attends with layer
    L-1's indices (layer 1 with its own); combined with IndexCache's FSSS FSSS
    pattern, the second F layer attends with the first F layer's tensor and the
    S layers after it with the second's."""
    g = gold("mli_shift.json")
    assert oracle.mli_source_layers(g["all_F_pattern"]) == g["all_F_source_layer_1based"]
    assert oracle.mli_source_layers(g["fsss_pattern"]) == g["fsss_source_layer_1based"]


@pytest.mark.parametrize("pattern", ["F", "FF", "FSSSFSSS", "FFSFSSF", syn.DECODE_PATTERN,
                                     syn.SEARCHED_PATTERNS_47["1/8"]])
def test_mli_sources_against_indexcache(pattern):
    """Invariants tying the shift to IndexCache's sources: an S layer keeps the
    source IndexCache gives it; an F layer l > 1 takes the source IndexCache gives
    layer l - 1; every source except layer 1's lies strictly before its layer."""
    ic = oracle.source_layers(pattern)
    mli = oracle.mli_source_layers(pattern)
    assert mli[0] == 1
    for l in range(2, len(pattern) + 1):
        c = pattern[l - 1]
        assert mli[l - 1] < l
        assert pattern[mli[l - 1] - 1] == "F"
        assert mli[l - 1] == (ic[l - 1] if c == "S" else ic[l - 2])


def test_mli_forward_uses_the_shifted_tensor():
    """The loop calls the indexer on F layers only, and layer l's attention sees
    the tensor of its shifted source, never one computed after it."""
    pattern = "FSFFSSFS"
    made = {}

    def indexer(l):
        made[l] = ("T", l)
        return made[l]

    seen = []

    def attn(l, T):
        assert T[1] in made                      # produced already
        seen.append(T[1])
        return ("O", l, T[1])

    src, Ts, outs, calls = oracle.mli_forward(pattern, indexer, attn)
    assert calls == [l for l, c in enumerate(pattern, start=1) if c == "F"]
    assert seen == src == oracle.mli_source_layers(pattern)
    assert [t[1] for t in Ts] == src
    assert outs == [("O", l, s) for l, s in enumerate(src, start=1)]
    with pytest.raises(ValueError):
        oracle.mli_source_layers("SF")
