"""Pins of the distillation-loss oracle (training-aware IndexCache) against the
pages' worked examples, Proposition 1 and finite differences."""
import json
import os

import numpy as np

from oracle import distill as od

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    return json.load(open(os.path.join(GOLD, "distill_worked_example.json")))


def test_worked_example_delta_and_wq_gradient():
    """[DSA-NOTES] §7.2: pi = (0.7, 0.3), p = (0.2, 0.8) -> delta = (0.5, -0.5); with
    x = (1, 0), k_A = (1, 0), k_B = (0, 1): dL/dW_q = [[0.5, 0], [-0.5, 0]]."""
    g = _gold()
    z = np.log(np.array(g["pi"]))
    loss, pi, delta = od.kl_multi(z, np.array([g["p"]]))
    assert np.allclose(pi, g["pi"], atol=1e-15)
    assert np.allclose(delta, g["delta"], atol=1e-15)
    # the same through the indexer path: one head, w = 1, q chosen so that both dot
    # products are positive (ReLU open) and softmax(q.k_A, q.k_B) = (0.7, 0.3)
    kA, kB, x = np.array(g["k_A"]), np.array(g["k_B"]), np.array(g["x"])
    qv = np.array([1.0 + np.log(0.7 / 0.3), 1.0])
    out = od.indexer_distill(qv[None, None, :], np.stack([kA, kB]), np.ones((1, 1)), np.array([[0, 1]]),
                             np.array(g["p"])[None, None, :], q_pos0=1)
    assert np.allclose(out["delta"][0], g["delta"], atol=1e-12)
    dq = out["dq"][0, 0]
    assert np.allclose(np.outer(dq, x), g["dL_dWq"], atol=1e-12)
    # single-head key side, [DSA-NOTES] §7.1: dL/dk_s = delta_s q
    assert np.allclose(out["dk"], np.outer(g["delta"], qv), atol=1e-12)
    # KL(p || pi) by hand
    p, q_ = np.array(g["p"]), np.array(g["pi"])
    assert np.isclose(loss, float((p * np.log(p / q_)).sum()), rtol=1e-14)


def test_proposition_1_gradient_equals_average_target_gradient():
    """[IC-SUMMARY] §3.2 Proposition 1 / [DSA-NOTES] §5.2: the gradient of the
    multi-layer loss w.r.t. the scores equals that of KL(p_bar || pi); the loss
    values themselves differ.  Checked by central differences."""
    rng = np.random.default_rng(11)
    z = rng.normal(size=7)
    P = rng.random((3, 7)) ** 2
    P /= P.sum(axis=1, keepdims=True)
    loss, pi, delta = od.kl_multi(z, P)
    loss_avg, delta_avg = od.kl_average(z, P)
    h = 1e-6
    num_multi = np.array([(od.kl_multi(z + h * e, P)[0] - od.kl_multi(z - h * e, P)[0]) / (2 * h)
                          for e in np.eye(7)])
    num_avg = np.array([(od.kl_average(z + h * e, P)[0] - od.kl_average(z - h * e, P)[0]) / (2 * h)
                        for e in np.eye(7)])
    assert np.allclose(num_multi, delta, atol=1e-8)
    assert np.allclose(num_avg, delta, atol=1e-8)
    assert np.allclose(delta_avg, delta, atol=1e-15)
    assert np.allclose(delta, pi - P.mean(axis=0), atol=1e-15)     # the pages' pi - p_bar
    assert loss > loss_avg + 1e-3                                  # values differ (mean KL >= KL of mean)


def test_centroid_is_the_stationary_point_of_the_shared_loss():
    """[DSA-NOTES] §5.3: two layers (0.8, 0.2, 0) and (0.2, 0.1, 0.7) average to
    (0.5, 0.15, 0.35); an indexer that matches that average has zero gradient."""
    g = _gold()
    P = np.array([g["layer1"], g["layer2"]])
    assert np.allclose(P.mean(axis=0), g["average"], atol=1e-15)
    loss, pi, delta = od.kl_multi(np.log(np.array(g["average"])), P)
    assert np.allclose(delta, 0.0, atol=1e-15)
    pb = np.array(g["average"])
    expect = 0.5 * sum(float((p[p > 0] * np.log(p[p > 0] / pb[p > 0])).sum()) for p in P)
    assert np.isclose(loss, expect, rtol=1e-14) and loss > 0


def test_loss_nonnegative_and_zero_at_the_teacher():
    rng = np.random.default_rng(3)
    for _ in range(5):
        z = rng.normal(size=9)
        P = rng.random((4, 9))
        P /= P.sum(axis=1, keepdims=True)
        assert od.kl_multi(z, P)[0] >= 0
    z = rng.normal(size=9)
    pi = np.exp(z - z.max())
    pi /= pi.sum()
    loss, _, delta = od.kl_multi(z, np.stack([pi, pi]))
    assert abs(loss) < 1e-14 and np.allclose(delta, 0, atol=1e-15)


def _total_loss(q, k, w, idx, T, q_pos0):
    return od.indexer_distill(q, k, w, idx, T, q_pos0=q_pos0)["loss"].sum()


def test_backward_matches_finite_differences():
    """dq, dw and dk of indexer_distill against central differences of the summed
    row losses (random inputs: no dot product sits on a ReLU kink)."""
    rng = np.random.default_rng(5)
    n_q, H, d, n_k, topk, r = 3, 3, 4, 7, 5, 2
    q = rng.normal(size=(n_q, H, d))
    k = rng.normal(size=(n_k, d))
    w = rng.normal(size=(n_q, H))
    q_pos0 = 4
    idx = np.full((n_q, topk), -1)
    for i in range(n_q):
        t = q_pos0 + i
        sel = np.sort(rng.choice(t + 1, size=min(topk - 1, t + 1), replace=False))
        idx[i, :len(sel)] = sel
    T = rng.random((r, n_q, topk))
    T[:, idx < 0] = 0.0
    T /= T.sum(axis=2, keepdims=True)
    out = od.indexer_distill(q, k, w, idx, T, q_pos0=q_pos0)
    h = 1e-6
    for name, arr, grad in (("q", q, out["dq"]), ("w", w, out["dw"]), ("k", k, out["dk"])):
        num = np.zeros_like(arr)
        it = np.nditer(arr, flags=["multi_index"])
        for _ in it:
            m = it.multi_index
            a1, a2 = arr.copy(), arr.copy()
            a1[m] += h
            a2[m] -= h
            args1 = {"q": q, "k": k, "w": w}
            args2 = dict(args1)
            args1[name], args2[name] = a1, a2
            num[m] = (_total_loss(args1["q"], args1["k"], args1["w"], idx, T, q_pos0)
                      - _total_loss(args2["q"], args2["k"], args2["w"], idx, T, q_pos0)) / (2 * h)
        assert np.allclose(num, grad, atol=1e-7, rtol=1e-6), name


def test_padding_and_future_positions_take_no_part():
    """Entries that select nothing (-1 padding, positions after t) get delta = 0 and
    leave loss and gradients unchanged."""
    rng = np.random.default_rng(9)
    H, d, n_k = 2, 3, 10
    q = rng.normal(size=(1, H, d))
    k = rng.normal(size=(n_k, d))
    w = rng.random((1, H))
    T = np.array([[[0.2, 0.5, 0.3, 0.0, 0.0]]])
    base = od.indexer_distill(q, k, w, np.array([[1, 3, 6, -1, -1]]), T, q_pos0=6)
    # position 8 is after t = 6: it selects nothing
    more = od.indexer_distill(q, k, w, np.array([[1, 3, 6, 8, -1]]), T, q_pos0=6)
    for key in ("loss", "dq", "dw", "dk", "delta"):
        assert np.allclose(base[key], more[key], atol=1e-15), key
    assert base["delta"][0, 3] == 0 and base["delta"][0, 4] == 0
