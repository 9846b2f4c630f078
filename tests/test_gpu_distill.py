"""GPU parity of the distillation loss over the selected Top-k and its backward
(training-aware IndexCache) against the float64 oracle.

Tolerances (fp32 accumulation of bf16 products, float atomics for dk):
  * loss: |l_gpu - l_ref| <= 1e-4 * (1 + |l_ref|)
  * delta: |d_gpu - d_ref| <= 1e-4 * max |d_ref| of the row
  * dq, dw, dk: |g_gpu - g_ref| <= 1e-3 * (the same sum taken over absolute terms)
    + 1e-6 * max of that scale (a ReLU mask may flip where q.k rounds across 0)
"""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dsa():
    import dsa_lightning_indexer_amd as m
    return m


def make(dev, *, B, n_q, n_k, heads, topk, r, q_pos0, seed, w_dist="u8"):
    ix = syn.indexer_inputs(B=B, n_q=n_q, n_k=n_k, H=heads, d=128, q_pos0=q_pos0, dtype=syn.BF16,
                            values="normal", w_dist=w_dist, seed=seed, device=dev)
    idx = syn.random_sorted_indices(B=B, n_q=n_q, topk=topk, q_pos0=q_pos0, n_k=n_k, seed=seed + 1, device=dev)
    T = syn.teacher_weights(idx, r=r, seed=seed + 2, device=dev)
    return ix, idx, T


def check(got, ref, rows=None, b=0):
    sel = slice(None) if rows is None else rows
    loss = got["loss"][b].cpu().double().numpy()[sel]
    assert np.all(np.abs(loss - ref["loss"]) <= 1e-4 * (1 + np.abs(ref["loss"]))), "loss"
    dl = got["delta"][b].cpu().double().numpy()[sel]
    rmax = np.abs(ref["delta"]).max(axis=1, keepdims=True)
    assert np.all(np.abs(dl - ref["delta"]) <= 1e-4 * rmax + 1e-12), "delta"
    for name in ("dq", "dw"):
        g = got[name][b].cpu().double().numpy()[sel]
        sc = ref[name + "_scale"]
        err = np.abs(g - ref[name])
        assert np.all(err <= 1e-3 * sc + 1e-6 * sc.max()), (name, float((err / (sc + 1e-30)).max()))


@pytest.mark.parametrize("heads,topk,r,q_pos0", [(64, 64, 3, 20), (40, 100, 1, 150), (64, 2048, 4, 2000)])
def test_distill_matches_oracle(dsa, dev, heads, topk, r, q_pos0):
    """Every output against the oracle on whole small problems: rows with fewer
    candidates than topk (padding), topk not a multiple of 16, heads not a
    multiple of 16, one teacher, a full 2048-entry row."""
    B, n_q = 2, 24
    n_k = q_pos0 + n_q
    ix, idx, T = make(dev, B=B, n_q=n_q, n_k=n_k, heads=heads, topk=topk, r=r, q_pos0=q_pos0, seed=50 + heads)
    got = dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T, q_pos0=q_pos0)
    torch.cuda.synchronize()
    for b in range(B):
        q, k, w = H.indexer_f64(ix, b)
        ref = oracle.indexer_distill(q, k, w, idx[b].cpu().numpy(), T[:, b].cpu().double().numpy(), q_pos0=q_pos0)
        check(got, ref, b=b)
        g = got["dk"][b].cpu().double().numpy()
        sc = ref["dk_scale"]
        err = np.abs(g - ref["dk"])
        assert np.all(err <= 1e-3 * sc + 1e-6 * sc.max()), ("dk", float((err / (sc + 1e-30)).max()))


def test_distill_signed_weights_and_worked_example_shape(dsa, dev):
    """Signed head weights (negative w flips the ReLU's contribution) and a row
    whose index set holds the same key for several queries (dk accumulates)."""
    B, n_q, n_k, topk = 1, 32, 48, 32
    ix, idx, T = make(dev, B=B, n_q=n_q, n_k=n_k, heads=64, topk=topk, r=2, q_pos0=16, seed=71, w_dist="normal")
    got = dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T, q_pos0=16)
    torch.cuda.synchronize()
    q, k, w = H.indexer_f64(ix, 0)
    ref = oracle.indexer_distill(q, k, w, idx[0].cpu().numpy(), T[:, 0].cpu().double().numpy(), q_pos0=16)
    check(got, ref)
    g = got["dk"][0].cpu().double().numpy()
    sc = ref["dk_scale"]
    assert np.all(np.abs(g - ref["dk"]) <= 1e-3 * sc + 1e-6 * sc.max())


def test_distill_full_size_sampled_and_homogeneity(dsa, dev):
    """One F layer at the bf16 prefill shape (L = 16384, H = 64, d = 128, k = 2048) with
    four teachers: sampled rows against the oracle; dk through identities that
    hold at any size (z is degree-1 homogeneous in q, w and k):
        sum_j w_j dw_j = sum_j q_j . dq_j = sum_e delta_e z_e   per row,
        sum_s k_s . dk_s = sum over rows of the above."""
    L, topk, r = 16384, 2048, 4
    ix, idx, T = make(dev, B=1, n_q=L, n_k=L, heads=64, topk=topk, r=r, q_pos0=0, seed=81)
    got = dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T, q_pos0=0)
    torch.cuda.synchronize()
    rows = np.array([0, 1, 2047, 2048, 9000, L - 1])
    q, k, w = H.indexer_f64(ix, 0)
    ref = oracle.indexer_distill(q, k, w, idx[0].cpu().numpy(), T[:, 0].cpu().double().numpy(), rows=rows)
    check(got, ref, rows=rows)
    qf = ix.q[0].float()
    wf = ix.w[0].float()
    a = (wf * got["dw"][0]).double().sum(dim=1)                      # per row
    c = (qf * got["dq"][0]).double().sum(dim=(1, 2))
    sa = (wf.abs() * got["dw"][0].abs()).double().sum(dim=1)
    assert torch.all((a - c).abs() <= 1e-3 * sa + 1e-6), "w.dw vs q.dq"
    kdk = (ix.k[0].float().double() * got["dk"][0].double()).sum()
    assert abs(float(kdk - c.sum())) <= 1e-3 * float(sa.sum()), "k.dk vs sum of q.dq"


def test_distill_repeat_is_stable(dsa, dev):
    """Two calls: loss, delta, dq and dw bit-identical; dk equal up to the float
    atomics' summation order."""
    ix, idx, T = make(dev, B=1, n_q=64, n_k=600, heads=64, topk=512, r=2, q_pos0=536, seed=91)
    a = dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T, q_pos0=536)
    b = dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T, q_pos0=536)
    torch.cuda.synchronize()
    for name in ("loss", "delta", "dq", "dw"):
        assert torch.equal(a[name], b[name]), name
    assert torch.allclose(a["dk"], b["dk"], rtol=1e-5, atol=1e-6)
