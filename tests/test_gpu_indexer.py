"""GPU parity of the indexer and Top-k against the CPU oracle.

Integer-valued inputs: indices bit-exact, scores exactly equal.  Float inputs:
scores within 1e-3 * A and the index-set tie-window rule (see helpers)."""
import dataclasses

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


def sample_rows(n_q, k, seed, n_random=24):
    """rows near 0, around k-1, a random sample and the last rows."""
    r = np.random.default_rng(seed)
    rows = set(range(min(8, n_q)))
    rows |= {x for x in range(k - 3, k + 3) if 0 <= x < n_q}
    rows |= set(r.integers(0, n_q, n_random).tolist())
    rows |= set(range(max(0, n_q - 4), n_q))
    return np.array(sorted(rows))


def oracle_rows(ixi, b, rows, topk):
    q, k, w = H.indexer_f64(ixi, b)
    idx, I, A = oracle.indexer_topk(q, k, w, topk, q_pos0=ixi.q_pos0, rows=rows)
    return idx, I, A


def run_topk(dsa, ixi, topk):
    out = dsa.topk(ixi.q, ixi.k, ixi.w, topk, q_scale=ixi.q_scale, k_scale=ixi.k_scale, q_pos0=ixi.q_pos0)
    torch.cuda.synchronize()
    return out


def check_exact(dsa, ixi, topk, rows=None, seed=0):
    B, n_q = ixi.q.shape[:2]
    got = run_topk(dsa, ixi, topk).cpu().numpy()
    for b in range(B):
        rr = np.arange(n_q) if rows is None else rows
        ref, _, _ = oracle_rows(ixi, b, rr, topk)
        mism = np.flatnonzero((got[b, rr] != ref).any(axis=1))
        assert mism.size == 0, f"batch {b}: {mism.size} rows differ, first row {rr[mism[0]]}"
    return got


def check_float(dsa, ixi, topk, rows):
    B = ixi.q.shape[0]
    got = run_topk(dsa, ixi, topk).cpu().numpy()
    for b in range(B):
        ref, I, _ = oracle_rows(ixi, b, rows, topk)
        for j, i in enumerate(rows):
            t = ixi.q_pos0 + i
            H.check_ascending_padded(got[b, i], min(t, ixi.k.shape[1] - 1), topk)
            n = min(t + 1, ixi.k.shape[1])
            msg = H.check_index_set(got[b, i], ref[j], I[j, :n], topk)
            assert msg is None, f"batch {b} row {i}: {msg}"
    return got


# --------------------------------------------------------------------------- tiny fp32 layer (L=512)
def test_tiny_fp32_exact(dsa, dev):
    c = syn.WORKLOADS["tiny_fp32_L512"]
    ixi = syn.indexer_inputs(n_q=c["L"], H=c["H"], d=c["d"], dtype=syn.F32, values="int",
                             w_dist="pow2", seed=c["seed"], device=dev)
    check_exact(dsa, ixi, c["topk"])
    # materialised scores equal the oracle's exactly
    sc = dsa.indexer_scores(ixi.q, ixi.k, ixi.w).cpu().numpy()[0]
    q, k, w = H.indexer_f64(ixi)
    I, _ = oracle.indexer_scores(q, k, w)
    assert np.array_equal(sc.astype(np.float64), I)


# --------------------------------------------------------------------------- fused prefill
@pytest.mark.parametrize("dtype", [syn.BF16, syn.FP8])
@pytest.mark.parametrize("L,topk", [(700, 64), (3500, 128), (5000, 2048)])
def test_fused_prefill_integer_exact(dsa, dev, dtype, L, topk):
    """Integer-valued q, k and power-of-two w: every score is exact in fp32, so
    the selection (with many ties) must equal the oracle's bit for bit.  L spans
    many 64-key tiles with a ragged tail; L=3500 and 5000 exercise the
    candidate-buffer compaction."""
    ixi = syn.indexer_inputs(B=2, n_q=L, dtype=dtype, values="int", w_dist="pow2", seed=L + topk, device=dev)
    rows = sample_rows(L, topk, seed=L)
    check_exact(dsa, ixi, topk, rows=rows)


@pytest.mark.parametrize("dtype", [syn.BF16, syn.FP8])
def test_fused_prefill_float(dsa, dev, dtype):
    L, topk = 4100, 2048
    ixi = syn.indexer_inputs(B=1, n_q=L, dtype=dtype, values="normal", w_dist="u8", seed=7, device=dev)
    check_float(dsa, ixi, topk, sample_rows(L, topk, seed=3))


def test_fused_prefill_small_heads_and_dims(dsa, dev):
    for H_, d, dt in ((16, 64, syn.BF16), (40, 32, syn.BF16), (64, 64, syn.FP8), (1, 128, syn.FP8)):
        ixi = syn.indexer_inputs(B=1, n_q=333, H=H_, d=d, dtype=dt, values="int", w_dist="pow2", seed=H_ + d,
                                 device=dev)
        check_exact(dsa, ixi, 50)


@pytest.mark.parametrize("heads", [33, 40, 50, 64])
def test_fused_prefill_two_row_kernel_edges(dsa, dev, heads):
    """bf16 d=128 with more than 32 heads runs two query rows per wave, eight rows
    per workgroup: head counts that leave partial 16-head tiles, and row counts
    (n_q = 333, 8 * 41 + 5) whose last workgroup has a wave with only its first
    row valid."""
    ixi = syn.indexer_inputs(B=2, n_q=333, H=heads, d=128, dtype=syn.BF16, values="int", w_dist="pm_pow2",
                             seed=heads, device=dev)
    check_exact(dsa, ixi, 100)


def test_fused_prefill_signed_weights_and_offset(dsa, dev):
    """Signed w (negative heads) and a query window that starts at q_pos0 > 0
    (chunked prefill: the keys before the window are already cached)."""
    ixi = syn.indexer_inputs(B=2, n_q=300, n_k=1200, q_pos0=900, dtype=syn.BF16, values="int",
                             w_dist="pm_pow2", seed=11, device=dev)
    check_exact(dsa, ixi, 256)


@pytest.mark.parametrize("H_,d,dt", [(64, 128, syn.BF16), (64, 128, syn.FP8), (16, 64, syn.BF16)])
def test_fused_prefill_rows_shorter_than_k(dsa, dev, H_, d, dt):
    """Row blocks whose every row has at most k candidates write 0..t without
    scoring; the block that straddles t = k - 1 scores for its longer rows only.
    Then a key cache shorter than k, with query rows past its end (each of those
    selects all n_k keys).  Two-row kernel (64 heads, d = 128) and one-row kernel."""
    ixi = syn.indexer_inputs(B=2, n_q=700, H=H_, d=d, dtype=dt, values="int", w_dist="pow2", seed=H_ + d + 5,
                             device=dev)
    check_exact(dsa, ixi, 517)
    ixi = syn.indexer_inputs(B=2, n_q=90, n_k=70, H=H_, d=d, dtype=dt, values="int", w_dist="pow2",
                             seed=H_ + d + 6, device=dev)
    check_exact(dsa, ixi, 128)


@pytest.mark.parametrize("k", [1, 2, 7])
def test_small_k_with_ties(dsa, dev, k):
    """k far below the tile width on integer-valued inputs (many tied scores, so
    the lower-position tie-break decides): two-row kernel (bf16 and fp8, through
    the candidate compaction at L = 9000), one-row kernel, and the few-row decode
    select over a 5000-key cache."""
    ixi = syn.indexer_inputs(B=1, n_q=9000, dtype=syn.BF16, values="int", w_dist="pow2", seed=40 + k, device=dev)
    check_exact(dsa, ixi, k, rows=sample_rows(9000, k, seed=k))
    ixi = syn.indexer_inputs(B=2, n_q=333, dtype=syn.FP8, values="int", w_dist="pm_pow2", seed=50 + k, device=dev)
    check_exact(dsa, ixi, k)
    ixi = syn.indexer_inputs(B=2, n_q=333, H=16, d=64, dtype=syn.BF16, values="int", w_dist="pow2", seed=60 + k,
                             device=dev)
    check_exact(dsa, ixi, k)
    ixi = syn.indexer_inputs(B=3, n_q=1, n_k=5000, q_pos0=4999, dtype=syn.FP8, values="int", w_dist="pow2",
                             seed=70 + k, device=dev)
    check_exact(dsa, ixi, k)


def _periodic_keys(ixi, period):
    """The same inputs with key s replaced by key s mod period (and its scale):
    every score recurs down the row, so the Top-k is decided by position."""
    n_k = ixi.k.shape[1]
    src = torch.arange(n_k, device=ixi.k.device) % period
    ks = None if ixi.k_scale is None else ixi.k_scale[:, src].contiguous()
    return dataclasses.replace(ixi, k=ixi.k[:, src].contiguous(), k_scale=ks)


@pytest.mark.parametrize("dtype", [syn.BF16, syn.FP8])
@pytest.mark.parametrize("k", [1, 2, 7, 100])
def test_repeated_keys_tie_break(dsa, dev, dtype, k):
    """Keys repeating with period 37: each row's best scores occur at several
    positions and only the lowest ones may be selected.  Rows long enough to pass
    the candidate compaction (L = 9000) and a decode row over 5000 keys."""
    ixi = _periodic_keys(syn.indexer_inputs(B=1, n_q=9000, dtype=dtype, values="int", w_dist="pm_pow2",
                                            seed=80 + k, device=dev), 37)
    got = check_exact(dsa, ixi, k, rows=sample_rows(9000, k, seed=k))
    # the best key pattern occurs at least k times below position 37 k, and ties go
    # to the lower position: a long row selects nothing at or above 37 k
    assert got[0, 8999, :k].max() < 37 * k
    ixi = _periodic_keys(syn.indexer_inputs(B=2, n_q=1, n_k=5000, q_pos0=4999, dtype=dtype, values="int",
                                            w_dist="pm_pow2", seed=90 + k, device=dev), 37)
    check_exact(dsa, ixi, k)


# --------------------------------------------------------------------------- materialised paths
@pytest.mark.parametrize("dtype", [syn.BF16, syn.FP8])
def test_indexer_scores_window(dsa, dev, dtype):
    ixi = syn.indexer_inputs(B=2, n_q=600, dtype=dtype, values="normal", w_dist="normal", seed=5, device=dev)
    row0, rows = 123, 77
    sc = dsa.indexer_scores(ixi.q, ixi.k, ixi.w, q_scale=ixi.q_scale, k_scale=ixi.k_scale,
                            row0=row0, rows=rows).cpu().numpy()
    for b in range(2):
        q, k, w = H.indexer_f64(ixi, b)
        I, A = oracle.indexer_scores(q, k, w, rows=np.arange(row0, row0 + rows))
        fin = np.isfinite(I)
        assert np.array_equal(np.isfinite(sc[b]), fin)
        err = np.abs(sc[b][fin] - I[fin])
        assert (err <= H.SCORE_RTOL * A[fin] + 1e-30).all(), float((err / np.maximum(A[fin], 1e-30)).max())


def test_indexer_scores_integer_exact(dsa, dev):
    ixi = syn.indexer_inputs(B=1, n_q=500, dtype=syn.FP8, values="int", w_dist="pm_pow2", seed=6, device=dev)
    sc = dsa.indexer_scores(ixi.q, ixi.k, ixi.w, q_scale=ixi.q_scale, k_scale=ixi.k_scale).cpu().numpy()[0]
    q, k, w = H.indexer_f64(ixi)
    I, _ = oracle.indexer_scores(q, k, w)
    assert np.array_equal(sc.astype(np.float64), I)


def test_select_from_given_scores_with_ties(dsa, dev):
    """dsa_topk over caller scores: heavy ties (small integers), +-0.0 and long
    rows; both sides decide on the same fp32 values, so the result is exact."""
    g = torch.Generator(device=dev).manual_seed(9)
    B, n_q, n_k, topk = 2, 40, 9000, 700
    sc = torch.randint(-3, 4, (B, n_q, n_k), generator=g, device=dev).float()
    sc[0, 5] = 0.0
    sc[0, 6] = -0.0
    sc[1, 7] = torch.where(torch.arange(n_k, device=dev) % 2 == 0, torch.tensor(-0.0, device=dev),
                           torch.tensor(0.0, device=dev))
    sc[1, 8] = torch.randn(n_k, generator=g, device=dev)
    q_pos0 = n_k - n_q - 5
    dummy_q = torch.zeros((B, n_q, 1, 32), dtype=torch.bfloat16, device=dev)
    dummy_k = torch.zeros((B, n_k, 32), dtype=torch.bfloat16, device=dev)
    dummy_w = torch.zeros((B, n_q, 1), device=dev)
    got = dsa.topk(dummy_q, dummy_k, dummy_w, topk, q_pos0=q_pos0, scores=sc).cpu().numpy()
    s64 = sc.cpu().double().numpy()
    for b in range(B):
        for i in range(n_q):
            n = min(q_pos0 + i + 1, n_k)
            ref = oracle.topk_row(s64[b, i, :n], topk)
            assert np.array_equal(got[b, i], ref), (b, i)


def test_select_few_rows_histogram_paths(dsa, dev):
    """Few long rows go through the key-histogram select (the bin of the k-th
    key, its candidates, an exact select over them).  Rows: 0 ordinary float
    scores; 1 a crowded k-th bin (6000 scores in [3, 3.01): one 12-bit key bin
    that still fits the candidate buffer); 2 all scores equal (more candidates
    than the buffer holds: whole-row select, ties by position); 3 integer scores
    0..49 (thousands of ties at the k-th key spread over every chunk); 4
    increasing scores (every candidate in the last chunk); 5 negative scores only.
    Exact against the oracle."""
    g = torch.Generator(device=dev).manual_seed(13)
    n_k, topk, R = 204800, 2048, 6
    sc = torch.randn((R, 1, n_k), generator=g, device=dev)
    crowd = torch.randperm(n_k, generator=g, device=dev)[:6000]
    sc[1, 0, crowd] = 3.0 + 0.01 * torch.rand(6000, generator=g, device=dev)
    sc[2, 0] = 0.5
    sc[3, 0] = torch.randint(0, 50, (n_k,), generator=g, device=dev).float()
    sc[4, 0] = torch.arange(n_k, device=dev).float() / n_k
    sc[5, 0] = -1.0 - torch.rand(n_k, generator=g, device=dev)
    dummy_q = torch.zeros((R, 1, 1, 32), dtype=torch.bfloat16, device=dev)
    dummy_k = torch.zeros((R, n_k, 32), dtype=torch.bfloat16, device=dev)
    dummy_w = torch.zeros((R, 1, 1), device=dev)
    got = dsa.topk(dummy_q, dummy_k, dummy_w, topk, q_pos0=n_k - 1, scores=sc).cpu().numpy()
    s64 = sc.cpu().double().numpy()
    for b in range(R):
        assert np.array_equal(got[b, 0], oracle.topk_row(s64[b, 0], topk)), b
    # a second call gives the same rows
    again = dsa.topk(dummy_q, dummy_k, dummy_w, topk, q_pos0=n_k - 1, scores=sc).cpu().numpy()
    assert np.array_equal(again, got)


# --------------------------------------------------------------------------- decode scan
@pytest.mark.parametrize("dtype", [syn.FP8, syn.BF16])
def test_decode_scan_integer_exact_and_matches_prefill_row(dsa, dev, dtype):
    S, topk = 6000, 2048
    pre = syn.indexer_inputs(B=3, n_q=S, dtype=dtype, values="int", w_dist="pm_pow2", seed=21, device=dev)
    dec = syn.IndexerInputs(dtype=dtype, q=pre.q[:, S - 1:].contiguous(), k=pre.k, w=pre.w[:, S - 1:].contiguous(),
                            q_scale=None if pre.q_scale is None else pre.q_scale[:, S - 1:].contiguous(),
                            k_scale=pre.k_scale, q_pos0=S - 1)
    got_dec = check_exact(dsa, dec, topk)
    got_pre = run_topk(dsa, pre, topk).cpu().numpy()
    assert np.array_equal(got_dec[:, 0], got_pre[:, S - 1])


def test_decode_scan_float_signed_w(dsa, dev):
    ixi = syn.decode_layer_indexer(0, B=4, S=7000, device=dev)
    check_float(dsa, ixi, 2048, np.array([0]))


def test_decode_full_size_layer(dsa, dev):
    """One decode F layer at full size: B=8 sequences, 204800 cached fp8 keys."""
    ixi = syn.decode_layer_indexer(0, device=dev)
    check_float(dsa, ixi, 2048, np.array([0]))
    ixi = syn.decode_layer_indexer(1, device=dev, values="int")
    check_exact(dsa, ixi, 2048)


def test_determinism(dsa, dev):
    ixi = syn.indexer_inputs(B=1, n_q=3000, dtype=syn.BF16, values="normal", seed=4, device=dev)
    a = run_topk(dsa, ixi, 2048)
    b = run_topk(dsa, ixi, 2048)
    assert torch.equal(a, b)


# --------------------------------------------------------------------------- long rows
@pytest.mark.parametrize("dtype", [syn.BF16, syn.FP8])
def test_fused_prefill_compaction_integer_exact(dsa, dev, dtype):
    """Rows longer than the candidate buffer force compactions (rows shorter than
    32768 keys compact first at 8192 candidates, longer ones at 16384: rows on
    both sides of both limits).  With integer scores ties are massive, so the
    16-bit-prefix shrink cannot free space and the exact select (ties to the
    lower position) takes over."""
    L = 40000
    ixi = syn.indexer_inputs(B=1, n_q=L, dtype=dtype, values="int", w_dist="pow2", seed=31, device=dev)
    rows = np.array([0, 2047, 8191, 8192, 8300, 16383, 16384, 16400, 20000, 32766, 32767, 32768, 33333,
                     L - 2, L - 1])
    check_exact(dsa, ixi, 2048, rows=rows)


def test_fused_prefill_compaction_float(dsa, dev):
    L = 40000
    ixi = syn.indexer_inputs(B=1, n_q=L, dtype=syn.BF16, values="normal", w_dist="u8", seed=32, device=dev)
    check_float(dsa, ixi, 2048, np.array([8191, 8192, 16383, 16384, 25000, 32767, 32768, L - 1]))


@pytest.mark.parametrize("wl", ["prefill_bf16_L16384", "prefill_fp8_L65536"])
def test_full_size_prefill_sampled(dsa, dev, wl):
    """The bf16 L=16384 and fp8 L=65536 prefill layers at full size, in the launch
    configuration the benchmark uses; sampled rows against the oracle."""
    c = syn.WORKLOADS[wl]
    ixi = syn.indexer_inputs(B=1, n_q=c["L"], dtype=c["dtype"], values="normal", w_dist="u8", seed=c["seed"],
                             device=dev)
    rows = np.array([0, 2046, 2047, 2048, c["L"] // 2, c["L"] - 1])
    check_float(dsa, ixi, c["topk"], rows)


def test_full_size_stack_layer_integer_exact(dsa, dev):
    """One F layer of the 8-layer L=131072 stack, integer-valued variant."""
    layers = syn.prefill_stack_layers(L=131072, n_layers=1, seed=4, device=dev, values="int", with_sa=False)
    ixi = layers[0][0]
    check_exact(dsa, ixi, 2048, rows=np.array([5, 4095, 65536, 131070, 131071]))
