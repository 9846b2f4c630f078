"""Parity at the full sizes of the measured workloads, on the bench's own inputs.

Each test builds its inputs exactly as bench.py does (same generators, seeds and
shapes), runs them through the same entry point and launch configuration, and
compares sampled query rows with the CPU oracle:
  * indices (float inputs): the tie-window rule against the float64 oracle on
    the same bf16 / fp8 bytes (rows t < k, t = k - 1, t = k, random rows, the
    last row);
  * attention: per (row, head) max |o - o_ref| <= 2e-3 max |o_ref|, computed by
    the oracle on the GPU's own index row ([DSA-NOTES] §3 equation for o_t),
    so that selection and attention errors are separated.
The oracle only sees the rows it needs (dequantised one query row at a time,
and the selected latent rows only), so every check is a few seconds of CPU."""
import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu

TOPK = 2048


@pytest.fixture(scope="module")
def dsa():
    import dsa_lightning_indexer_amd as m
    return m


def sample_rows(L, seed, n_random=3):
    r = np.random.default_rng(seed)
    rows = {0, 5, TOPK - 2, TOPK - 1, TOPK, L - 1}
    rows |= set(r.integers(TOPK + 1, L - 1, n_random).tolist())
    return np.array(sorted(rows))


def check_index_rows(ixi, got, rows, b=0):
    """got: the GPU's [n_q, k] index tensor of batch b (numpy)."""
    k64 = H.deq(ixi.k[b], None if ixi.k_scale is None else ixi.k_scale[b])
    n_k = k64.shape[0]
    for i in rows:
        q64 = H.deq(ixi.q[b, i:i + 1], None if ixi.q_scale is None else ixi.q_scale[b, i:i + 1])
        w64 = ixi.w[b, i:i + 1].detach().cpu().double().numpy()
        t = ixi.q_pos0 + int(i)
        ref, I, _ = oracle.indexer_topk(q64, k64, w64, TOPK, q_pos0=t)
        H.check_ascending_padded(got[i], min(t, n_k - 1), TOPK)
        msg = H.check_index_set(got[i], ref[0], I[0, :min(t + 1, n_k)], TOPK)
        assert msg is None, f"batch {b} row {i} (t={t}): {msg}"


def check_attention_rows(sa, idx_np, out, rows, b=0):
    """Oracle attention on the GPU's index rows, over only the selected latent rows."""
    kv_raw, dt = H.raw(sa.kv[b])                       # [n_k, 1, 576] raw bf16
    worst = 0.0
    for i in rows:
        sel = idx_np[i][idx_np[i] >= 0]
        KV = oracle.dequantize(kv_raw[sel], dt)          # the selected rows only
        Q = H.deq(sa.q[b, i:i + 1])
        ref = oracle.sparse_attn(Q, KV, KV[..., :sa.d_v], np.arange(sel.size)[None, :], sa.scale)
        got = out[b, i:i + 1].detach().cpu().numpy()
        err = H.attn_close(got, ref)
        worst = max(worst, err)
        assert err <= H.ATTN_RTOL, f"batch {b} row {i}: relative error {err:.3g}"
    return worst


def test_prefill_stack_layers_full_size(dsa, dev):
    """The 8-layer prefill stack at L = 131072 as the benchmark builds it: its
    first two layers (F then S) through indexcache_forward.  The float F layer's
    indices follow the tie-window rule, and both layers' attention outputs match
    the oracle on that index tensor."""
    L = 131072
    layers = syn.prefill_stack_layers(L=L, n_layers=2, seed=4, device=dev)
    specs = []
    for l, (ix, sa) in enumerate(layers):
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.empty((1, L, 16, 512), dtype=torch.float32, device=dev)}}
        if l == 0:
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w}
            spec["idx_out"] = torch.empty((1, L, TOPK), dtype=torch.int32, device=dev)
        specs.append(spec)
    src = dsa.indexcache_forward("FS", specs, TOPK)
    torch.cuda.synchronize()
    assert src == [0, 0]
    idx = specs[0]["idx_out"][0].cpu().numpy()
    rows = sample_rows(L, seed=41)
    check_index_rows(layers[0][0], idx, rows)
    for l in range(2):
        check_attention_rows(layers[l][1], idx, specs[l]["sa"]["out"], rows)


def test_fp8_prefill_layer_and_attention_full_size(dsa, dev):
    """The fp8 prefill layer at L = 65536 (per-token key scales, per-(token, head)
    query scales) and its 16-head MLA attention, as timed by the benchmark's
    single-layer mode: fused indexer+Top-k, then sparse attention over its
    index tensor."""
    c = syn.WORKLOADS["prefill_fp8_L65536"]
    L = c["L"]
    ixi = syn.indexer_inputs(B=1, n_q=L, H=c["H"], d=c["d"], dtype=c["dtype"], values=c["values"],
                             w_dist=c["w_dist"], seed=c["seed"], device=dev)
    idx = dsa.topk(ixi.q, ixi.k, ixi.w, TOPK, q_scale=ixi.q_scale, k_scale=ixi.k_scale)
    sa = syn.sa_inputs(B=1, n_q=L, n_k=L, heads=c["sa_heads"], d_qk=c["sa_d_qk"], d_v=c["sa_d_v"], seed=c["seed"],
                       device=dev)
    out = dsa.sparse_attn(sa.q, sa.kv, idx, sa.scale, d_v=sa.d_v)
    torch.cuda.synchronize()
    idx_np = idx[0].cpu().numpy()
    rows = sample_rows(L, seed=42)
    check_index_rows(ixi, idx_np, rows)
    check_attention_rows(sa, idx_np, out, rows)


def test_decode_stack_layers_full_size(dsa, dev):
    """The decode stack's first two layers (F then S) at B = 8 sequences x 204800
    cached tokens, as the benchmark builds them: every sequence's fp8 decode
    Top-k follows the tie-window rule, and both layers' split-k decode attention
    matches the oracle on every sequence."""
    B, S = 8, 204800
    specs, ixs, sas = [], [], []
    for l in range(2):
        sa = syn.decode_layer_sa(l, B=B, S=S, device=dev)
        sas.append(sa)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.empty((B, 1, 16, 512), dtype=torch.float32, device=dev)}}
        if l == 0:
            ix = syn.decode_layer_indexer(l, B=B, S=S, device=dev)
            ixs.append(ix)
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w, "q_scale": ix.q_scale, "k_scale": ix.k_scale,
                          "q_pos0": ix.q_pos0}
            spec["idx_out"] = torch.empty((B, 1, TOPK), dtype=torch.int32, device=dev)
        specs.append(spec)
    src = dsa.indexcache_forward("FS", specs, TOPK)
    torch.cuda.synchronize()
    assert src == [0, 0]
    idx = specs[0]["idx_out"].cpu().numpy()            # [B, 1, k]
    for b in range(B):
        check_index_rows(ixs[0], idx[b], np.array([0]), b=b)
        for l in range(2):
            check_attention_rows(sas[l], idx[b], specs[l]["sa"]["out"], np.array([0]), b=b)
