"""GPU parity of the multi-layer-indexer shift ([MLI] 核心思路) against the
oracle's shifted loop: layer l attends with the nearest earlier F layer's index
tensor (layer 0 with its own) while F-layer indexers run on a second stream.
Integer-valued indexer inputs, so every index tensor is bit-exact; attention
within 2e-3 on the oracle's own index tensors."""
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


def prefill_specs(dev, pattern, L, topk):
    layers = syn.prefill_stack_layers(L=L, n_layers=len(pattern), seed=41, device=dev, values="int")
    specs = []
    for l, (ix, sa) in enumerate(layers):
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.full((1, L, 16, 512), float("nan"), device=dev)}}
        if pattern[l] == "F":
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w}
            spec["idx_out"] = torch.full((1, L, topk), -7, dtype=torch.int32, device=dev)
        specs.append(spec)
    return layers, specs


def fresh_outputs(specs):
    for s in specs:
        s["sa"]["out"].fill_(float("nan"))
        if "idx_out" in s:
            s["idx_out"].fill_(-7)


@pytest.mark.parametrize("pattern", ["FSFFS", "FFFF", "FSSSFSSS"])
def test_mli_prefill_stack_matches_shifted_oracle(dsa, dev, pattern):
    L, topk = 700, 128
    layers, specs = prefill_specs(dev, pattern, L, topk)
    side = torch.cuda.Stream(device=dev)
    src = dsa.indexcache_forward_mli(pattern, specs, topk, index_stream=side)
    torch.cuda.synchronize()
    want = [s - 1 for s in oracle.mli_source_layers(pattern)]
    assert src == want
    T = {}
    for l, c in enumerate(pattern):
        if c == "F":
            q, k, w = H.indexer_f64(layers[l][0])
            T[l] = oracle.indexer_topk(q, k, w, topk)[0]
            assert np.array_equal(specs[l]["idx_out"][0].cpu().numpy(), T[l]), f"layer {l}: index tensor"
    rows = np.array([0, 3, topk - 1, topk, 333, L - 1])
    for l in range(len(pattern)):
        sa = layers[l][1]
        Q, K, V = H.sa_f64(sa)
        ref = oracle.sparse_attn(Q, K, V, T[want[l]], sa.scale, rows=rows)
        got = specs[l]["sa"]["out"][0].cpu().numpy()[rows]
        assert H.attn_close(got, ref) <= H.ATTN_RTOL, f"layer {l}"
    # one stream (in order) gives the same bits
    outs = [s["sa"]["out"].clone() for s in specs]
    fresh_outputs(specs)
    assert dsa.indexcache_forward_mli(pattern, specs, topk) == want
    torch.cuda.synchronize()
    for l in range(len(pattern)):
        assert torch.equal(specs[l]["sa"]["out"], outs[l]), f"layer {l}: one stream differs from two"


def test_mli_decode_stack_matches_shifted_oracle(dsa, dev):
    """Decode layers (fp8 K cache scan + select, split-k attention) in the
    overlapped loop: FSSSFSSSF, B = 2, 5000 cached tokens."""
    pattern, B, S, topk = "FSSSFSSSF", 2, 5000, 2048
    specs, ixs, sas = [], [], []
    for l, c in enumerate(pattern):
        sa = syn.decode_layer_sa(l, B=B, S=S, device=dev)
        sas.append(sa)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.full((B, 1, 16, 512), float("nan"), device=dev)}}
        ix = syn.decode_layer_indexer(l, B=B, S=S, device=dev, values="int") if c == "F" else None
        ixs.append(ix)
        if ix is not None:
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w, "q_scale": ix.q_scale, "k_scale": ix.k_scale,
                          "q_pos0": ix.q_pos0}
            spec["idx_out"] = torch.full((B, 1, topk), -7, dtype=torch.int32, device=dev)
        specs.append(spec)
    side = torch.cuda.Stream(device=dev)
    src = dsa.indexcache_forward_mli(pattern, specs, topk, index_stream=side)
    torch.cuda.synchronize()
    want = [s - 1 for s in oracle.mli_source_layers(pattern)]
    assert src == want == [0, 0, 0, 0, 0, 4, 4, 4, 4]
    for b in range(B):
        T = {}
        for l, c in enumerate(pattern):
            if c == "F":
                q, k, w = H.indexer_f64(ixs[l], b)
                T[l] = oracle.indexer_topk(q, k, w, topk, q_pos0=S - 1)[0]
                assert np.array_equal(specs[l]["idx_out"][b].cpu().numpy(), T[l])
        for l in range(len(pattern)):
            Q, K, V = H.sa_f64(sas[l], b)
            ref = oracle.sparse_attn(Q, K, V, T[want[l]], sas[l].scale)
            got = specs[l]["sa"]["out"][b].cpu().numpy()
            assert H.attn_close(got, ref) <= H.ATTN_RTOL, (b, l)
