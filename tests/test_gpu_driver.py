"""GPU parity of the IndexCache layer loop against the oracle's loop."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from synth import inputs as syn
from tests import helpers as H

pytestmark = pytest.mark.gpu
GOLD = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def dsa():
    import dsa_lightning_indexer_amd as m
    return m


def build_stack(dev, pattern, L, topk, values="int"):
    layers = syn.prefill_stack_layers(L=L, n_layers=len(pattern), seed=40, device=dev, values=values)
    specs = []
    for l, (ix, sa) in enumerate(layers):
        out = torch.zeros((1, L, 16, 512), dtype=torch.float32, device=dev)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "out": out, "d_v": 512}}
        if pattern[l] == "F":
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w}
            spec["idx_out"] = torch.full((1, L, topk), -7, dtype=torch.int32, device=dev)
        specs.append(spec)
    return layers, specs


def test_fsss_trace_on_gpu(dsa, dev):
    """The FSSS FSSS trace: F layers 1 and 5 run the indexer, layers 2-4 and 6-8
    reuse their index tensor.  S layers get no indexer inputs at all (NULL
    pointers, no output buffer); each layer's attention uses its own Q/KV."""
    g = json.load(open(os.path.join(GOLD, "fsss_trace.json")))
    pattern, L, topk = g["pattern"], 700, 128
    layers, specs = build_stack(dev, pattern, L, topk)
    src = dsa.indexcache_forward(pattern, specs, topk)
    torch.cuda.synchronize()
    assert [s + 1 for s in src] == g["source_layer_1based"]

    def indexer_fn(l):
        ix = layers[l - 1][0]
        q, k, w = H.indexer_f64(ix)
        return oracle.indexer_topk(q, k, w, topk)[0]

    rows = np.array([0, 1, 100, 127, 128, 300, L - 1])

    def attn_fn(l, T):
        Q, K, V = H.sa_f64(layers[l - 1][1])
        return oracle.sparse_attn(Q, K, V, T, layers[l - 1][1].scale, rows=rows)

    osrc, Ts, outs, calls = oracle.indexcache_forward(pattern, indexer_fn, attn_fn)
    assert calls == g["indexer_layers_1based"]
    for l in range(len(pattern)):
        if pattern[l] == "F":
            got = specs[l]["idx_out"][0].cpu().numpy()
            assert np.array_equal(got, Ts[l]), f"layer {l + 1} index tensor differs"
        got = specs[l]["sa"]["out"][0].cpu().numpy()[rows]
        assert H.attn_close(got, outs[l]) <= H.ATTN_RTOL, f"layer {l + 1} attention"


def test_s_layers_equal_their_f_layer_and_all_f_differs(dsa, dev):
    L, topk = 900, 256
    pat_s, pat_f = "FSSSFSSS", "FFFFFFFF"
    _, s_specs = build_stack(dev, pat_s, L, topk, values="normal")
    _, f_specs = build_stack(dev, pat_f, L, topk, values="normal")
    dsa.indexcache_forward(pat_s, s_specs, topk)
    dsa.indexcache_forward(pat_f, f_specs, topk)
    torch.cuda.synchronize()
    # F layers of both runs saw identical inputs -> identical tensors
    assert torch.equal(s_specs[0]["idx_out"], f_specs[0]["idx_out"])
    assert torch.equal(s_specs[4]["idx_out"], f_specs[4]["idx_out"])
    # S layer attention equals attention run directly on the F layer's tensor
    for l in (1, 2, 3, 5, 6, 7):
        f = 0 if l < 4 else 4
        sa = s_specs[l]["sa"]
        direct = dsa.sparse_attn(sa["q"], sa["kv"], s_specs[f]["idx_out"], sa["scale"], d_v=512)
        torch.cuda.synchronize()
        assert torch.equal(direct, sa["out"]), l
    # overlap between adjacent all-F layers is high but not 1 (keys differ by noise)
    k = topk
    tot = dsa.index_overlap(f_specs[0]["idx_out"][0, k - 1:], f_specs[1]["idx_out"][0, k - 1:], k)
    ov = int(tot.item()) / ((L - k + 1) * k)
    assert 0.3 < ov < 1.0, ov


def test_decode_stack_fsss(dsa, dev):
    """Decode through the layer loop: 9 layers FSSSFSSSF, B=2, 5000 cached tokens."""
    pattern, B, S, topk = "FSSSFSSSF", 2, 5000, 2048
    specs, ixs, sas = [], [], []
    for l, c in enumerate(pattern):
        sa = syn.decode_layer_sa(l, B=B, S=S, device=dev)
        sas.append(sa)
        out = torch.zeros((B, 1, 16, 512), device=dev)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "out": out, "d_v": 512}}
        ix = syn.decode_layer_indexer(l, B=B, S=S, device=dev, values="int") if c == "F" else None
        ixs.append(ix)
        if ix is not None:
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w, "q_scale": ix.q_scale, "k_scale": ix.k_scale,
                          "q_pos0": ix.q_pos0}
            spec["idx_out"] = torch.empty((B, 1, topk), dtype=torch.int32, device=dev)
        specs.append(spec)
    src = dsa.indexcache_forward(pattern, specs, topk)
    torch.cuda.synchronize()
    assert src == [0, 0, 0, 0, 4, 4, 4, 4, 8]
    for b in range(B):
        T = None
        for l, c in enumerate(pattern):
            if c == "F":
                q, k, w = H.indexer_f64(ixs[l], b)
                T = oracle.indexer_topk(q, k, w, topk, q_pos0=S - 1)[0]
                assert np.array_equal(specs[l]["idx_out"][b].cpu().numpy(), T)
            Q, K, V = H.sa_f64(sas[l], b)
            ref = oracle.sparse_attn(Q, K, V, T, sas[l].scale)
            got = specs[l]["sa"]["out"][b].cpu().numpy()
            assert H.attn_close(got, ref) <= H.ATTN_RTOL


@pytest.mark.parametrize("retention", ["1/4", "1/8"])
def test_searched_47_layer_pattern_on_gpu(dsa, dev, retention):
    """A searched 47-layer sharing pattern ([IC-SUMMARY] Appendix B) through the
    driver: every F layer's index tensor is bit-exact against the oracle on
    integer inputs, every layer attends with the tensor of its source layer
    (compared on sampled rows), and no S layer gets indexer inputs."""
    pattern = syn.SEARCHED_PATTERNS_47[retention]
    L, topk = 320, 64
    layers, specs = build_stack(dev, pattern, L, topk)
    src = dsa.indexcache_forward(pattern, specs, topk)
    torch.cuda.synchronize()
    assert [s + 1 for s in src] == oracle.source_layers(pattern)

    def indexer_fn(l):
        ix = layers[l - 1][0]
        q, k, w = H.indexer_f64(ix)
        return oracle.indexer_topk(q, k, w, topk)[0]

    rows = np.array([0, 63, 64, 200, L - 1])

    def attn_fn(l, T):
        Q, K, V = H.sa_f64(layers[l - 1][1])
        return oracle.sparse_attn(Q, K, V, T, layers[l - 1][1].scale, rows=rows)

    osrc, Ts, outs, calls = oracle.indexcache_forward(pattern, indexer_fn, attn_fn)
    assert calls == [l + 1 for l, c in enumerate(pattern) if c == "F"]
    for l in range(len(pattern)):
        if pattern[l] == "F":
            assert np.array_equal(specs[l]["idx_out"][0].cpu().numpy(), Ts[l]), f"layer {l + 1} index"
        got = specs[l]["sa"]["out"][0].cpu().numpy()[rows]
        assert H.attn_close(got, outs[l]) <= H.ATTN_RTOL, f"layer {l + 1} attention"


def test_decode_stack_graph_replay(dsa, dev):
    """The decode layer loop captured once in a HIP graph and replayed: every
    replay (with eager writes over the outputs and host synchronisation between
    replays) reproduces the eager run bit for bit, and the eager run matches the
    oracle on the F layers' index tensors."""
    pattern, B, S, topk = "FSSSFSSSF", 2, 6000, 2048
    specs, ixs = [], []
    for l, c in enumerate(pattern):
        sa = syn.decode_layer_sa(l, B=B, S=S, device=dev)
        out = torch.zeros((B, 1, 16, 512), device=dev)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "out": out, "d_v": 512}}
        ix = syn.decode_layer_indexer(l, B=B, S=S, device=dev, values="int") if c == "F" else None
        ixs.append(ix)
        if ix is not None:
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w, "q_scale": ix.q_scale, "k_scale": ix.k_scale,
                          "q_pos0": ix.q_pos0}
            spec["idx_out"] = torch.empty((B, 1, topk), dtype=torch.int32, device=dev)
        specs.append(spec)
    ws = torch.empty(max(dsa.indexcache_forward_workspace_size(pattern, specs, topk), 256),
                     dtype=torch.uint8, device=dev)
    dsa.indexcache_forward(pattern, specs, topk, ws=ws)
    torch.cuda.synchronize()
    eager_idx = [s["idx_out"].clone() for s in specs if "idx_out" in s]
    eager_out = [s["sa"]["out"].clone() for s in specs]
    for l, c in enumerate(pattern):
        if c == "F":
            q, k, w = H.indexer_f64(ixs[l], 1)
            T = oracle.indexer_topk(q, k, w, topk, q_pos0=S - 1)[0]
            assert np.array_equal(specs[l]["idx_out"][1].cpu().numpy(), T)

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dsa.indexcache_forward(pattern, specs, topk, ws=ws)
    for rep in range(3):
        for s in specs:
            s["sa"]["out"].fill_(float("nan"))
            if "idx_out" in s:
                s["idx_out"].fill_(-7)
        ws.fill_(0xA5)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got_idx = [s["idx_out"] for s in specs if "idx_out" in s]
        for a, b in zip(got_idx, eager_idx):
            assert torch.equal(a, b), f"replay {rep}: index tensor differs from the eager run"
        for l, s in enumerate(specs):
            assert torch.equal(s["sa"]["out"], eager_out[l]), f"replay {rep}: layer {l + 1} attention differs"
