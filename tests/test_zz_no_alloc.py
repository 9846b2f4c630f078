"""indexcache_forward_noalloc (static per-GPU scratch, no workspace argument)
against indexcache_forward with a caller workspace.  Both run the same kernels
with the same launch shapes, so outputs are compared bit for bit: two calls in
a row, the second with a smaller input (the scratch still holds the first
call's contents), and a graph capture replayed several times."""
import pytest
import torch

from synth import inputs as syn

pytestmark = pytest.mark.gpu

TOPK = 2048


@pytest.fixture(scope="module")
def dsa():
    import dsa_lightning_indexer_amd as m
    return m


def decode_stack(dev, B, S, pattern, seed):
    specs = []
    for l, c in enumerate(pattern):
        sa = syn.decode_layer_sa(l, B=B, S=S, seed=seed, device=dev)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.full((B, 1, 16, 512), float("nan"), device=dev)}}
        if c == "F":
            ix = syn.decode_layer_indexer(l, B=B, S=S, seed=seed, device=dev)
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w, "q_scale": ix.q_scale, "k_scale": ix.k_scale,
                          "q_pos0": ix.q_pos0}
            spec["idx_out"] = torch.full((B, 1, TOPK), -7, dtype=torch.int32, device=dev)
        specs.append(spec)
    return specs


def twin(specs):
    """The same inputs with fresh output tensors."""
    out = []
    for s in specs:
        t = {"sa": dict(s["sa"], out=torch.full_like(s["sa"]["out"], float("nan")))}
        if "ix" in s:
            t["ix"] = s["ix"]
            t["idx_out"] = torch.full_like(s["idx_out"], -7)
        out.append(t)
    return out


def assert_same(a, b, pattern):
    for l, c in enumerate(pattern):
        if c == "F":
            assert torch.equal(a[l]["idx_out"], b[l]["idx_out"]), f"layer {l}: index tensors differ"
        assert torch.equal(a[l]["sa"]["out"], b[l]["sa"]["out"]), f"layer {l}: attention outputs differ"


@pytest.mark.parametrize("B,S,pattern", [(8, 60000, "FSSSFS"), (3, 9000, "FSF")])
def test_noalloc_matches_workspace_driver(dsa, dev, B, S, pattern):
    ref = decode_stack(dev, B, S, pattern, seed=11)
    got = twin(ref)
    src_ref = dsa.indexcache_forward(pattern, ref, TOPK)
    src = dsa.indexcache_forward_noalloc(pattern, got, TOPK)
    torch.cuda.synchronize()
    assert src == src_ref
    assert_same(ref, got, pattern)


def test_noalloc_two_calls_second_smaller(dsa, dev):
    big = decode_stack(dev, 8, 120000, "FSSF", seed=12)
    small = decode_stack(dev, 2, 5000, "FS", seed=13)
    big_ref, small_ref = twin(big), twin(small)
    dsa.indexcache_forward("FSSF", big_ref, TOPK)
    dsa.indexcache_forward("FS", small_ref, TOPK)
    dsa.indexcache_forward_noalloc("FSSF", big, TOPK)
    dsa.indexcache_forward_noalloc("FS", small, TOPK)
    torch.cuda.synchronize()
    assert_same(big_ref, big, "FSSF")
    assert_same(small_ref, small, "FS")


def test_noalloc_graph_replay(dsa, dev):
    """Captured into a HIP graph (after a first eager call on the device), every
    replay equals the eager workspace-driver result."""
    pattern = "FSSSF"
    ref = decode_stack(dev, 4, 30000, pattern, seed=14)
    got = twin(ref)
    dsa.indexcache_forward(pattern, ref, TOPK)
    dsa.indexcache_forward_noalloc(pattern, got, TOPK)
    torch.cuda.synchronize()
    assert_same(ref, got, pattern)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        dsa.indexcache_forward_noalloc(pattern, got, TOPK)
    for _ in range(3):
        for s in got:
            s["sa"]["out"].fill_(float("nan"))
            if "idx_out" in s:
                s["idx_out"].fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_same(ref, got, pattern)
