"""GPU parity of sparse attention and the overlap measure against the oracle.
Sparse attention: per (row, head) max_c|o_gpu - o_ref| <= 2e-3 * max_c|o_ref|,
with the index tensor drawn by the seeded generator (never produced by the GPU)."""
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


def run_sa(dsa, sa, idx):
    out = dsa.sparse_attn(sa.q, sa.kv, idx, sa.scale, d_v=sa.d_v, v=sa.v)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_sa(dsa, sa, idx, rows=None):
    got = run_sa(dsa, sa, idx)
    B, n_q = sa.q.shape[:2]
    worst = 0.0
    for b in range(B):
        Q, K, V = H.sa_f64(sa, b)
        rr = np.arange(n_q) if rows is None else rows
        ref = oracle.sparse_attn(Q, K, V, idx[b].cpu().numpy(), sa.scale, rows=rr)
        worst = max(worst, H.attn_close(got[b, rr], ref))
    assert worst <= H.ATTN_RTOL, worst
    return got


def test_tiny_fp32_mha(dsa, dev):
    c = syn.WORKLOADS["tiny_fp32_L512"]
    L = c["L"]
    sa = syn.sa_inputs(n_q=L, n_k=L, heads=4, kv_heads=4, d_qk=64, d_v=64, latent=False, dtype=syn.F32,
                       seed=c["seed"], device=dev)
    idx = syn.random_sorted_indices(n_q=L, topk=c["topk"], seed=12, device=dev)
    check_sa(dsa, sa, idx)


def test_mla_prefill_short_and_full_rows(dsa, dev):
    """16 heads over the 576-wide latent (V = first 512 columns); rows t < 2047
    carry -1 padding, later rows a full 2048 selection."""
    n = 2600
    sa = syn.sa_inputs(n_q=n, n_k=n, seed=3, device=dev)
    idx = syn.random_sorted_indices(n_q=n, topk=2048, seed=4, device=dev)
    rows = np.array(sorted(set([0, 1, 2, 15, 16, 17, 500, 2046, 2047, 2048, 2300, n - 1])))
    check_sa(dsa, sa, idx, rows)


def test_mla_decode_split(dsa, dev):
    """Decode shape (1 query per sequence): the index row is split across
    workgroups and merged by the combine kernel."""
    B, S = 3, 9000
    sa = syn.sa_inputs(B=B, n_q=1, n_k=S, seed=5, device=dev)
    idx = syn.random_sorted_indices(B=B, n_q=1, topk=2048, q_pos0=S - 1, seed=6, device=dev)
    check_sa(dsa, sa, idx)


@pytest.mark.parametrize("B,topk", [(5, 1000), (1, 700), (8, 130), (2, 100)])
def test_mla_decode_ragged_splits(dsa, dev, B, topk):
    """Decode shapes whose index rows split unevenly: 1000 entries over 15
    splits of 67 (the last 62), 700 over 10 of 70, 130 over 2 of 65; 100
    entries give a single split (no combine).  Splits end inside 16-position
    steps."""
    S = 5000
    sa = syn.sa_inputs(B=B, n_q=1, n_k=S, seed=21, device=dev)
    idx = syn.random_sorted_indices(B=B, n_q=1, topk=topk, q_pos0=S - 1, seed=22, device=dev)
    check_sa(dsa, sa, idx)


@pytest.mark.parametrize("n", [300, 1103])
def test_mla_invalid_entries_and_empty_rows(dsa, dev, n):
    """Empty rows, out-of-range entries and ragged row counts.  300 rows run the
    four-waves-per-row kernel with split index rows; 1103 rows the
    one-wave-per-row kernel (from 1024 rows), whose last workgroup has three
    rows."""
    sa = syn.sa_inputs(n_q=n, n_k=n, seed=7, device=dev)
    idx = syn.random_sorted_indices(n_q=n, topk=2048, seed=8, device=dev)
    idx[0, 10] = -1                      # an empty row -> zeros
    idx[0, 11, :] = n + 5                # out of range -> selects nothing
    idx[0, 12, 5] = 10 ** 9              # one bad entry among valid ones
    idx[0, n - 2, 100:] = -1             # a row that ends early
    rows = np.concatenate([np.arange(0, 40), np.arange(n - 5, n)])
    got = check_sa(dsa, sa, idx, rows)
    assert (got[0, 10] == 0).all() and (got[0, 11] == 0).all()


@pytest.mark.parametrize("topk", [1, 17, 100, 700])
def test_mla_rows_kernel_short_index_rows(dsa, dev, topk):
    """The one-wave-per-row kernel (from 1024 rows) on index rows of other
    lengths than 2048: a row ending inside a 16-position step and inside a
    64-entry block of the index ring; 1030 rows leave the last workgroup two
    rows."""
    n = 1030
    sa = syn.sa_inputs(n_q=n, n_k=n, seed=13, device=dev)
    idx = syn.random_sorted_indices(n_q=n, topk=topk, seed=14, device=dev)
    rows = np.array(sorted(set([0, 1, topk - 1, topk, 511, 1000, n - 2, n - 1])))
    check_sa(dsa, sa, idx, rows)


def test_mla_rows_kernel_batched(dsa, dev):
    """Two batches of 600 query rows (1200 rows: the one-wave-per-row kernel),
    queries at positions 100..699 of a 700-row latent cache per batch: each
    row gathers from its own batch's rows."""
    B, n_q, n_k = 2, 600, 700
    sa = syn.sa_inputs(B=B, n_q=n_q, n_k=n_k, seed=15, device=dev)
    idx = syn.random_sorted_indices(B=B, n_q=n_q, topk=2048, q_pos0=n_k - n_q, n_k=n_k, seed=16, device=dev)
    check_sa(dsa, sa, idx, np.array([0, 1, 299, 598, 599]))


@pytest.mark.parametrize("latent,kv_heads,dtype", [(False, 2, syn.BF16), (True, 4, syn.BF16), (False, 1, syn.F32)])
def test_generic_paths(dsa, dev, latent, kv_heads, dtype):
    n = 200
    sa = syn.sa_inputs(n_q=n, n_k=n, heads=8, kv_heads=kv_heads, d_qk=96, d_v=80 if not latent else 64,
                       latent=latent, dtype=dtype, seed=9, device=dev)
    idx = syn.random_sorted_indices(n_q=n, topk=100, seed=10, device=dev)
    check_sa(dsa, sa, idx)


def test_sa_determinism(dsa, dev):
    sa = syn.sa_inputs(B=2, n_q=1, n_k=5000, seed=11, device=dev)
    idx = syn.random_sorted_indices(B=2, n_q=1, topk=2048, q_pos0=4999, seed=12, device=dev)
    a = run_sa(dsa, sa, idx)
    b = run_sa(dsa, sa, idx)
    assert np.array_equal(a, b)


def test_overlap_counts(dsa, dev):
    k = 256
    a = syn.random_sorted_indices(n_q=700, topk=k, seed=1, device=dev)[0]
    b = syn.random_sorted_indices(n_q=700, topk=k, seed=2, device=dev)[0]
    b[300:400] = a[300:400]
    counts = torch.zeros(700, dtype=torch.int32, device=dev)
    total = dsa.index_overlap(a, b, k, row_counts=counts)
    an, bn = a.cpu().numpy(), b.cpu().numpy()
    ref = [len(set(an[r][an[r] >= 0]) & set(bn[r][bn[r] >= 0])) for r in range(700)]
    assert counts.cpu().numpy().tolist() == ref
    assert int(total.item()) == sum(ref)
    rows = np.arange(k - 1, 700)
    ov = sum(ref[r] for r in rows) / (len(rows) * k)
    assert ov == pytest.approx(oracle.overlap(an, bn, k, rows))


@pytest.mark.parametrize("mode", range(11))
def test_gather_probe_reads_every_selected_row(dsa, dev, mode):
    """The gather probe (measurement helper) reads each valid selected 1152-byte
    row exactly once per query: the XOR of its per-wave checksums equals the XOR
    of every 32-bit word of the query's selected rows; -1 padding and entries
    past the table read nothing.  Covers a partial last workgroup (37 queries)
    and index rows that end mid-step (300 entries)."""
    n_rows, n_q, topk = 5000, 37, 300
    g = torch.Generator(device=dev)
    g.manual_seed(mode)
    kv = torch.randint(-(1 << 15), 1 << 15, (n_rows, 576), dtype=torch.int32, generator=g, device=dev)
    kv = kv.to(torch.int16).view(torch.bfloat16).contiguous()
    idx = syn.random_sorted_indices(B=1, n_q=n_q, topk=topk, q_pos0=280, n_k=n_rows, seed=5, device=dev)[0]
    idx[3, -1] = n_rows + 7                      # past the table: read nothing
    idx[4, 10] = -1
    out = dsa.gather_probe(kv, idx.contiguous(), mode)
    torch.cuda.synchronize()
    words = kv.view(torch.int16).cpu().numpy().view(np.uint32)   # [n_rows, 288]
    got = out.cpu().numpy().view(np.uint32)
    ix = idx.cpu().numpy()
    for q in range(n_q):
        sel = ix[q][(ix[q] >= 0) & (ix[q] < n_rows)]
        want = np.bitwise_xor.reduce(words[sel].ravel()) if sel.size else np.uint32(0)
        have = np.bitwise_xor.reduce(got[4 * q:4 * q + 4]) if mode in (0, 3, 6, 7, 8) else got[q]
        assert have == want, (mode, q)


@pytest.mark.parametrize("wgs,unroll", [(1, 1), (7, 2), (300, 4), (4096, 4)])
def test_stream_probe_reads_every_byte_once(dsa, dev, wgs, unroll):
    """The streaming read probe (measurement helper) reads the whole buffer
    exactly once: the XOR of its per-wave checksums equals the XOR of every
    32-bit word, for grids smaller and larger than the number of chunks."""
    n = 16384 * 101
    g = torch.Generator(device=dev)
    g.manual_seed(wgs)
    buf = torch.randint(-(1 << 30), 1 << 30, (n // 4,), dtype=torch.int32, generator=g, device=dev)
    out = dsa.stream_probe(buf, wgs, unroll)
    torch.cuda.synchronize()
    want = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    have = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert have == want
