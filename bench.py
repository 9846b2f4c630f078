"""Benchmark of the DSA step with IndexCache reuse on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill stack: L = 131072 tokens, 8 layers, pattern FSSSFSSS, k = 2048,
    bf16 indexer (64 heads x 128), 16-head MLA sparse attention (576/512 latent);
  * decode stack:  8 sequences x 204800 cached tokens, 47 layers, F at layers
    1,5,...,45 (12 F), fp8 indexer K cache, 16-head MLA sparse decode attention.
Both stacks go through indexcache_forward (the C ABI), inputs resident in HBM.

Prints one JSON line.  `value` is indexer+Top-k score-pairs per second of the
whole step (causal pairs scored by every F layer of both stacks / step time);
sparse-attention tokens per second are reported beside it.
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer+Top-k score-pairs/s & sparse-attn tokens/s at 128K-200K; % MFMA/HBM peak"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=5)
    p.add_argument("--warmup", type=int, default=1)
    p.add_argument("--prefill-len", type=int, default=131072)
    p.add_argument("--decode-len", type=int, default=204800)
    p.add_argument("--decode-batch", type=int, default=8)
    p.add_argument("--decode-layers", type=int, default=47)
    p.add_argument("--kernel-reps", type=int, default=5)
    p.add_argument("--cpu-seconds", type=float, default=15.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-report", action="store_true", help="skip the all-F comparison and overlap matrix")
    p.add_argument("--distill", action="store_true",
                   help="training-aware IndexCache instead of the bench line: the distillation loss over "
                        "the selected Top-k and its backward at L=16384 (H=64, d=128, k=2048, 4 teachers); "
                        "prints one JSON object")
    p.add_argument("--sweep", action="store_true",
                   help="retention sweep instead of the bench line: both stacks under all-F, uniform 1/2, 1/4, "
                        "1/8 and (decode) the searched 47-layer patterns; prints one JSON object")
    p.add_argument("--similarity", action="store_true",
                   help="similarity-based pattern search instead of the bench line: the similarity matrix "
                        "of a 47-layer calibration prefill (L=--similarity-len, drifting indexer keys) and "
                        "the dynamic-program patterns at 24/12/7 F layers; prints one JSON object")
    p.add_argument("--mli", action="store_true",
                   help="multi-layer-indexer shift instead of the bench line: the prefill stack (FSSSFSSS) and "
                        "the decode stack (FSSS) under plain IndexCache and under the shifted loop (indexers on a "
                        "second stream beside attention, and on one stream), same inputs; prints one JSON object")
    p.add_argument("--similarity-len", type=int, default=16384)
    p.add_argument("--similarity-layers", type=int, default=47)
    p.add_argument("--layer", choices=["prefill_bf16_L16384", "prefill_fp8_L65536"], default=None,
                   help="one prefill F layer of a named workload instead of the bench line: the fused "
                        "indexer+Top-k (and, for the fp8 layer, its 16-head MLA sparse attention) timed with HIP "
                        "events over --kernel-reps launches; prints one JSON object")
    p.add_argument("--profile", choices=["indexer", "indexer_fp8", "attn", "copy", "gather", "decode", "stream"],
                   default=None,
                   help="counter-collection runs: 'indexer' launches only the prefill F layer's fused "
                        "indexer+Top-k (3 launches, the first a warm-up); 'attn' that layer's prefill "
                        "sparse attention (3 launches after one indexer launch); 'copy' runs a 1 GiB read + "
                        "1 GiB write elementwise kernel, the calibration for the HBM byte counters; 'gather' "
                        "times the prefill attention of that layer and the gather probe's access patterns over the "
                        "same index tensor and latent rows, and prints one JSON object; 'decode' runs the decode "
                        "stack's first three F layers' indexer+Top-k (scan + select) and their attention, each on "
                        "its own cold K cache, once each; 'stream' times the decode scan of one F layer on a cold "
                        "cache (evicted by a 1 GiB read right before, no host sync between) against the gather "
                        "probe reading the same number of bytes in order, also cold, and prints one JSON object")
    return p.parse_args()


def prefill_stack(dsa, syn, L, pattern, topk, dev):
    layers = syn.prefill_stack_layers(L=L, n_layers=len(pattern), seed=4, device=dev)
    specs = []
    for l, (ix, sa) in enumerate(layers):
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.empty((1, L, 16, 512), dtype=torch.float32, device=dev)}}
        if pattern[l] == "F":
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w}
            spec["idx_out"] = torch.empty((1, L, topk), dtype=torch.int32, device=dev)
        specs.append(spec)
    return layers, specs


def decode_stack(dsa, syn, B, S, n_layers, topk, dev):
    pattern = syn.uniform_pattern(n_layers, 4)
    specs = []
    for l, c in enumerate(pattern):
        sa = syn.decode_layer_sa(l, B=B, S=S, device=dev)
        spec = {"sa": {"q": sa.q, "kv": sa.kv, "scale": sa.scale, "d_v": 512,
                       "out": torch.empty((B, 1, 16, 512), dtype=torch.float32, device=dev)}}
        if c == "F":
            ix = syn.decode_layer_indexer(l, B=B, S=S, device=dev)
            spec["ix"] = {"q": ix.q, "k": ix.k, "w": ix.w, "q_scale": ix.q_scale, "k_scale": ix.k_scale,
                          "q_pos0": ix.q_pos0}
            spec["idx_out"] = torch.empty((B, 1, topk), dtype=torch.int32, device=dev)
        specs.append(spec)
    return pattern, specs


def time_launches(fn, reps):
    """Average duration of fn() with HIP events on torch's current stream (the
    stream the library launches on)."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in evs:
        a.record(st)
        fn()
        b.record(st)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def time_batch(fn, reps):
    """Average duration of fn() over reps back-to-back calls between one pair of
    HIP events (the queue stays full, so host call overhead is not counted for
    kernels that run longer than it)."""
    st = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(st)
    for _ in range(reps):
        fn()
    b.record(st)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def cpu_baseline(ix, topk, seconds):
    """The oracle as it stands, on host cores, over a bounded sample of query rows
    of the prefill stack's first F layer (rows spread over the causal range)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_info
    threads = max([d.get("num_threads", 1) for d in threadpool_info()] + [1])
    L = ix.q.shape[1]
    qraw = ix.q[0].detach().cpu().view(torch.int16).numpy().view(np.uint16)
    kraw = ix.k[0].detach().cpu().view(torch.int16).numpy().view(np.uint16)
    k64 = oracle.dequantize(kraw, "bf16")
    w64 = ix.w[0].detach().cpu().double().numpy()
    rng = np.random.default_rng(0)
    order = rng.permutation(L)
    pairs = 0
    rows = 0
    t0 = time.perf_counter()
    for i in order:
        q64 = oracle.dequantize(qraw[i:i + 1], "bf16")
        oracle.indexer_topk(q64, k64, w64[i:i + 1], topk, q_pos0=int(i))
        pairs += int(i) + 1
        rows += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": pairs / dt, "unit": "score-pairs/s", "cores": int(threads), "kind": "oracle",
            "host_cpu_count": os.cpu_count(), "blas_threads": int(threads),
            "sample": f"{rows} random query rows of the L={L} bf16 F layer (indexer + Top-k k={topk}), "
                      f"{pairs} causal pairs in {dt:.1f} s, float64 NumPy; `cores` = the BLAS threads the "
                      f"oracle ran on ({os.cpu_count()} logical CPUs on the host)"}


PROBE_MODES = {0: "quarter rows, 2 steps in flight (the attention kernel's pattern)",
               1: "whole rows per wave, 64 B of 16 rows per load, 2 steps",
               2: "whole rows per wave, rows end to end, 2 steps",
               3: "quarter rows, 4 steps in flight",
               4: "whole rows per wave, 64 B of 16 rows per load, 3 steps",
               5: "whole rows per wave, rows end to end, 3 steps",
               6: "the attention kernel's pattern: 256-B V slices of 4 rows per load + rope, 2 steps",
               7: "mode 6 with each rope line read whole by one wave (rows 4w..4w+3)",
               8: "four waves per query, wave w reads rows 4w..4w+3 whole, end to end",
               9: "the one-wave-per-query attention pattern: one instruction per row's V KiB + 2 rope-line loads, 2 steps",
               10: "mode 9's instructions landing in LDS by DMA, with the DMA attention kernel's two tiles per wave and index ring"}


def gather_ceiling(dsa, kv, idx, reps):
    """Rate at which the chip gathers the selected 1152-byte latent rows of idx
    from kv with no arithmetic (the gather probe, every access pattern it has);
    returns {mode: (ms per launch, gathered GB/s)}."""
    n_sel = int((idx >= 0).sum().item())
    out = {}
    for mode in PROBE_MODES:
        dsa.gather_probe(kv, idx, mode)
        torch.cuda.synchronize()
        ms = time_batch(lambda: dsa.gather_probe(kv, idx, mode), reps)
        out[mode] = (ms, n_sel * 1152 / (ms * 1e-3) / 1e9)
    return out


def sa_roofline(sa_ms, n_sel, probe):
    """Prefill sparse attention against its two bounds: the gather rate of the
    selected latent rows (against the probe's best pattern on the same index
    tensor, and against HBM peak for scale) and the bf16 MFMA rate of its
    2 x 16 x (576 + 512) flop per (query, selected position)."""
    gathered = n_sel * 1152
    flop = n_sel * 2 * 16 * (576 + 512)
    gbs = gathered / (sa_ms * 1e-3) / 1e9
    best_mode = max(probe, key=lambda m: probe[m][1])
    ceiling = probe[best_mode][1]
    tflops = flop / (sa_ms * 1e-3) / 1e12
    return {
        "kernel": "sa_mla1_kernel (prefill sparse attention, bf16 MLA 16 heads 576/512, one wave per query row)",
        "bound": "gather", "achieved": gbs, "peak": ceiling, "unit": "GB/s", "frac": gbs / ceiling,
        "peak_source": f"gather probe, best pattern: mode {best_mode} ({PROBE_MODES[best_mode]}), measured live "
                       "on the same index tensor and latent rows",
        "hbm_peak_frac": gbs / PEAK_HBM_GBS,
        "mfma_achieved_TFLOPs": tflops, "mfma_peak_TFLOPs": PEAK_BF16_TFLOPS, "mfma_frac": tflops / PEAK_BF16_TFLOPS,
        "algorithmic_per_launch": f"{n_sel} (query, selected position) pairs x 1152 B = {gathered:.4g} B; "
                                  f"x 34816 flop = {flop:.4g} flop",
        "launch_ms": sa_ms,
        "probe_GBs": {str(m): round(v[1], 1) for m, v in probe.items()},
    }


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fused_indexer_topk_bf16_L131072_traffic.md")


def kernel_source_sha():
    import hashlib
    h = hashlib.sha256()
    for f in ("indexer.hip", "common.hpp"):
        with open(os.path.join(ROOT, "dsa_lightning_indexer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per fused-kernel launch from the committed counter summary, or
    None when it is missing or was taken on other kernel sources."""
    try:
        text = open(TRAFFIC_FILE).read()
    except OSError:
        return None
    vals = {}
    for line in text.splitlines():
        if line.startswith("- ") and ": " in line:
            k, v = line[2:].split(": ", 1)
            vals[k.strip()] = v.strip().strip("`")
    if vals.get("kernel_source_sha256") != kernel_source_sha():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_run(args, dev):
    if args.profile == "copy":
        n = 1 << 28                                      # 2^28 floats = 1 GiB
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(2):
            torch.mul(src, 1.0, out=dst)
        torch.cuda.synchronize()
        print("profile copy: 2 launches of a 1 GiB read + 1 GiB write kernel", flush=True)
        return
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn
    L = args.prefill_len
    if args.profile == "indexer_fp8":
        c = syn.WORKLOADS["prefill_fp8_L65536"]
        ix = syn.indexer_inputs(B=1, n_q=c["L"], H=c["H"], d=c["d"], dtype=c["dtype"], values=c["values"],
                                w_dist=c["w_dist"], seed=c["seed"], device=dev)
        out = torch.empty((1, c["L"], c["topk"]), dtype=torch.int32, device=dev)
        torch.cuda.synchronize()
        for i in range(3):
            dsa.topk(ix.q, ix.k, ix.w, c["topk"], q_scale=ix.q_scale, k_scale=ix.k_scale, out=out)
            torch.cuda.synchronize()
            print(f"profile indexer_fp8: fused indexer+Top-k L={c['L']} launch {i + 1}/3 done", flush=True)
        return
    if args.profile == "stream":
        B, S = args.decode_batch, args.decode_len
        ix = syn.decode_layer_indexer(0, B=B, S=S, device=dev)
        scores = torch.empty((B, 1, 2048), dtype=torch.int32, device=dev)
        # eviction by a 1 GiB read (written once, long before): it leaves clean lines behind, as
        # the stack does (a large write right before would leave the cache full of dirty lines
        # whose write-back halves the scan's read rate)
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        flush_sum = torch.empty((), dtype=torch.float32, device=dev)
        for _ in range(2):
            torch.sum(flush, dim=0, out=flush_sum)
        nbytes = B * S * (128 + 4)
        # the same bytes as rows of 1152 B read in position order, 64 rows per probe "query"
        rows = nbytes // 1152 // 64 * 64
        table = torch.empty(rows * 1152, dtype=torch.uint8, device=dev).view(rows, 1152)
        table.fill_(1)
        seq = torch.arange(rows, dtype=torch.int32, device=dev).view(-1, 64)
        st = torch.cuda.current_stream()

        def cold(fn, reps=7):
            ts = []
            for _ in range(reps):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.sum(flush, dim=0, out=flush_sum)
                a.record(st)
                fn()
                b.record(st)
                torch.cuda.synchronize()
                ts.append(a.elapsed_time(b))
            return sorted(ts)[len(ts) // 2]
        scan = lambda: dsa.topk(ix.q, ix.k, ix.w, 2048, q_scale=ix.q_scale, k_scale=ix.k_scale,
                                q_pos0=ix.q_pos0, out=scores)
        scan()
        for m in (2, 5):
            dsa.gather_probe(table, seq, m)
        torch.cuda.synchronize()
        res = {"workload": f"decode F layer B={B} x S={S} fp8 K cache ({nbytes} B of keys and scales), cold",
               "decode_indexer_topk_ms": cold(scan)}
        # the streaming read probe over the same number of bytes, over grid sizes and depths
        sbytes = nbytes // 16384 * 16384
        sbuf = torch.ones(sbytes // 4, dtype=torch.int32, device=dev)
        best = None
        for wgs in (512, 1024, 2048, 4096):
            for unroll in (1, 2, 4):
                dsa.stream_probe(sbuf, wgs, unroll)
                ms = cold(lambda: dsa.stream_probe(sbuf, wgs, unroll), reps=5)
                gbs = sbytes / (ms * 1e-3) / 1e9
                res[f"stream_wg{wgs}_u{unroll}_GBs"] = gbs
                if best is None or gbs > best[2]:
                    best = (wgs, unroll, gbs, ms)
        res["stream_best"] = {"workgroups": best[0], "unroll": best[1], "GBs": best[2], "ms": best[3],
                              "bytes": sbytes}
        for m in (2, 5):
            ms = cold(lambda: dsa.gather_probe(table, seq, m))
            res[f"probe_mode{m}_ms"] = ms
            res[f"probe_mode{m}_GBs"] = rows * 1152 / (ms * 1e-3) / 1e9
        print(json.dumps(res), flush=True)
        return
    if args.profile == "decode":
        B, S = args.decode_batch, args.decode_len
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)    # evicts the inputs from L2 and MALL
        for n, l in enumerate((0, 4, 8)):
            ix = syn.decode_layer_indexer(l, B=B, S=S, device=dev)
            sa = syn.decode_layer_sa(l, B=B, S=S, device=dev)
            flush.fill_(n)
            torch.cuda.synchronize()
            idx = dsa.topk(ix.q, ix.k, ix.w, 2048, q_scale=ix.q_scale, k_scale=ix.k_scale, q_pos0=ix.q_pos0)
            dsa.sparse_attn(sa.q, sa.kv, idx, sa.scale, d_v=512)
            torch.cuda.synchronize()
            print(f"profile decode: F layer {l} (B={B}, S={S}) indexer+Top-k and attention done ({n + 1}/3)",
                  flush=True)
            del ix, sa, idx
        return
    if args.profile == "gather":
        ix, sa = syn.prefill_stack_layers(L=L, n_layers=1, seed=4, device=dev)[0]
        idx = dsa.topk(ix.q, ix.k, ix.w, 2048)
        out = torch.empty((1, L, 16, 512), dtype=torch.float32, device=dev)
        dsa.sparse_attn(sa.q, sa.kv, idx, sa.scale, d_v=512, out=out)
        torch.cuda.synchronize()
        reps = max(args.kernel_reps, 3)
        sa_ms = time_batch(lambda: dsa.sparse_attn(sa.q, sa.kv, idx, sa.scale, d_v=512, out=out), reps)
        kv = sa.kv[0, :, 0]
        probe = gather_ceiling(dsa, kv, idx[0], reps)
        for m, (ms, gbs) in probe.items():
            print(f"profile gather: mode {m} ({PROBE_MODES[m]}): {ms:.3f} ms, {gbs:.1f} GB/s", flush=True)
        n_sel = int((idx >= 0).sum().item())
        print(json.dumps({"workload": f"prefill layer L={L}, k=2048, latent rows 1152 B",
                          "roofline_sa": sa_roofline(sa_ms, n_sel, probe)}), flush=True)
        return
    if args.profile == "attn":
        # the step's first prefill layer: its sparse attention over its F layer's index tensor
        ix, sa = syn.prefill_stack_layers(L=L, n_layers=1, seed=4, device=dev)[0]
        idx = dsa.topk(ix.q, ix.k, ix.w, 2048)
        out = torch.empty((1, L, 16, 512), dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        for i in range(3):
            dsa.sparse_attn(sa.q, sa.kv, idx, sa.scale, d_v=512, out=out)
            torch.cuda.synchronize()
            print(f"profile attn: prefill sparse attention L={L} launch {i + 1}/3 done", flush=True)
        return
    ix = syn.prefill_stack_layers(L=L, n_layers=1, seed=4, device=dev, with_sa=False)[0][0]   # the step's first F layer
    out = torch.empty((1, L, 2048), dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    for i in range(3):
        dsa.topk(ix.q, ix.k, ix.w, 2048, out=out)
        torch.cuda.synchronize()
        print(f"profile indexer: fused indexer+Top-k L={L} launch {i + 1}/3 done", flush=True)


def layer_run(args, dev):
    """One prefill F layer of a named workload: fused indexer+Top-k, plus (fp8
    layer) the sparse attention over its index tensor."""
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn
    c = syn.WORKLOADS[args.layer]
    L, topk = c["L"], c["topk"]
    ix = syn.indexer_inputs(B=1, n_q=L, H=c["H"], d=c["d"], dtype=c["dtype"], values=c["values"],
                            w_dist=c["w_dist"], seed=c["seed"], device=dev)
    out = torch.empty((1, L, topk), dtype=torch.int32, device=dev)
    run = lambda: dsa.topk(ix.q, ix.k, ix.w, topk, q_scale=ix.q_scale, k_scale=ix.k_scale, out=out)
    run()
    torch.cuda.synchronize()
    ts = time_launches(run, max(args.kernel_reps, 3))
    ms = sum(ts) / len(ts)
    flop = L * (L + 1) / 2 * 2 * c["H"] * c["d"]
    fp8 = c["dtype"] == syn.FP8
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    rec = {"metric": "indexer+Top-k score-pairs/s", "value": L * (L + 1) / 2 / (ms * 1e-3), "unit": "score-pairs/s",
           "n_gpus": 1, "higher_is_better": True, "ms_per_launch": ms, "launches": len(ts),
           "dtype": c["dtype"], "data": "synthetic", "config": {"workload": c["name"]},
           "roofline": {"bound": "mfma", "achieved": flop / (ms * 1e-3) / 1e12, "peak": peak, "unit": "TFLOP/s",
                        "frac": flop / (ms * 1e-3) / 1e12 / peak,
                        "algorithmic_per_launch": f"{L * (L + 1) // 2} causal pairs x {2 * c['H'] * c['d']} flop"}}
    log(f"{args.layer}: fused indexer+Top-k {ms:.3f} ms/launch")
    if fp8:
        sa = syn.sa_inputs(B=1, n_q=L, n_k=L, heads=c["sa_heads"], d_qk=c["sa_d_qk"], d_v=c["sa_d_v"], seed=c["seed"],
                           device=dev)
        o = torch.empty((1, L, c["sa_heads"], c["sa_d_v"]), dtype=torch.float32, device=dev)
        sa_run = lambda: dsa.sparse_attn(sa.q, sa.kv, out, sa.scale, d_v=sa.d_v, out=o)
        sa_run()
        torch.cuda.synchronize()
        t_sa = time_launches(sa_run, max(args.kernel_reps, 3))
        sa_ms = sum(t_sa) / len(t_sa)
        gathered = int((out >= 0).sum().item()) * c["sa_d_qk"] * 2
        rec["sparse_attn"] = {"ms_per_launch": sa_ms, "gathered_bytes": gathered,
                              "gathered_TBps": gathered / (sa_ms * 1e-3) / 1e12,
                              "tokens_per_s": L / (sa_ms * 1e-3)}
        log(f"{args.layer}: sparse attention {sa_ms:.3f} ms/launch")
    print(json.dumps(rec), flush=True)


def distill_run(args, dev):
    """Distillation loss + backward over one F layer's index tensor: kernel time
    with HIP events on the launch stream, algorithmic work per (query, selected
    entry) pair, and the oracle timed on a sample of rows."""
    import numpy as np
    import oracle
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn
    from threadpoolctl import threadpool_info
    L, topk, r, H, d = 16384, 2048, 4, 64, 128
    ix = syn.indexer_inputs(B=1, n_q=L, H=H, d=d, dtype=syn.BF16, values="normal", w_dist="u8", seed=2,
                            device=dev)
    idx = syn.random_sorted_indices(B=1, n_q=L, topk=topk, seed=3, device=dev)
    T = syn.teacher_weights(idx, r=r, seed=4, device=dev)
    pairs = int((idx >= 0).sum().item())
    for _ in range(2):
        dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T)
    torch.cuda.synchronize()
    ts = time_launches(lambda: dsa.indexer_distill(ix.q, ix.k, ix.w, idx, T), max(args.kernel_reps, 3))
    ms = sum(ts) / len(ts)
    flop_alg = pairs * 3 * 2 * H * d                  # scores, dq, dk: one contraction over d each
    flop_done = pairs * 7 * 2 * H * d                 # + the pass-2 score recompute (two layouts) + hi/lo halves
    log(f"distillation L={L} k={topk} r={r}: {ms:.3f} ms, {pairs / (ms * 1e-3):.4g} pairs/s")
    # the oracle on a bounded sample of rows
    threads = max([dd.get("num_threads", 1) for dd in threadpool_info()] + [1])
    qraw = ix.q[0].detach().cpu().view(torch.int16).numpy().view(np.uint16)
    k64 = oracle.dequantize(ix.k[0].detach().cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
    w64 = ix.w[0].detach().cpu().double().numpy()
    idx_np = idx[0].cpu().numpy()
    T_np = T[:, 0].cpu().double().numpy()
    rng = np.random.default_rng(0)
    done = rows = 0
    t0 = time.perf_counter()
    for i in rng.permutation(L):
        q64 = oracle.dequantize(qraw[i:i + 1], "bf16")
        oracle.indexer_distill(q64, k64, w64[i:i + 1], idx_np[i:i + 1], T_np[:, i:i + 1], q_pos0=int(i))
        done += int((idx_np[i] >= 0).sum())
        rows += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = time.perf_counter() - t0
    rec = {
        "metric": "distillation loss + backward, (query, selected entry) pairs/s",
        "value": pairs / (ms * 1e-3), "unit": "pairs/s", "n_gpus": 1, "higher_is_better": True,
        "ms_per_call": ms, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"one F layer: L={L} queries, H={H}, d={d}, k={topk} selected entries per row, "
                               f"{r} teacher distributions", "pairs": pairs},
        "roofline": {"bound": "mfma", "achieved": flop_alg / (ms * 1e-3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": flop_alg / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                     "algorithmic_per_call": f"{pairs} pairs x 3 x {2 * H * d} flop = {flop_alg:.4g} flop",
                     "executed_mfma_flop": f"{flop_done:.4g}",
                     "key_bytes_gathered": pairs * d * 2 * 2, "dk_float_atomics": pairs * d,
                     "dk_float_atomics_per_s": pairs * d / (ms * 1e-3)},
        "cpu_baseline": {"value": done / dt, "unit": "pairs/s", "cores": int(threads), "kind": "oracle",
                         "sample": f"{rows} random rows, {done} pairs in {dt:.1f} s, float64 NumPy"},
    }
    print(json.dumps(rec), flush=True)


def similarity_run(args, dev):
    """Similarity matrix + pattern search ([IC-SUMMARY] Appendix C) on a drifting
    calibration stack: whole-matrix time with HIP events, the per-kernel
    durations of its attention and cosine launches, the host dynamic program,
    and the oracle timed on a sample of rows of one matrix entry."""
    import numpy as np
    import oracle
    from oracle import pattern_search as ps
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn
    from threadpoolctl import threadpool_info
    L, n, topk = args.similarity_len, args.similarity_layers, 2048
    layers, jumps = syn.drift_stack(n_layers=n, n_q=L, seed=6, device=dev)
    ixs = [dict(q=ix.q, k=ix.k, w=ix.w) for ix, _ in layers]
    sas = [dict(q=sa.q, kv=sa.kv, scale=sa.scale, d_v=sa.d_v) for _, sa in layers]
    idx = [torch.empty((1, L, topk), dtype=torch.int32, device=dev) for _ in range(n)]
    ws = torch.empty(dsa.similarity_matrix_workspace_size(ixs, sas, topk), dtype=torch.uint8, device=dev)
    for _ in range(max(args.warmup, 1)):
        S, _ = dsa.similarity_matrix(ixs, sas, topk, idx_out=idx, ws=ws)
    torch.cuda.synchronize()
    ts = time_launches(lambda: dsa.similarity_matrix(ixs, sas, topk, idx_out=idx, ws=ws), max(args.steps, 1))
    ms = sum(ts) / len(ts)
    S, _ = dsa.similarity_matrix(ixs, sas, topk, idx_out=idx, ws=ws)
    Sh = S.cpu().numpy()
    # per-kernel durations of the launches the matrix is made of
    sa = layers[1][1]
    o_own = dsa.sparse_attn(sa.q, sa.kv, idx[1], sa.scale, d_v=sa.d_v)
    o_re = torch.empty_like(o_own)
    reps = max(args.kernel_reps, 3)
    flat_own, flat_re = o_own.reshape(L, -1), o_re.reshape(L, -1)
    row_cos = torch.empty(L, dtype=torch.float32, device=dev)
    sa_ms = time_batch(lambda: dsa.sparse_attn(sa.q, sa.kv, idx[0], sa.scale, d_v=sa.d_v, out=o_re), reps)
    cos_ms = time_batch(lambda: dsa.row_cosine(flat_own, flat_re, row_cos=row_cos), 4 * reps)   # + row mean
    sel = int((idx[0] >= 0).sum().item())
    gather = sel * 576 * 2
    cos_bytes = 2 * o_own.numel() * 4
    pairs = n * (n - 1) // 2
    # dynamic program at the printed retention counts
    pats = {}
    for m in (24, 12, 7):
        t0 = time.perf_counter()
        pat, score = dsa.pattern_search(Sh, m)
        dp_us = (time.perf_counter() - t0) * 1e6
        r = {24: 2, 12: 4, 7: 8}[m]
        uni = "".join("F" if i % r == 0 else "S" for i in range(n))
        pats[str(m)] = {"pattern": pat, "score": score, "dp_us": dp_us,
                        "uniform_1/%d" % r: {"pattern": uni, "F": uni.count("F"),
                                             "score": ps.pattern_objective(Sh, uni)}}
    log(f"similarity matrix {n} layers L={L}: {ms:.1f} ms; attention {sa_ms:.3f} ms, cosine {cos_ms * 1e3:.1f} us")
    # the oracle: one matrix entry (layer 1 vs layer 0) on a bounded sample of rows
    threads = max([dd.get("num_threads", 1) for dd in threadpool_info()] + [1])

    def f64(t):
        return oracle.dequantize(t.detach().cpu().view(torch.int16).numpy().view(np.uint16), "bf16")
    ix0, ix1 = layers[0][0], layers[1][0]
    k0, k1 = f64(ix0.k[0]), f64(ix1.k[0])
    w64 = ix0.w[0].detach().cpu().double().numpy()
    KV = f64(sa.kv[0])
    rng = np.random.default_rng(0)
    rows = 0
    t0 = time.perf_counter()
    for i in ([] if args.no_cpu_baseline else rng.permutation(L)):
        q64 = f64(ix0.q[0, i:i + 1])
        T0, _, _ = oracle.indexer_topk(q64, k0, w64[i:i + 1], topk, q_pos0=int(i))
        T1, _, _ = oracle.indexer_topk(q64, k1, w64[i:i + 1], topk, q_pos0=int(i))
        Q = f64(sa.q[0, i:i + 1])
        own = oracle.sparse_attn(Q, KV, KV[..., :sa.d_v], T1, sa.scale)
        other = oracle.sparse_attn(Q, KV, KV[..., :sa.d_v], T0, sa.scale)
        ps.row_cosine(own, other)
        rows += 1
        if time.perf_counter() - t0 >= args.cpu_seconds:
            break
    dt = max(time.perf_counter() - t0, 1e-9)
    rec = {
        "metric": "similarity-matrix (calibration row, layer pair) entries/s",
        "value": L * pairs / (ms * 1e-3), "unit": "row-pairs/s", "n_gpus": 1, "higher_is_better": True,
        "ms_per_matrix": ms, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"{n}-layer calibration prefill L={L} (drifting bf16 indexer keys, 64 heads x 128, "
                               f"k={topk}; 16-head MLA attention 576/512)", "layer_pairs": pairs,
                   "jump_layers": [l for l, j in enumerate(jumps) if j]},
        "kernels": {"sparse_attn_ms": sa_ms, "sparse_attn_gathered_TBps": gather / (sa_ms * 1e-3) / 1e12,
                    "row_cosine_plus_mean_us": cos_ms * 1e3, "row_cosine_GBps": cos_bytes / (cos_ms * 1e-3) / 1e9,
                    "launches_per_matrix": {"topk": n, "sparse_attn": n - 1 + pairs, "row_cosine+mean": pairs}},
        "roofline": {"bound": "hbm", "kernel": "sa_mla1_kernel (one layer pair)",
                     "achieved": gather / (sa_ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gather / (sa_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                     "algorithmic_per_launch": f"{sel} selected (row, position) pairs x 1152 B = {gather:.4g} B",
                     "traffic": None},
        "row_cosine_roofline": {"bound": "hbm", "achieved": cos_bytes / (cos_ms * 1e-3) / 1e9,
                                "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                "frac": cos_bytes / (cos_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                "algorithmic_per_launch": f"2 x {L} rows x {o_own[0].numel()} fp32 = {cos_bytes} B"},
        "patterns": pats,
        "cpu_baseline": None if args.no_cpu_baseline else {
            "value": rows / dt, "unit": "row-pairs/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} random rows of entry S[1, 0] (both layers' indexer + Top-k, two attention rows, "
                      f"one cosine) in {dt:.1f} s, float64 NumPy"},
    }
    print(json.dumps(rec), flush=True)


def mli_run(args, dev):
    """Plain IndexCache against the multi-layer-indexer shift at equal retention
    (same kernels, same inputs): stack time with HIP events on the attention
    stream, which the shifted loop joins with its indexer stream at the end."""
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn
    topk = 2048
    side = torch.cuda.Stream(device=dev)
    res = {"metric": "stack time, plain IndexCache vs the multi-layer-indexer shift", "unit": "ms",
           "data": "synthetic"}

    def measure(pattern, specs, reps):
        ws = torch.empty(max(dsa.indexcache_forward_workspace_size(pattern, specs, topk), 256),
                         dtype=torch.uint8, device=dev)
        ws2 = torch.empty(max(dsa.indexcache_forward_mli_workspace_size(pattern, specs, topk), 256),
                          dtype=torch.uint8, device=dev)
        runs = {"indexcache": lambda: dsa.indexcache_forward(pattern, specs, topk, ws=ws),
                "mli_two_streams": lambda: dsa.indexcache_forward_mli(pattern, specs, topk, index_stream=side,
                                                                      ws=ws2),
                "mli_one_stream": lambda: dsa.indexcache_forward_mli(pattern, specs, topk, ws=ws2)}
        for f in runs.values():
            f()
        torch.cuda.synchronize()
        out = {}
        # interleaved repetitions so that clock drift hits every variant alike
        times = {k: [] for k in runs}
        for _ in range(reps):
            for k, f in runs.items():
                times[k].append(time_launches(f, 1)[0])
        for k, t in times.items():
            t = sorted(t)
            out[k] = {"median_ms": t[len(t) // 2], "min_ms": t[0]}
        base = out["indexcache"]["median_ms"]
        for k in out:
            out[k]["speedup_vs_indexcache"] = base / out[k]["median_ms"]
        return out

    B, S, NL = args.decode_batch, args.decode_len, args.decode_layers
    pattern_d, dspecs = decode_stack(dsa, syn, B, S, NL, topk, dev)
    torch.cuda.synchronize()
    r = measure(pattern_d, dspecs, 9)
    log(f"mli decode: " + ", ".join(f"{k} {v['median_ms']:.3f} ms" for k, v in r.items()))
    res["decode"] = {"workload": f"decode stack B={B} x S={S} x {NL} layers {pattern_d.count('F')} F (FSSS), fp8 "
                                 f"indexer K cache, k={topk}", "pattern": pattern_d, "results": r}
    del dspecs
    torch.cuda.empty_cache()
    L = args.prefill_len
    pattern_p = "FSSSFSSS"
    _, pspecs = prefill_stack(dsa, syn, L, pattern_p, topk, dev)
    torch.cuda.synchronize()
    r = measure(pattern_p, pspecs, 3)
    log(f"mli prefill: " + ", ".join(f"{k} {v['median_ms']:.1f} ms" for k, v in r.items()))
    res["prefill"] = {"workload": f"prefill stack L={L} x 8 layers {pattern_p}, bf16 indexer, k={topk}",
                      "pattern": pattern_p, "results": r}
    print(json.dumps(res), flush=True)


def sweep_run(args, dev):
    """Stack time per sharing pattern (same kernels and driver as the bench line)."""
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn
    topk = 2048
    res = {"metric": "stack time per sharing pattern (retention sweep)", "unit": "ms", "data": "synthetic"}

    def run(pattern, specs, reps):
        ws = torch.empty(max(dsa.indexcache_forward_workspace_size(pattern, specs, topk), 256),
                         dtype=torch.uint8, device=dev)
        dsa.indexcache_forward(pattern, specs, topk, ws=ws)
        torch.cuda.synchronize()
        t = time_launches(lambda: dsa.indexcache_forward(pattern, specs, topk, ws=ws), reps)
        return sum(t) / len(t)

    # decode stack: every layer has attention inputs; indexer inputs for any layer a pattern makes F
    B, S, NL = args.decode_batch, args.decode_len, args.decode_layers
    sa = [syn.decode_layer_sa(l, B=B, S=S, device=dev) for l in range(NL)]
    ix = [syn.decode_layer_indexer(l, B=B, S=S, device=dev) for l in range(NL)]
    outs = [torch.empty((B, 1, 16, 512), dtype=torch.float32, device=dev) for _ in range(NL)]
    idxs = [torch.empty((B, 1, topk), dtype=torch.int32, device=dev) for _ in range(NL)]
    torch.cuda.synchronize()
    log("sweep: decode inputs ready")

    def dspecs(pattern):
        specs = []
        for l, c in enumerate(pattern):
            spec = {"sa": {"q": sa[l].q, "kv": sa[l].kv, "scale": sa[l].scale, "d_v": 512, "out": outs[l]}}
            if c == "F":
                x = ix[l]
                spec["ix"] = {"q": x.q, "k": x.k, "w": x.w, "q_scale": x.q_scale, "k_scale": x.k_scale,
                              "q_pos0": x.q_pos0}
                spec["idx_out"] = idxs[l]
            specs.append(spec)
        return specs

    pats = [("all-F", "F" * NL)]
    for r, name in ((2, "1/2"), (4, "1/4"), (8, "1/8")):
        pats.append((f"uniform {name}", syn.uniform_pattern(NL, r)))
        if NL == 47:
            pats.append((f"searched {name}", syn.SEARCHED_PATTERNS_47[name]))
    rows = []
    for name, pat in pats:
        ms = run(pat, dspecs(pat), 5)
        rows.append({"pattern": name, "F_layers": pat.count("F"), "ms": ms})
        log(f"sweep decode {name:13s} F={pat.count('F'):2d}: {ms:.3f} ms")
    base = rows[0]["ms"]
    for r in rows:
        r["speedup_vs_all_F"] = base / r["ms"]
    res["decode"] = {"workload": f"decode stack B={B} x S={S} x {NL} layers, fp8 indexer K cache, k={topk}",
                     "rows": rows}
    del sa, ix, outs, idxs
    torch.cuda.empty_cache()

    # prefill stack
    L = args.prefill_len
    layers = syn.prefill_stack_layers(L=L, n_layers=8, seed=4, device=dev)
    pouts = [torch.empty((1, L, 16, 512), dtype=torch.float32, device=dev) for _ in range(8)]
    pidx = [torch.empty((1, L, topk), dtype=torch.int32, device=dev) for _ in range(8)]
    torch.cuda.synchronize()
    log("sweep: prefill inputs ready")

    def pspecs(pattern):
        specs = []
        for l, c in enumerate(pattern):
            x, a = layers[l]
            spec = {"sa": {"q": a.q, "kv": a.kv, "scale": a.scale, "d_v": 512, "out": pouts[l]}}
            if c == "F":
                spec["ix"] = {"q": x.q, "k": x.k, "w": x.w}
                spec["idx_out"] = pidx[l]
            specs.append(spec)
        return specs

    rows = []
    for name, pat in (("all-F", "FFFFFFFF"), ("uniform 1/2", "FSFSFSFS"), ("uniform 1/4", "FSSSFSSS"),
                      ("uniform 1/8", "FSSSSSSS")):
        ms = run(pat, pspecs(pat), 2)
        rows.append({"pattern": name, "F_layers": pat.count("F"), "ms": ms})
        log(f"sweep prefill {name:13s} F={pat.count('F')}: {ms:.1f} ms")
    base = rows[0]["ms"]
    for r in rows:
        r["speedup_vs_all_F"] = base / r["ms"]
    res["prefill"] = {"workload": f"prefill stack L={L} x 8 layers, bf16 indexer, k={topk}", "rows": rows}
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.profile:
        profile_run(args, dev)
        return
    if args.sweep:
        sweep_run(args, dev)
        return
    if args.mli:
        mli_run(args, dev)
        return
    if args.distill:
        distill_run(args, dev)
        return
    if args.similarity:
        similarity_run(args, dev)
        return
    if args.layer:
        layer_run(args, dev)
        return
    import dsa_lightning_indexer_amd as dsa
    from synth import inputs as syn

    topk = 2048
    L = args.prefill_len
    pattern_p = "FSSSFSSS"
    t0 = time.time()
    players, pspecs = prefill_stack(dsa, syn, L, pattern_p, topk, dev)
    B, S = args.decode_batch, args.decode_len
    pattern_d, dspecs = decode_stack(dsa, syn, B, S, args.decode_layers, topk, dev)
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f} s; "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB resident")

    ws_p = torch.empty(max(dsa.indexcache_forward_workspace_size(pattern_p, pspecs, topk), 256),
                       dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(dsa.indexcache_forward_workspace_size(pattern_d, dspecs, topk), 256),
                       dtype=torch.uint8, device=dev)

    def step():
        dsa.indexcache_forward(pattern_p, pspecs, topk, ws=ws_p)
        dsa.indexcache_forward(pattern_d, dspecs, topk, ws=ws_d)

    for i in range(args.warmup):
        step()
        torch.cuda.synchronize()
        log(f"warmup step {i + 1}/{args.warmup} done")
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    e0.record(st)
    for i in range(args.steps):
        step()
    e1.record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    log(f"timed {args.steps} steps: {ms_step:.2f} ms/step (wall {wall:.2f} s)")

    # phase times (same calls, events per phase)
    ms_prefill = sum(time_launches(lambda: dsa.indexcache_forward(pattern_p, pspecs, topk, ws=ws_p), 2)) / 2
    ms_decode = sum(time_launches(lambda: dsa.indexcache_forward(pattern_d, dspecs, topk, ws=ws_d), 3)) / 3
    # the same decode layer loop captured once in a HIP graph and replayed
    dgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(dgraph):
        dsa.indexcache_forward(pattern_d, dspecs, topk, ws=ws_d)
    dgraph.replay()
    torch.cuda.synchronize()
    ms_decode_graph = sum(time_launches(dgraph.replay, 5)) / 5
    log(f"decode stack: {ms_decode:.3f} ms eager, {ms_decode_graph:.3f} ms as a HIP graph")

    # dominant kernel: the fused indexer+Top-k launch of an F prefill layer
    ix0 = players[0][0]
    idx_tmp = pspecs[0]["idx_out"]
    ktimes = time_launches(lambda: dsa.topk(ix0.q, ix0.k, ix0.w, topk, out=idx_tmp), args.kernel_reps)
    k_ms = sum(ktimes) / len(ktimes)
    pairs_layer = L * (L + 1) // 2
    flop_layer = pairs_layer * 2 * 64 * 128
    achieved_tflops = flop_layer / (k_ms * 1e-3) / 1e12
    log(f"fused indexer+Top-k L={L}: {k_ms:.2f} ms/launch, {achieved_tflops:.1f} TFLOP/s")
    traffic = measured_traffic() if L == 131072 else None

    # decode F-layer indexer+Top-k (scan + select) and one decode attention layer
    dF = [i for i, c in enumerate(pattern_d) if c == "F"][0]
    dix = dspecs[dF]["ix"]
    dtimes = time_launches(lambda: dsa.topk(dix["q"], dix["k"], dix["w"], topk, q_scale=dix["q_scale"],
                                            k_scale=dix["k_scale"], q_pos0=dix["q_pos0"],
                                            out=dspecs[dF]["idx_out"]), args.kernel_reps)
    d_ms = sum(dtimes) / len(dtimes)
    scan_bytes = B * S * (128 + 4)

    # prefill sparse attention (layer 1 over layer 0's index tensor) and its gather ceiling
    sa1 = pspecs[1]["sa"]
    idx0 = pspecs[0]["idx_out"]
    sa_ms = sum(time_launches(lambda: dsa.sparse_attn(sa1["q"], sa1["kv"], idx0, sa1["scale"], d_v=512,
                                                      out=sa1["out"]), args.kernel_reps)) / args.kernel_reps
    n_sel = int((idx0 >= 0).sum().item())
    probe = gather_ceiling(dsa, sa1["kv"][0, :, 0], idx0[0], max(args.kernel_reps, 3))
    roof_sa = sa_roofline(sa_ms, n_sel, probe)
    log(f"prefill sparse attention: {sa_ms:.2f} ms/launch, {roof_sa['achieved']:.0f} GB/s gathered "
        f"({roof_sa['frac']:.3f} of the probe's {roof_sa['peak']:.0f} GB/s), MFMA {roof_sa['mfma_frac']:.3f}")

    n_f_p = pattern_p.count("F")
    n_f_d = pattern_d.count("F")
    pairs_step = n_f_p * pairs_layer + n_f_d * B * S
    sa_tokens_step = len(pattern_p) * L + len(pattern_d) * B
    value = pairs_step / (ms_step * 1e-3)

    rec = {
        "metric": METRIC,
        "value": value,
        "unit": "score-pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"IndexCache DSA step: prefill stack L={L} x {len(pattern_p)} layers {pattern_p} "
                        f"(bf16 indexer H_I=64 d_I=128, k={topk}, MLA sparse attention 16 heads 576/512) + "
                        f"decode stack B={B} x S={S} x {len(pattern_d)} layers FSSS ({n_f_d} F, fp8 indexer "
                        f"K cache, k={topk})",
            "prefill_len": L, "decode_batch": B, "decode_len": S, "topk": topk,
        },
        "sparse_attn_tokens_per_s": sa_tokens_step / (ms_step * 1e-3),
        "phases": {
            "prefill_stack_ms": ms_prefill,
            "decode_stack_ms": ms_decode,
            "decode_stack_graph_ms": ms_decode_graph,
            "decode_tokens_per_s": B / (ms_decode * 1e-3),
            "prefill_indexer_topk_ms_per_F_layer": k_ms,
            "decode_indexer_topk_ms_per_F_layer": d_ms,
            "decode_scan_select_hbm_GBs": scan_bytes / (d_ms * 1e-3) / 1e9,
        },
        "roofline": {
            "kernel": "fused indexer+Top-k (prefill, bf16)",
            "bound": "mfma",
            "achieved": achieved_tflops,
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": achieved_tflops / PEAK_BF16_TFLOPS,
            "traffic": traffic,
            "traffic_unit": "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "algorithmic_per_launch": f"{pairs_layer} causal pairs x 16384 flop = {flop_layer:.4g} flop",
            "launch_ms": k_ms,
        },
        "roofline_sa": roof_sa,
    }

    if not args.no_report:
        # S-vs-F: the same stack with every layer F, plus the all-F overlap matrix
        pattern_f = "F" * len(pattern_p)
        fspecs = []
        for l, (ix, sa) in enumerate(players):
            fspecs.append({"ix": {"q": ix.q, "k": ix.k, "w": ix.w}, "sa": pspecs[l]["sa"],
                           "idx_out": pspecs[l].get("idx_out") if pattern_p[l] == "F" else
                           torch.empty((1, L, topk), dtype=torch.int32, device=dev)})
        ws_f = torch.empty(max(dsa.indexcache_forward_workspace_size(pattern_f, fspecs, topk), 256),
                           dtype=torch.uint8, device=dev)
        ms_allf = time_launches(lambda: dsa.indexcache_forward(pattern_f, fspecs, topk, ws=ws_f), 1)[0]
        rows = L - topk + 1
        M = [[1.0] * len(pattern_f) for _ in pattern_f]
        for i in range(len(pattern_f)):
            for j in range(i + 1, len(pattern_f)):
                tot = dsa.index_overlap(fspecs[i]["idx_out"][0, topk - 1:], fspecs[j]["idx_out"][0, topk - 1:],
                                        topk)
                M[i][j] = M[j][i] = int(tot.item()) / (rows * topk)
        rec["report"] = {
            "all_F_stack_ms": ms_allf,
            "FSSSFSSS_stack_ms": ms_prefill,
            "stack_speedup": ms_allf / ms_prefill,
            "F_layer_ms": k_ms + sa_ms,
            "S_layer_ms": sa_ms,
            "S_over_F_layer_speedup": (k_ms + sa_ms) / sa_ms,
            "sparse_attn_prefill_ms_per_layer": sa_ms,
            "sparse_attn_gathered_GBs": L * topk * 1152 / (sa_ms * 1e-3) / 1e9,
            "overlap_matrix_all_F": [[round(x, 4) for x in r] for r in M],
        }
        log(f"all-F stack {ms_allf:.1f} ms vs FSSSFSSS {ms_prefill:.1f} ms; SA {sa_ms:.2f} ms/layer")

    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        rec["cpu_baseline"] = cpu_baseline(players[0][0], topk, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
