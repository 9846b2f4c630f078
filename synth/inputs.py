"""Seeded synthetic workloads with the shapes and value distributions of the five
configurations this library is measured on.

Everything here is random-number drawing and storage-format conversion
(bf16 rounding, OCP fp8 e4m3fn encoding with per-vector ``amax/448`` scales).
No step of the indexer, Top-k, sparse attention or layer driver is computed
here; both the HIP path and the CPU oracle consume exactly these tensors.

Shapes follow the library's layouts:
  indexer q  [B, n_q, H, d]   (+ q_scale [B, n_q, H] fp32 for fp8)
  indexer k  [B, n_k, d]      (+ k_scale [B, n_k]   fp32 for fp8)
  indexer w  [B, n_q, H]      fp32
  attention Q  [B, n_q, heads, d_qk]
  attention KV [B, n_k, kv_heads, d_qk]   (MLA latent: V = first d_v columns)
  attention V  [B, n_k, kv_heads, d_v] or None
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import torch

F32, BF16, FP8 = "f32", "bf16", "fp8"
FP8_MAX = 448.0

__all__ = [
    "F32", "BF16", "FP8", "IndexerInputs", "SAInputs", "generator",
    "fp8_encode_vectors", "indexer_inputs", "sa_inputs", "random_sorted_indices",
    "prefill_stack_layers", "decode_layer_indexer", "decode_layer_sa", "WORKLOADS", "DECODE_PATTERN",
    "uniform_pattern", "SEARCHED_PATTERNS_47", "drift_stack",
]


def generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(int(seed))
    return g


def fp8_encode_vectors(x: torch.Tensor):
    """Encode fp32 ``x`` to e4m3fn codes with one fp32 scale per vector along the
    last dim: scale = amax/448, code = RNE(x/scale) saturated to +-448."""
    amax = x.abs().amax(dim=-1, keepdim=True).float()
    scale = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    codes = (x.float() / scale).clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn)
    return codes, scale.squeeze(-1).contiguous()


@dataclasses.dataclass
class IndexerInputs:
    dtype: str
    q: torch.Tensor
    k: torch.Tensor
    w: torch.Tensor
    q_scale: Optional[torch.Tensor] = None
    k_scale: Optional[torch.Tensor] = None
    q_pos0: int = 0

    @property
    def shape(self):
        B, n_q, H, d = self.q.shape
        return B, n_q, self.k.shape[1], H, d


@dataclasses.dataclass
class SAInputs:
    dtype: str
    q: torch.Tensor
    kv: torch.Tensor
    v: Optional[torch.Tensor]
    d_v: int
    scale: float


def _draw(g, shape, device, values: str):
    if values == "int":
        return torch.randint(-3, 4, shape, generator=g, device=device).float()
    if values == "normal":
        return torch.randn(shape, generator=g, device=device)
    raise ValueError(values)


def _draw_w(g, shape, device, w_dist: str):
    if w_dist == "pow2":   # {0.25, 0.5, 1, 2}
        e = torch.randint(0, 4, shape, generator=g, device=device).float()
        return torch.exp2(e - 2.0)
    if w_dist == "u8":     # U(0,1)/8
        return torch.rand(shape, generator=g, device=device) / 8.0
    if w_dist == "normal":
        return torch.randn(shape, generator=g, device=device)
    if w_dist == "pm_pow2":  # signed {+-0.25, +-0.5, +-1, +-2}
        e = torch.randint(0, 4, shape, generator=g, device=device).float()
        s = torch.randint(0, 2, shape, generator=g, device=device).float() * 2 - 1
        return s * torch.exp2(e - 2.0)
    raise ValueError(w_dist)


def _store(x: torch.Tensor, dtype: str, values: str):
    """Store fp32 draws as ``dtype``.  Integer draws keep scale 1.0 for fp8 so
    every code is exact."""
    if dtype == F32:
        return x.contiguous(), None
    if dtype == BF16:
        return x.to(torch.bfloat16).contiguous(), None
    if dtype == FP8:
        if values == "int":
            return x.to(torch.float8_e4m3fn).contiguous(), torch.ones(
                x.shape[:-1], dtype=torch.float32, device=x.device)
        return fp8_encode_vectors(x)
    raise ValueError(dtype)


def indexer_inputs(*, B=1, n_q, n_k=None, H=64, d=128, q_pos0=0, dtype=BF16,
                   values="normal", w_dist="u8", seed=0, device="cpu",
                   k_source: Optional[torch.Tensor] = None) -> IndexerInputs:
    """One F layer's indexer inputs.  ``n_k`` defaults to ``q_pos0 + n_q``
    (prefill: every query's causal predecessors are present)."""
    if n_k is None:
        n_k = q_pos0 + n_q
    g = generator(seed, device)
    qf = _draw(g, (B, n_q, H, d), device, values)
    if k_source is None:
        kf = _draw(g, (B, n_k, d), device, values)
    else:
        kf = k_source
    w = _draw_w(g, (B, n_q, H), device, w_dist).float().contiguous()
    q, qs = _store(qf, dtype, values)
    del qf
    k, ks = _store(kf, dtype, values) if k_source is None else (k_source, None)
    return IndexerInputs(dtype=dtype, q=q, k=k, w=w, q_scale=qs, k_scale=ks, q_pos0=q_pos0)


def sa_inputs(*, B=1, n_q, n_k, heads=16, kv_heads=1, d_qk=576, d_v=512,
              latent=True, dtype=BF16, seed=0, device="cpu", scale=None) -> SAInputs:
    """Sparse-attention inputs, Q/K/V ~ N(0,1).  ``latent`` stores one row of
    ``d_qk`` values per (token, kv head) whose first ``d_v`` columns are V."""
    g = generator(seed, device)
    tdt = torch.float32 if dtype == F32 else torch.bfloat16
    q = torch.randn((B, n_q, heads, d_qk), generator=g, device=device).to(tdt)
    kv = torch.randn((B, n_k, kv_heads, d_qk), generator=g, device=device).to(tdt)
    v = None if latent else torch.randn((B, n_k, kv_heads, d_v), generator=g,
                                        device=device).to(tdt)
    if scale is None:
        scale = 1.0 / float(d_qk) ** 0.5
    return SAInputs(dtype=dtype, q=q.contiguous(), kv=kv.contiguous(),
                    v=None if v is None else v.contiguous(), d_v=d_v, scale=scale)


def random_sorted_indices(*, B=1, n_q, topk, q_pos0=0, n_k=None, seed=0, device="cpu"):
    """Index tensors with the structure of a Top-k result: row (b, i) holds
    min(topk, t+1) distinct positions of [0, t] (t = q_pos0 + i, capped at
    n_k-1) in ascending order, then -1 padding."""
    g = generator(seed, device)
    t = torch.arange(n_q, device=device) + q_pos0
    if n_k is not None:
        t = t.clamp(max=n_k - 1)
    m = (t + 1).view(1, n_q, 1)                      # candidates per row
    u, _ = torch.rand((B, n_q, topk), generator=g, device=device).sort(dim=-1)
    j = torch.arange(topk, device=device).view(1, 1, topk)
    span = (m - topk + 1).clamp(min=1)
    sampled = (u * span).floor().long().clamp(max=span - 1) + j   # strictly increasing
    dense = j.expand(B, n_q, topk)
    idx = torch.where(m > topk, sampled, torch.where(j < m, dense, torch.full_like(dense, -1)))
    return idx.to(torch.int32).contiguous()


def teacher_weights(idx: torch.Tensor, *, r: int, seed=0, device="cpu"):
    """Synthetic teacher distributions for the distillation loss: r random
    probability vectors per index row, [r, B, n_q, topk] fp32, over the row's
    entries that hold a position (>= 0); zero on the -1 padding.  Weights are
    U(0,1)^4 (a few entries carry most of the mass, as attention does),
    normalised per row."""
    g = generator(seed, device)
    u = torch.rand((r,) + tuple(idx.shape), generator=g, device=device) ** 4
    u = u * (idx >= 0).to(u.dtype).unsqueeze(0)
    return (u / u.sum(dim=-1, keepdim=True).clamp(min=1e-30)).contiguous()


def uniform_pattern(n_layers: int, r: int) -> str:
    """Keep every r-th indexer (F), share the rest (S): FSSSFSSS... for r=4."""
    return "".join("F" if i % r == 0 else "S" for i in range(n_layers))


DECODE_PATTERN = uniform_pattern(47, 4)   # F at layers 1,5,...,45 (1-based): 12 F layers

# Greedy-searched sharing patterns of the 47-layer GLM-4.7-Flash 30B DSA model at
# retention 1/2, 1/4 and 1/8 ([IC-SUMMARY] Appendix B, "搜索到的模式"), as printed
# (47 characters each): data for the pattern driver (layer l is F or S), not
# method arithmetic.
SEARCHED_PATTERNS_47 = {
    "1/2": "FSFSFSSSSFSFFFFSFFSSFFSFFFSSFFSSFSSSSFSFFFSFSSF",
    "1/4": "FSFSFSSSSFSSSFSSFFSSFSSFSSSSFSSSFSSSSFSSSSSSSSS",
    "1/8": "FSSSFSSSSSSSSFSSSFSSSSSFSSSSFSSSSSSSSFSSSSSSSSS",
}


# --- named workloads ---------------------------------------------------------
WORKLOADS = {
    "tiny_fp32_L512": dict(name="tiny fp32 F layer L=512 H_I=4 d_I=32 k=64", L=512, H=4, d=32, dtype=F32,
            values="int", w_dist="pow2", topk=64, sa_heads=4, sa_kv_heads=4, sa_d=64, seed=1),
    "prefill_bf16_L16384": dict(name="bf16 prefill indexer L=16384 H_I=64 d_I=128 k=2048", L=16384, H=64, d=128,
            dtype=BF16, values="normal", w_dist="u8", topk=2048, seed=2),
    "prefill_fp8_L65536": dict(name="fp8 prefill indexer+SA L=65536 H_I=64 d_I=128 k=2048, SA 16 heads 576/512",
            L=65536, H=64, d=128, dtype=FP8, values="normal", w_dist="u8", topk=2048,
            sa_heads=16, sa_d_qk=576, sa_d_v=512, seed=3),
    "stack_bf16_L131072": dict(name="8-layer IndexCache prefill stack L=131072 FSSSFSSS vs FFFFFFFF", L=131072,
            H=64, d=128, dtype=BF16, topk=2048, layers=8, sa_heads=16, sa_d_qk=576,
            sa_d_v=512, seed=4),
    "decode_fp8_B8_S204800": dict(name="47-layer decode stack B=8 S=204800 FSSS k=2048", B=8, S=204800, layers=47,
            H=64, d=128, dtype=FP8, topk=2048, sa_heads=16, sa_d_qk=576, sa_d_v=512, seed=5),
}


def prefill_stack_layers(*, L, n_layers=8, H=64, d=128, noise=0.3, seed=4, device="cpu", values="normal",
             with_sa=True, sa_heads=16, d_qk=576, d_v=512):
    """8-layer prefill stack (L = 131072 in the benchmark): q and w drawn once and shared by every layer; layer l's
    indexer keys are bf16(base_k + noise * N(0,1)_l) with base_k ~ N(0,1) in bf16;
    every layer has independent sparse-attention Q/KV."""
    g = generator(seed, device)
    base = _draw(g, (1, L, d), device, values).to(torch.bfloat16)
    shared = indexer_inputs(B=1, n_q=L, n_k=L, H=H, d=d, dtype=BF16, values=values,
                            w_dist="u8" if values == "normal" else "pow2",
                            seed=seed * 1000 + 1, device=device, k_source=base)
    layers = []
    for l in range(n_layers):
        gl = generator(seed * 1000 + 10 + l, device)
        if values == "int":
            flip = torch.randint(0, 10, (1, L, d), generator=gl, device=device) == 0
            kl = torch.where(flip, _draw(gl, (1, L, d), device, "int").to(torch.bfloat16), base)
        else:
            kl = (base.float() + noise * torch.randn((1, L, d), generator=gl, device=device)
                  ).to(torch.bfloat16)
        ix = IndexerInputs(dtype=BF16, q=shared.q, k=kl.contiguous(), w=shared.w)
        sa = None
        if with_sa:
            sa = sa_inputs(B=1, n_q=L, n_k=L, heads=sa_heads, kv_heads=1, d_qk=d_qk, d_v=d_v,
                           latent=True, dtype=BF16, seed=seed * 1000 + 100 + l, device=device)
        layers.append((ix, sa))
    return layers


def decode_layer_indexer(layer: int, *, B=8, S=204800, H=64, d=128, seed=5, device="cpu",
                     values="normal"):
    """Decode F layer: one new query per sequence at position S-1 against an fp8
    e4m3fn indexer K cache [B, S, d] with per-token scales; w ~ N(0,1) (signed)."""
    return indexer_inputs(B=B, n_q=1, n_k=S, H=H, d=d, q_pos0=S - 1, dtype=FP8, values=values,
                          w_dist="normal" if values == "normal" else "pm_pow2",
                          seed=seed * 1000 + 200 + layer, device=device)


def decode_layer_sa(layer: int, *, B=8, S=204800, heads=16, d_qk=576, d_v=512, seed=5, device="cpu"):
    return sa_inputs(B=B, n_q=1, n_k=S, heads=heads, kv_heads=1, d_qk=d_qk, d_v=d_v,
                     latent=True, dtype=BF16, seed=seed * 1000 + 300 + layer, device=device)


def drift_stack(*, n_layers, B=1, n_q, n_k=None, q_pos0=0, H=64, d=128, dtype=BF16, values="normal",
                rho=0.9, rho_jump=0.2, p_jump=0.15, seed=6, device="cpu", sa_heads=16, d_qk=576, d_v=512):
    """Calibration stack for the similarity-based pattern search.  The indexer
    queries and head weights are drawn once and shared by every layer; the
    indexer keys drift with depth, so nearby layers select overlapping index
    sets and distant ones less:
      normal: k_0 ~ N(0, 1);   k_l = rho_l k_{l-1} + sqrt(1 - rho_l^2) e_l,  e_l ~ N(0, 1)
      int:    k_0 ~ U{-3..3};  k_l = k_{l-1} with each entry redrawn with probability 1 - rho_l
    rho_l = rho_jump on "jump" layers (each layer >= 1 is one with probability
    p_jump), else rho.  Keys are stored as ``dtype`` (fp8 with per-token
    scales).  Every layer has its own sparse-attention inputs (MLA latent rows).
    Returns (layers [(IndexerInputs, SAInputs)], jumps [bool])."""
    if n_k is None:
        n_k = q_pos0 + n_q
    g = generator(seed, device)
    shared = indexer_inputs(B=B, n_q=n_q, n_k=1, H=H, d=d, q_pos0=q_pos0, dtype=dtype, values=values,
                            w_dist="u8" if values == "normal" else "pow2", seed=seed * 1000 + 1, device=device)
    jumps = (torch.rand(n_layers, generator=g, device=device) < p_jump).cpu().tolist()
    jumps[0] = False
    kf = _draw(g, (B, n_k, d), device, values)
    layers = []
    for l in range(n_layers):
        if l > 0:
            r = rho_jump if jumps[l] else rho
            if values == "int":
                redraw = torch.rand((B, n_k, d), generator=g, device=device) < (1.0 - r)
                kf = torch.where(redraw, _draw(g, (B, n_k, d), device, "int"), kf)
            else:
                kf = r * kf + (1.0 - r * r) ** 0.5 * _draw(g, (B, n_k, d), device, values)
        k, ks = _store(kf, dtype, values)
        ix = IndexerInputs(dtype=dtype, q=shared.q, k=k, w=shared.w, q_scale=shared.q_scale, k_scale=ks,
                           q_pos0=q_pos0)
        sa = sa_inputs(B=B, n_q=n_q, n_k=n_k, heads=sa_heads, kv_heads=1, d_qk=d_qk, d_v=d_v, latent=True,
                       dtype=BF16, seed=seed * 1000 + 100 + l, device=device)
        layers.append((ix, sa))
    return layers, jumps
