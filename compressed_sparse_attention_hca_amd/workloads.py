"""Workload definitions and seeded synthetic inputs for the compressed attention layer.

This module holds the shapes of the DeepSeek-V4-Flash compressed attention layer and
draws seeded random inputs of those shapes.  It contains none of the layer's own
arithmetic: the CPU oracle and the HIP path both consume the tensors drawn here, and
neither imports the other.

Shapes follow "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
Primus", section "The DeepSeek-V4-Flash architecture" (64 query heads sharing one
512-wide latent that is both key and value) and subsection "Three attention types,
interleaved" (CSA pools 4 tokens per entry with overlapping groups and keeps the best
512 entries from a lightning indexer; HCA pools 128 tokens per entry and attends
densely; every layer adds a 128-token sliding window).  The RoPE base 40000 and the
plain head_dim**-0.5 scale come from "fix(deepseek-v4): correct V4-Flash attention
math", Part 1, items 1 and 2.

Distributions: values, gates and raw latents are N(0, 1); the per-position pooling
bias is N(0, 0.1^2) (standard deviation 0.1); queries are N(0, 1) and then
RMS-normalised per head in fp32 before the cast to the activation dtype; indexer
queries and keys are N(0, 1); indexer head weights are U(0, 1) in fp32.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

F32 = "f32"
BF16 = "bf16"

CSA = "csa"
HCA = "hca"
SWA = "swa"


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    """One attention layer's shape.  Field names follow the pages' notation."""

    name: str
    kind: str  # "csa" | "hca" | "swa"
    B: int
    S: int
    H: int = 64  # query heads
    D: int = 512  # latent width = head dim (K = V)
    rope_dim: int = 64  # RoPE on the last rope_dim dims
    ratio: int = 4  # compress ratio (tokens per compressed entry)
    window: int = 128  # sliding-window length
    topk: int = 512  # entries kept by the indexer (CSA only)
    idx_heads: int = 64
    idx_dim: int = 128
    dtype: str = BF16
    rope_theta: float = 40000.0
    rms_eps: float = 1e-6
    pos0: int = 0
    norm_window: bool = False  # RMS-normalise window latents before rotation
    index_prologue: bool = False  # indexer RoPE + Hadamard + temperature (CSA)
    index_fp8: bool = False  # indexer QK on per-row E4M3 operands (CSA)
    seed: int = 0

    @property
    def overlap(self) -> int:
        return 1 if self.kind == CSA else 0

    @property
    def span(self) -> int:
        return 2 * self.ratio if self.overlap else self.ratio

    @property
    def n_entries(self) -> int:
        return self.S // self.ratio if self.kind != SWA else 0

    @property
    def softmax_scale(self) -> float:
        return self.D ** -0.5

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


# The five workloads.  C0 is the tiny fp32 case the oracle finishes in a second.
C0 = LayerConfig(name="tiny_csa_f32_S256", kind=CSA, B=1, S=256, H=4, D=64, rope_dim=16,
                 ratio=4, window=32, topk=16, idx_heads=4, idx_dim=16, dtype=F32, seed=1000)
C1 = LayerConfig(name="v4flash_csa_bf16_S4096", kind=CSA, B=1, S=4096, seed=2000)
C2 = LayerConfig(name="v4flash_hca_bf16_S65536", kind=HCA, B=1, S=65536, ratio=128,
                 topk=0, seed=3000)
C3 = LayerConfig(name="v4flash_csa_bf16_S65536", kind=CSA, B=1, S=65536, seed=4000)

CONFIGS = {"C0": C0, "C1": C1, "C2": C2, "C3": C3}


def stack_layers(B: int = 4, S: int = 8192, n_layers: int = 43, seed: int = 5000):
    """The 43-layer V4-Flash pattern: layers 0-1 window-only, then CSA on even and HCA
    on odd layer indices, so the last layer (42) is CSA (21 CSA, 20 HCA)."""
    layers = []
    for l in range(n_layers):
        if l < 2:
            layers.append(LayerConfig(name=f"stack_l{l}_swa", kind=SWA, B=B, S=S, topk=0,
                                      seed=seed + 100 * l))
        elif l % 2 == 0:
            layers.append(LayerConfig(name=f"stack_l{l}_csa", kind=CSA, B=B, S=S,
                                      seed=seed + 100 * l))
        else:
            layers.append(LayerConfig(name=f"stack_l{l}_hca", kind=HCA, B=B, S=S, ratio=128,
                                      topk=0, seed=seed + 100 * l))
    return layers


def torch_dtype(dtype: str) -> torch.dtype:
    return {F32: torch.float32, BF16: torch.bfloat16}[dtype]


_TENSOR_IDS = {"va": 1, "ga": 2, "vb": 3, "gb": 4, "bias": 5, "q": 6, "kv_raw": 7,
               "q_idx": 8, "w_idx": 9, "k_idx": 10}


def _gen(seed: int, name: str, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 131 + _TENSOR_IDS[name])
    return g


def _normal(shape, seed, name, device, std=1.0, chunk_rows=None):
    g = _gen(seed, name, device)
    out = torch.empty(shape, dtype=torch.float32, device=device)
    if chunk_rows is None:
        out.normal_(0.0, std, generator=g)
    else:
        flat = out.view(shape[0] * shape[1], -1) if len(shape) > 2 else out
        for r0 in range(0, flat.shape[0], chunk_rows):
            flat[r0:r0 + chunk_rows].normal_(0.0, std, generator=g)
    return out


def _cast(x: torch.Tensor, dtype: str) -> torch.Tensor:
    return x.to(torch_dtype(dtype))


def make_inputs(cfg: LayerConfig, device="cpu", seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw every input of one layer.  Returns contiguous tensors on `device`.

    Keys: q [B,S,H,D], kv_raw [B,S,D]; for CSA/HCA also va, ga [B,S,D], bias [span,D]
    fp32; CSA also vb, gb [B,S,D], q_idx [B,S,H_I,D_I], w_idx [B,S,H_I] fp32 and
    k_idx [B,S/ratio,D_I].  Activations use cfg.dtype.
    """
    seed = cfg.seed if seed is None else seed
    B, S, H, D = cfg.B, cfg.S, cfg.H, cfg.D
    out: Dict[str, torch.Tensor] = {}
    dt = cfg.dtype

    # Queries: N(0,1), RMS-normalised per head over D in fp32, then cast.  Drawn in
    # row chunks so the fp32 temporary stays small at long sequence lengths.
    q = torch.empty((B, S, H, D), dtype=torch_dtype(dt), device=device)
    g = _gen(seed, "q", device)
    rows = B * S
    qv = q.view(rows, H, D)
    step = max(1, (1 << 24) // (H * D))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.empty((r1 - r0, H, D), dtype=torch.float32, device=device).normal_(0.0, 1.0, generator=g)
        x = x * torch.rsqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
        qv[r0:r1] = x.to(q.dtype)
    out["q"] = q
    out["kv_raw"] = _cast(_normal((B, S, D), seed, "kv_raw", device), dt)

    if cfg.kind in (CSA, HCA):
        out["va"] = _cast(_normal((B, S, D), seed, "va", device), dt)
        out["ga"] = _cast(_normal((B, S, D), seed, "ga", device), dt)
        out["bias"] = _normal((cfg.span, D), seed, "bias", device, std=0.1)
    if cfg.kind == CSA:
        out["vb"] = _cast(_normal((B, S, D), seed, "vb", device), dt)
        out["gb"] = _cast(_normal((B, S, D), seed, "gb", device), dt)
        HI, DI = cfg.idx_heads, cfg.idx_dim
        qi = torch.empty((B, S, HI, DI), dtype=torch_dtype(dt), device=device)
        g = _gen(seed, "q_idx", device)
        qiv = qi.view(B * S, HI, DI)
        step = max(1, (1 << 24) // (HI * DI))
        for r0 in range(0, B * S, step):
            r1 = min(B * S, r0 + step)
            qiv[r0:r1] = torch.empty((r1 - r0, HI, DI), dtype=torch.float32,
                                     device=device).normal_(0.0, 1.0, generator=g).to(qi.dtype)
        out["q_idx"] = qi
        gw = _gen(seed, "w_idx", device)
        out["w_idx"] = torch.empty((B, S, HI), dtype=torch.float32, device=device).uniform_(0.0, 1.0, generator=gw)
        out["k_idx"] = _cast(_normal((B, S // cfg.ratio, DI), seed, "k_idx", device), dt)
    return out


# ----------------------------------------------------------------------------------
# Algorithmic work counts (causally visible pairs only).
# ----------------------------------------------------------------------------------

def visible_entries(t: int, ratio: int) -> int:
    """Entries whose whole group has been seen by query t: (s+1)*ratio - 1 <= t."""
    return (t + 1) // ratio


def keys_per_query(cfg: LayerConfig, t: int) -> int:
    win = min(cfg.window, t + 1)
    if cfg.kind == SWA:
        return win
    n = visible_entries(t, cfg.ratio)
    sel = n if cfg.kind == HCA else min(cfg.topk, n)
    return sel + win


def layer_flops(cfg: LayerConfig) -> Dict[str, float]:
    """Algorithmic FLOPs: attention 4*H*D per (query, key); indexer 2*H_I*D_I per
    visible (query, entry) pair.  Closed-form sums over t for speed."""
    S, B = cfg.S, cfg.B
    r, W = cfg.ratio, cfg.window
    # sum_t min(W, t+1)
    win = sum(min(W, t + 1) for t in range(0, min(S, W))) + max(0, S - W) * W
    sel = 0
    vis = 0
    if cfg.kind != SWA:
        # sum_t n_t with n_t = floor((t+1)/r); n_t = j for r rows (t+1 in [j r, j r + r - 1])
        n_max = S // r
        vis = sum(j * r for j in range(n_max)) + n_max * (S - n_max * r + 1)
        if cfg.kind == HCA:
            sel = vis
        else:
            K = cfg.topk
            # rows with n_t <= K contribute n_t, else K
            sel = 0
            for j in range(0, n_max + 1):
                cnt = r if j < n_max else (S + 1 - n_max * r)
                if j == 0:
                    cnt = r - 1  # t = 0 .. r-2 have n_t = 0
                sel += cnt * min(j, K)
    attn = 4.0 * cfg.H * cfg.D * (sel + win) * B
    idx = 2.0 * cfg.idx_heads * cfg.idx_dim * vis * B if cfg.kind == CSA else 0.0
    return {"attention": attn, "indexer": idx, "total": attn + idx,
            "keys": float((sel + win) * B), "visible_pairs": float(vis * B),
            "selected_pairs": float(sel * B)}


def page_convention_attention_flops(cfg: LayerConfig) -> float:
    """The pages' kernel-table convention: 4*H*D*(K+W) per query, causality ignored."""
    if cfg.kind == SWA:
        keys = cfg.window
    elif cfg.kind == HCA:
        keys = cfg.S // cfg.ratio + cfg.window
    else:
        keys = cfg.topk + cfg.window
    return 4.0 * cfg.H * cfg.D * keys * cfg.S * cfg.B
