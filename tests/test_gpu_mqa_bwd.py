"""GPU-versus-oracle parity of the attention backward's query side
(csa_sparse_mqa_bwd_dq: dQ with delta = rowsum(o * do) inside the kernel;
"Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus",
"Attention kernels for the three layer types").

Inputs of the kernel: the seeded layer inputs, the GPU's compressed entries, the
oracle's own selection for the checked rows (-1 elsewhere, so no oracle input comes
from the GPU), the GPU forward's output o over that selection, and a seeded dL/do.  The
oracle (oracle.csa_oracle.layer_dq_rows) differentiates its own fp64 forward.
Acceptance as for the forward outputs: max |dq_gpu - dq_ora| <= 1e-2 of the largest
|dq_ora| over the checked rows for bf16 activations, 1e-5 for fp32.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_hca_amd import workloads as wl
from oracle import csa_oracle as O
from gpu_util import assert_close_rel, lazy_inputs, sample_rows, tol
from test_gpu_parity import DEV, gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def bd():
    from compressed_sparse_attention_hca_amd import binding
    return binding


EDGE = wl.LayerConfig(name="dq_edge", kind="csa", B=2, S=44, H=20, D=128, rope_dim=32, ratio=4,
                      window=7, topk=5, idx_heads=8, idx_dim=16, dtype=wl.BF16, pos0=1_000_003, seed=991)

# name: (config, sampled rows (None: every row), with sinks)
CASES = {
    "C0": (wl.C0, None, False),
    "C0_sink": (wl.C0, None, True),
    "C1": (wl.C1, 32, False),
    "C1_sink": (wl.C1, 24, True),
    "hca_4096": (wl.C2.replace(S=4096, name="hca_4096"), 24, False),
    "swa_1024": (wl.C1.replace(kind="swa", topk=0, S=1024, name="swa_1024"), 24, False),
    "edge": (EDGE, None, False),
    "hd_h40": (wl.C1.replace(H=40, S=512, name="dq_h40"), None, False),   # head-group kernel, padded heads
    "C2": (wl.C2, 12, False),                                            # HCA, S=65536
    "C3": (wl.C3, 12, False),
}


def dq_check(bd, cfg, n_rows, with_sink, edit=None, rel=None, mutate_sel=None, split_dim0=None):
    """mutate_sel(idx, sel): edit the selection handed to the kernels ([B,S,K] int32
    numpy) and return the entries the oracle attends to (dict of rows).  split_dim0:
    compare dims 1.. at `rel` and dim 0 at this bound (both relative to the largest
    |dq_ora| over dims 1..)."""
    inp = gen(cfg)
    if edit is not None:
        edit(inp)
    p = bd.params(cfg)
    rows = [(b, t) for b in range(cfg.B) for t in range(cfg.S)] if n_rows is None else sample_rows(cfg, n_rows)
    lz = lazy_inputs(inp)
    rng = np.random.default_rng(cfg.seed + 17)
    sinks = rng.normal(size=cfg.H).astype(np.float32) if with_sink else None
    sinks_d = torch.from_numpy(sinks).to(DEV) if with_sink else None
    sinks64 = sinks.astype(np.float64) if with_sink else None
    dev = "cpu" if inp["q"].numel() <= (1 << 26) else DEV
    g = torch.Generator(device=dev).manual_seed(cfg.seed + 23)
    d_o = torch.randn(inp["q"].shape, generator=g, dtype=torch.float32, device=dev).to(inp["q"].dtype).to(DEV)

    if cfg.kind == "swa":
        kv, idx_d, sel, kv_ora = None, None, {k: np.zeros(0, dtype=np.int64) for k in rows}, None
    else:
        kv = bd.compress(p, inp["va"], inp["ga"], inp.get("vb"), inp.get("gb"), inp["bias"])
        ora = O.layer_rows(cfg, lz, rows)                 # the oracle's kv_c and selection
        sel, kv_ora = ora["sel"], ora["kv_c"]
        idx_d = None
        if cfg.kind == "csa":
            idx = np.full((cfg.B, cfg.S, cfg.topk), -1, dtype=np.int32)
            for k in rows:
                idx[k[0], k[1], :len(sel[k])] = sel[k]
            if mutate_sel is not None:
                sel = mutate_sel(idx, sel)
            idx_d = torch.from_numpy(idx).to(DEV)
    o = bd.sparse_mqa_fwd(p, inp["q"], kv, inp["kv_raw"], idx_d, sinks=sinks_d)
    dq = bd.sparse_mqa_bwd_dq(p, inp["q"], kv, inp["kv_raw"], idx_d, o, d_o, sinks=sinks_d)
    torch.cuda.synchronize()
    assert torch.isfinite(dq.float()).all()

    do_np = {(b, t): d_o[b, t].float().cpu().double().numpy() for (b, t) in rows}
    want = O.layer_dq_rows(cfg, lz, rows, do_np, sel, kv_ora if kv_ora is not None else {}, sinks=sinks64)
    got = np.stack([dq[b, t].float().cpu().double().numpy() for (b, t) in rows])
    want = np.stack([want[k] for k in rows])
    if split_dim0 is not None:
        scale = float(np.max(np.abs(want[..., 1:])))
        err0 = float(np.max(np.abs(got[..., 0] - want[..., 0])))
        assert err0 <= split_dim0 * scale, f"dq dim 0: {err0:.3e} > {split_dim0} * {scale:.3e}"
        return assert_close_rel(got[..., 1:], want[..., 1:], rel or tol(cfg), f"dq {cfg.name} dims 1..")
    return assert_close_rel(got, want, rel or tol(cfg), f"dq {cfg.name}")


@pytest.mark.parametrize("name", list(CASES))
def test_dq_parity(bd, name):
    cfg, n, with_sink = CASES[name]
    dq_check(bd, cfg, n, with_sink)


def test_dq_empty_batch_is_noop(bd):
    cfg = wl.C0.replace(B=0)
    p = bd.params(cfg)
    z = torch.empty((0, cfg.S, cfg.H, cfg.D), dtype=torch.float32, device=DEV)
    kvr = torch.empty((0, cfg.S, cfg.D), dtype=torch.float32, device=DEV)
    kv = torch.empty((0, cfg.S // cfg.ratio, cfg.D), dtype=torch.float32, device=DEV)
    idx = torch.empty((0, cfg.S, cfg.topk), dtype=torch.int32, device=DEV)
    bd.sparse_mqa_bwd_dq(p, z, kv, kvr, idx, z, z, dq=z)
    torch.cuda.synchronize()


def test_dq_deterministic(bd):
    """Two calls on the same inputs give bit-identical dq (no atomics in the kernel)."""
    cfg = wl.C1.replace(S=1024, name="dq_det")
    inp = gen(cfg)
    p = bd.params(cfg)
    kv = bd.compress(p, inp["va"], inp["ga"], inp["vb"], inp["gb"], inp["bias"])
    idx, _ = bd.index_topk(p, inp["q_idx"], inp["w_idx"], inp["k_idx"])
    o = bd.sparse_mqa_fwd(p, inp["q"], kv, inp["kv_raw"], idx)
    d_o = torch.randn_like(o)
    a = bd.sparse_mqa_bwd_dq(p, inp["q"], kv, inp["kv_raw"], idx, o, d_o)
    b = bd.sparse_mqa_bwd_dq(p, inp["q"], kv, inp["kv_raw"], idx, o, d_o)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dq_large_logit_range_recomputes_exactly(bd):
    """q[..., 0] = 4 and the window latents' dim 0 raised by 100 lift every window logit
    by about 72 (log2 units) over the selected entries, which fill the first tile of the
    rows t >= 127 (topk 40): the kernel must run its second pass with the exact
    reference.  fp32, no RoPE.  dq's dim 0 is a sum of terms of size ~3 that cancel
    (the common offset), so the bound is 1e-3 of the largest |dq| instead of 1e-5 (one
    run measured 4.9e-4); a second pass that kept the first pass's sums or reference
    would be off by O(1)."""
    cfg = wl.C0.replace(topk=40, rope_dim=0, name="dq_wide_logits")

    def edit(inp):
        inp["q"][..., 0] = 4.0
        inp["kv_raw"][..., 0] += 100.0
    dq_check(bd, cfg, None, False, edit=edit, rel=1e-3)


def test_dq_bf16_second_pass(bd):
    """The head-group kernel (bf16, D=512, 64 heads) on a logit range that forces the
    second pass: q[..., 0] = 64 and the window latents' dim 0 raised by 24 lift every
    window logit by 64 * 24 * 512**-0.5 = 68 (98 log2 units) over the selected
    entries, which fill the first tile of the rows t >= 127, while the softmax over the
    window stays spread (a few units of spread from dim 0 and the other dims).  RoPE is
    off, so keys are exact bf16 values.  Dims 1.. are held to the bf16 bound.  Dim 0
    is the common component 24 of every window key: dq's dim 0 is 24 times a sum of dz
    that cancels exactly, and dz is rounded to bf16 (2^-9 relative) before that
    product, so it is held to 24 * 2^-8 of the largest |dq|."""
    cfg = wl.C1.replace(S=512, rope_dim=0, name="dq_wide_logits_bf16")

    def edit(inp):
        inp["q"][..., 0] = 64.0
        inp["kv_raw"][..., 0] += 24.0
    dq_check(bd, cfg, None, False, edit=edit, split_dim0=24 * 2.0 ** -8)


def test_dq_invalid_selection_entries_are_masked(bd):
    """Selection entries outside 0..n_t-1 inside the selection (-1, n_t, n_t + 1000,
    -7) are masked out of the backward as of the forward.  The first 40 entries of every
    row are made invalid, so the first 32-key tile of each query holds no valid entry
    (the reference then starts at 0 and the end-of-pass check decides on a second
    pass), and every seventh row's whole selection is invalid (window keys only)."""
    cfg = wl.C1.replace(S=1024, name="dq_masked")
    junk = [-1, None, "far", -7]

    def mutate(idx, sel):
        out = {}
        for (b, t), s_ in sel.items():
            n_t = O.visible_entries(t, cfg.ratio)
            m = len(s_)
            k = m if t % 7 == 0 else min(40, m)
            for j in range(k):
                v = junk[j % 4]
                idx[b, t, j] = n_t if v is None else (n_t + 1000 if v == "far" else v)
            r = idx[b, t, :m]
            out[(b, t)] = r[(r >= 0) & (r < n_t)].astype(np.int64)
        return out
    dq_check(bd, cfg, None, False, mutate_sel=mutate)
