"""GPU-versus-oracle parity of the attention backward's key side and of the forward's
log-denominators (csa_sparse_mqa_bwd_dkv, csa_sparse_mqa_fwd_lse; "Enabling
DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus", "Attention kernels
for the three layer types": interm, the contraction over heads that gives each key's
gradient, and the scatter back to the entries; "fix(deepseek-v4): correct V4-Flash
attention math", Part 1 item 6f: the sink logit).

Inputs: the seeded layer inputs, the GPU's compressed entries, the oracle's own
selection for the checked rows (-1 elsewhere, so no oracle input comes from the GPU),
the GPU forward's o and lse over that selection, and a seeded dL/do that is zero on
every row the oracle does not evaluate.  Such a row contributes nothing (its du and
delta are 0), so the oracle's gradients over the checked rows (oracle.csa_oracle.
layer_bwd_rows, fp64) are the exact full tables: dkv_c [B, S/ratio, D] and dkv_raw
[B, S, D] are compared entry by entry, zeros included, and dsinks per head.
Acceptance as for the forward: max |gpu - oracle| <= 1e-2 of the table's largest
|oracle| for bf16 activations, 1e-5 for fp32; lse within 2e-2 (bf16) or 1e-4 (fp32)
in absolute terms (a relative error of the denominator).
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


EDGE = wl.LayerConfig(name="dkv_edge", kind="csa", B=2, S=44, H=20, D=128, rope_dim=32, ratio=4,
                      window=7, topk=5, idx_heads=8, idx_dim=16, dtype=wl.BF16, pos0=1_000_003, seed=991)
# three sequences of 3000 rows: the 6528-row chunks of the selected mode end inside
# the third sequence, so window tokens and entries are summed across a chunk boundary
CHUNKS = wl.C1.replace(B=3, S=3000, name="dkv_chunks", seed=2300)
CHUNK_ROWS = [(0, 5), (0, 2999), (1, 0), (1, 130), (1, 2999), (2, 0), (2, 400), (2, 500), (2, 520),
              (2, 527), (2, 528), (2, 529), (2, 600), (2, 655), (2, 2999)]

# name: (config, rows: None = every row, int = sample_rows(n), list = those rows; sinks)
CASES = {
    "C0": (wl.C0, None, False),
    "C0_sink": (wl.C0, None, True),
    "C0_norm_window_sink": (wl.C0.replace(norm_window=True, name="c0_nw"), None, True),
    "C1": (wl.C1, 24, False),
    "C1_sink": (wl.C1, 16, True),
    "hca_4096": (wl.C2.replace(S=4096, name="hca_4096"), 16, True),
    "swa_1024": (wl.C1.replace(kind="swa", topk=0, S=1024, name="swa_1024"), 16, False),
    "swa_norm_window": (wl.C1.replace(kind="swa", topk=0, S=512, norm_window=True, name="swa_nw"), 12, True),
    "edge": (EDGE, None, True),
    "h8_one_wave": (wl.C1.replace(H=8, S=512, name="dkv_h8"), None, False),
    "h40_padded": (wl.C1.replace(H=40, S=512, name="dkv_h40"), None, True),
    "fp32_d256": (wl.C0.replace(D=256, H=20, rope_dim=64, S=512, name="dkv_f32_d256"), None, True),
    "chunks": (CHUNKS, CHUNK_ROWS, True),
    "C2": (wl.C2, 8, True),
    "C3": (wl.C3, 10, True),
}


def _np(t):
    return t.detach().to(torch.float32).cpu().double().numpy()


def run_case(bd, cfg, rows_spec, with_sink, edit=None, mutate_sel=None):
    """GPU forward (o, lse) and key-side backward, and the oracle's gradients over the
    checked rows.  Returns (gpu dict, oracle dict, rows)."""
    inp = gen(cfg)
    if edit is not None:
        edit(inp)
    p = bd.params(cfg)
    if rows_spec is None:
        rows = [(b, t) for b in range(cfg.B) for t in range(cfg.S)]
    elif isinstance(rows_spec, int):
        rows = sample_rows(cfg, rows_spec)
    else:
        rows = list(rows_spec)
    lz = lazy_inputs(inp)
    rng = np.random.default_rng(cfg.seed + 31)
    sinks = rng.normal(size=cfg.H).astype(np.float32) if with_sink else None
    sinks_d = torch.from_numpy(sinks).to(DEV) if with_sink else None
    d_o = torch.zeros(inp["q"].shape, dtype=inp["q"].dtype, device=DEV)
    g = torch.Generator().manual_seed(cfg.seed + 37)
    do_np = {}
    for (b, t) in rows:
        x = torch.randn((cfg.H, cfg.D), generator=g).to(inp["q"].dtype)
        d_o[b, t] = x.to(DEV)
        do_np[(b, t)] = x.double().numpy()

    if cfg.kind == "swa":
        kv, idx_d, sel, kv_ora = None, None, None, None
    else:
        kv = bd.compress(p, inp["va"], inp["ga"], inp.get("vb"), inp.get("gb"), inp["bias"])
        ora = O.layer_rows(cfg, lz, rows)
        sel, kv_ora = ora["sel"], ora["kv_c"]
        idx_d = None
        if cfg.kind == "csa":
            idx = np.full((cfg.B, cfg.S, cfg.topk), -1, dtype=np.int32)
            for k in rows:
                idx[k[0], k[1], :len(sel[k])] = sel[k]
            if mutate_sel is not None:
                sel = mutate_sel(idx, sel)
            idx_d = torch.from_numpy(idx).to(DEV)
    o, lse = bd.sparse_mqa_fwd_lse(p, inp["q"], kv, inp["kv_raw"], idx_d, sinks=sinks_d)
    dkv_c, dkv_raw, dsinks = bd.sparse_mqa_bwd_dkv(p, inp["q"], kv, inp["kv_raw"], idx_d, o, lse, d_o,
                                                   sinks=sinks_d)
    torch.cuda.synchronize()
    gpu = {"o": o, "lse": lse, "dkv_c": dkv_c, "dkv_raw": dkv_raw, "dsinks": dsinks, "kv": kv, "idx": idx_d,
           "inp": inp, "p": p, "sinks": sinks_d, "d_o": d_o}
    want = O.layer_bwd_rows(cfg, lz, rows, do_np, sel, kv_ora, sinks=None if sinks is None else sinks.astype(np.float64))
    return gpu, want, rows


def check_case(cfg, gpu, want, rows):
    rel = tol(cfg)
    lse_tol = 1e-4 if cfg.dtype == wl.F32 else 2e-2
    got_lse = np.stack([_np(gpu["lse"][b, t]) for (b, t) in rows])
    want_lse = np.stack([want["lse"][k] for k in rows])
    assert np.all(np.isfinite(got_lse) == np.isfinite(want_lse))
    fin = np.isfinite(want_lse)
    err = float(np.max(np.abs(got_lse[fin] - want_lse[fin]))) if fin.any() else 0.0
    assert err <= lse_tol, f"lse {cfg.name}: max err {err:.3e}"
    if cfg.kind != "swa":
        got = _np(gpu["dkv_c"])
        ref = np.stack([want["dkv_c"].get(b, np.zeros_like(got[0])) for b in range(cfg.B)])
        assert np.isfinite(got).all()
        assert_close_rel(got, ref, rel, f"dkv_c {cfg.name}")
    else:
        assert gpu["dkv_c"] is None
    got = _np(gpu["dkv_raw"])
    ref = np.stack([want["dkv_raw"].get(b, np.zeros_like(got[0])) for b in range(cfg.B)])
    assert np.isfinite(got).all()
    assert_close_rel(got, ref, rel, f"dkv_raw {cfg.name}")
    if want["dsinks"] is not None:
        assert_close_rel(_np(gpu["dsinks"]), want["dsinks"], rel, f"dsinks {cfg.name}")


@pytest.mark.parametrize("name", list(CASES))
def test_dkv_parity(bd, name):
    cfg, rows, with_sink = CASES[name]
    print(f"[dkv] {name}: B={cfg.B} S={cfg.S} H={cfg.H} D={cfg.D} {cfg.dtype} {cfg.kind}", flush=True)
    gpu, want, rows = run_case(bd, cfg, rows, with_sink)
    check_case(cfg, gpu, want, rows)


@pytest.mark.parametrize("name", ["C0_sink", "C1_sink", "hca_4096", "swa_1024"])
def test_fwd_lse_keeps_the_forward_output(bd, name):
    """The forward that keeps lse writes the same o, bit for bit, as the plain one."""
    cfg, _, with_sink = CASES[name]
    inp = gen(cfg.replace(S=min(cfg.S, 1024)))
    cfg = cfg.replace(S=min(cfg.S, 1024))
    p = bd.params(cfg)
    sinks = torch.linspace(-1.0, 1.5, cfg.H, device=DEV) if with_sink else None
    kv = None if cfg.kind == "swa" else bd.compress(p, inp["va"], inp["ga"], inp.get("vb"), inp.get("gb"), inp["bias"])
    idx = bd.index_topk(p, inp["q_idx"], inp["w_idx"], inp["k_idx"])[0] if cfg.kind == "csa" else None
    o1 = bd.sparse_mqa_fwd(p, inp["q"], kv, inp["kv_raw"], idx, sinks=sinks)
    o2, lse = bd.sparse_mqa_fwd_lse(p, inp["q"], kv, inp["kv_raw"], idx, sinks=sinks)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.isfinite(lse).all()


def test_dkv_deterministic(bd):
    """Two calls on the same inputs give bit-identical gradients: the inverse index keeps
    each entry's pairs in row order and every sum runs in a fixed order."""
    cfg = wl.C1.replace(S=2048, name="dkv_det")
    inp = gen(cfg)
    p = bd.params(cfg)
    kv = bd.compress(p, inp["va"], inp["ga"], inp["vb"], inp["gb"], inp["bias"])
    idx, _ = bd.index_topk(p, inp["q_idx"], inp["w_idx"], inp["k_idx"])
    sinks = torch.linspace(-2.0, 2.0, cfg.H, device=DEV)
    o, lse = bd.sparse_mqa_fwd_lse(p, inp["q"], kv, inp["kv_raw"], idx, sinks=sinks)
    d_o = torch.randn_like(o)
    a = bd.sparse_mqa_bwd_dkv(p, inp["q"], kv, inp["kv_raw"], idx, o, lse, d_o, sinks=sinks)
    b = bd.sparse_mqa_bwd_dkv(p, inp["q"], kv, inp["kv_raw"], idx, o, lse, d_o, sinks=sinks)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_dkv_invalid_selection_entries_are_masked(bd):
    """Selection entries outside 0..n_t-1 (-1, n_t, n_t + 1000, -7) are left out of the
    backward as of the forward: the first 40 entries of every checked row are made
    invalid and every seventh checked row's whole selection is (window keys only)."""
    cfg = wl.C1.replace(S=1024, name="dkv_masked")
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
    gpu, want, rows = run_case(bd, cfg, 40, True, mutate_sel=mutate)
    check_case(cfg, gpu, want, rows)


def test_dkv_repeated_entry_in_a_row_counts_twice(bd):
    """An entry listed twice in one row's selection is attended twice by the forward
    (two keys), so it gathers both key gradients."""
    cfg = wl.C1.replace(S=512, name="dkv_repeat")

    def mutate(idx, sel):
        out = {}
        for (b, t), s_ in sel.items():
            if len(s_) >= 4:
                idx[b, t, 1] = idx[b, t, 0]
                idx[b, t, 3] = idx[b, t, 0]
            m = len(s_)
            out[(b, t)] = idx[b, t, :m].astype(np.int64)
        return out
    gpu, want, rows = run_case(bd, cfg, 16, False, mutate_sel=mutate)
    check_case(cfg, gpu, want, rows)


def test_dkv_empty_batch_zeroes_the_sink_gradient(bd):
    cfg = wl.C0.replace(B=0)
    p = bd.params(cfg)
    z = torch.empty((0, cfg.S, cfg.H, cfg.D), dtype=torch.float32, device=DEV)
    kvr = torch.empty((0, cfg.S, cfg.D), dtype=torch.float32, device=DEV)
    kv = torch.empty((0, cfg.S // cfg.ratio, cfg.D), dtype=torch.float32, device=DEV)
    idx = torch.empty((0, cfg.S, cfg.topk), dtype=torch.int32, device=DEV)
    lse = torch.empty((0, cfg.S, cfg.H), dtype=torch.float32, device=DEV)
    sinks = torch.ones(cfg.H, device=DEV)
    dsinks = torch.full((cfg.H,), 7.0, device=DEV)
    bd.sparse_mqa_bwd_dkv(p, z, kv, kvr, idx, z, lse, z, sinks=sinks, dsinks=dsinks)
    torch.cuda.synchronize()
    assert torch.equal(dsinks, torch.zeros_like(dsinks))


def test_fused_layer_keeps_the_same_lse(bd):
    """csa_fwd with lse_out keeps the log-denominators csa_sparse_mqa_fwd_lse writes for
    the same entries and selection, bit for bit, and the same output."""
    cfg = wl.C1.replace(S=1024, name="dkv_fused_lse")
    inp = gen(cfg)
    inp["sinks"] = torch.linspace(-1.0, 1.0, cfg.H, device=DEV)
    p = bd.params(cfg)
    n = cfg.S // cfg.ratio
    kv = torch.empty((cfg.B, n, cfg.D), dtype=torch.bfloat16, device=DEV)
    idx = torch.empty((cfg.B, cfg.S, cfg.topk), dtype=torch.int32, device=DEV)
    lse = torch.empty((cfg.B, cfg.S, cfg.H), dtype=torch.float32, device=DEV)
    o = bd.layer_fwd(p, inp, kv_c_out=kv, idx_out=idx, lse_out=lse)
    o2, lse2 = bd.sparse_mqa_fwd_lse(p, inp["q"], kv, inp["kv_raw"], idx, sinks=inp["sinks"])
    torch.cuda.synchronize()
    assert torch.equal(o, o2)
    assert torch.equal(lse, lse2)
