"""GPU-versus-oracle parity of the indexer distillation target (csa_kl_target).

The target ("fix(deepseek-v4): correct V4-Flash attention math", Part 1 items 5 and
11): per query, the head mean of each head's softmax over the selected entries'
logits.  The selection fed to the kernel is the oracle's own top-k (no oracle input
comes from the GPU); the kernel reads the GPU's compressed entries, the oracle its own
fp64 ones.  Acceptance as for the layer outputs: max |T_gpu - T_ora| <= 1e-2 of the
row's largest target for bf16 inputs and 1e-5 for fp32; every row sums to 1; slots
past the selection and invalid indices hold 0.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_hca_amd import workloads as wl
from oracle import csa_oracle as O
from gpu_util import lazy_inputs, sample_rows, tol
from test_gpu_parity import DEV, gen

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def bd():
    from compressed_sparse_attention_hca_amd import binding
    return binding


CASES = {
    "C0": (wl.C0, None),
    "C1": (wl.C1, 48),
    "C3": (wl.C3, 12),
    "edge": (wl.LayerConfig(name="kl_edge", kind="csa", B=2, S=44, H=20, D=128, rope_dim=32, ratio=4,
                            window=7, topk=5, idx_heads=8, idx_dim=16, dtype=wl.BF16, pos0=1_000_003,
                            seed=990), None),
    # bf16 D = 512, every row of a short sequence: 0 to 4 tiles of 32 selected entries,
    # the last one partial
    "short_all_rows": (wl.C1.replace(S=512, name="kl_short"), None),
    # 40 heads: the second head group is partly padding
    "h40": (wl.C1.replace(H=40, S=1024, name="kl_h40"), 32),
    # more than 512 selected entries: the two-pass kernel
    "topk1024": (wl.C1.replace(topk=1024, S=8192, name="kl_topk1024"), 12),
}


def kl_check(bd, cfg, n, edit=None, rel=None):
    inp = gen(cfg)
    if edit is not None:
        edit(inp)
    p = bd.params(cfg)
    rows = [(b, t) for b in range(cfg.B) for t in range(cfg.S)] if n is None else sample_rows(cfg, n)
    lz = lazy_inputs(inp)
    ora = O.layer_rows(cfg, lz, rows)                      # the oracle's kv_c and selection
    idx = np.full((cfg.B, cfg.S, cfg.topk), -1, dtype=np.int32)
    for k in rows:
        sel = ora["sel"][k]
        idx[k[0], k[1], :len(sel)] = sel
    idx_d = torch.from_numpy(idx).to(DEV)
    kv = bd.compress(p, inp["va"], inp["ga"], inp["vb"], inp["gb"], inp["bias"])
    tgt = bd.kl_target(p, inp["q"], kv, idx_d)
    torch.cuda.synchronize()
    got = tgt.cpu().double().numpy()
    want = O.kl_target(cfg, lz, rows, ora["sel"], ora["kv_c"])
    rel = rel or tol(cfg)
    for (b, t) in rows:
        m = len(want[(b, t)])
        assert not got[b, t, m:].any()
        if m:
            w = want[(b, t)]
            assert np.abs(got[b, t, :m] - w).max() <= rel * w.max(), (b, t)
            assert abs(got[b, t, :m].sum() - 1.0) < 1e-5


@pytest.mark.parametrize("name", list(CASES))
def test_kl_target_parity(bd, name):
    cfg, n = CASES[name]
    kl_check(bd, cfg, n)


def test_kl_target_wide_logit_range(bd):
    """q scaled by 64 (exact in bf16) spreads each head's logits over about +-250 log2
    units, so in most rows some later tile's maximum lies more than 64 log2 units above
    the first tile's: the bf16 D = 512 kernel must take its second pass with the exact
    maximum.  Amplified logits would also amplify any difference between the entries the
    two sides read, so here both read the same seeded bf16 entries (not the compressor's
    output, which the oracle forms in fp64) and a seeded random selection of each row's
    visible entries; RoPE is off, so the query operand is the exact input.  The
    remaining difference is fp32 against fp64 accumulation, well inside 1e-2 of the
    row's largest target.  Every row of S = 1024 (up to 8 tiles)."""
    cfg = wl.C1.replace(S=1024, rope_dim=0, name="kl_wide_logits")
    inp = gen(cfg)
    inp["q"].mul_(64.0)
    p = bd.params(cfg)
    lz = lazy_inputs(inp)
    n = cfg.S // cfg.ratio
    g = torch.Generator().manual_seed(cfg.seed + 31)
    kv = torch.randn((1, n, cfg.D), generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(cfg.seed + 37)
    idx = np.full((1, cfg.S, cfg.topk), -1, dtype=np.int32)
    rows, sels = [], {}
    for t in range(cfg.S):
        n_t = O.visible_entries(t, cfg.ratio)
        sel = rng.permutation(n_t)[:min(cfg.topk, n_t)]
        idx[0, t, :len(sel)] = sel
        rows.append((0, t))
        sels[(0, t)] = sel
    tgt = bd.kl_target(p, inp["q"], kv.to(DEV), torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    got = tgt.cpu().double().numpy()
    want = O.kl_target(cfg, lz, rows, sels, {0: kv[0].double().numpy()})
    for (b, t) in rows:
        m = len(want[(b, t)])
        assert not got[b, t, m:].any()
        if m:
            w = want[(b, t)]
            assert np.abs(got[b, t, :m] - w).max() <= tol(cfg) * w.max(), (b, t)
            assert abs(got[b, t, :m].sum() - 1.0) < 1e-5


@pytest.mark.parametrize("name", ["C0", "C1"])
def test_kl_target_masks_invalid_indices(bd, name):
    """-1 and out-of-range indices are left out of the softmax and get 0; the rest of
    the row is the target over the valid entries alone (C0: the generic kernel, C1:
    the bf16 D = 512 one)."""
    cfg = wl.CONFIGS[name]
    inp = gen(cfg)
    p = bd.params(cfg)
    lz = lazy_inputs(inp)
    t = 200                                                # n_t = 50
    sel = np.array([3, 7, 19, 31, 44])
    idx = np.full((1, cfg.S, cfg.topk), -1, dtype=np.int32)
    idx[0, t, :8] = [3, -1, 7, 19, 9999, 31, -7, 44]
    kv = bd.compress(p, inp["va"], inp["ga"], inp["vb"], inp["gb"], inp["bias"])
    tgt = bd.kl_target(p, inp["q"], kv, torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    got = tgt[0, t].cpu().double().numpy()
    kvo = O.compress(lz["va"][0], lz["ga"][0], lz["vb"][0], lz["gb"][0], lz["bias"][:], cfg.ratio, True,
                     cfg.rope_dim, cfg.rope_theta, cfg.rms_eps, cfg.pos0)
    want = O.kl_target(cfg, lz, [(0, t)], {(0, t): sel}, {0: kvo})[(0, t)]
    assert got[1] == 0 and got[4] == 0 and got[6] == 0 and not got[8:].any()
    assert np.abs(got[[0, 2, 3, 5, 7]] - want).max() <= tol(cfg) * want.max()


def test_kl_target_first_tile_masked(bd):
    """The bf16 D = 512 kernel takes its reference from the first tile of 32 entries;
    with all of them invalid it starts from 0 and its end-of-pass check decides whether
    a second pass is needed.  Rows t = 1000 and 4095 of C1 get 40 invalid entries
    (-1 and n_t) ahead of 100 valid ones."""
    cfg = wl.C1
    inp = gen(cfg)
    p = bd.params(cfg)
    lz = lazy_inputs(inp)
    kv = bd.compress(p, inp["va"], inp["ga"], inp["vb"], inp["gb"], inp["bias"])
    kvo = O.compress(lz["va"][0], lz["ga"][0], lz["vb"][0], lz["gb"][0], lz["bias"][:], cfg.ratio, True,
                     cfg.rope_dim, cfg.rope_theta, cfg.rms_eps, cfg.pos0)
    idx = np.full((1, cfg.S, cfg.topk), -1, dtype=np.int32)
    rng = np.random.default_rng(5)
    sels = {}
    for t in (1000, 4095):
        n_t = O.visible_entries(t, cfg.ratio)
        sel = np.sort(rng.choice(n_t, size=100, replace=False))
        idx[0, t, :40] = [(-1 if j % 2 else n_t) for j in range(40)]
        idx[0, t, 40:140] = sel
        sels[(0, t)] = sel
    tgt = bd.kl_target(p, inp["q"], kv, torch.from_numpy(idx).to(DEV))
    torch.cuda.synchronize()
    for (b, t), sel in sels.items():
        got = tgt[b, t].cpu().double().numpy()
        want = O.kl_target(cfg, lz, [(b, t)], {(b, t): sel}, {0: kvo})[(b, t)]
        assert not got[:40].any() and not got[140:].any()
        assert np.abs(got[40:140] - want).max() <= tol(cfg) * want.max(), t
        assert abs(got.sum() - 1.0) < 1e-5
