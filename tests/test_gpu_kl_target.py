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
}


@pytest.mark.parametrize("name", list(CASES))
def test_kl_target_parity(bd, name):
    cfg, n = CASES[name]
    inp = gen(cfg)
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
    rel = tol(cfg)
    for (b, t) in rows:
        m = len(want[(b, t)])
        assert not got[b, t, m:].any()
        if m:
            w = want[(b, t)]
            assert np.abs(got[b, t, :m] - w).max() <= rel * w.max(), (b, t)
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
