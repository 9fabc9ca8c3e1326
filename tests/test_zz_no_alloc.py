"""csa_fwd_noalloc (the fused CSA layer on the library's static workspace) against
csa_fwd with a caller workspace: two calls in a row, the second on a smaller input,
each compared with csa_fwd on the same inputs.  The kernels are the same, so the
outputs must be identical (and the selections, which are integer work, bit-exact).
A shape whose workspace exceeds the static one is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

from compressed_sparse_attention_hca_amd import workloads as wl

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def bd():
    from compressed_sparse_attention_hca_amd import binding
    return binding


def _outs(cfg, inp):
    B, S = cfg.B, cfg.S
    return dict(kv_c_out=torch.empty((B, S // cfg.ratio, cfg.D), dtype=inp["q"].dtype, device=DEV),
                idx_out=torch.empty((B, S, cfg.topk), dtype=torch.int32, device=DEV),
                n_visible_out=torch.empty((B, S), dtype=torch.int32, device=DEV))


def _compare(bd, cfg, inp, o_na, outs_na):
    p = bd.params(cfg)
    outs = _outs(cfg, inp)
    o = bd.layer_fwd(p, inp, **outs)
    torch.cuda.synchronize()
    for k in outs:
        assert torch.equal(outs[k], outs_na[k]), f"{cfg.name}: {k} differs"
    d = (o.float() - o_na.float()).abs().max().item()
    scale = o.float().abs().max().item()
    assert d <= (1e-2 if cfg.dtype == wl.BF16 else 1e-5) * scale, (cfg.name, d, scale)
    assert torch.equal(o, o_na), f"{cfg.name}: output differs from csa_fwd ({d:.3e})"


def test_noalloc_matches_csa_fwd_twice_then_smaller(bd):
    big = wl.C1  # CSA, S=4096, 64 heads x 512, top-512, bf16
    small = wl.C1.replace(S=1024, B=2, seed=2077, name="c1_small_b2")
    assert bd.workspace_bytes(bd.params(big), bd.OP_CSA_FWD) <= bd.NOALLOC_SCRATCH_BYTES
    runs = []
    for cfg in (big, small):
        inp = {k: v.to(DEV) for k, v in wl.make_inputs(cfg, "cpu").items()}
        outs = _outs(cfg, inp)
        o = bd.csa_fwd_noalloc(bd.params(cfg), inp, **outs)
        torch.cuda.synchronize()
        runs.append((cfg, inp, o, outs))
    for cfg, inp, o, outs in runs:
        _compare(bd, cfg, inp, o, outs)


def test_noalloc_fp32_and_headline_shape_fit(bd):
    """The tiny fp32 layer, and the size check of the S=65536 shape (no launch)."""
    cfg = wl.C0
    inp = {k: v.to(DEV) for k, v in wl.make_inputs(cfg, "cpu").items()}
    outs = _outs(cfg, inp)
    o = bd.csa_fwd_noalloc(bd.params(cfg), inp, **outs)
    torch.cuda.synchronize()
    _compare(bd, cfg, inp, o, outs)
    for c in (wl.C3, wl.C3.replace(index_fp8=True), wl.C3.replace(index_prologue=True)):
        assert bd.workspace_bytes(bd.params(c), bd.OP_CSA_FWD) <= bd.NOALLOC_SCRATCH_BYTES


def test_noalloc_refuses_oversized_shapes_before_launch(bd):
    p = bd.params(wl.C3.replace(B=2))
    assert bd.workspace_bytes(p, bd.OP_CSA_FWD) > bd.NOALLOC_SCRATCH_BYTES
    st = bd.lib.csa_fwd_noalloc(ctypes.byref(p), ctypes.byref(bd.Inputs()), None, None)
    assert st == bd.CSA_ERR_WORKSPACE
    assert "static workspace" in bd.last_error()
    # invalid params keep csa_fwd's status; an empty batch is a no-op
    bad = bd.params(wl.C1, topk=0)
    assert bd.lib.csa_fwd_noalloc(ctypes.byref(bad), ctypes.byref(bd.Inputs()), None, None) == bd.CSA_ERR_INVALID_ARG
    empty = bd.params(wl.C1.replace(B=0))
    assert bd.lib.csa_fwd_noalloc(ctypes.byref(empty), ctypes.byref(bd.Inputs()), None, None) == bd.CSA_OK
