"""Host-side checks of the workload shapes, the generator and the FLOP accounting
against constants the pages print (tests/golden/page_constants.json)."""
import json
import os

import numpy as np
import torch

from compressed_sparse_attention_hca_amd import workloads as wl

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")))


def test_configs_carry_page_constants():
    for c in (wl.C1, wl.C3):
        assert c.H == GOLD["query_heads"]["value"] and c.D == GOLD["latent_dim"]["value"]
        assert c.ratio == GOLD["csa_ratio"]["value"] and c.topk == GOLD["topk"]["value"]
        assert c.window == GOLD["window"]["value"] and c.rope_dim == GOLD["derotate_dims"]["value"]
        assert c.rope_theta == GOLD["rope_theta_flash"]["value"]
        assert abs(c.softmax_scale - 512 ** -0.5) < 1e-15
    assert wl.C2.ratio == GOLD["hca_ratio"]["value"]


def test_stack_pattern_matches_pages():
    layers = wl.stack_layers()
    kinds = [l.kind for l in layers]
    g = GOLD["layers"]["value"]
    assert kinds.count("swa") == g["swa"] and kinds.count("csa") == g["csa"]
    assert kinds.count("hca") == g["hca"] and len(kinds) == g["total"] and kinds[-1] == g["last"]


def test_page_flop_convention_reproduces_kernel_table():
    """ms x TFLOP/s in the forward kernel table equals 4*H*D*(K+W)*S for CSA, with
    (S/128 + W) keys for HCA and W keys for the window-only layer, to rounding."""
    tab = GOLD["forward_kernel_table_flash"]["value"]
    S = GOLD["forward_kernel_table_flash"]["workload"]["S"]
    for kind, cfg in (("csa", wl.C1), ("hca", wl.C2.replace(S=S)), ("swa", wl.C1.replace(kind="swa", topk=0))):
        f = wl.page_convention_attention_flops(cfg.replace(S=S))
        for ms, tf in tab[kind]:
            implied = ms * 1e-3 * tf * 1e12
            assert abs(implied / f - 1) < 0.05, (kind, implied, f)


def test_algorithmic_flops_closed_form_vs_loop():
    for cfg in (wl.C0, wl.C1.replace(S=1000), wl.C2.replace(S=4096), wl.C1.replace(kind="swa", topk=0, S=300)):
        f = wl.layer_flops(cfg)
        keys = sum(wl.keys_per_query(cfg, t) for t in range(cfg.S))
        assert f["keys"] == keys
        vis = sum((t + 1) // cfg.ratio for t in range(cfg.S)) if cfg.kind != "swa" else 0
        assert f["visible_pairs"] == vis
    f3 = wl.layer_flops(wl.C3)
    assert abs(f3["indexer"] - 8.80e12) / 8.80e12 < 0.005
    assert abs(f3["attention"] - 5.43e12) / 5.43e12 < 0.005


def test_generator_is_seeded_and_shaped():
    a = wl.make_inputs(wl.C0)
    b = wl.make_inputs(wl.C0)
    for k in a:
        assert torch.equal(a[k], b[k])
    assert a["q"].shape == (1, 256, 4, 64) and a["q"].dtype == torch.float32
    assert a["k_idx"].shape == (1, 64, 16) and a["bias"].shape == (8, 64)
    rms = a["q"].pow(2).mean(-1).sqrt()
    assert torch.allclose(rms, torch.ones_like(rms), atol=1e-5)
    assert float(a["bias"].std()) < 0.2 and 0.0 <= float(a["w_idx"].min())
    small = wl.make_inputs(wl.C1.replace(S=64))
    assert small["q"].dtype == torch.bfloat16 and small["w_idx"].dtype == torch.float32
