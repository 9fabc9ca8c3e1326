"""GPU-versus-oracle parity of the indexer prologue, through the C ABI.

The prologue ("fix(deepseek-v4): correct V4-Flash attention math", Part 1 items 6a and
6e): partial RoPE of q_I at pos0 + t and of k_I at pos0 + s*ratio, then the normalised
Hadamard, rounded to the activation dtype, and the temperature (H_I * D_I)^-1/2 on the
head weights.  Acceptance as for the plain indexer: rotated keys equal the oracle's up to
the fp32 arithmetic of the transform (one unit in the last place plus 2^-16 of the
largest value; at most 1% of values differ); scores within 1e-4 of the row's largest; top-k
exact up to near-ties (1e-3 of the k-th score); layer outputs within the usual bounds.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_hca_amd import workloads as wl
from oracle import csa_oracle as O
from gpu_util import Lazy, check_selection, full_np, sample_rows
from test_gpu_parity import DEV, gen, layer_check

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def bd():
    from compressed_sparse_attention_hca_amd import binding
    return binding


def pro(cfg, **kw):
    return cfg.replace(index_prologue=True, name=cfg.name + "_pro", **kw)


KEY_CASES = {
    "C0": pro(wl.C0),
    "C1": pro(wl.C1),
    "C1_pos0": pro(wl.C1, pos0=999_999_937),
    "idx64_rope32_B2": pro(wl.C1, B=2, S=512, idx_dim=64, rope_dim=32, D=128),
    "idx32_norope": pro(wl.C1, S=256, idx_dim=32, rope_dim=0, D=64),
    "idx16_f32": pro(wl.C0, idx_dim=16, rope_dim=8, pos0=12345),
}


def oracle_keys(cfg, k_idx_b):
    n = k_idx_b.shape[0]
    pos = cfg.pos0 + np.arange(n, dtype=np.int64) * cfg.ratio
    return O.index_prologue(k_idx_b, pos, cfg.rope_dim, cfg.rope_theta, cfg.dtype)


def assert_rounded_alike(got, want, dtype, what):
    """Equal up to the fp32 arithmetic of the kernel's transform: every value within
    one unit in the last place of the activation dtype plus 2^-16 of the largest
    magnitude (cancellation leaves an absolute fp32 error of about 1e-6, which exceeds
    the ulp of a value near zero), and at most 1% of the values rounded to the
    neighbouring representable number."""
    scale = np.abs(want).max()
    diff = np.abs(got - want)
    if dtype == wl.F32:
        assert diff.max() <= 1e-6 * scale, f"{what}: {diff.max()}"
        return
    mag = np.maximum(np.abs(got), np.abs(want))
    ulp = np.ldexp(1.0, np.frexp(mag)[1] - 8)
    excess = diff - (ulp + 2.0 ** -16 * scale)
    k = np.unravel_index(np.argmax(excess), diff.shape)
    assert excess.max() <= 0, f"{what}: at {k} got {got[k]!r} want {want[k]!r}"
    assert np.count_nonzero(diff) <= diff.size // 100, f"{what}: {np.count_nonzero(diff)} of {diff.size} differ"


@pytest.mark.parametrize("name", list(KEY_CASES))
def test_key_prologue_parity(bd, name):
    cfg = KEY_CASES[name]
    inp = gen(cfg)
    kr = bd.index_keys(bd.params(cfg), inp["k_idx"])
    torch.cuda.synchronize()
    for b in range(cfg.B):
        got = kr[b].float().cpu().double().numpy()
        assert_rounded_alike(got, oracle_keys(cfg, Lazy(inp["k_idx"])[b]), cfg.dtype, f"keys {name} b{b}")


def oracle_scores(cfg, inp, b, t, k_rot):
    n = O.visible_entries(t, cfg.ratio)
    q = O.index_prologue(Lazy(inp["q_idx"])[b, t], cfg.pos0 + t, cfg.rope_dim, cfg.rope_theta, cfg.dtype)
    w = Lazy(inp["w_idx"])[b, t] * O.index_temperature(cfg.idx_heads, cfg.idx_dim)
    return O.indexer_scores_row(q, w, k_rot, n)


@pytest.mark.parametrize("name", ["C0", "C1", "idx64_rope32_B2"])
def test_prologue_scores_parity(bd, name):
    """csa_index_scores with the flag (queries rotated and weights scaled in-kernel) on
    keys from csa_index_keys, against the oracle's prologue scores."""
    cfg = KEY_CASES[name]
    inp = gen(cfg)
    p = bd.params(cfg)
    kr = bd.index_keys(p, inp["k_idx"])
    sc = bd.index_scores(p, inp["q_idx"], inp["w_idx"], kr)
    torch.cuda.synchronize()
    got = sc.cpu().double().numpy()
    rows = range(cfg.S) if cfg.S <= 512 else sorted(set(range(0, cfg.S, 7)) | {cfg.S - 1})
    rel = []
    for b in range(cfg.B):
        k_rot = oracle_keys(cfg, Lazy(inp["k_idx"])[b])
        for t in rows:
            want = oracle_scores(cfg, inp, b, t, k_rot)
            n = want.size
            if n:
                rel.append(float(np.abs(got[b, t, :n] - want).max() / np.abs(want).max()))
            assert np.all(np.isnan(got[b, t, n:]))
    # a rotated operand that rounds to the other neighbour moves one product term by an
    # ulp; rows of a few entries feel that most
    rel = np.array(rel)
    assert rel.max() <= 1e-3 and np.median(rel) <= 1e-4, (rel.max(), np.median(rel))


@pytest.mark.parametrize("name,topk", [("C0", None), ("C1", None), ("C1", 1024)])
def test_prologue_topk_parity(bd, name, topk):
    """csa_index_topk with the flag (the key prologue runs into the workspace), fused
    selection and, above 512, the chunked scores + selection path."""
    cfg = KEY_CASES[name] if topk is None else KEY_CASES[name].replace(S=8192, topk=topk)
    inp = gen(cfg)
    idx, nv = bd.index_topk(bd.params(cfg), inp["q_idx"], inp["w_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    idx, nv = idx.cpu().numpy(), nv.cpu().numpy()
    k_rot = oracle_keys(cfg, Lazy(inp["k_idx"])[0])
    rows = range(cfg.S) if topk is None else list(range(0, cfg.S, 97)) + [4095, 4096, 8191]
    swaps = 0
    for t in rows:
        n = O.visible_entries(t, cfg.ratio)
        assert nv[0, t] == n
        sc = oracle_scores(cfg, inp, 0, t, k_rot)
        swaps += check_selection(idx[0, t], n, cfg.topk, sc, O.topk_row(sc, cfg.topk))
    assert swaps <= max(2, len(rows) // 100), swaps


def test_prologue_changes_the_selection(bd):
    """The rotation changes which entries are picked (unlike the temperature alone): the
    selections with and without the prologue differ on most long rows."""
    cfg = wl.C1
    inp = gen(cfg)
    a, _ = bd.index_topk(bd.params(cfg), inp["q_idx"], inp["w_idx"], inp["k_idx"])
    b, _ = bd.index_topk(bd.params(pro(cfg)), inp["q_idx"], inp["w_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    differ = (a[0, 3000:] != b[0, 3000:]).any(dim=1).float().mean().item()
    assert differ > 0.9, differ


def test_prologue_layer_C0_full(bd):
    layer_check(bd, pro(wl.C0))


def test_prologue_layer_C1_sampled(bd):
    layer_check(bd, pro(wl.C1), sample_rows(wl.C1, 32))


def test_prologue_layer_C3_sampled(bd):
    """The metric's shape at full size, in the bench's launch configuration, with the
    prologue on."""
    layer_check(bd, pro(wl.C3), sample_rows(wl.C3, 16))


PRO_EDGE = [
    # ragged S, two batches, offset positions, rope over every indexer dim (fp32)
    dict(kind="csa", B=2, S=44, H=5, D=64, rope_dim=16, ratio=4, window=7, topk=3, idx_heads=3,
         idx_dim=16, dtype=wl.F32, pos0=1_000_003),
    # partial rope in the indexer (32 of 64 dims), heads padded, window beyond S
    dict(kind="csa", B=1, S=96, H=20, D=128, rope_dim=32, ratio=4, window=200, topk=5, idx_heads=40,
         idx_dim=64, dtype=wl.BF16, pos0=5),
    # no rope at all: Hadamard and temperature only; top-k covering every entry
    dict(kind="csa", B=1, S=64, H=16, D=256, rope_dim=0, ratio=2, window=1, topk=64, idx_heads=64,
         idx_dim=32, dtype=wl.BF16),
]


@pytest.mark.parametrize("i", range(len(PRO_EDGE)))
def test_prologue_edge_cases_full(bd, i):
    layer_check(bd, wl.LayerConfig(name=f"pro_edge{i}", seed=950 + i, index_prologue=True, **PRO_EDGE[i]))
