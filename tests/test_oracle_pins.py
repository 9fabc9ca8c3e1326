"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics.

None of these re-types the oracle's formula: each checks a closed form, an
invariant, a library special case, a printed constant, or the independent
pure-Python brute force.
"""
import math

import numpy as np
import pytest
import torch

from conftest import to_np
from compressed_sparse_attention_hca_amd import workloads as wl
from oracle import csa_oracle as O
from oracle import brute


def tiny(kind="csa", **kw):
    base = dict(name="t", kind=kind, B=1, S=32, H=2, D=16, rope_dim=8, ratio=4, window=6,
                topk=3, idx_heads=3, idx_dim=4, dtype=wl.F32, seed=7)
    if kind == "hca":
        base.update(ratio=8, topk=0)
    if kind == "swa":
        base.update(topk=0)
    base.update(kw)
    return wl.LayerConfig(**base)


# ---------------------------------------------------------------- pooling ----------

def test_pool_uniform_gates_zero_bias_is_plain_mean(rng):
    """Uniform gate logits and zero bias make pooling a plain mean of the tokens the
    entry covers; CSA entry 0 (no previous group) averages only its own 4 tokens."""
    S, D, r = 24, 5, 4
    va, vb = rng.normal(size=(S, D)), rng.normal(size=(S, D))
    g = np.full((S, D), 0.37)
    p = O.gated_pool(va, g, vb, g, np.zeros((2 * r, D)), r, True)
    assert np.allclose(p[0], va[0:4].mean(0), atol=1e-14)
    for s in range(1, S // r):
        want = (vb[s * r - r:s * r].sum(0) + va[s * r:s * r + r].sum(0)) / 8
        assert np.allclose(p[s], want, atol=1e-14)
    ph = O.gated_pool(va, g, None, None, np.zeros((8, D)), 8, False)
    for s in range(S // 8):
        assert np.allclose(ph[s], va[s * 8:s * 8 + 8].mean(0), atol=1e-14)


@pytest.mark.parametrize("j", range(8))
def test_pool_dominant_gate_selects_slot_token(rng, j):
    """A +60 gate on slot j makes the entry equal to that slot's token: slots 0-3 are
    the previous group from the b projections, slots 4-7 the own group from a."""
    S, D, r = 20, 3, 4
    va, vb = rng.normal(size=(S, D)), rng.normal(size=(S, D))
    ga, gb = np.zeros((S, D)), np.zeros((S, D))
    s = 3
    tok = s * r - r + j
    if j < r:
        gb[tok] = 60.0
        want = vb[tok]
    else:
        ga[tok] = 60.0
        want = va[tok]
    p = O.gated_pool(va, ga, vb, gb, np.zeros((8, D)), r, True)
    assert np.allclose(p[s], want, atol=1e-20 + 1e-12)


@pytest.mark.parametrize("j", [0, 3, 5, 7])
def test_pool_bias_row_is_slot(rng, j):
    """Bias row j weights slot j (token order), not a transposed or reversed row."""
    S, D, r = 16, 4, 4
    va, vb = rng.normal(size=(S, D)), rng.normal(size=(S, D))
    z = np.zeros((S, D))
    bias = np.zeros((8, D))
    bias[j] = 80.0
    p = O.gated_pool(va, z, vb, z, bias, r, True)
    s = 2
    want = vb[s * r - r + j] if j < r else va[s * r - r + j]
    assert np.allclose(p[s], want, atol=1e-12)


def test_pool_hca_ratio1_is_identity(rng):
    va = rng.normal(size=(9, 6))
    p = O.gated_pool(va, rng.normal(size=(9, 6)), None, None, rng.normal(size=(1, 6)), 1, False)
    assert np.array_equal(p, va)


def test_pool_convex_combination(rng):
    """Per channel the weights sum to 1: pooling constant values returns the constant."""
    S, D = 16, 7
    c = rng.normal(size=(1, D))
    v = np.repeat(c, S, axis=0)
    p = O.gated_pool(v, rng.normal(size=(S, D)), v, rng.normal(size=(S, D)),
                     rng.normal(size=(8, D)), 4, True)
    assert np.allclose(p, np.repeat(c, S // 4, axis=0), atol=1e-14)


# ------------------------------------------------------------ norm & RoPE ----------

def test_rms_norm_unit_rms(rng):
    x = rng.normal(size=(10, 64)) * 3
    n = O.rms_norm(x, 0.0)
    assert np.allclose(np.sqrt((n * n).mean(-1)), 1.0, atol=1e-14)
    n2 = O.rms_norm(x, 1e-6)
    ms = (x * x).mean(-1)
    assert np.allclose(np.sqrt((n2 * n2).mean(-1)), np.sqrt(ms / (ms + 1e-6)), atol=1e-14)


def test_rope_closed_form_interleaved_last_dims():
    """A unit pair (1, 0) at pair i comes out as (cos a, sin a), a = P*40000**(-2i/R);
    the first D-R dims are untouched (partial RoPE on the last dims, interleaved)."""
    D, R, P = 12, 8, 17
    for i in range(R // 2):
        x = np.zeros(D)
        x[:D - R] = np.arange(1, D - R + 1)
        x[D - R + 2 * i] = 1.0
        y = O.rope(x, P, R, 40000.0)
        a = P * 40000.0 ** (-(2 * i) / R)
        assert np.array_equal(y[:D - R], x[:D - R])
        assert abs(y[D - R + 2 * i] - math.cos(a)) < 1e-15
        assert abs(y[D - R + 2 * i + 1] - math.sin(a)) < 1e-15
        others = [k for k in range(D - R, D) if k not in (D - R + 2 * i, D - R + 2 * i + 1)]
        assert np.all(y[others] == 0)


def test_rope_inverse_zero_and_relative(rng):
    D, R = 32, 16
    x = rng.normal(size=(5, D))
    assert np.allclose(O.rope(O.rope(x, 12345, R, 4e4), -12345, R, 4e4), x, atol=1e-12)
    assert np.array_equal(O.rope(x, 0, R, 4e4), x)
    a, b = rng.normal(size=D), rng.normal(size=D)
    d1 = O.rope(a, 100, R, 4e4) @ O.rope(b, 37, R, 4e4)
    d2 = O.rope(a, 1063, R, 4e4) @ O.rope(b, 1000, R, 4e4)
    assert abs(d1 - d2) < 1e-11


def test_compressed_position_is_s_times_ratio():
    """Position probe (uses ratio > 1 and entry index > 0, where the two conventions
    differ): after pooling to a known vector, entry s carries rotation pos0 + s*r."""
    D, R, r, pos0 = 8, 4, 4, 5
    S = 16
    # every token's value is the same vector, so every pooled entry equals it
    base = np.array([1.0, -1.0, 1.0, -1.0, 1.0, 0.0, 1.0, 0.0])
    v = np.repeat(base[None], S, axis=0)
    z = np.zeros((S, D))
    kv = O.compress(v, z, v, z, np.zeros((8, D)), r, True, R, 40000.0, 0.0, pos0)
    rms = math.sqrt((base ** 2).mean())
    for s in range(S // r):
        P = pos0 + s * r
        for i in range(R // 2):
            a = P * 40000.0 ** (-(2 * i) / R)
            assert abs(kv[s, D - R + 2 * i] - math.cos(a) / rms) < 1e-14
            assert abs(kv[s, D - R + 2 * i + 1] - math.sin(a) / rms) < 1e-14
        wrong = pos0 + s
        if s > 0:
            assert abs(kv[s, D - R] - math.cos(wrong) / rms) > 1e-3


# ------------------------------------------------------------- indexer -------------

def test_indexer_hand_example():
    """I[t,s] = sum_h w_h ReLU(q_h . k_s) on a hand-computed case."""
    q = np.array([[1.0, 2.0], [-1.0, 0.5]])  # 2 heads x 2 dims
    w = np.array([0.5, 2.0])
    k = np.array([[1.0, 1.0], [2.0, -1.0], [-3.0, 1.0]])
    # head0 dots: 3, 0, -1 -> relu 3, 0, 0 ; head1 dots: -0.5, -2.5, 3.5 -> 0, 0, 3.5
    want = np.array([0.5 * 3, 0.0, 2.0 * 3.5])
    assert np.allclose(O.indexer_scores_row(q, w, k, 3), want, atol=0)
    assert np.allclose(O.indexer_scores_row(q, w, k, 2), want[:2], atol=0)


def test_indexer_block_matches_rows(rng):
    """The block form gives, row by row, the pinned per-row scores (hand example
    included), for ragged visible counts."""
    q = np.array([[[1.0, 2.0], [-1.0, 0.5]]])
    w = np.array([[0.5, 2.0]])
    k = np.array([[1.0, 1.0], [2.0, -1.0], [-3.0, 1.0]])
    assert np.array_equal(O.indexer_scores_block(q, w, k, [3])[0], np.array([1.5, 0.0, 7.0]))
    R, HI, DI, n = 9, 5, 12, 40
    q, w, k = rng.normal(size=(R, HI, DI)), rng.uniform(size=(R, HI)), rng.normal(size=(n, DI))
    nv = [0, 1, 7, 40, 13, 0, 39, 2, 40]
    got = O.indexer_scores_block(q, w, k, nv)
    for r in range(R):
        want = O.indexer_scores_row(q[r], w[r], k, nv[r])
        assert got[r].shape == (nv[r],)
        assert np.allclose(got[r], want, rtol=1e-13, atol=1e-13)
    # scalar loops (a third transcription of the definition)
    r = 3
    for s_ in range(0, 40, 7):
        acc = 0.0
        for h in range(HI):
            d = sum(q[r, h, j] * k[s_, j] for j in range(DI))
            acc += w[r, h] * max(d, 0.0)
        assert abs(got[r][s_] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_visibility_and_window_layout():
    assert [O.visible_entries(t, 4) for t in range(10)] == [0, 0, 0, 1, 1, 1, 1, 2, 2, 2]
    assert O.visible_entries(127, 128) == 1 and O.visible_entries(126, 128) == 0
    assert O.window_bounds(0, 128) == (0, 0)
    assert O.window_bounds(200, 128) == (73, 200)


def test_topk_ties_and_small_rows():
    sc = np.array([1.0, 3.0, 3.0, 2.0, 3.0])
    assert list(O.topk_row(sc, 2)) == [1, 2]
    assert list(O.topk_row(sc, 4)) == [1, 2, 3, 4]
    assert list(O.topk_row(sc, 9)) == [0, 1, 2, 3, 4]
    assert list(O.topk_row(np.zeros(0), 3)) == []


def test_topk_matches_python_sorted(rng):
    for n in [1, 5, 50, 300]:
        sc = np.round(rng.normal(size=n), 1)  # many exact ties
        k = 17
        want = sorted(sorted(range(n), key=lambda j: (-sc[j], j))[:k])
        assert list(O.topk_row(sc, k)) == want


def test_topk_invariant_to_positive_weight_scale(rng):
    """Scaling every head weight by c > 0 (e.g. the 1/90.5 temperature) leaves the
    selection unchanged."""
    q, k = rng.normal(size=(4, 8)), rng.normal(size=(40, 8))
    w = rng.uniform(size=4)
    a = O.topk_row(O.indexer_scores_row(q, w, k, 40), 7)
    b = O.topk_row(O.indexer_scores_row(q, w / 90.5, k, 40), 7)
    assert np.array_equal(a, b)


# ----------------------------------------------------------- attention -------------

def _sdpa_causal(q, k, v, scale):
    """torch fp64 SDPA, q [S,H,D], k,v [S,D] shared across heads (MQA)."""
    qt = torch.from_numpy(q).permute(1, 0, 2)[None]  # [1,H,S,D]
    H = q.shape[1]
    kt = torch.from_numpy(k)[None, None].expand(1, H, -1, -1).contiguous()
    vt = torch.from_numpy(v)[None, None].expand(1, H, -1, -1).contiguous()
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def test_hca_ratio1_no_rope_is_causal_sdpa(rng):
    """Library special case: ratio 1 disjoint pooling of unit-RMS rows (eps 0) with no
    window and no RoPE is plain causal multi-query attention over the entries."""
    S, H, D = 24, 3, 8
    va = rng.choice([-1.0, 1.0], size=(S, D))
    cfg = tiny("hca", S=S, H=H, D=D, rope_dim=0, ratio=1, window=0, rms_eps=0.0)
    # window 0 means no window keys; the oracle's window_bounds(t, 0) is (t+1, t): empty
    inp = {"va": va[None], "ga": rng.normal(size=(1, S, D)), "bias": rng.normal(size=(1, D)),
           "q": rng.normal(size=(1, S, H, D)), "kv_raw": rng.normal(size=(1, S, D))}
    out = O.layer_forward(cfg, inp)["o_full"][0]
    want = _sdpa_causal(inp["q"][0], va, va, D ** -0.5)
    assert np.allclose(out, want, atol=1e-12)


def test_swa_full_window_no_rope_is_causal_sdpa(rng):
    S, H, D = 20, 2, 8
    cfg = tiny("swa", S=S, H=H, D=D, rope_dim=0, window=S)
    inp = {"q": rng.normal(size=(1, S, H, D)), "kv_raw": rng.normal(size=(1, S, D))}
    out = O.layer_forward(cfg, inp)["o_full"][0]
    want = _sdpa_causal(inp["q"][0], inp["kv_raw"][0], inp["kv_raw"][0], D ** -0.5)
    assert np.allclose(out, want, atol=1e-12)


def test_swa_with_rope_matches_sdpa_on_rotated_then_derotated(rng):
    """With RoPE: SDPA on queries rotated at t and keys rotated at t', then the output
    rotated back at -t, equals the layer (the de-rotation step of the output)."""
    S, H, D, R = 16, 2, 8, 4
    cfg = tiny("swa", S=S, H=H, D=D, rope_dim=R, window=S, pos0=3)
    inp = {"q": rng.normal(size=(1, S, H, D)), "kv_raw": rng.normal(size=(1, S, D))}
    out = O.layer_forward(cfg, inp)["o_full"][0]
    t = np.arange(S) + 3
    qr = O.rope(inp["q"][0], t[:, None], R, 4e4)
    kr = O.rope(inp["kv_raw"][0], t, R, 4e4)
    u = _sdpa_causal(qr, kr, kr, D ** -0.5)
    want = O.rope(u, -t[:, None], R, 4e4)
    assert np.allclose(out, want, atol=1e-12)


def test_t0_output_is_raw_latent():
    """Closed form: at t = 0 no entry is visible (ratio > 1) and the window holds only
    token 0, so o[0,h] = RoPE(RoPE(x0, pos0), -pos0) = x0 for every head."""
    cfg = tiny("csa", pos0=977)
    inp = to_np(wl.make_inputs(cfg))
    r = O.layer_rows(cfg, inp, [(0, 0)])
    for h in range(cfg.H):
        assert np.allclose(r["o"][(0, 0)][h], inp["kv_raw"][0, 0], atol=1e-13)


def test_uniform_logits_average_union_of_keys():
    """Zero queries make every logit 0: the output is the plain mean over the union of
    selected entries and window keys (one softmax), de-rotated."""
    cfg = tiny("hca", S=40, window=5)
    inp = to_np(wl.make_inputs(cfg))
    inp["q"][:] = 0.0
    rows = [(0, t) for t in (4, 15, 16, 39)]
    r = O.layer_rows(cfg, inp, rows)
    kv_c = r["kv_c"][0]
    for (b, t) in rows:
        n = O.visible_entries(t, cfg.ratio)
        lo = max(0, t - cfg.window + 1)
        wk = O.rope(inp["kv_raw"][0, lo:t + 1], np.arange(lo, t + 1), cfg.rope_dim, 4e4)
        keys = np.concatenate([kv_c[:n], wk])
        want = O.rope(keys.mean(0), -t, cfg.rope_dim, 4e4)
        assert np.allclose(r["o"][(b, t)], want[None].repeat(cfg.H, 0), atol=1e-13)
        assert len(keys) == n + min(cfg.window, t + 1)


def test_position_shift_invariance():
    """Shifting pos0 by a multiple of the ratio leaves attention probabilities and the
    de-rotated output unchanged."""
    cfg = tiny("csa", S=48)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(0, 48, 5)]
    a = O.layer_rows(cfg, inp, rows, want_p=True)
    b = O.layer_rows(cfg.replace(pos0=4 * 1013), inp, rows, want_p=True)
    for k in rows:
        assert np.allclose(a["P"][k], b["P"][k], atol=1e-10)
        assert np.allclose(a["o"][k], b["o"][k], atol=1e-10)


def test_csa_with_topk_covering_all_equals_dense():
    """With top-k >= visible entries for every query, CSA equals dense attention over
    all visible entries."""
    cfg = tiny("csa", S=48, topk=64)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(48)]
    a = O.layer_rows(cfg, inp, rows)
    dense_sel = {(0, t): np.arange(O.visible_entries(t, 4)) for t in range(48)}
    b = O.layer_rows(cfg, inp, rows, sel_override=dense_sel)
    for k in rows:
        assert np.array_equal(a["sel"][k], dense_sel[k])
        assert np.allclose(a["o"][k], b["o"][k], atol=0)


# ---------------------------------------------------------------- sink -------------
# The softmax sink: one fp32 logit per head that joins the softmax with no value
# ("Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus",
# "Kernel fusions", row "SWA / CSA / HCA attention"; "fix(deepseek-v4)", Part 1 item 6f).

def test_sink_closed_form_scales_the_uniform_average():
    """Zero queries make every logit 0.  A sink of ln(n * c) for n keys gives every key
    probability 1 / (n (1 + c)), so the output is the plain mean divided by 1 + c."""
    cfg = tiny("hca", S=40, H=3, window=5)
    inp = to_np(wl.make_inputs(cfg))
    inp["q"][:] = 0.0
    t = 21
    n = O.visible_entries(t, cfg.ratio) + min(cfg.window, t + 1)
    c = np.array([0.5, 1.0, 3.0])
    r0 = O.layer_rows(cfg, inp, [(0, t)])
    r1 = O.layer_rows(cfg, inp, [(0, t)], sinks=np.log(n * c))
    for h in range(cfg.H):
        assert np.allclose(r1["o"][(0, t)][h], r0["o"][(0, t)][h] / (1.0 + c[h]), atol=1e-13)


def test_sink_minus_infinity_is_no_sink_and_large_sink_silences():
    cfg = tiny("csa", S=48)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in (3, 17, 47)]
    a = O.layer_rows(cfg, inp, rows, want_p=True)
    b = O.layer_rows(cfg, inp, rows, want_p=True, sinks=np.full(cfg.H, -np.inf))
    c = O.layer_rows(cfg, inp, rows, sinks=np.full(cfg.H, 800.0))
    for k in rows:
        assert np.array_equal(a["o"][k], b["o"][k]) and np.array_equal(a["P"][k], b["P"][k])
        assert np.abs(c["o"][k]).max() == 0.0  # exp(z - 800) underflows: all mass on the sink
        assert np.all(np.asarray(b["P"][k]).sum(1) <= 1.0 + 1e-12)


def test_sink_with_no_key_gives_zero():
    """No key at all (window 0, t < ratio - 1): with a sink the softmax is defined and
    all of its mass is on the sink, so the output is 0."""
    cfg = tiny("hca", S=16, ratio=8, window=0)
    inp = to_np(wl.make_inputs(cfg))
    r = O.layer_rows(cfg, inp, [(0, 3)], sinks=np.zeros(cfg.H))
    assert np.array_equal(r["o"][(0, 3)], np.zeros((cfg.H, cfg.D)))


@pytest.mark.parametrize("kind", ["csa", "hca", "swa"])
def test_oracle_with_sink_matches_brute_force(kind, rng):
    cfg = tiny(kind, S=24, pos0=5)
    inp = to_np(wl.make_inputs(cfg))
    sinks = rng.normal(size=cfg.H) * 2.0
    ora = O.layer_forward(cfg, inp, sinks=sinks)
    bf = brute.brute_layer(cfg, inp, sinks=sinks)
    assert np.allclose(ora["o_full"][0], np.array(bf["o"]), atol=1e-12)


# ------------------------------------------------------------ brute force ----------

@pytest.mark.parametrize("kind", ["csa", "hca", "swa"])
def test_oracle_matches_brute_force(kind):
    cfg = tiny(kind, S=32, pos0=9 if kind != "swa" else 2, norm_window=(kind == "hca"))
    inp = to_np(wl.make_inputs(cfg))
    ora = O.layer_forward(cfg, inp)
    bf = brute.brute_layer(cfg, inp)
    assert np.allclose(ora["o_full"][0], np.array(bf["o"]), atol=1e-12)
    for t in range(cfg.S):
        assert list(ora["sel"][(0, t)]) == bf["sel"][t]
        if kind == "csa":
            assert np.allclose(ora["scores"][(0, t)], bf["scores"][t], atol=1e-12)
    if kind != "swa":
        assert np.allclose(ora["kv_c"][0], np.array(bf["kv_c"]), atol=1e-13)


def test_keys_per_query_matches_pages():
    """Keys per query: min(K, n_t) + min(W, t+1).  At long context CSA reads 512 + 128
    = 640 keys and HCA at 1M tokens reads 10^6/128 + 128, about 7,900 ("Three
    attention types, interleaved")."""
    c1 = wl.C1
    assert wl.keys_per_query(c1, 4095) == 640
    hca_1m = wl.C2.replace(S=1_000_448)
    assert abs(wl.keys_per_query(hca_1m, hca_1m.S - 1) - 7900) < 100


# ---------------------------------------------------- indexer prologue ----------
# "fix(deepseek-v4): correct V4-Flash attention math", Part 1 items 6a (temperature
# folded into the head weights) and 6e (partial RoPE at the compressed base, queries at
# t and keys at s*ratio, then a normalised Hadamard, indexer only).

def popcount(x):
    return bin(x).count("1")


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 32, 64, 128])
def test_hadamard_is_the_walsh_matrix_and_orthogonal(n):
    """Sylvester's matrix has entry (-1)^popcount(i & j); H H^T = n I exactly in fp64
    (the pages' test list pins the Hadamard's orthogonality in float64); and it is the
    matrix scipy builds."""
    import scipy.linalg
    H = O.hadamard(n)
    walsh = np.array([[(-1.0) ** popcount(i & j) for j in range(n)] for i in range(n)])
    assert np.array_equal(H, walsh)
    assert np.array_equal(H @ H.T, n * np.eye(n))
    assert np.array_equal(H, scipy.linalg.hadamard(n).astype(np.float64))


def test_round_to_matches_torch_casts_and_ties_to_even(rng):
    """For values that are exactly fp32, rounding to bf16 is torch's fp32 -> bf16 cast
    (round to nearest even), subnormals included; fp32 rounding is numpy's cast."""
    x32 = np.concatenate([rng.normal(size=4000) * 10.0 ** rng.integers(-6, 6, size=4000),
                          rng.normal(size=200) * 1e-39, [0.0, -0.0, 1.0, -2.5]]).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to(x32.astype(np.float64), "bf16"), want)
    # ties go to the even neighbour: 1 + 2^-8 -> 1; 1 + 3 * 2^-8 -> 1 + 2^-6
    got = O.round_to(np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)]), "bf16")
    assert list(got) == [1.0, 1 + 2.0 ** -6, -1.0]
    x = rng.normal(size=100)
    assert np.array_equal(O.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_index_temperature_constant():
    """At Flash widths (64 heads x 128) the temperature is a factor of about 90.5."""
    assert abs(1.0 / O.index_temperature(64, 128) - 90.5) < 0.05
    assert O.index_temperature(4, 16) == 0.125


@pytest.mark.parametrize("P", [0, 37, 65535, 1_000_003])
def test_index_prologue_unit_pair_closed_form(P):
    """A unit pair (1, 0) on the last rope pair becomes (cos phi, sin phi) with
    phi = P * theta^-(R-2)/R, and the normalised Hadamard then gives every component i
    the value (cos phi (-1)^popcount(i & (n-2)) + sin phi (-1)^popcount(i & (n-1))) /
    sqrt(n).  A component outside the rope dims is not rotated: a unit vector on dim 0
    becomes the constant 1/sqrt(n)."""
    n, R, theta = 16, 8, 40000.0
    x = np.zeros(n)
    x[n - 2] = 1.0
    phi = P * theta ** (-(R - 2) / R)
    y = O.index_prologue(x, P, R, theta, "f32")
    for i in range(n):
        want = (math.cos(phi) * (-1) ** popcount(i & (n - 2)) + math.sin(phi) * (-1) ** popcount(i & (n - 1))) / 4
        assert abs(y[i] - want) < 1e-7
    e0 = np.zeros(n)
    e0[0] = 1.0
    assert np.allclose(O.index_prologue(e0, P, R, theta, "f32"), 0.25, atol=1e-12)
    yb = O.index_prologue(x, P, R, theta, "bf16")
    assert np.array_equal(O.round_to(yb, "bf16"), yb)        # bf16-representable
    assert np.abs(yb - y).max() < 2.0 ** -9                  # and the nearest such value


def prologue_cfg(**kw):
    base = dict(idx_dim=16, rope_dim=8, idx_heads=3, index_prologue=True)
    base.update(kw)
    return tiny("csa", **base)


@pytest.mark.parametrize("pos0", [0, 1000])
def test_prologue_scores_follow_relative_position(pos0):
    """Unit pairs on the last rope pair of every q_I head and every k_I entry, w = 1:
    the Hadamard keeps inner products, so I[t,s] = H_I * T * ReLU(cos((t - s*r) f)),
    with T = (H_I * D_I)^-1/2 and f = theta^-(R-2)/R, for any pos0."""
    cfg = prologue_cfg(S=64, pos0=pos0, topk=64)
    inp = to_np(wl.make_inputs(cfg))
    n = cfg.idx_dim
    inp["q_idx"][:] = 0.0
    inp["q_idx"][..., n - 2] = 1.0
    inp["k_idx"][:] = 0.0
    inp["k_idx"][..., n - 2] = 1.0
    inp["w_idx"][:] = 1.0
    f = cfg.rope_theta ** (-(cfg.rope_dim - 2) / cfg.rope_dim)
    T = (cfg.idx_heads * cfg.idx_dim) ** -0.5
    rows = [(0, t) for t in (3, 17, 40, 63)]
    r = O.layer_rows(cfg, inp, rows)
    for (_, t) in rows:
        sc = r["scores"][(0, t)]
        want = [cfg.idx_heads * T * max(0.0, math.cos((t - s * cfg.ratio) * f)) for s in range(len(sc))]
        assert np.allclose(sc, want, atol=1e-6)


def test_prologue_pos0_shift_keeps_scores():
    """Queries and keys move together under a pos0 shift, so the scores keep their
    values up to the fp32 rounding of the rotated vectors."""
    cfg = prologue_cfg(S=48)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(3, 48, 4)]
    a = O.layer_rows(cfg, inp, rows)
    b = O.layer_rows(cfg.replace(pos0=4 * 12345), inp, rows)
    for k in rows:
        assert np.allclose(a["scores"][k], b["scores"][k], rtol=1e-5, atol=1e-6)


def test_prologue_changes_scores_but_temperature_alone_does_not_change_selection():
    """Without RoPE (R = 0) the rotated scores are the plain scores times the
    temperature, up to the rounding of the Hadamard outputs; the selection then agrees
    except at near-ties.  With RoPE the scores change."""
    cfg0 = prologue_cfg(S=64, index_prologue=False, topk=5)
    inp = to_np(wl.make_inputs(cfg0))
    rows = [(0, t) for t in range(7, 64, 8)]
    plain = O.layer_rows(cfg0, inp, rows)
    T = (cfg0.idx_heads * cfg0.idx_dim) ** -0.5
    # rope_dim 0 leaves only the Hadamard and the temperature (main layer keys unrotated too)
    nr = O.layer_rows(cfg0.replace(index_prologue=True, rope_dim=0), inp, rows)
    for k in rows:
        assert np.allclose(nr["scores"][k], T * plain["scores"][k], rtol=1e-5, atol=1e-6)
    wr = O.layer_rows(cfg0.replace(index_prologue=True), inp, rows)
    assert max(np.abs(wr["scores"][k] - T * plain["scores"][k]).max() for k in rows) > 1e-2


@pytest.mark.parametrize("dtype", [wl.F32, wl.BF16])
def test_prologue_oracle_matches_brute_force(dtype):
    cfg = prologue_cfg(S=24, pos0=7, dtype=dtype)
    inp = to_np(wl.make_inputs(cfg))
    ora = O.layer_forward(cfg, inp)
    bf = brute.brute_layer(cfg, inp)
    for t in range(cfg.S):
        assert np.allclose(ora["scores"][(0, t)], bf["scores"][t], atol=1e-12)
        assert list(ora["sel"][(0, t)]) == bf["sel"][t]
    assert np.allclose(ora["o_full"][0], np.array(bf["o"]), atol=1e-12)


# -------------------------------------------------------------- FP8 indexer ----------
# "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus",
# closing remarks (an E4M3 path for the indexer QK); "fix(deepseek-v4): correct
# V4-Flash attention math", Part 1 item 4 (quantization changes the selection).

def test_e4m3_matches_torch_cast_and_the_code_table(rng):
    """Rounding to E4M3 is torch's float8_e4m3fn cast (round to nearest even) on
    in-range fp32 values, normal and subnormal, and the table search of the brute force."""
    x = np.concatenate([rng.normal(size=3000) * 60.0, rng.normal(size=1000) * 2.0 ** -8,
                        [448.0, -448.0, 0.0, 2.0 ** -9, 3 * 2.0 ** -10, 1.0625, 1.1875]])
    x32 = x[np.abs(x) < 440].astype(np.float32)
    want = torch.from_numpy(x32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = O.e4m3(x32.astype(np.float64))
    assert np.array_equal(got, want)
    assert np.array_equal(got[:300], [brute.brute_e4m3(float(v)) for v in x32[:300]])
    # ties: 1 + 1/16 is halfway between 1 and 1.125 -> 1 (even); 1.1875 -> 1.25
    assert list(O.e4m3(np.array([1.0625, 1.1875, 3 * 2.0 ** -10]))) == [1.0, 1.25, 2.0 ** -8]


def test_quant_rows_closed_forms():
    """The largest magnitude of a row maps to +-448 and the scale is absmax / 448;
    values that are E4M3 numbers times the scale come back exactly; a zero row has
    codes 0 and scale 0; scaling a row by a power of two keeps its codes."""
    row = np.array([[3.5, -1.75, 0.4375, 0.0, 2.0 ** -7]]) * 0.5
    codes, sc = O.quant_e4m3_rows(row)
    assert codes[0, 0] == 448.0 and sc[0] == np.float32(1.75 / 448.0)
    assert np.allclose(codes[0] * sc[0], row[0], rtol=0, atol=1e-12)
    z, zs = O.quant_e4m3_rows(np.zeros((2, 8)))
    assert not z.any() and not zs.any()
    r = np.random.default_rng(3).normal(size=(4, 64)).astype(np.float32)
    c1, s1 = O.quant_e4m3_rows(r)
    c2, s2 = O.quant_e4m3_rows(r * np.float32(8.0))
    assert np.array_equal(c1, c2) and np.array_equal(s2, s1 * 8)


def test_quant_rows_error_bound_and_brute_force(rng):
    """Decoding loses at most half a unit of the 3-bit mantissa (2^-4 relative) plus
    half the subnormal spacing (2^-10 times the scale); the brute force's per-step fp32
    quantization gives the same codes and scales."""
    x = (rng.normal(size=(16, 128)) * np.exp(rng.normal(size=(16, 1)))).astype(np.float32).astype(np.float64)
    codes, sc = O.quant_e4m3_rows(x)
    err = np.abs(codes * sc[:, None] - x)
    assert np.all(err <= 2.0 ** -4 * np.abs(x) + 2.0 ** -10 * sc[:, None] * 1.0000001)
    for i in range(4):
        bc, bs = brute.brute_quant_row(list(x[i]))
        assert list(codes[i]) == bc and sc[i] == bs


@pytest.mark.parametrize("prologue", [False, True])
def test_fp8_indexer_oracle_matches_brute_force(prologue):
    cfg = tiny("csa", S=24, pos0=3, idx_dim=16, rope_dim=8, idx_heads=3, dtype=wl.BF16,
               index_fp8=True, index_prologue=prologue)
    inp = to_np(wl.make_inputs(cfg))
    ora = O.layer_forward(cfg, inp)
    bf = brute.brute_layer(cfg, inp)
    for t in range(cfg.S):
        assert np.allclose(ora["scores"][(0, t)], bf["scores"][t], atol=1e-12)
        assert list(ora["sel"][(0, t)]) == bf["sel"][t]
    assert np.allclose(ora["o_full"][0], np.array(bf["o"]), atol=1e-12)


def test_fp8_scores_track_the_exact_scores():
    """The quantized scores stay within the error bound of the operands (each element
    within 2^-4 of itself plus 2^-10 of its row scale; ReLU and the positive weights
    do not enlarge the difference), and most of the selection survives."""
    cfg = tiny("csa", S=256, idx_dim=64, rope_dim=8, idx_heads=8, topk=16, dtype=wl.BF16)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(150, 256, 15)]
    a = O.layer_rows(cfg, inp, rows)
    b = O.layer_rows(cfg.replace(index_fp8=True), inp, rows)
    q, k, w = inp["q_idx"][0], inp["k_idx"][0], inp["w_idx"][0]
    keep = []
    for (_, t) in rows:
        n = len(a["scores"][(0, t)])
        # per element |error| <= 2^-4 |x| + 2^-10 * scale (normal and subnormal range)
        sq = np.abs(q[t]).max(1, keepdims=True) / 448
        sk = np.abs(k[:n]).max(1, keepdims=True) / 448
        eq, ek = 2.0 ** -4 * np.abs(q[t]) + 2.0 ** -10 * sq, 2.0 ** -4 * np.abs(k[:n]) + 2.0 ** -10 * sk
        dot_err = eq @ (np.abs(k[:n]) + ek).T + np.abs(q[t]) @ ek.T
        bound = np.abs(w[t]) @ dot_err * 1.001
        assert np.all(np.abs(b["scores"][(0, t)] - a["scores"][(0, t)]) <= bound)
        keep.append(len(set(a["sel"][(0, t)]) & set(b["sel"][(0, t)])) / cfg.topk)
    assert np.mean(keep) > 0.6


# ----------------------------------------------------------- KL target ----------
# "fix(deepseek-v4): correct V4-Flash attention math", Part 1 items 5 and 11.

def test_kl_target_closed_forms(rng):
    """Zero queries give the uniform target 1/|Sel|; one selected entry gets 1; the
    target sums to 1 and is positive; relabelling the selection permutes it."""
    H, D, n = 3, 16, 9
    kv = rng.normal(size=(n, D))
    sel = np.array([1, 4, 5, 8])
    assert np.allclose(O.kl_target_row(np.zeros((H, D)), kv, sel, 0.25), 0.25, atol=1e-15)
    q = rng.normal(size=(H, D))
    assert np.allclose(O.kl_target_row(q, kv, [6], 0.25), [1.0], atol=1e-15)
    t = O.kl_target_row(q, kv, sel, 0.25)
    assert abs(t.sum() - 1) < 1e-14 and np.all(t > 0)
    perm = np.array([2, 0, 3, 1])
    assert np.allclose(O.kl_target_row(q, kv, sel[perm], 0.25), t[perm], atol=1e-15)


def test_kl_target_is_the_attention_restricted_to_the_selection():
    """Without a window the layer's softmax runs over the selected entries alone, so the
    target is the head mean of the layer's own probabilities P."""
    cfg = tiny("csa", S=40, window=0, topk=4)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in (7, 23, 39)]
    r = O.layer_rows(cfg, inp, rows, want_p=True)
    kt = O.kl_target(cfg, inp, rows, r["sel"], r["kv_c"])
    for k in rows:
        assert np.allclose(kt[k], np.mean(r["P"][k], axis=0), atol=1e-14)


def test_kl_target_reading_with_a_window():
    """With a window the layer's softmax also covers the window keys, and two readings
    of "the attention over the selected entries" part ways: (A) each head's
    probabilities restricted to the selection and renormalised per head, then the mean
    over heads (the same as a softmax over the selected entries alone); (B) the head
    sum of the restricted probabilities, L1-normalised.  The target is (A): the page's
    target branch gathers only the selected entries ([B, S, K, head_dim], item 11) and
    sums heads over softmaxes formed from those gathered logits.  Here the two differ
    by more than 1e-2, so a target built as (B) fails this pin."""
    cfg = tiny("csa", S=40, window=6, topk=4, H=4)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in (11, 23, 39)]
    r = O.layer_rows(cfg, inp, rows, want_p=True)
    kt = O.kl_target(cfg, inp, rows, r["sel"], r["kv_c"])
    sep = 0.0
    for k in rows:
        m = len(r["sel"][k])
        ps = r["P"][k][:, :m]  # the selected entries come first in the layer's key list
        a = np.mean(ps / ps.sum(axis=1, keepdims=True), axis=0)
        b_ = ps.sum(axis=0) / ps.sum()
        assert np.allclose(kt[k], a, atol=1e-14)
        sep = max(sep, float(np.max(np.abs(a - b_))))
    assert sep > 1e-2, sep


def test_kl_target_matches_brute_force():
    cfg = tiny("csa", S=24, pos0=11)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(3, 24, 4)]
    r = O.layer_rows(cfg, inp, rows)
    kt = O.kl_target(cfg, inp, rows, r["sel"], r["kv_c"])
    for (b, t) in rows:
        want = brute.brute_kl_target(cfg, inp, r["kv_c"][0], t, list(r["sel"][(b, t)]))
        assert np.allclose(kt[(b, t)], want, atol=1e-13)


# ------------------------------------------------------------ dQ backward ----------
# "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus",
# "Attention kernels for the three layer types": the backward's dQ kernel with delta.

@pytest.mark.parametrize("kind,with_sink", [("csa", False), ("hca", False), ("swa", False), ("csa", True)])
def test_dq_matches_finite_differences(kind, with_sink, rng):
    """Central differences of the forward oracle's loss L = sum(o * do) in each query
    coordinate (the selection is held fixed, as the backward holds it)."""
    cfg = tiny(kind, S=24, pos0=5, H=2, D=8, rope_dim=4)
    inp = to_np(wl.make_inputs(cfg))
    t = 17
    rows = [(0, t)]
    base = O.layer_rows(cfg, inp, rows)
    sel = base["sel"]
    do = {(0, t): rng.normal(size=(cfg.H, cfg.D))}
    sinks = rng.normal(size=cfg.H) if with_sink else None
    dq = O.layer_dq_rows(cfg, inp, rows, do, sel, base["kv_c"], sinks=sinks)[(0, t)]
    eps = 1e-6
    for h in range(cfg.H):
        for d in range(cfg.D):
            qp, qm = inp["q"].copy(), inp["q"].copy()
            qp[0, t, h, d] += eps
            qm[0, t, h, d] -= eps
            lp = np.sum(O.layer_rows(cfg, dict(inp, q=qp), rows, sel_override=sel,
                                     sinks=sinks)["o"][(0, t)] * do[(0, t)])
            lm = np.sum(O.layer_rows(cfg, dict(inp, q=qm), rows, sel_override=sel,
                                     sinks=sinks)["o"][(0, t)] * do[(0, t)])
            assert abs((lp - lm) / (2 * eps) - dq[h, d]) < 1e-7


def test_dq_matches_torch_autograd(rng):
    """torch autograd through an fp64 softmax attention written with torch ops."""
    H, D, nk, scale = 3, 16, 11, 0.25
    q = rng.normal(size=(H, D))
    keys = rng.normal(size=(nk, D))
    du = rng.normal(size=(H, D))
    qt = torch.tensor(q, requires_grad=True)
    kt = torch.tensor(keys)
    u = torch.softmax((qt @ kt.T) * scale, dim=1) @ kt
    (u * torch.tensor(du)).sum().backward()
    dqr, delta = O.attend_row_bwd_dq(q, keys, scale, du)
    assert np.allclose(dqr, qt.grad.numpy(), atol=1e-12)
    assert np.allclose(delta, np.sum(u.detach().numpy() * du, axis=1), atol=1e-12)


def test_dq_closed_forms(rng):
    """One key: the softmax is constant, so dq = 0; equal keys: likewise; delta is
    rowsum(u * du)."""
    H, D = 2, 6
    q, du = rng.normal(size=(H, D)), rng.normal(size=(H, D))
    k1 = rng.normal(size=(1, D))
    dq, delta = O.attend_row_bwd_dq(q, k1, 0.5, du)
    assert np.allclose(dq, 0, atol=1e-15) and np.allclose(delta, du @ k1[0], atol=1e-15)
    dq2, _ = O.attend_row_bwd_dq(q, np.repeat(k1, 4, axis=0), 0.5, du)
    assert np.allclose(dq2, 0, atol=1e-14)


# ----------------------------------------------------- key-side backward -----------
# "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with Primus",
# "Attention kernels for the three layer types": interm, the contraction over heads
# that gives each key's gradient; "fix(deepseek-v4): correct V4-Flash attention
# math", Part 1 item 6f: the sink is an fp32 logit of the softmax.

def _loss(cfg, inp, rows, sel, kv_c, do, sinks):
    r = O.layer_rows(cfg, inp, rows, sel_override=sel, kv_c=kv_c, sinks=sinks)
    return sum(float(np.sum(r["o"][k] * do[k])) for k in rows)


@pytest.mark.parametrize("kind,with_sink,norm_window", [
    ("csa", False, False), ("csa", True, False), ("hca", True, False), ("swa", False, True),
    ("csa", True, True)])
def test_key_grads_match_finite_differences(kind, with_sink, norm_window, rng):
    """Central differences of L = sum over every row of sum(o * do), through the
    forward oracle, in sampled coordinates of the rotated entries kv_c, of the raw
    window latents kv_raw (each feeds the windows of up to W queries) and in every
    sink.  The selection is held fixed, as the backward holds it."""
    cfg = tiny(kind, S=24, pos0=5, H=2, D=8, rope_dim=4, window=5, norm_window=norm_window)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(cfg.S)]
    base = O.layer_rows(cfg, inp, rows)
    sel, kv_c = base["sel"], base["kv_c"]
    do = {k: rng.normal(size=(cfg.H, cfg.D)) for k in rows}
    sinks = rng.normal(size=cfg.H) if with_sink else None
    g = O.layer_bwd_rows(cfg, inp, rows, do, sel, kv_c, sinks=sinks)
    eps = 1e-6

    def fd(edit):
        return (_loss(*edit(+eps)) - _loss(*edit(-eps))) / (2 * eps)

    if kind != "swa":
        n = kv_c[0].shape[0]
        for _ in range(12):
            s, d = int(rng.integers(0, n)), int(rng.integers(0, cfg.D))

            def edit(e, s=s, d=d):
                kv = {0: kv_c[0].copy()}
                kv[0][s, d] += e
                return cfg, inp, rows, sel, kv, do, sinks
            assert abs(fd(edit) - g["dkv_c"][0][s, d]) < 1e-7, (s, d)
    for _ in range(12):
        t, d = int(rng.integers(0, cfg.S)), int(rng.integers(0, cfg.D))

        def edit(e, t=t, d=d):
            kr = inp["kv_raw"].copy()
            kr[0, t, d] += e
            return cfg, dict(inp, kv_raw=kr), rows, sel, kv_c, do, sinks
        assert abs(fd(edit) - g["dkv_raw"][0][t, d]) < 1e-7, (t, d)
    if with_sink:
        for h in range(cfg.H):
            def edit(e, h=h):
                sk = sinks.copy()
                sk[h] += e
                return cfg, inp, rows, sel, kv_c, do, sk
            assert abs(fd(edit) - g["dsinks"][h]) < 1e-7, h
    # the query side agrees with the dQ oracle
    dq = O.layer_dq_rows(cfg, inp, rows, do, sel, kv_c, sinks=sinks)
    for k in rows:
        assert np.allclose(g["dq"][k], dq[k], atol=1e-12)


def _torch_rope(x, pos, R, theta):
    """Interleaved RoPE on the last R dims, written with torch ops (pairs 2i, 2i+1)."""
    if R == 0:
        return x
    D = x.shape[-1]
    i = torch.arange(R // 2, dtype=torch.float64)
    ang = torch.as_tensor(pos, dtype=torch.float64)[..., None] * theta ** (-2.0 * i / R)
    c, s = torch.cos(ang), torch.sin(ang)
    x0, x1 = x[..., D - R::2], x[..., D - R + 1::2]
    rot = torch.stack([x0 * c - x1 * s, x0 * s + x1 * c], dim=-1).reshape(*x.shape[:-1], R)
    return torch.cat([x[..., :D - R], rot], dim=-1)


@pytest.mark.parametrize("norm_window", [False, True])
def test_layer_grads_match_torch_autograd(norm_window, rng):
    """torch autograd through the layer's attention written with torch ops in fp64
    (RoPE of queries and window tokens, optional window RMSNorm, entries gathered by the
    fixed selection, one softmax with a sink, de-rotation), for every input the
    backward differentiates: q, kv_c, kv_raw and the sinks."""
    cfg = tiny("csa", S=28, pos0=11, H=3, D=8, rope_dim=4, window=6, topk=3, norm_window=norm_window)
    inp = to_np(wl.make_inputs(cfg))
    rows = [(0, t) for t in range(cfg.S)]
    base = O.layer_rows(cfg, inp, rows)
    sel, kv_c = base["sel"], base["kv_c"]
    do = {k: rng.normal(size=(cfg.H, cfg.D)) for k in rows}
    sinks = rng.normal(size=cfg.H)
    g = O.layer_bwd_rows(cfg, inp, rows, do, sel, kv_c, sinks=sinks)

    q = torch.tensor(inp["q"][0], requires_grad=True)
    kc = torch.tensor(kv_c[0], requires_grad=True)
    kr = torch.tensor(inp["kv_raw"][0], requires_grad=True)
    sk = torch.tensor(sinks, requires_grad=True)
    R, th, scale = cfg.rope_dim, cfg.rope_theta, cfg.D ** -0.5
    loss = torch.zeros((), dtype=torch.float64)
    for (_, t) in rows:
        lo = max(0, t - cfg.window + 1)
        w = kr[lo:t + 1]
        if norm_window:
            w = w / torch.sqrt((w * w).mean(-1, keepdim=True) + cfg.rms_eps)
        w = _torch_rope(w, cfg.pos0 + torch.arange(lo, t + 1), R, th)
        keys = torch.cat([kc[torch.as_tensor(sel[(0, t)], dtype=torch.long)], w], 0)
        qr = _torch_rope(q[t], torch.full((cfg.H,), cfg.pos0 + t), R, th)
        z = torch.cat([(qr @ keys.T) * scale, sk[:, None]], 1)
        p = torch.softmax(z, dim=1)[:, :-1]
        o = _torch_rope(p @ keys, torch.full((cfg.H,), -(cfg.pos0 + t)), R, th)
        loss = loss + (o * torch.tensor(do[(0, t)])).sum()
    loss.backward()
    assert np.allclose(np.stack([g["dq"][k] for k in rows]), q.grad.numpy(), atol=1e-11)
    assert np.allclose(g["dkv_c"][0], kc.grad.numpy(), atol=1e-11)
    assert np.allclose(g["dkv_raw"][0], kr.grad.numpy(), atol=1e-11)
    assert np.allclose(g["dsinks"], sk.grad.numpy(), atol=1e-11)


def test_key_grads_closed_forms(rng):
    """Without a sink, moving every key by one vector c moves u by c and leaves the
    softmax unchanged, so sum_k dkey_k = sum_h du[h]; with one key and a sink,
    L = Pk (du . key) and dL/dsink = -Pk Ps (du . key); the lse of all-zero keys is
    log(nk), or log(nk + e^s) with a sink."""
    H, D, nk, scale = 3, 6, 7, 0.4
    qr, keys, du = rng.normal(size=(H, D)), rng.normal(size=(nk, D)), rng.normal(size=(H, D))
    g = O.attend_row_bwd(qr, keys, scale, du)
    assert np.allclose(g["dkeys"].sum(0), du.sum(0), atol=1e-13)
    assert np.allclose(g["dsink"], 0.0)
    key = rng.normal(size=(1, D))
    s = rng.normal(size=H)
    g1 = O.attend_row_bwd(qr, key, scale, du, sink=s)
    z = (qr @ key[0]) * scale
    pk, ps = np.exp(z) / (np.exp(z) + np.exp(s)), np.exp(s) / (np.exp(z) + np.exp(s))
    assert np.allclose(g1["dsink"], -pk * ps * (du @ key[0]), atol=1e-14)
    assert np.allclose(O.attend_row_lse(qr, np.zeros((nk, D)), scale), np.log(nk), atol=1e-14)
    assert np.allclose(O.attend_row_lse(qr, np.zeros((nk, D)), scale, s), np.log(nk + np.exp(s)), atol=1e-14)
    assert np.all(O.attend_row_lse(qr, np.zeros((0, D)), scale) == -np.inf)


def test_lse_reproduces_the_forward_probabilities(rng):
    """exp(z - lse) is the forward's softmax (attend_row's P) and, with a sink, the
    keys' probabilities sum to 1 - exp(sink - lse)."""
    H, D, nk, scale = 4, 8, 9, 0.3
    qr, keys = rng.normal(size=(H, D)), rng.normal(size=(nk, D)) * 3
    s = rng.normal(size=H)
    for sink in (None, s):
        _, P = O.attend_row(qr, keys, scale, sink)
        lse = O.attend_row_lse(qr, keys, scale, sink)
        assert np.allclose(np.exp((qr @ keys.T) * scale - lse[:, None]), P, atol=1e-14)
        rest = 0.0 if sink is None else np.exp(sink - lse)
        assert np.allclose(P.sum(1) + rest, 1.0, atol=1e-14)
