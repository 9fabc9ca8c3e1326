"""Pure-Python scalar brute force of the compressed attention layer, for tiny inputs.

TEST INFRASTRUCTURE ONLY.  A second transcription of the same definition with scalar
loops and the `math` module, written token by token rather than with array reshapes,
so that an indexing slip in the vectorised oracle (csa_oracle) shows up as a mismatch.
Use only for S <= 64 and D <= 32.

Sources as in csa_oracle: "fix(deepseek-v4): correct V4-Flash attention math",
Part 1 items 1-3; "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs
with Primus", subsection "Three attention types, interleaved".
"""
from __future__ import annotations

import math
import struct


def _rot_pair(x0, x1, P, i, R, theta):
    ang = P * (theta ** (-(2.0 * i) / R))
    c, s = math.cos(ang), math.sin(ang)
    return x0 * c - x1 * s, x0 * s + x1 * c


def brute_rope(vec, P, R, theta):
    D = len(vec)
    out = list(vec)
    for i in range(R // 2):
        a = D - R + 2 * i
        out[a], out[a + 1] = _rot_pair(vec[a], vec[a + 1], P, i, R, theta)
    return out


def _round_scalar(x, dtype):
    """Nearest value of the activation dtype, ties to even (struct for float32; for
    bf16, 8 significant bits from frexp and Python's round-half-even)."""
    if dtype == "f32":
        return struct.unpack("f", struct.pack("f", x))[0]
    m, e = math.frexp(x)
    if e < -125:  # below the smallest normal: fixed spacing 2**-133
        m, e = math.ldexp(m, e + 125), -125
    return math.ldexp(round(m * 256.0), e - 8)


def brute_index_prologue(vec, P, R, theta, dtype):
    """RoPE at P, then (1/sqrt(n)) * sum_j (-1)^popcount(i & j) x_j for every i (the
    Walsh form of the Sylvester Hadamard), rounded to the activation dtype."""
    x = brute_rope(vec, P, R, theta)
    n = len(x)
    out = []
    for i in range(n):
        acc = 0.0
        for j in range(n):
            acc += -x[j] if bin(i & j).count("1") % 2 else x[j]
        out.append(_round_scalar(acc / math.sqrt(n), dtype))
    return out


def _f32(x):
    return struct.unpack("f", struct.pack("f", x))[0]


def _e4m3_table():
    """Every finite non-negative OCP E4M3 value with its code: exponent field E and
    mantissa M give M * 2**-9 for E = 0, else (1 + M/8) * 2**(E - 7); E = 15, M = 7 is
    NaN and left out, so the largest is 448."""
    vals = []
    for E in range(16):
        for M in range(8):
            if E == 15 and M == 7:
                continue
            v = M * 2.0 ** -9 if E == 0 else (1 + M / 8) * 2.0 ** (E - 7)
            vals.append((v, E * 8 + M))
    return vals


_E4M3 = _e4m3_table()


def brute_e4m3(x):
    """Nearest E4M3 value by search over the table; a tie takes the code with an even
    mantissa."""
    a = abs(x)
    best = min(_E4M3, key=lambda vc: (abs(vc[0] - a), vc[1] & 1))
    return math.copysign(best[0], x) if best[0] else 0.0


def brute_quant_row(row):
    """Per-row E4M3 codes and scale, each step rounded to fp32 (a float64 result of
    one division or product rounds to the correctly rounded fp32 value)."""
    m = max(abs(_f32(v)) for v in row)
    if m == 0:
        return [0.0] * len(row), 0.0
    inv = _f32(448.0 / m)
    return [brute_e4m3(_f32(_f32(v) * inv)) for v in row], _f32(m / 448.0)


def brute_entry(va, ga, vb, gb, bias, s, r, overlap, D):
    """Pooled entry s (list of D floats).  Slots enumerated token by token."""
    slots = []  # (value row, gate row, bias row index)
    if overlap:
        for j in range(2 * r):
            tok = s * r - r + j
            if tok < 0:
                continue
            if j < r:
                slots.append((vb[tok], gb[tok], j))
            else:
                slots.append((va[tok], ga[tok], j))
    else:
        for j in range(r):
            tok = s * r + j
            slots.append((va[tok], ga[tok], j))
    p = []
    for c in range(D):
        logits = [g[c] + bias[j][c] for (_, g, j) in slots]
        mx = max(logits)
        ws = [math.exp(l - mx) for l in logits]
        tot = sum(ws)
        p.append(sum(w / tot * v[c] for w, (v, _, _) in zip(ws, slots)))
    return p


def brute_layer(cfg, inp, b=0, sinks=None):
    """Returns dict with o[t][h][d], sel[t] (sorted list), kv_c[s][d] for batch b.
    sinks: optional per-head softmax sink logits (a key with no value)."""
    S, H, D, R, r = cfg.S, cfg.H, cfg.D, cfg.rope_dim, cfg.ratio
    theta, eps, pos0 = cfg.rope_theta, cfg.rms_eps, cfg.pos0
    scale = cfg.softmax_scale
    L = lambda a: [[float(x) for x in row] for row in a]  # noqa: E731
    kv_raw = L(inp["kv_raw"][b])
    q = [[[float(x) for x in hrow] for hrow in inp["q"][b][t]] for t in range(S)]
    kv_c = []
    if cfg.kind in ("csa", "hca"):
        va, ga = L(inp["va"][b]), L(inp["ga"][b])
        vb = L(inp["vb"][b]) if cfg.kind == "csa" else None
        gb = L(inp["gb"][b]) if cfg.kind == "csa" else None
        bias = L(inp["bias"])
        for s in range(S // r):
            p = brute_entry(va, ga, vb, gb, bias, s, r, cfg.kind == "csa", D)
            ms = sum(x * x for x in p) / D
            inv = 1.0 / math.sqrt(ms + eps)
            kv_c.append(brute_rope([x * inv for x in p], pos0 + s * r, R, theta))
    res = {"o": [], "sel": [], "kv_c": kv_c, "scores": []}
    for t in range(S):
        # visible entries: whole group seen
        vis = [s for s in range(len(kv_c)) if (s + 1) * r - 1 <= t]
        if cfg.kind == "csa":
            qi, wi, ki = inp["q_idx"][b][t], inp["w_idx"][b][t], inp["k_idx"][b]
            if getattr(cfg, "index_prologue", False):
                qi = [brute_index_prologue([float(v) for v in qi[h]], pos0 + t, R, theta, cfg.dtype)
                      for h in range(cfg.idx_heads)]
                ki = [brute_index_prologue([float(v) for v in ki[s]], pos0 + s * r, R, theta, cfg.dtype)
                      for s in range(len(ki))]
                temp = 1.0 / math.sqrt(cfg.idx_heads * cfg.idx_dim)
                wi = [float(wi[h]) * temp for h in range(cfg.idx_heads)]
            if getattr(cfg, "index_fp8", False):
                def deq(row):
                    codes, sc = brute_quant_row([float(v) for v in row])
                    return [c * sc for c in codes]
                qi = [deq(qi[h]) for h in range(cfg.idx_heads)]
                ki = [deq(ki[s]) for s in range(len(ki))]
            sc = []
            for s in vis:
                tot = 0.0
                for h in range(cfg.idx_heads):
                    dot = sum(float(qi[h][d]) * float(ki[s][d]) for d in range(cfg.idx_dim))
                    tot += float(wi[h]) * (dot if dot > 0 else 0.0)
                sc.append(tot)
            ranked = sorted(range(len(vis)), key=lambda j: (-sc[j], vis[j]))
            sel = sorted(vis[j] for j in ranked[: cfg.topk])
            res["scores"].append(sc)
        elif cfg.kind == "hca":
            sel = list(vis)
        else:
            sel = []
        res["sel"].append(sel)
        keys = [kv_c[s] for s in sel]
        for tp in range(max(0, t - cfg.window + 1), t + 1):
            x = kv_raw[tp]
            if cfg.norm_window:
                inv = 1.0 / math.sqrt(sum(v * v for v in x) / D + eps)
                x = [v * inv for v in x]
            keys.append(brute_rope(x, pos0 + tp, R, theta))
        o_t = []
        for h in range(H):
            qh = brute_rope(q[t][h], pos0 + t, R, theta)
            z = [sum(qh[d] * k[d] for d in range(D)) * scale for k in keys]
            mx = max(z) if z else float(sinks[h])
            if sinks is not None:
                mx = max(mx, float(sinks[h]))
            e = [math.exp(v - mx) for v in z]
            tot = sum(e)
            if sinks is not None:
                tot += math.exp(float(sinks[h]) - mx)
            u = [sum(e[j] / tot * keys[j][d] for j in range(len(keys))) for d in range(D)]
            o_t.append(brute_rope(u, -(pos0 + t), R, theta))
        res["o"].append(o_t)
    return res


def brute_kl_target(cfg, inp, kv_c, t, sel, b=0):
    """Head-mean of the per-head softmax over the selected entries' logits, scalar loops."""
    H, D = cfg.H, cfg.D
    q = [[float(x) for x in inp["q"][b][t][h]] for h in range(H)]
    tot = [0.0] * len(sel)
    for h in range(H):
        qh = brute_rope(q[h], cfg.pos0 + t, cfg.rope_dim, cfg.rope_theta)
        z = [sum(qh[d] * kv_c[s][d] for d in range(D)) * cfg.softmax_scale for s in sel]
        mx = max(z)
        e = [math.exp(v - mx) for v in z]
        den = sum(e)
        for k in range(len(sel)):
            tot[k] += e[k] / den / H
    return tot
