"""fp64 numpy oracle of the compressed attention layer: forward and attention backward.

TEST INFRASTRUCTURE ONLY: imported by tests, the smoke check and the CPU-baseline
leg of the benchmark; never by the product path.

Every function consumes float64 arrays (bf16 or fp32 inputs are upcast losslessly by
the caller) and computes in float64.  No online softmax, no fusion, no blocking
beyond looping over queries.  Sources, cited by page title and section:

  [PR930] "fix(deepseek-v4): correct V4-Flash attention math, wire the MoE balance
          loss", Part 1 "Attention correctness", items 1 (scale), 2 (compressed RoPE
          positions and base), 3 (output de-rotation), 4 (indexer precision).
  [BLOG]  "Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
          Primus", section "The DeepSeek-V4-Flash architecture", subsection "Three
          attention types, interleaved" (pooling, overlap, indexer, window), and
          section "Kernel fusions" (compressor pooling, interleaved partial RoPE,
          RMSNorm).

Readings taken where the pages leave a step open:
  * CSA entry 0 has no previous group: those slots get logit -inf.
  * Bias row j is pooling slot j in token order (CSA: rows 0..r-1 are the previous
    group read from the b projections, rows r..2r-1 the entry's own group read from
    the a projections).
  * Entry s is visible to query t iff its whole group is seen: (s+1)*r - 1 <= t.
  * RMSNorm has weight 1 and eps 1e-6, applied before RoPE.
  * RoPE is interleaved (adjacent pairs) on the last R dims, angle
    P * theta**(-2i/R), no frequency interpolation.
  * Window keys are the raw latents of tokens t-W+1..t (clipped at 0), rotated at
    their own positions and not normalised (unless norm_window is set).
  * One softmax over the union of selected entries and window keys.
  * Top-k ties break to the smaller entry index.
  * Indexer prologue (optional, index_prologue): the RoPE of the layer (same R and
    theta, last R dims) on q_I at pos0 + t and on k_I at pos0 + s*r, then the
    normalised Sylvester Hadamard over D_I, the result rounded to the activation dtype
    (the tensor the scoring consumes); the per-head weights are scaled by
    (H_I * D_I)**-0.5.
  * FP8 indexer (optional, index_fp8): each q_I[t,h] and k_I[s] row is quantized to
    OCP E4M3 (max 448, round to nearest even) with its own scale, absmax / 448; the
    code is decided in fp32 (the multiplier 448 / absmax and the product rounded to
    fp32, as the kernel does); the scores use the decoded values code * scale.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope_angles", "rope", "gated_pool", "rms_norm", "compress", "visible_entries",
    "window_bounds", "indexer_scores_row", "indexer_scores_block", "indexer_scores", "topk_row", "topk",
    "rotate_queries", "rotate_window", "attend_row", "layer_forward", "layer_rows",
    "hadamard", "round_to", "index_prologue", "index_temperature", "e4m3", "quant_e4m3_rows",
    "kl_target_row", "kl_target", "attend_row_bwd_dq", "layer_dq_rows",
    "attend_row_lse", "attend_row_bwd", "rms_norm_bwd", "layer_bwd_rows",
]


def rope_angles(pos, rope_dim: int, theta: float) -> np.ndarray:
    """Angles P * theta**(-2i/R) for i = 0..R/2-1 ([PR930] item 2: the compressed base
    theta = 40000 for Flash).  `pos` is an integer array; result has shape
    pos.shape + (R/2,)."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    inv_freq = np.power(np.float64(theta), -2.0 * i / rope_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x: np.ndarray, pos, rope_dim: int, theta: float) -> np.ndarray:
    """Interleaved partial RoPE on the last `rope_dim` dims of x ([BLOG] "Kernel
    fusions": interleaved partial RoPE).  Pair i is (x[D-R+2i], x[D-R+2i+1]) and is
    rotated by +angle: (x0 cos - x1 sin, x0 sin + x1 cos).  `pos` broadcasts against
    x.shape[:-1]; a negative position is the inverse rotation."""
    x = np.array(x, dtype=np.float64, copy=True)
    if rope_dim == 0:
        return x
    D = x.shape[-1]
    ang = rope_angles(pos, rope_dim, theta)
    c, s = np.cos(ang), np.sin(ang)
    lo = D - rope_dim
    x0 = x[..., lo::2].copy()
    x1 = x[..., lo + 1::2].copy()
    x[..., lo::2] = x0 * c - x1 * s
    x[..., lo + 1::2] = x0 * s + x1 * c
    return x


def gated_pool(va, ga, vb, gb, bias, ratio: int, overlap: bool) -> np.ndarray:
    """Softmax-gated pooling ([BLOG] "Three attention types, interleaved": a softmax
    over the group of gate plus a learnable per-position bias weights the sum of the
    values; CSA entries pool their own `ratio` tokens plus the previous `ratio`).

    va, ga, vb, gb: [S, D] (vb, gb unused when overlap is False); bias [span, D].
    Returns p [S/ratio, D].

    Entry s, slot j:
      overlap: token tau_j = s*r - r + j; j < r reads (vb, gb), j >= r reads (va, ga);
               a slot whose token is before 0 gets logit -inf.
      disjoint: token tau_j = s*r + j, read from (va, ga).
    """
    S, D = va.shape
    r = ratio
    n = S // r
    own_v = va[: n * r].reshape(n, r, D)
    own_g = ga[: n * r].reshape(n, r, D)
    if overlap:
        prev_v = np.zeros((n, r, D))
        prev_g = np.full((n, r, D), -np.inf)
        if n > 1:
            prev_v[1:] = vb[: (n - 1) * r].reshape(n - 1, r, D)
            prev_g[1:] = gb[: (n - 1) * r].reshape(n - 1, r, D)
        v = np.concatenate([prev_v, own_v], axis=1)  # [n, 2r, D]
        logit = np.concatenate([prev_g, own_g], axis=1) + bias[None, :, :]
    else:
        v = own_v
        logit = own_g + bias[None, :, :]
    m = np.max(logit, axis=1, keepdims=True)
    e = np.exp(logit - m)
    alpha = e / np.sum(e, axis=1, keepdims=True)
    return np.sum(alpha * v, axis=1)


def rms_norm(x: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) over the last axis, weight 1 ([PR930] item 1: V4
    RMS-normalises the KV entries directly)."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def compress(va, ga, vb, gb, bias, ratio, overlap, rope_dim, theta, eps, pos0=0):
    """Pool, RMS-normalise, then rotate entry s at its original-sequence position
    pos0 + s*ratio ([PR930] item 2: entry s covers the window starting at s*ratio).
    Returns kv_c [S/ratio, D]."""
    p = gated_pool(va, ga, vb, gb, bias, ratio, overlap)
    nrm = rms_norm(p, eps)
    pos = pos0 + np.arange(p.shape[0], dtype=np.int64) * ratio
    return rope(nrm, pos, rope_dim, theta)


def visible_entries(t: int, ratio: int) -> int:
    """n_t: entries whose last token (s+1)*ratio - 1 is at or before t."""
    return (t + 1) // ratio


def window_bounds(t: int, window: int):
    """Window tokens lo..t inclusive, lo = max(0, t - W + 1)."""
    return max(0, t - window + 1), t


def indexer_scores_row(q_i_t, w_t, k_i, n_vis: int) -> np.ndarray:
    """Lightning-indexer scores of query t over its visible entries ([PR930] item 6a
    and [BLOG] "Three attention types": I[t,s] = sum_h w[t,h] * ReLU(q_I[t,h].k_I[s])),
    in fp64 ([PR930] item 4 keeps the indexer product in high precision).
    q_i_t [H_I, D_I], w_t [H_I], k_i [n, D_I].  Returns [n_vis]."""
    if n_vis == 0:
        return np.zeros(0)
    dots = q_i_t @ k_i[:n_vis].T  # [H_I, n_vis]
    return w_t @ np.maximum(dots, 0.0)


def indexer_scores_block(q_i, w, k_i, n_vis) -> list:
    """indexer_scores_row for a block of queries at once (one matrix product for the
    block; the same definition, for speed at long sequence lengths).
    q_i [R, H_I, D_I], w [R, H_I], k_i [n, D_I], n_vis: R visible-entry counts.
    Returns R rows, row r of length n_vis[r]."""
    R, HI, DI = q_i.shape
    nmax = int(max(n_vis)) if R else 0
    if nmax == 0:
        return [np.zeros(0) for _ in range(R)]
    dots = (q_i.reshape(R * HI, DI) @ k_i[:nmax].T).reshape(R, HI, nmax)
    np.maximum(dots, 0.0, out=dots)  # ReLU (in place: the block can be large)
    sc = np.matmul(w[:, None, :], dots)[:, 0, :]  # sum_h w[r,h] ReLU(q . k)
    return [sc[r, : int(n_vis[r])].copy() for r in range(R)]


def hadamard(n: int) -> np.ndarray:
    """Sylvester Hadamard matrix of order n (a power of two), built by the doubling
    H_1 = [1], H_2m = [[H_m, H_m], [H_m, -H_m]].  Symmetric, with H H^T = n I."""
    if n < 1 or n & (n - 1):
        raise ValueError(f"Hadamard order {n} is not a power of two")
    h = np.ones((1, 1))
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def round_to(x, dtype: str) -> np.ndarray:
    """Round fp64 values to the activation dtype and return them as fp64: "f32" to the
    nearest float32; "bf16" to the nearest value with 8 significant bits (ties to
    even), with the fixed spacing 2**-133 below the smallest normal 2**-126."""
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype != "bf16":
        raise ValueError(dtype)
    _, e = np.frexp(x)                      # x = m * 2**e with 0.5 <= |m| < 1
    ulp = np.ldexp(1.0, np.maximum(e, -125) - 8)
    return np.rint(x / ulp) * ulp


def index_prologue(x, pos, rope_dim: int, theta: float, dtype: str) -> np.ndarray:
    """Indexer prologue of one set of indexer vectors ([PR930] item 6e): the partial
    RoPE at `pos` (queries at their own position, keys at s * ratio), then the
    normalised Hadamard H / sqrt(D_I) over the whole vector, rounded to `dtype` (the
    activation dtype of the tensor the bf16 scoring reads, [PR930] item 4).
    x [..., D_I]; pos broadcasts against x.shape[:-1]."""
    n = np.asarray(x).shape[-1]
    y = rope(x, pos, rope_dim, theta)
    y = y @ (hadamard(n) / np.sqrt(n))      # H is symmetric: row-vector form of H y
    return round_to(y, dtype)


def index_temperature(idx_heads: int, idx_dim: int) -> float:
    """Score temperature folded into the per-head weights ([PR930] item 6a):
    idx_heads**-0.5 * idx_dim**-0.5 (1/90.5 at 64 x 128)."""
    return float(idx_heads) ** -0.5 * float(idx_dim) ** -0.5


E4M3_MAX = 448.0


def e4m3(x) -> np.ndarray:
    """Nearest OCP E4M3 value (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
    largest finite 448), ties to even.  Normal numbers |x| >= 2**-6 keep 4 significant
    bits; below that the spacing is 2**-9.  Magnitudes above 448 saturate to 448 (the
    quantizer below never produces them)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    ulp = np.ldexp(1.0, np.maximum(e, -5) - 4)
    return np.clip(np.rint(x / ulp) * ulp, -E4M3_MAX, E4M3_MAX)


def quant_e4m3_rows(x):
    """Per-row E4M3 quantization of the indexer operands ("Enabling DeepSeek-V4-Flash
    Training ...", closing remarks: an E4M3 path for the indexer QK; "fix(deepseek-v4)
    ...", Part 1 item 4: it changes the selection, so it is opt-in).  Over the last
    axis: m = max |x|, codes = E4M3(fp32(x * fp32(448 / m))) and scale = fp32(m / 448),
    both divisions and the product rounded to fp32; a zero row gets codes 0 and scale 0.
    x holds fp32-representable values.  Returns (codes, scale) as fp64 arrays; the row
    decodes to codes * scale."""
    x32 = np.asarray(x, dtype=np.float32)
    m = np.max(np.abs(x32), axis=-1, keepdims=True)
    with np.errstate(divide="ignore"):
        inv = np.where(m > 0, np.float32(E4M3_MAX) / np.where(m > 0, m, 1), np.float32(0)).astype(np.float32)
    y = (x32 * inv).astype(np.float32)
    scale = (m / np.float32(E4M3_MAX)).astype(np.float32)
    return e4m3(y.astype(np.float64)), scale[..., 0].astype(np.float64)


def indexer_scores(q_i, w, k_i, ratio: int) -> list:
    """Scores for every query, as a list of rows of length n_t."""
    S = q_i.shape[0]
    return [indexer_scores_row(q_i[t], w[t], k_i, visible_entries(t, ratio)) for t in range(S)]


def topk_row(scores_row: np.ndarray, k: int) -> np.ndarray:
    """Indices of the min(k, n) largest scores, ordered by (-score, index): ties go to
    the smaller index.  Returned sorted ascending."""
    n = scores_row.shape[0]
    if n == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(n), -scores_row))
    return np.sort(order[: min(k, n)])


def topk(scores_rows: list, k: int) -> list:
    return [topk_row(r, k) for r in scores_rows]


def rotate_queries(q, rope_dim, theta, pos0=0):
    """q [S, H, D] rotated at pos0 + t."""
    S = q.shape[0]
    pos = (pos0 + np.arange(S, dtype=np.int64))[:, None]
    return rope(q, pos, rope_dim, theta)


def rotate_window(kv_raw, rope_dim, theta, eps, pos0=0, norm_window=False):
    """Raw per-token latents rotated at their own positions (optionally normalised)."""
    x = rms_norm(kv_raw, eps) if norm_window else kv_raw
    pos = pos0 + np.arange(kv_raw.shape[0], dtype=np.int64)
    return rope(x, pos, rope_dim, theta)


def attend_row(qr_t, keys, scale: float, sink=None):
    """One query's multi-query attention: z = (q.key) * scale for every head and key,
    one softmax over all keys, u = sum P key (K = V, [BLOG] "The DeepSeek-V4-Flash
    architecture").  qr_t [H, D] (already rotated), keys [nk, D].  Returns (u [H, D],
    P [H, nk]).

    sink [H] (optional): one fp32 logit per head that joins each head's softmax as a
    key with no value, i.e. exp(sink_h) is added to the denominator.  [BLOG] "Kernel
    fusions", row "SWA / CSA / HCA attention" (the attention kernel folds in the
    softmax sink); [PR930] Part 1 item 6f (the sink is an FP32 logit that feeds the
    softmax directly).  With a sink, a query with no key gives u = 0."""
    z = (qr_t @ keys.T) * scale
    if sink is None:
        m = np.max(z, axis=1, keepdims=True)
        e = np.exp(z - m)
        P = e / np.sum(e, axis=1, keepdims=True)
        return P @ keys, P
    sk = np.asarray(sink, dtype=np.float64).reshape(-1, 1)
    m = sk if z.shape[1] == 0 else np.maximum(np.max(z, axis=1, keepdims=True), sk)
    e = np.exp(z - m)
    P = e / (np.sum(e, axis=1, keepdims=True) + np.exp(sk - m))
    return P @ keys, P


def kl_target_row(qr_t, kv_c, sel, scale: float) -> np.ndarray:
    """Target distribution of the indexer's distillation loss for one query
    ("fix(deepseek-v4): correct V4-Flash attention math", Part 1 item 5: KL(attention
    || indexer) over the selected entries, kept in [B, S, K]; item 11: the head sum
    taken inside the loop, never forming the per-head tensor).  The main attention's
    logits over the selected entries only, z[h,k] = (q~[h] . kv_c[sel[k]]) * scale, a
    softmax per head over those entries, then the mean over heads:
        T[k] = (1/H) sum_h softmax_k(z[h, :])[k],  summing to 1 over the selection.
    qr_t [H, D] rotated query, kv_c [n, D], sel the selected indices.  Returns [len(sel)]."""
    if len(sel) == 0:
        return np.zeros(0)
    z = (qr_t @ kv_c[np.asarray(sel)].T) * scale
    m = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - m)
    return np.mean(e / np.sum(e, axis=1, keepdims=True), axis=0)


def kl_target(cfg, inp: dict, rows, sel: dict, kv_c: dict) -> dict:
    """kl_target_row for each (b, t) in rows, with the query rotated at pos0 + t, the
    scale D**-0.5, and sel[(b, t)] / kv_c[b] from the layer (layer_rows)."""
    out = {}
    for (b, t) in rows:
        qr = rope(_as64(inp["q"][b, t]), cfg.pos0 + t, cfg.rope_dim, cfg.rope_theta)
        out[(b, t)] = kl_target_row(qr, np.asarray(kv_c[b], dtype=np.float64), sel[(b, t)], cfg.D ** -0.5)
    return out


def attend_row_bwd_dq(qr_t, keys, scale: float, du, sink=None):
    """Gradient of one query's attention output with respect to its rotated query
    (the dQ part of the backward, "Enabling DeepSeek-V4-Flash Training on AMD Instinct
    MI355X GPUs with Primus", section "Attention kernels for the three layer types":
    dQ, with delta = rowsum(O * dO) computed inside it).  With P = softmax(z),
    z = (qr . key) * scale and u = sum P key:
        dP[h,k] = du[h] . key_k,  delta[h] = sum_k P dP = du[h] . u[h],
        dz = P (dP - delta),      dqr[h] = scale * sum_k dz[h,k] key_k.
    qr_t [H, D] rotated query, keys [nk, D], du [H, D] the gradient of u.  A sink
    (attend_row) only changes P's denominator: it carries no value, so it adds no term
    to dP or delta.  Returns (dqr [H, D], delta [H])."""
    _, P = attend_row(qr_t, keys, scale, sink)
    dP = du @ keys.T
    delta = np.sum(P * dP, axis=1)
    dz = P * (dP - delta[:, None])
    return scale * (dz @ keys), delta


def layer_dq_rows(cfg, inp: dict, rows, do: dict, sel: dict = None, kv_c=None, sinks=None) -> dict:
    """dL/dq for the query rows `rows` given dL/do[(b, t)] [H, D]: the output's
    de-rotation transposes to a rotation of do by +(pos0 + t) (du), the query's
    rotation to a rotation of dqr by -(pos0 + t).  Keys, selection and window as in
    layer_rows (`sel` and `kv_c` may come from a layer_rows result)."""
    R, theta, pos0 = cfg.rope_dim, cfg.rope_theta, cfg.pos0
    scale = cfg.D ** -0.5 if getattr(cfg, "softmax_scale", None) is None else cfg.softmax_scale
    if sel is None or kv_c is None:
        r = layer_rows(cfg, inp, rows, sel_override=sel)
        sel = r["sel"] if sel is None else sel
        kv_c = r["kv_c"] if kv_c is None else kv_c
    out = {}
    for (b, t) in rows:
        lo, hi = window_bounds(t, cfg.window)
        win = rotate_window(_as64(inp["kv_raw"][b][lo:hi + 1]), R, theta, cfg.rms_eps, pos0 + lo,
                            bool(getattr(cfg, "norm_window", False)))
        ent = np.asarray(kv_c[b], dtype=np.float64)[np.asarray(sel[(b, t)], dtype=np.int64)] \
            if cfg.kind != "swa" else np.zeros((0, cfg.D))
        keys = np.concatenate([ent, win], axis=0)
        qr = rope(_as64(inp["q"][b, t]), pos0 + t, R, theta)
        du = rope(np.asarray(do[(b, t)], dtype=np.float64), pos0 + t, R, theta)
        dqr, _ = attend_row_bwd_dq(qr, keys, scale, du, sinks)
        out[(b, t)] = rope(dqr, -(pos0 + t), R, theta)
    return out


def attend_row_lse(qr_t, keys, scale: float, sink=None) -> np.ndarray:
    """Natural log of each head's softmax denominator, the statistic a training forward
    keeps for its backward: lse[h] = log( sum_k exp(z[h,k]) + exp(sink[h]) ) with
    z = (qr . key) * scale as in attend_row (the sink term only with a sink).  Then
    P[h,k] = exp(z[h,k] - lse[h]).  A head with no key and no sink gets -inf."""
    z = (qr_t @ keys.T) * scale
    H = qr_t.shape[0]
    cols = [z]
    if sink is not None:
        cols.append(np.asarray(sink, dtype=np.float64).reshape(H, 1))
    allz = np.concatenate(cols, axis=1)
    if allz.shape[1] == 0:
        return np.full(H, -np.inf)
    m = np.max(allz, axis=1, keepdims=True)
    return m[:, 0] + np.log(np.sum(np.exp(allz - m), axis=1))


def attend_row_bwd(qr_t, keys, scale: float, du, sink=None) -> dict:
    """Backward of one query's attention with the query, every key and the sink as
    variables ("Enabling DeepSeek-V4-Flash Training on AMD Instinct MI355X GPUs with
    Primus", section "Attention kernels for the three layer types": dQ with delta,
    and interm, the contraction over heads that gives each key's gradient;
    "fix(deepseek-v4): correct V4-Flash attention math", Part 1 item 6f: the sink is a
    logit of the softmax).  K = V, so a key gets a logit term and a value term:
        dP[h,k] = du[h] . key_k,   delta[h] = sum_k P dP,   dz = P (dP - delta)
        dqr[h]  = scale sum_k dz[h,k] key_k
        dkey_k  = scale sum_h dz[h,k] qr[h]  +  sum_h P[h,k] du[h]
    The sink is a logit with a zero value, so its dP is 0 and its dz is
        dsink[h] = -Ps[h] delta[h],   Ps[h] = exp(sink[h] - lse[h]).
    qr_t [H, D] rotated query, keys [nk, D], du [H, D] the gradient of u.  Returns
    dqr [H, D], dkeys [nk, D], dsink [H] (zeros without a sink), lse [H], delta [H]."""
    _, P = attend_row(qr_t, keys, scale, sink)
    dP = du @ keys.T
    delta = np.sum(P * dP, axis=1)
    dz = P * (dP - delta[:, None])
    lse = attend_row_lse(qr_t, keys, scale, sink)
    if sink is None:
        dsink = np.zeros(qr_t.shape[0])
    else:
        dsink = -np.exp(np.asarray(sink, dtype=np.float64) - lse) * delta
    return {"dqr": scale * (dz @ keys), "dkeys": scale * (dz.T @ qr_t) + P.T @ du,
            "dsink": dsink, "lse": lse, "delta": delta}


def rms_norm_bwd(x, dy, eps: float) -> np.ndarray:
    """Gradient through rms_norm: with r = (mean(x^2) + eps)**-0.5 and y = x r,
    dx = r (dy - y mean(dy * y)) over the last axis."""
    r = 1.0 / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * np.mean(dy * y, axis=-1, keepdims=True))


def layer_bwd_rows(cfg, inp: dict, rows, do: dict, sel: dict = None, kv_c=None, sinks=None) -> dict:
    """Gradients of L = sum over the query rows `rows` of sum(do[(b,t)] * o[b,t]) with
    the selection held fixed (top-k has no gradient):
      dq {(b,t): [H,D]}, lse {(b,t): [H]},
      dkv_c {b: [n, D]}   with respect to the rotated entries the attention reads
                          (the selected entries of each row gather their key gradient),
      dkv_raw {b: [S, D]} with respect to the raw window latents: the key gradients of
                          token t' over every row whose window holds it, rotated back
                          by -(pos0 + t') (the transpose of its rotation) and, with
                          norm_window, taken through the RMSNorm,
      dsinks [H] or None.
    Keys, selection and window as in layer_rows (`sel` and `kv_c` may come from a
    layer_rows result)."""
    R, theta, pos0, eps = cfg.rope_dim, cfg.rope_theta, cfg.pos0, cfg.rms_eps
    scale = cfg.D ** -0.5 if getattr(cfg, "softmax_scale", None) is None else cfg.softmax_scale
    norm_window = bool(getattr(cfg, "norm_window", False))
    if cfg.kind != "swa" and (sel is None or kv_c is None):
        r = layer_rows(cfg, inp, rows, sel_override=sel)
        sel = r["sel"] if sel is None else sel
        kv_c = r["kv_c"] if kv_c is None else kv_c
    n = cfg.S // cfg.ratio if cfg.kind != "swa" else 0
    out = {"dq": {}, "lse": {}, "dkv_c": {}, "dkv_raw": {},
           "dsinks": None if sinks is None else np.zeros(cfg.H)}
    gwin = {}
    for b in sorted({b for b, _ in rows}):
        out["dkv_c"][b] = np.zeros((n, cfg.D))
        gwin[b] = np.zeros((cfg.S, cfg.D))
    for (b, t) in rows:
        lo, hi = window_bounds(t, cfg.window)
        win = rotate_window(_as64(inp["kv_raw"][b][lo:hi + 1]), R, theta, eps, pos0 + lo, norm_window)
        if cfg.kind == "swa":
            s_t = np.zeros(0, dtype=np.int64)
            ent = np.zeros((0, cfg.D))
        else:
            s_t = np.asarray(sel[(b, t)], dtype=np.int64)
            ent = np.asarray(kv_c[b], dtype=np.float64)[s_t]
        keys = np.concatenate([ent, win], axis=0)
        qr = rope(_as64(inp["q"][b, t]), pos0 + t, R, theta)
        du = rope(np.asarray(do[(b, t)], dtype=np.float64), pos0 + t, R, theta)
        g = attend_row_bwd(qr, keys, scale, du, sinks)
        out["dq"][(b, t)] = rope(g["dqr"], -(pos0 + t), R, theta)
        out["lse"][(b, t)] = g["lse"]
        if len(s_t):
            np.add.at(out["dkv_c"][b], s_t, g["dkeys"][:len(s_t)])
        gwin[b][lo:hi + 1] += g["dkeys"][len(s_t):]
        if sinks is not None:
            out["dsinks"] += g["dsink"]
    for b, gw in gwin.items():
        pos = pos0 + np.arange(cfg.S, dtype=np.int64)
        d = rope(gw, -pos, R, theta)
        if norm_window:
            d = rms_norm_bwd(_as64(inp["kv_raw"][b]), d, eps)
        out["dkv_raw"][b] = d
    return out


def _as64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def layer_rows(cfg, inp: dict, rows, sel_override: dict = None, kv_c=None, want_p=False, sinks=None):
    """Oracle outputs for the query rows `rows` of batch 0..B-1 (rows is a list of
    (b, t) pairs).  `inp` holds numpy arrays (any float dtype) with the shapes of
    workloads.make_inputs.  `sel_override` maps (b, t) to a selection to use instead
    of the oracle's own top-k (for re-evaluating on another admissible selection).
    `sinks` [H] (optional): per-head softmax sink logits (see attend_row).
    With cfg.index_prologue set, the indexer reads index_prologue(q_I) at pos0 + t,
    index_prologue(k_I) at pos0 + s*r and w * index_temperature (CSA only).  With
    cfg.index_fp8 set it scores the E4M3-decoded operands (quant_e4m3_rows), after the
    prologue when both are set.

    Returns a dict: o {(b,t): [H,D]}, sel {(b,t): indices}, scores {(b,t): row},
    n_visible {(b,t): int}, win {(b,t): (lo, hi)}, kv_c {b: [n, D]}, lse {(b,t): [H]}
    (attend_row_lse), and P when want_p.  Steps, per [PR930] Part 1 and [BLOG] "Three attention types":
      1 pool + norm + rotate entries at pos0 + s*r   (CSA, HCA)
      2 rotate queries at pos0 + t and window tokens at pos0 + t'
      3 indexer scores over visible entries          (CSA)
      4 top-k (CSA) / all visible (HCA) / none (window-only)
      5 one softmax over selected entries plus window, scale D**-0.5 ([PR930] item 1)
      6 de-rotate the output at -(pos0 + t)          ([PR930] item 3)
    """
    kind = cfg.kind
    R, theta, eps, pos0 = cfg.rope_dim, cfg.rope_theta, cfg.rms_eps, cfg.pos0
    scale = cfg.D ** -0.5 if getattr(cfg, "softmax_scale", None) is None else cfg.softmax_scale
    norm_window = bool(getattr(cfg, "norm_window", False))
    out = {"o": {}, "sel": {}, "scores": {}, "n_visible": {}, "win": {}, "kv_c": {}, "P": {}, "lse": {}}
    batches = sorted({b for b, _ in rows})
    for b in batches:
        if kind in ("csa", "hca"):
            if kv_c is not None:
                kvb = np.asarray(kv_c[b], dtype=np.float64)
            else:
                kvb = compress(_as64(inp["va"][b]), _as64(inp["ga"][b]),
                               _as64(inp["vb"][b]) if kind == "csa" else None,
                               _as64(inp["gb"][b]) if kind == "csa" else None,
                               _as64(inp["bias"]), cfg.ratio, kind == "csa", R, theta, eps, pos0)
            out["kv_c"][b] = kvb
        kv_raw_b = inp["kv_raw"][b]
        ts = [t for bb, t in rows if bb == b]
        prologue = kind == "csa" and bool(getattr(cfg, "index_prologue", False))
        fp8 = kind == "csa" and bool(getattr(cfg, "index_fp8", False))
        if kind == "csa":
            k_i_b = _as64(inp["k_idx"][b])
            if prologue:
                k_pos = pos0 + np.arange(k_i_b.shape[0], dtype=np.int64) * cfg.ratio
                k_i_b = index_prologue(k_i_b, k_pos, R, theta, cfg.dtype)
            if fp8:
                codes, sc = quant_e4m3_rows(k_i_b)
                k_i_b = codes * sc[:, None]

        def index_row(t, n_vis):
            q_i, w_i = _as64(inp["q_idx"][b, t]), _as64(inp["w_idx"][b, t])
            if prologue:
                q_i = index_prologue(q_i, pos0 + t, R, theta, cfg.dtype)
                w_i = w_i * index_temperature(cfg.idx_heads, cfg.idx_dim)
            if fp8:
                codes, sc = quant_e4m3_rows(q_i)
                q_i = codes * sc[:, None]
            return indexer_scores_row(q_i, w_i, k_i_b, n_vis)

        for t in ts:
            lo, hi = window_bounds(t, cfg.window)
            win_keys = rotate_window(_as64(kv_raw_b[lo:hi + 1]), R, theta, eps, pos0 + lo, norm_window)
            if kind == "swa":
                n_vis, sel = 0, np.zeros(0, dtype=np.int64)
                ent_keys = np.zeros((0, cfg.D))
            else:
                n_vis = visible_entries(t, cfg.ratio)
                if sel_override is not None and (b, t) in sel_override:
                    sel = np.sort(np.asarray(sel_override[(b, t)], dtype=np.int64))
                    if kind == "csa":
                        out["scores"][(b, t)] = index_row(t, n_vis)
                elif kind == "csa":
                    sc = index_row(t, n_vis)
                    out["scores"][(b, t)] = sc
                    sel = topk_row(sc, cfg.topk)
                else:
                    sel = np.arange(n_vis, dtype=np.int64)
                ent_keys = kvb[sel]
            keys = np.concatenate([ent_keys, win_keys], axis=0)
            qr = rope(_as64(inp["q"][b, t]), pos0 + t, R, theta)
            u, P = attend_row(qr, keys, scale, sinks)
            out["o"][(b, t)] = rope(u, -(pos0 + t), R, theta)
            out["lse"][(b, t)] = attend_row_lse(qr, keys, scale, sinks)
            out["sel"][(b, t)] = sel
            out["n_visible"][(b, t)] = n_vis
            out["win"][(b, t)] = (lo, hi)
            if want_p:
                out["P"][(b, t)] = P
    return out


def layer_forward(cfg, inp: dict, want_p=False, sinks=None) -> dict:
    """Whole-layer oracle: o [B, S, H, D] plus kv_c, selections, scores and layout."""
    rows = [(b, t) for b in range(cfg.B) for t in range(cfg.S)]
    r = layer_rows(cfg, inp, rows, want_p=want_p, sinks=sinks)
    o = np.zeros((cfg.B, cfg.S, cfg.H, cfg.D))
    for (b, t), v in r["o"].items():
        o[b, t] = v
    r["o_full"] = o
    return r
