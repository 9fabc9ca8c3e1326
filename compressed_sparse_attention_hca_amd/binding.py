"""Thin ctypes binding of libcsa.so (include/csa.h).

Argument marshalling only: every step of the layer runs in the HIP kernels behind
the C ABI.  PyTorch supplies device memory and the current stream.  There is no CPU
fallback; if the library is missing or fails to load, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from . import workloads as wl

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa.so")

CSA_OK, CSA_ERR_INVALID_ARG, CSA_ERR_WORKSPACE, CSA_ERR_UNSUPPORTED, CSA_ERR_HIP = range(5)
CSA_F32, CSA_BF16 = 0, 1
OP_COMPRESS, OP_INDEX_TOPK, OP_SPARSE_MQA, OP_CSA_FWD, OP_HCA_FWD, OP_SPARSE_MQA_BWD = range(6)
FLAG_NORM_WINDOW = 1
FLAG_INDEX_PROLOGUE = 2
FLAG_INDEX_FP8 = 4


class Params(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "S", "H", "D", "rope_dim", "ratio", "overlap", "window", "topk",
                 "idx_heads", "idx_dim", "dtype")] + [
        ("rope_theta", ctypes.c_double), ("rms_eps", ctypes.c_float),
        ("softmax_scale", ctypes.c_float), ("pos0", ctypes.c_int64), ("flags", ctypes.c_uint32)]


class Inputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("q", "kv_raw", "va", "ga", "vb", "gb", "bias", "q_idx", "w_idx", "k_idx",
                 "kv_c_out", "idx_out", "n_visible_out", "sinks", "lse_out")]


class CsaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_names.get(status, status)}: {msg}")
        self.status = status


_status_names = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_WORKSPACE",
                 3: "CSA_ERR_UNSUPPORTED", 4: "CSA_ERR_HIP"}


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run "
                          "`python -m compressed_sparse_attention_hca_amd.build_lib`")
    lib = ctypes.CDLL(LIB_PATH)
    P, V, I32, I64, SZ = ctypes.POINTER(Params), ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "csa_compress": [P, V, V, V, V, V, V, V],
        "csa_index_scores": [P, V, V, V, V, I64, I32, I32, V],
        "csa_index_topk": [P, V, V, V, V, V, V, SZ, V],
        "csa_index_keys": [P, V, V, V],
        "csa_kl_target": [P, V, V, V, V, V],
        "csa_sparse_mqa_fwd": [P, V, V, V, V, V, V, SZ, V],
        "csa_sparse_mqa_fwd_sink": [P, V, V, V, V, V, V, V, SZ, V],
        "csa_sparse_mqa_fwd_lse": [P, V, V, V, V, V, V, V, V, SZ, V],
        "csa_sparse_mqa_bwd_dq": [P, V, V, V, V, V, V, V, V, V, SZ, V],
        "csa_sparse_mqa_bwd_dkv": [P, V, V, V, V, V, V, V, V, V, V, V, V, SZ, V],
        "csa_fwd": [P, ctypes.POINTER(Inputs), V, V, SZ, V],
        "csa_fwd_noalloc": [P, ctypes.POINTER(Inputs), V, V],
        "hca_fwd": [P, ctypes.POINTER(Inputs), V, V, SZ, V],
        "csa_debug_layout": [P, V, V, V, V],
        "csa_fwd_traced": [P, ctypes.POINTER(Inputs), V, V, SZ, V, ctypes.POINTER(V),
                           ctypes.POINTER(I32), I32],
        "hca_fwd_traced": [P, ctypes.POINTER(Inputs), V, V, SZ, V, ctypes.POINTER(V),
                           ctypes.POINTER(I32), I32],
    }
    for name, args in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.csa_trace_events.argtypes = [P, I32]
    lib.csa_trace_events.restype = I32
    lib.csa_workspace_bytes.argtypes = [P, I32]
    lib.csa_workspace_bytes.restype = SZ
    lib.csa_status_str.argtypes = [ctypes.c_int]
    lib.csa_status_str.restype = ctypes.c_char_p
    lib.csa_last_error.argtypes = []
    lib.csa_last_error.restype = ctypes.c_char_p
    lib.csa_abi_version.argtypes = []
    lib.csa_abi_version.restype = ctypes.c_int32
    return lib


lib = _load()

EXPORTS = ("csa_compress", "csa_index_scores", "csa_index_topk", "csa_index_keys",
           "csa_sparse_mqa_fwd",
           "csa_sparse_mqa_fwd_sink", "csa_sparse_mqa_fwd_lse", "csa_sparse_mqa_bwd_dq",
           "csa_sparse_mqa_bwd_dkv", "csa_kl_target", "csa_fwd",
           "csa_fwd_noalloc",
           "hca_fwd", "csa_fwd_traced", "hca_fwd_traced", "csa_trace_events",
           "csa_workspace_bytes", "csa_debug_layout", "csa_status_str", "csa_last_error",
           "csa_abi_version")

KERNEL_NAMES = {0: "compress", 1: "window_rope", 2: "indexer", 3: "topk", 4: "attention",
                5: "index_topk", 6: "index_keys"}


def last_error() -> str:
    return lib.csa_last_error().decode()


def check(status: int):
    if status != CSA_OK:
        raise CsaError(status, last_error())


def params(cfg: wl.LayerConfig, **over) -> Params:
    """csa_params_t for a workload config (fields may be overridden by keyword)."""
    p = Params(B=cfg.B, S=cfg.S, H=cfg.H, D=cfg.D, rope_dim=cfg.rope_dim, ratio=cfg.ratio,
               overlap=cfg.overlap, window=cfg.window, topk=max(cfg.topk, 1),
               idx_heads=cfg.idx_heads, idx_dim=cfg.idx_dim,
               dtype=CSA_BF16 if cfg.dtype == wl.BF16 else CSA_F32,
               rope_theta=cfg.rope_theta, rms_eps=cfg.rms_eps, softmax_scale=cfg.softmax_scale,
               pos0=cfg.pos0, flags=(FLAG_NORM_WINDOW if cfg.norm_window else 0)
               | (FLAG_INDEX_PROLOGUE if cfg.index_prologue else 0)
               | (FLAG_INDEX_FP8 if cfg.index_fp8 else 0))
    for k, v in over.items():
        setattr(p, k, v)
    return p


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _act(p: Params) -> torch.dtype:
    return torch.bfloat16 if p.dtype == CSA_BF16 else torch.float32


def _chk(t: Optional[torch.Tensor], name: str, shape, dtype: torch.dtype, required: bool = True):
    """The C ABI sees only pointers, so a tensor of the wrong dtype or size would make a
    kernel read or write past its end: check both against the params here."""
    if t is None:
        if required:
            raise ValueError(f"{name}: a tensor is required")
        return
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    n = 1
    for s in shape:
        n *= int(s)
    if t.numel() != n:
        raise ValueError(f"{name}: {t.numel()} elements (shape {tuple(t.shape)}), expected "
                         f"{n} for shape {tuple(int(s) for s in shape)}")


def _key_rows(p: Params):
    """Shape and dtype of the indexer keys after csa_index_keys for p.flags."""
    n = p.S // p.ratio
    if p.flags & FLAG_INDEX_FP8:
        return (p.B, n, p.idx_dim + 16), torch.uint8
    return (p.B, n, p.idx_dim), _act(p)


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(p: Params, op: int) -> int:
    return int(lib.csa_workspace_bytes(ctypes.byref(p), op))


def workspace(p: Params, op: int, device="cuda") -> torch.Tensor:
    n = workspace_bytes(p, op)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device)


def compress(p: Params, va, ga, vb, gb, bias, kv_c=None, stream=None) -> torch.Tensor:
    n = p.S // p.ratio
    if kv_c is None:
        kv_c = torch.empty((p.B, n, p.D), dtype=va.dtype, device=va.device)
    act, bsd = _act(p), (p.B, p.S, p.D)
    for t, nm in ((va, "va"), (ga, "ga")):
        _chk(t, nm, bsd, act)
    for t, nm in ((vb, "vb"), (gb, "gb")):
        _chk(t, nm, bsd, act, required=False)
    _chk(bias, "bias", ((2 if p.overlap else 1) * p.ratio, p.D), torch.float32)
    _chk(kv_c, "kv_c", (p.B, n, p.D), act)
    check(lib.csa_compress(ctypes.byref(p), _ptr(va), _ptr(ga), _ptr(vb), _ptr(gb), _ptr(bias),
                           _ptr(kv_c), _stream(stream)))
    return kv_c


def index_scores(p: Params, q_idx, w_idx, k_idx, t0=0, nrows=None, scores=None, stream=None):
    nrows = p.S - t0 if nrows is None else nrows
    ld = max(p.S // p.ratio, 1)
    if scores is None:
        scores = torch.full((p.B, nrows, ld), float("nan"), dtype=torch.float32, device=q_idx.device)
    _chk_indexer(p, q_idx, w_idx)
    kshape, kdt = _key_rows(p) if p.flags & (FLAG_INDEX_FP8 | FLAG_INDEX_PROLOGUE) else \
        ((p.B, p.S // p.ratio, p.idx_dim), _act(p))
    _chk(k_idx, "k_idx", kshape, kdt)
    if scores.dtype != torch.float32 or scores.dim() != 3 or scores.shape[0] != p.B or \
            scores.shape[1] < nrows or scores.shape[2] < max(p.S // p.ratio, 1):
        raise ValueError(f"scores: need fp32 [B, >= nrows, >= S/ratio], got {scores.dtype} {tuple(scores.shape)}")
    if t0 < 0 or nrows < 0 or t0 + nrows > p.S:
        raise ValueError(f"rows {t0}..{t0 + nrows} outside 0..{p.S}")
    check(lib.csa_index_scores(ctypes.byref(p), _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(scores),
                               scores.shape[-1], t0, nrows, _stream(stream)))
    return scores


def _chk_indexer(p: Params, q_idx, w_idx):
    _chk(q_idx, "q_idx", (p.B, p.S, p.idx_heads, p.idx_dim), _act(p))
    _chk(w_idx, "w_idx", (p.B, p.S, p.idx_heads), torch.float32)


def index_keys(p: Params, k_idx, k_out=None, stream=None) -> torch.Tensor:
    """csa_index_keys: the key pass of the indexer prologue and/or the FP8 indexer
    (p.flags).  Returns the activation-dtype keys, or with FP8 a uint8 tensor of
    [B, S/ratio, idx_dim + 16] rows (codes in the MFMA order, fp32 scale, padding)."""
    if k_out is None:
        if p.flags & FLAG_INDEX_FP8:
            k_out = torch.empty((p.B, p.S // p.ratio, p.idx_dim + 16), dtype=torch.uint8, device=k_idx.device)
        else:
            k_out = torch.empty_like(k_idx)
    _chk(k_idx, "k_idx", (p.B, p.S // p.ratio, p.idx_dim), _act(p))
    kshape, kdt = _key_rows(p)
    _chk(k_out, "k_out", kshape, kdt)
    check(lib.csa_index_keys(ctypes.byref(p), _ptr(k_idx), _ptr(k_out), _stream(stream)))
    return k_out


def index_topk(p: Params, q_idx, w_idx, k_idx, idx=None, n_visible=None, ws=None, stream=None):
    dev = q_idx.device
    if idx is None:
        idx = torch.empty((p.B, p.S, p.topk), dtype=torch.int32, device=dev)
    if n_visible is None:
        n_visible = torch.empty((p.B, p.S), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(p, OP_INDEX_TOPK, dev)
    _chk_indexer(p, q_idx, w_idx)
    _chk(k_idx, "k_idx", (p.B, p.S // p.ratio, p.idx_dim), _act(p))
    _chk(idx, "idx", (p.B, p.S, p.topk), torch.int32)
    _chk(n_visible, "n_visible", (p.B, p.S), torch.int32)
    _chk_ws(ws)
    check(lib.csa_index_topk(ctypes.byref(p), _ptr(q_idx), _ptr(w_idx), _ptr(k_idx), _ptr(idx),
                             _ptr(n_visible), _ptr(ws), ws.numel(), _stream(stream)))
    return idx, n_visible


def _chk_ws(ws):
    if ws is not None and ws.dtype != torch.uint8:
        raise ValueError(f"ws: dtype {ws.dtype}, expected torch.uint8")


def _chk_attn(p: Params, q, kv_c, kv_raw, idx, sinks, **outs):
    act = _act(p)
    bshd = (p.B, p.S, p.H, p.D)
    _chk(q, "q", bshd, act)
    _chk(kv_c, "kv_c", (p.B, p.S // p.ratio, p.D), act, required=False)
    _chk(kv_raw, "kv_raw", (p.B, p.S, p.D), act)
    _chk(idx, "idx", (p.B, p.S, p.topk), torch.int32, required=False)
    _chk(sinks, "sinks", (p.H,), torch.float32, required=False)
    for nm, t in outs.items():
        _chk(t, nm, bshd, act)


def sparse_mqa_fwd(p: Params, q, kv_c, kv_raw, idx=None, o=None, ws=None, stream=None, sinks=None):
    """sinks: optional [H] fp32 softmax-sink logits (csa_sparse_mqa_fwd_sink)."""
    if o is None:
        o = torch.empty_like(q)
    if ws is None:
        ws = workspace(p, OP_SPARSE_MQA, q.device)
    _chk_attn(p, q, kv_c, kv_raw, idx, sinks, o=o)
    _chk_ws(ws)
    if sinks is None:
        check(lib.csa_sparse_mqa_fwd(ctypes.byref(p), _ptr(q), _ptr(kv_c), _ptr(kv_raw), _ptr(idx), _ptr(o),
                                     _ptr(ws), ws.numel(), _stream(stream)))
    else:
        check(lib.csa_sparse_mqa_fwd_sink(ctypes.byref(p), _ptr(q), _ptr(kv_c), _ptr(kv_raw), _ptr(idx),
                                          _ptr(sinks), _ptr(o), _ptr(ws), ws.numel(), _stream(stream)))
    return o


def sparse_mqa_bwd_dq(p: Params, q, kv_c, kv_raw, idx, o, d_o, dq=None, ws=None, stream=None,
                      sinks=None) -> torch.Tensor:
    """csa_sparse_mqa_bwd_dq: dL/dq [B,S,H,D] of sparse_mqa_fwd (same arguments and
    sinks), given its output o and dL/do."""
    if dq is None:
        dq = torch.empty_like(q)
    if ws is None:
        ws = workspace(p, OP_SPARSE_MQA, q.device)
    _chk_attn(p, q, kv_c, kv_raw, idx, sinks, o=o, d_o=d_o, dq=dq)
    _chk_ws(ws)
    check(lib.csa_sparse_mqa_bwd_dq(ctypes.byref(p), _ptr(q), _ptr(kv_c), _ptr(kv_raw), _ptr(idx),
                                    _ptr(sinks), _ptr(o), _ptr(d_o), _ptr(dq), _ptr(ws), ws.numel(),
                                    _stream(stream)))
    return dq


def sparse_mqa_fwd_lse(p: Params, q, kv_c, kv_raw, idx=None, sinks=None, o=None, lse=None, ws=None,
                       stream=None):
    """csa_sparse_mqa_fwd_lse: the forward's output o and lse [B,S,H] fp32, the natural
    log of each head's softmax denominator (what the backward reads)."""
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((p.B, p.S, p.H), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = workspace(p, OP_SPARSE_MQA, q.device)
    _chk_attn(p, q, kv_c, kv_raw, idx, sinks, o=o)
    _chk(lse, "lse", (p.B, p.S, p.H), torch.float32)
    _chk_ws(ws)
    check(lib.csa_sparse_mqa_fwd_lse(ctypes.byref(p), _ptr(q), _ptr(kv_c), _ptr(kv_raw), _ptr(idx),
                                     _ptr(sinks), _ptr(o), _ptr(lse), _ptr(ws), ws.numel(), _stream(stream)))
    return o, lse


def sparse_mqa_bwd_dkv(p: Params, q, kv_c, kv_raw, idx, o, lse, d_o, sinks=None, dkv_c=None, dkv_raw=None,
                       dsinks=None, ws=None, stream=None):
    """csa_sparse_mqa_bwd_dkv: dL/dkv_c [B,S/ratio,D] (None without kv_c), dL/dkv_raw
    [B,S,D] and dL/dsinks [H] (None without sinks), all fp32, for sparse_mqa_fwd_lse
    with the same arguments, given its o and lse and dL/do."""
    dev = q.device
    if dkv_c is None and kv_c is not None:
        dkv_c = torch.empty((p.B, p.S // p.ratio, p.D), dtype=torch.float32, device=dev)
    if dkv_raw is None:
        dkv_raw = torch.empty((p.B, p.S, p.D), dtype=torch.float32, device=dev)
    if dsinks is None and sinks is not None:
        dsinks = torch.empty((p.H,), dtype=torch.float32, device=dev)
    if ws is None:
        ws = workspace(p, OP_SPARSE_MQA_BWD, dev)
    _chk_attn(p, q, kv_c, kv_raw, idx, sinks, o=o, d_o=d_o)
    _chk(lse, "lse", (p.B, p.S, p.H), torch.float32)
    _chk(dkv_c, "dkv_c", (p.B, p.S // p.ratio, p.D), torch.float32, required=kv_c is not None)
    _chk(dkv_raw, "dkv_raw", (p.B, p.S, p.D), torch.float32)
    _chk(dsinks, "dsinks", (p.H,), torch.float32, required=sinks is not None)
    _chk_ws(ws)
    check(lib.csa_sparse_mqa_bwd_dkv(ctypes.byref(p), _ptr(q), _ptr(kv_c), _ptr(kv_raw), _ptr(idx), _ptr(sinks),
                                     _ptr(o), _ptr(lse), _ptr(d_o), _ptr(dkv_c), _ptr(dkv_raw), _ptr(dsinks),
                                     _ptr(ws), ws.numel(), _stream(stream)))
    return dkv_c, dkv_raw, dsinks


def kl_target(p: Params, q, kv_c, idx, target=None, stream=None) -> torch.Tensor:
    """csa_kl_target: [B, S, topk] fp32 target of the indexer's distillation loss."""
    if target is None:
        target = torch.empty((p.B, p.S, p.topk), dtype=torch.float32, device=q.device)
    _chk(q, "q", (p.B, p.S, p.H, p.D), _act(p))
    _chk(kv_c, "kv_c", (p.B, p.S // p.ratio, p.D), _act(p))
    _chk(idx, "idx", (p.B, p.S, p.topk), torch.int32)
    _chk(target, "target", (p.B, p.S, p.topk), torch.float32)
    check(lib.csa_kl_target(ctypes.byref(p), _ptr(q), _ptr(kv_c), _ptr(idx), _ptr(target), _stream(stream)))
    return target


def _chk_layer(p: Params, inp: dict, o, kv_c_out, idx_out, n_visible_out):
    act = _act(p)
    g = inp.get
    csa = bool(p.overlap)
    _chk_attn(p, g("q"), None, g("kv_raw"), None, g("sinks"), o=o)
    bsd = (p.B, p.S, p.D)
    _chk(g("va"), "va", bsd, act)
    _chk(g("ga"), "ga", bsd, act)
    _chk(g("vb"), "vb", bsd, act, required=csa)
    _chk(g("gb"), "gb", bsd, act, required=csa)
    _chk(g("bias"), "bias", ((2 if csa else 1) * p.ratio, p.D), torch.float32)
    if csa:
        _chk_indexer(p, g("q_idx"), g("w_idx"))
        _chk(g("k_idx"), "k_idx", (p.B, p.S // p.ratio, p.idx_dim), act)
        _chk(idx_out, "idx_out", (p.B, p.S, p.topk), torch.int32, required=False)
        _chk(n_visible_out, "n_visible_out", (p.B, p.S), torch.int32, required=False)
    _chk(kv_c_out, "kv_c_out", (p.B, p.S // p.ratio, p.D), act, required=False)


def make_inputs_struct(inp: dict, kv_c_out=None, idx_out=None, n_visible_out=None, lse_out=None) -> Inputs:
    g = inp.get
    return Inputs(q=_ptr(g("q")), kv_raw=_ptr(g("kv_raw")), va=_ptr(g("va")), ga=_ptr(g("ga")),
                  vb=_ptr(g("vb")), gb=_ptr(g("gb")), bias=_ptr(g("bias")), q_idx=_ptr(g("q_idx")),
                  w_idx=_ptr(g("w_idx")), k_idx=_ptr(g("k_idx")), kv_c_out=_ptr(kv_c_out),
                  idx_out=_ptr(idx_out), n_visible_out=_ptr(n_visible_out), sinks=_ptr(g("sinks")),
                  lse_out=_ptr(lse_out))


def layer_fwd(p: Params, inp: dict, o=None, ws=None, stream=None, kv_c_out=None, idx_out=None,
              n_visible_out=None, lse_out=None):
    """csa_fwd when p.overlap == 1, else hca_fwd.  lse_out: optional [B,S,H] fp32, the
    attention's log-denominators for the key-side backward."""
    q = inp["q"]
    if o is None:
        o = torch.empty_like(q)
    op = OP_CSA_FWD if p.overlap else OP_HCA_FWD
    if ws is None:
        ws = workspace(p, op, q.device)
    _chk_layer(p, inp, o, kv_c_out, idx_out, n_visible_out)
    _chk(lse_out, "lse_out", (p.B, p.S, p.H), torch.float32, required=False)
    _chk_ws(ws)
    s = make_inputs_struct(inp, kv_c_out, idx_out, n_visible_out, lse_out)
    f = lib.csa_fwd if p.overlap else lib.hca_fwd
    check(f(ctypes.byref(p), ctypes.byref(s), _ptr(o), _ptr(ws), ws.numel(), _stream(stream)))
    return o


def csa_fwd_noalloc(p: Params, inp: dict, o=None, stream=None, kv_c_out=None, idx_out=None,
                    n_visible_out=None):
    """csa_fwd_noalloc: the fused CSA layer with the library's static workspace (no ws
    argument; the call allocates nothing)."""
    q = inp["q"]
    if o is None:
        o = torch.empty_like(q)
    _chk_layer(p, inp, o, kv_c_out, idx_out, n_visible_out)
    s = make_inputs_struct(inp, kv_c_out, idx_out, n_visible_out)
    check(lib.csa_fwd_noalloc(ctypes.byref(p), ctypes.byref(s), _ptr(o), _stream(stream)))
    return o


NOALLOC_SCRATCH_BYTES = 256 << 20


class LayerTrace:
    """Caller-owned HIP events for the traced fused call; per-kernel times in ms."""

    def __init__(self, p: Params):
        op = OP_CSA_FWD if p.overlap else OP_HCA_FWD
        self.n = int(lib.csa_trace_events(ctypes.byref(p), op))
        if self.n <= 0:
            raise CsaError(CSA_ERR_INVALID_ARG, last_error())
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(self.n)]
        for e in self.events:  # materialise the underlying hipEvent_t
            e.record()
        torch.cuda.synchronize()
        self.handles = (ctypes.c_void_p * self.n)(*[e.cuda_event for e in self.events])
        self.kinds = (ctypes.c_int32 * self.n)()

    def kernel_ms(self) -> dict:
        """Per-kernel sums of launch durations (ms) from the last traced call, plus the
        number of launches of each kernel."""
        ms, launches = {}, {}
        for i in range(self.n - 1):
            name = KERNEL_NAMES[self.kinds[i]]
            ms[name] = ms.get(name, 0.0) + self.events[i].elapsed_time(self.events[i + 1])
            launches[name] = launches.get(name, 0) + 1
        return ms, launches


def layer_fwd_traced(p: Params, inp: dict, trace: LayerTrace, o=None, ws=None, stream=None,
                     kv_c_out=None, idx_out=None, n_visible_out=None, lse_out=None):
    q = inp["q"]
    if o is None:
        o = torch.empty_like(q)
    op = OP_CSA_FWD if p.overlap else OP_HCA_FWD
    if ws is None:
        ws = workspace(p, op, q.device)
    _chk_layer(p, inp, o, kv_c_out, idx_out, n_visible_out)
    _chk(lse_out, "lse_out", (p.B, p.S, p.H), torch.float32, required=False)
    _chk_ws(ws)
    s = make_inputs_struct(inp, kv_c_out, idx_out, n_visible_out, lse_out)
    f = lib.csa_fwd_traced if p.overlap else lib.hca_fwd_traced
    check(f(ctypes.byref(p), ctypes.byref(s), _ptr(o), _ptr(ws), ws.numel(), _stream(stream),
            trace.handles, trace.kinds, trace.n))
    return o


def debug_layout(p: Params, device="cuda", stream=None):
    n = max(p.S // p.ratio, 1)
    comp = torch.full((n,), -7, dtype=torch.int32, device=device)
    nv = torch.full((max(p.S, 1),), -7, dtype=torch.int32, device=device)
    wl_ = torch.full((max(p.S, 1),), -7, dtype=torch.int32, device=device)
    check(lib.csa_debug_layout(ctypes.byref(p), _ptr(comp), _ptr(nv), _ptr(wl_), _stream(stream)))
    return comp, nv, wl_
