"""C-ABI checks that need no GPU: the library loads and exports every entry point the
header declares, the binding's struct layout matches the C compiler's, and every
argument error is reported by host-side validation before anything is launched.

Only failing-validation calls are made here (plus pure host queries), so no kernel is
ever enqueued: these tests are safe with or without a GPU present.
"""
import ctypes
import os
import re
import subprocess

import pytest

from compressed_sparse_attention_hca_amd import binding as bd
from compressed_sparse_attention_hca_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa.h")


def header_functions():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(csa_\w+|hca_\w+)\s*\(", txt)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 10
    out = subprocess.run(["nm", "-D", "--defined-only", bd.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (\w+)$", out, flags=re.M))
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    for n in names:
        assert hasattr(bd.lib, n)
    assert set(bd.EXPORTS) == set(names)


def test_abi_version_and_status_strings():
    assert bd.lib.csa_abi_version() == 8
    for code, name in bd._status_names.items():
        assert bd.lib.csa_status_str(code).decode() == name


def test_struct_layout_matches_c_compiler(tmp_path):
    src = tmp_path / "layout.c"
    fields = [f for f, _ in bd.Params._fields_]
    ifields = [f for f, _ in bd.Inputs._fields_]
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "csa.h"', "int main(void){",
             'printf("%zu %zu\\n", sizeof(csa_params_t), sizeof(csa_inputs_t));']
    lines += [f'printf("%zu\\n", offsetof(csa_params_t, {f}));' for f in fields]
    lines += [f'printf("%zu\\n", offsetof(csa_inputs_t, {f}));' for f in ifields]
    lines += ["return 0;}"]
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(bd.Params) and vals[1] == ctypes.sizeof(bd.Inputs)
    offs = vals[2:]
    assert offs[:len(fields)] == [getattr(bd.Params, f).offset for f in fields]
    assert offs[len(fields):] == [getattr(bd.Inputs, f).offset for f in ifields]


# Fake, 16-byte aligned device addresses.  Every call below fails validation, so they
# are never dereferenced or passed to a kernel.
A = 0x10000


def p_c1(**kw):
    return bd.params(wl.C1, **kw)


def call_compress(p, va=A, ga=A, vb=A, gb=A, bias=A, out=A):
    return bd.lib.csa_compress(ctypes.byref(p) if p is not None else None, va, ga, vb, gb, bias, out, None)


@pytest.mark.parametrize("over,code", [
    (dict(D=96), bd.CSA_ERR_INVALID_ARG),
    (dict(D=1024), bd.CSA_ERR_INVALID_ARG),
    (dict(D=192), bd.CSA_ERR_UNSUPPORTED),
    (dict(rope_dim=7), bd.CSA_ERR_INVALID_ARG),
    (dict(rope_dim=576), bd.CSA_ERR_INVALID_ARG),
    (dict(rope_dim=256), bd.CSA_ERR_UNSUPPORTED),
    (dict(S=4097), bd.CSA_ERR_INVALID_ARG),
    (dict(ratio=0), bd.CSA_ERR_INVALID_ARG),
    (dict(overlap=2), bd.CSA_ERR_INVALID_ARG),
    (dict(dtype=5), bd.CSA_ERR_INVALID_ARG),
    (dict(flags=8), bd.CSA_ERR_INVALID_ARG),
    (dict(B=-1), bd.CSA_ERR_INVALID_ARG),
    (dict(rope_theta=0.0), bd.CSA_ERR_INVALID_ARG),
    (dict(rms_eps=float("nan")), bd.CSA_ERR_INVALID_ARG),
])
def test_compress_rejects_bad_params(over, code):
    assert call_compress(p_c1(**over)) == code
    assert bd.last_error()


def test_compress_rejects_null_and_misaligned_pointers():
    p = p_c1()
    assert call_compress(None) == bd.CSA_ERR_INVALID_ARG
    assert call_compress(p, va=None) == bd.CSA_ERR_INVALID_ARG and "va" in bd.last_error()
    assert call_compress(p, bias=A + 4) == bd.CSA_ERR_INVALID_ARG and "aligned" in bd.last_error()
    assert call_compress(p, out=None) == bd.CSA_ERR_INVALID_ARG and "kv_c" in bd.last_error()
    assert call_compress(p, gb=None) == bd.CSA_ERR_INVALID_ARG and "gb" in bd.last_error()
    ph = bd.params(wl.C2)
    assert call_compress(ph) == bd.CSA_ERR_INVALID_ARG and "NULL when overlap" in bd.last_error()


def test_index_topk_rejects():
    def call(p, ws_bytes=1 << 40, idx=A, ws=A):
        return bd.lib.csa_index_topk(ctypes.byref(p), A, A, A, idx, A, ws, ws_bytes, None)
    assert call(p_c1(topk=0)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(topk=4096)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(idx_heads=65)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(idx_dim=24)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(idx_dim=256)) == bd.CSA_ERR_UNSUPPORTED
    assert call(p_c1(S=4 * 40000)) == bd.CSA_ERR_UNSUPPORTED
    assert call(p_c1(), idx=None) == bd.CSA_ERR_INVALID_ARG
    # top-k <= 512 is selected inside the indexer kernel: no workspace
    assert bd.workspace_bytes(p_c1(), bd.OP_INDEX_TOPK) == 0
    # larger top-k scores query chunks into the workspace first
    need = bd.workspace_bytes(p_c1(topk=1024), bd.OP_INDEX_TOPK)
    assert need >= 64 * 1024 * 4  # at least 64 query rows of 1024 fp32 scores
    assert call(p_c1(topk=1024), ws_bytes=need - 1) == bd.CSA_ERR_WORKSPACE
    assert call(p_c1(topk=1024), ws=None) == bd.CSA_ERR_INVALID_ARG


def test_index_prologue_validation_and_workspace():
    """The indexer prologue rotates inside the indexer dims (rope_dim <= idx_dim), keeps
    the rotated keys in the workspace, and adds one launch to the traced fused call."""
    pro = dict(flags=bd.FLAG_INDEX_PROLOGUE)

    def topk(p, ws_bytes=1 << 40, ws=A):
        return bd.lib.csa_index_topk(ctypes.byref(p), A, A, A, A, A, ws, ws_bytes, None)
    assert topk(p_c1(rope_dim=130, D=512, **pro)) == bd.CSA_ERR_INVALID_ARG
    assert "rope_dim" in bd.last_error()
    c0 = bd.params(wl.C0, flags=bd.FLAG_INDEX_PROLOGUE, rope_dim=18)   # idx_dim 16
    assert topk(c0) == bd.CSA_ERR_INVALID_ARG
    need = bd.workspace_bytes(p_c1(**pro), bd.OP_INDEX_TOPK)
    assert need >= 1024 * 128 * 2                     # the rotated keys of C1, bf16
    assert bd.workspace_bytes(p_c1(), bd.OP_INDEX_TOPK) == 0
    assert topk(p_c1(**pro), ws_bytes=need - 1) == bd.CSA_ERR_WORKSPACE
    assert topk(p_c1(**pro), ws=None) == bd.CSA_ERR_INVALID_ARG
    assert (bd.workspace_bytes(p_c1(**pro), bd.OP_CSA_FWD)
            == bd.workspace_bytes(p_c1(), bd.OP_CSA_FWD) + need)
    assert bd.lib.csa_trace_events(ctypes.byref(p_c1(**pro)), bd.OP_CSA_FWD) == \
        bd.lib.csa_trace_events(ctypes.byref(p_c1()), bd.OP_CSA_FWD) + 1

    def keys(p, k=A, out=A + (1 << 30)):
        return bd.lib.csa_index_keys(ctypes.byref(p), k, out, None)
    assert keys(p_c1(**pro), out=A + 16) == bd.CSA_ERR_INVALID_ARG       # overlapping
    assert "overlaps" in bd.last_error()
    assert keys(p_c1(**pro), k=None) == bd.CSA_ERR_INVALID_ARG
    assert keys(p_c1(**pro), out=A + 8) == bd.CSA_ERR_INVALID_ARG        # misaligned
    assert keys(p_c1(rope_dim=130, **pro)) == bd.CSA_ERR_INVALID_ARG
    assert keys(p_c1(idx_dim=24, **pro)) == bd.CSA_ERR_INVALID_ARG
    assert keys(p_c1(rope_theta=-1.0, **pro)) == bd.CSA_ERR_INVALID_ARG
    assert keys(p_c1(flags=8)) == bd.CSA_ERR_INVALID_ARG                # unknown flag
    assert keys(p_c1()) == bd.CSA_ERR_INVALID_ARG and "needs" in bd.last_error()


def test_index_fp8_validation_and_workspace():
    """The FP8 indexer runs on idx_dim 64 and 128; its key rows (codes, scale and
    padding: idx_dim + 16 bytes) live in the workspace; the key pass's output rows
    must not overlap its input."""
    f8 = dict(flags=bd.FLAG_INDEX_FP8)

    def topk(p, ws_bytes=1 << 40, ws=A):
        return bd.lib.csa_index_topk(ctypes.byref(p), A, A, A, A, A, ws, ws_bytes, None)
    assert topk(p_c1(idx_dim=32, **f8)) == bd.CSA_ERR_UNSUPPORTED
    assert "FP8" in bd.last_error()
    assert bd.workspace_bytes(p_c1(**f8), bd.OP_INDEX_TOPK) == 1024 * (128 + 16)
    both = dict(flags=bd.FLAG_INDEX_FP8 | bd.FLAG_INDEX_PROLOGUE)
    assert bd.workspace_bytes(p_c1(**both), bd.OP_INDEX_TOPK) == 1024 * (128 + 16)
    need = bd.workspace_bytes(p_c1(**f8), bd.OP_INDEX_TOPK)
    assert topk(p_c1(**f8), ws_bytes=need - 1) == bd.CSA_ERR_WORKSPACE
    assert bd.lib.csa_trace_events(ctypes.byref(p_c1(**f8)), bd.OP_CSA_FWD) == \
        bd.lib.csa_trace_events(ctypes.byref(p_c1()), bd.OP_CSA_FWD) + 1
    # an output that starts inside the input (1024 rows of 256 bytes) overlaps it
    assert bd.lib.csa_index_keys(ctypes.byref(p_c1(**f8)), A, A + 1024 * 256 - 16, None) == bd.CSA_ERR_INVALID_ARG
    assert bd.lib.csa_index_keys(ctypes.byref(p_c1(idx_dim=16, **f8)), A, A + (1 << 30), None) == \
        bd.CSA_ERR_UNSUPPORTED


def test_index_scores_rejects_rows_and_ld():
    def call(p, ld=1024, t0=0, n=16):
        return bd.lib.csa_index_scores(ctypes.byref(p), A, A, A, A, ld, t0, n, None)
    assert call(p_c1(), t0=-1) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), t0=4090, n=10) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), ld=1000) == bd.CSA_ERR_INVALID_ARG


def test_sparse_mqa_rejects():
    def call(p, q=A, kv_c=A, kv_raw=A, idx=A, o=A, ws=A, ws_bytes=1 << 40):
        return bd.lib.csa_sparse_mqa_fwd(ctypes.byref(p), q, kv_c, kv_raw, idx, o, ws, ws_bytes, None)
    assert call(p_c1(H=0)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(H=65)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(window=-1)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(window=0), kv_c=None, idx=None) == bd.CSA_ERR_INVALID_ARG  # nothing to attend
    assert call(p_c1(), kv_c=None) == bd.CSA_ERR_INVALID_ARG  # idx without entries
    assert call(p_c1(softmax_scale=0.0)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), q=None) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), kv_raw=A + 8) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), ws_bytes=100) == bd.CSA_ERR_WORKSPACE
    def call_sink(p, sinks, ws_bytes=1 << 40):
        return bd.lib.csa_sparse_mqa_fwd_sink(ctypes.byref(p), A, A, A, A, sinks, A, A, ws_bytes, None)
    assert call_sink(p_c1(), A + 4) == bd.CSA_ERR_INVALID_ARG and "sinks" in bd.last_error()
    assert call_sink(p_c1(H=0), A) == bd.CSA_ERR_INVALID_ARG
    assert call_sink(p_c1(), A, ws_bytes=100) == bd.CSA_ERR_WORKSPACE


def test_fused_rejects():
    ins = bd.Inputs(q=A, kv_raw=A, va=A, ga=A, vb=A, gb=A, bias=A, q_idx=A, w_idx=A, k_idx=A)
    def call(f, p, inputs=ins, o=A, ws_bytes=1 << 40):
        return f(ctypes.byref(p), ctypes.byref(inputs) if inputs is not None else None, o, A, ws_bytes, None)
    assert call(bd.lib.csa_fwd, bd.params(wl.C2)) == bd.CSA_ERR_INVALID_ARG      # overlap 0
    assert call(bd.lib.hca_fwd, p_c1()) == bd.CSA_ERR_INVALID_ARG                 # overlap 1
    assert call(bd.lib.csa_fwd, p_c1(), inputs=None) == bd.CSA_ERR_INVALID_ARG
    assert call(bd.lib.csa_fwd, p_c1(), o=None) == bd.CSA_ERR_INVALID_ARG
    assert call(bd.lib.csa_fwd, p_c1(), ws_bytes=0) == bd.CSA_ERR_WORKSPACE
    bad = bd.Inputs(q=A, kv_raw=A, va=A, ga=A, vb=A, gb=A, bias=A, q_idx=None, w_idx=A, k_idx=A)
    assert call(bd.lib.csa_fwd, p_c1(), inputs=bad) == bd.CSA_ERR_INVALID_ARG and "q_idx" in bd.last_error()
    hca_in = bd.Inputs(q=A, kv_raw=A, va=A, ga=A, vb=A, gb=None, bias=A)
    assert call(bd.lib.hca_fwd, bd.params(wl.C2), inputs=hca_in) == bd.CSA_ERR_INVALID_ARG  # vb given


def test_workspace_bytes():
    p = p_c1()
    csa = bd.workspace_bytes(p, bd.OP_CSA_FWD)
    hca = bd.workspace_bytes(bd.params(wl.C2), bd.OP_HCA_FWD)
    assert bd.workspace_bytes(p, bd.OP_COMPRESS) == 0
    mqa = bd.workspace_bytes(p, bd.OP_SPARSE_MQA)
    assert mqa >= 4096 * 512 * 2                     # rotated window latents
    assert csa >= mqa + 1024 * 512 * 2 + 4096 * 512 * 4  # + entries + selection
    assert hca >= 65536 * 512 * 2 + 512 * 512 * 2
    assert bd.workspace_bytes(p_c1(D=96), bd.OP_CSA_FWD) == 0
    assert bd.workspace_bytes(p, 99) == 0
    # C3 stays well inside one GPU's memory
    assert bd.workspace_bytes(bd.params(wl.C3), bd.OP_CSA_FWD) < 2 << 30


def test_empty_problem_is_a_noop():
    p = p_c1(S=0)
    assert call_compress(p, va=None, ga=None, vb=None, gb=None, bias=None, out=None) == bd.CSA_OK
    p = p_c1(B=0)
    assert bd.lib.csa_sparse_mqa_fwd(ctypes.byref(p), None, None, None, None, None, None, 0, None) == bd.CSA_OK


def test_kl_target_rejects():
    def call(p, q=A, kv=A, idx=A, out=A):
        return bd.lib.csa_kl_target(ctypes.byref(p), q, kv, idx, out, None)
    assert call(p_c1(), idx=None) == bd.CSA_ERR_INVALID_ARG and "idx" in bd.last_error()
    assert call(p_c1(), out=None) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), q=A + 4) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(topk=0)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(H=65)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(D=192)) == bd.CSA_ERR_UNSUPPORTED


def test_bwd_dq_rejects():
    """Argument checks of csa_sparse_mqa_bwd_dq fail before any GPU call."""
    def call(p, q=A, kv=A, kvr=A, idx=A, o=A, d_o=A, dq=A):
        return bd.lib.csa_sparse_mqa_bwd_dq(ctypes.byref(p), q, kv, kvr, idx, None, o, d_o, dq, A, 1 << 30, None)
    assert call(p_c1(), d_o=None) == bd.CSA_ERR_INVALID_ARG and "d_o" in bd.last_error()
    assert call(p_c1(), dq=None) == bd.CSA_ERR_INVALID_ARG and "dq" in bd.last_error()
    assert call(p_c1(), o=None) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), q=A + 4) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), kv=None) == bd.CSA_ERR_INVALID_ARG and "idx" in bd.last_error()
    assert call(p_c1(H=65)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(D=192)) == bd.CSA_ERR_UNSUPPORTED
    z = ctypes.byref(p_c1(B=0))
    assert bd.lib.csa_sparse_mqa_bwd_dq(z, None, None, None, None, None, None, None, None, None, 0, None) == bd.CSA_OK


def test_bwd_dkv_rejects():
    """Argument checks of csa_sparse_mqa_bwd_dkv (and of the forward that keeps lse)
    fail before any GPU call."""
    W = 1 << 40

    def call(p, q=A, kv=A, kvr=A, idx=A, sinks=None, o=A, lse=A, d_o=A, dkv_c=A, dkv_raw=A, dsinks=None, wsb=W):
        return bd.lib.csa_sparse_mqa_bwd_dkv(ctypes.byref(p), q, kv, kvr, idx, sinks, o, lse, d_o, dkv_c, dkv_raw,
                                             dsinks, A, wsb, None)
    assert call(p_c1(), lse=None) == bd.CSA_ERR_INVALID_ARG and "lse" in bd.last_error()
    assert call(p_c1(), d_o=None) == bd.CSA_ERR_INVALID_ARG and "d_o" in bd.last_error()
    assert call(p_c1(), dkv_raw=None) == bd.CSA_ERR_INVALID_ARG and "dkv_raw" in bd.last_error()
    assert call(p_c1(), dkv_c=None) == bd.CSA_ERR_INVALID_ARG and "dkv_c" in bd.last_error()
    assert call(p_c1(), kv=None, idx=None) == bd.CSA_ERR_INVALID_ARG and "dkv_c" in bd.last_error()
    assert call(p_c1(), sinks=A) == bd.CSA_ERR_INVALID_ARG and "dsinks" in bd.last_error()
    assert call(p_c1(), dsinks=A) == bd.CSA_ERR_INVALID_ARG and "dsinks" in bd.last_error()
    assert call(p_c1(), lse=A + 4) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(), kv=None) == bd.CSA_ERR_INVALID_ARG and "idx" in bd.last_error()
    assert call(p_c1(), wsb=0) == bd.CSA_ERR_WORKSPACE
    assert call(p_c1(H=65)) == bd.CSA_ERR_INVALID_ARG
    assert call(p_c1(D=192)) == bd.CSA_ERR_UNSUPPORTED
    assert call(p_c1(dtype=bd.CSA_F32)) == bd.CSA_ERR_UNSUPPORTED and "D <= 256" in bd.last_error()
    z = ctypes.byref(p_c1(B=0))  # empty batch without sinks: nothing to launch
    assert bd.lib.csa_sparse_mqa_bwd_dkv(z, *([None] * 11), None, 0, None) == bd.CSA_OK
    assert bd.lib.csa_sparse_mqa_fwd_lse(ctypes.byref(p_c1()), A, A, A, A, None, A, None, A, W, None) \
        == bd.CSA_ERR_INVALID_ARG and "lse" in bd.last_error()


def test_bwd_dkv_workspace():
    """The key-side workspace holds the rotated window latents, the per-query sink terms
    and a chunk of per-pair key gradients of at most 4 GiB plus the chunk's inverse
    index; the chunk covers the whole problem when it fits."""
    c1 = bd.params(wl.C1)
    ws1 = bd.workspace_bytes(c1, bd.OP_SPARSE_MQA_BWD)
    win = 4096 * 512 * 2
    assert ws1 >= win + 4096 * (512 + 128) * 512 * 2      # every row's pairs of the selected mode
    assert ws1 <= win + (4 << 30) + (256 << 20)
    c3 = bd.params(wl.C3)
    ws3 = bd.workspace_bytes(c3, bd.OP_SPARSE_MQA_BWD)
    assert (4 << 30) - (1 << 20) <= ws3 - 65536 * 512 * 2 <= (4 << 30) + (256 << 20)
    c0 = bd.params(wl.C0)
    assert 0 < bd.workspace_bytes(c0, bd.OP_SPARSE_MQA_BWD) < 64 << 20
    swa = bd.params(wl.C1.replace(kind="swa", topk=0))
    assert bd.workspace_bytes(swa, bd.OP_SPARSE_MQA_BWD) >= win + 4096 * 128 * 512 * 2
    assert bd.workspace_bytes(p_c1(D=192), bd.OP_SPARSE_MQA_BWD) == 0


# ---- the binding checks dtype and size against the params before any call --------
def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def _attn_args(cfg, act):
    import torch
    B, S, H, D = cfg.B, cfg.S, cfg.H, cfg.D
    return dict(q=_t((B, S, H, D), act), kv_c=_t((B, S // cfg.ratio, D), act),
                kv_raw=_t((B, S, D), act), idx=_t((B, S, cfg.topk), torch.int32))


@pytest.mark.parametrize("bad", ["q_dtype", "q_size", "idx_dtype", "idx_size", "kv_raw_size",
                                 "sinks_dtype", "o_size"])
def test_binding_rejects_mismatched_attention_tensors(bad):
    import torch
    cfg = wl.C0.replace(S=32)
    p = bd.params(cfg)
    a = _attn_args(cfg, torch.float32)
    o = _t(a["q"].shape, torch.float32)
    sinks = None
    if bad == "q_dtype":
        a["q"] = a["q"].to(torch.bfloat16)
    elif bad == "q_size":
        a["q"] = _t((1, 32, cfg.H + 1, cfg.D), torch.float32)
    elif bad == "idx_dtype":
        a["idx"] = a["idx"].to(torch.int64)
    elif bad == "idx_size":
        a["idx"] = _t((1, 32, cfg.topk - 1), torch.int32)
    elif bad == "kv_raw_size":
        a["kv_raw"] = _t((1, 31, cfg.D), torch.float32)
    elif bad == "sinks_dtype":
        sinks = _t((cfg.H,), torch.float64)
    elif bad == "o_size":
        o = _t((1, 32, cfg.H, cfg.D // 2), torch.float32)
    name = bad.rsplit("_", 1)[0]
    with pytest.raises(ValueError, match=name):
        bd.sparse_mqa_fwd(p, a["q"], a["kv_c"], a["kv_raw"], a["idx"], o=o, ws=_t((256,), torch.uint8),
                          sinks=sinks)
    with pytest.raises(ValueError, match=name):
        bd.sparse_mqa_bwd_dq(p, a["q"], a["kv_c"], a["kv_raw"], a["idx"], o, o.clone(), dq=o.clone(),
                             ws=_t((256,), torch.uint8), sinks=sinks)


def test_binding_rejects_mismatched_indexer_and_compress_tensors():
    import torch
    cfg = wl.C1.replace(S=64)
    p = bd.params(cfg)
    bf = torch.bfloat16
    B, S, HI, DI, D = cfg.B, cfg.S, cfg.idx_heads, cfg.idx_dim, cfg.D
    q_idx, w_idx, k_idx = _t((B, S, HI, DI), bf), _t((B, S, HI), torch.float32), _t((B, S // 4, DI), bf)
    with pytest.raises(ValueError, match="w_idx"):
        bd.index_topk(p, q_idx, w_idx.to(bf), k_idx, idx=_t((B, S, cfg.topk), torch.int32),
                      n_visible=_t((B, S), torch.int32), ws=_t((256,), torch.uint8))
    with pytest.raises(ValueError, match="k_idx"):
        bd.index_topk(p, q_idx, w_idx, _t((B, S // 4, DI * 2), bf), idx=_t((B, S, cfg.topk), torch.int32),
                      n_visible=_t((B, S), torch.int32), ws=_t((256,), torch.uint8))
    with pytest.raises(ValueError, match="n_visible"):
        bd.index_topk(p, q_idx, w_idx, k_idx, idx=_t((B, S, cfg.topk), torch.int32),
                      n_visible=_t((B, S + 1), torch.int32), ws=_t((256,), torch.uint8))
    p8 = bd.params(cfg.replace(index_fp8=True))
    with pytest.raises(ValueError, match="k_out"):   # fp8 key rows are uint8 [B, n, DI + 16]
        bd.index_keys(p8, k_idx, k_out=_t((B, S // 4, DI), bf))
    with pytest.raises(ValueError, match="bias"):
        bd.compress(p, _t((B, S, D), bf), _t((B, S, D), bf), _t((B, S, D), bf), _t((B, S, D), bf),
                    _t((4, D), torch.float32), kv_c=_t((B, S // 4, D), bf))
    with pytest.raises(ValueError, match="target"):
        bd.kl_target(p, _t((B, S, cfg.H, D), bf), _t((B, S // 4, D), bf), _t((B, S, cfg.topk), torch.int32),
                     target=_t((B, S, cfg.topk), bf))


def test_binding_rejects_mismatched_layer_inputs():
    import torch
    cfg = wl.C0.replace(S=32)
    p = bd.params(cfg)
    inp = wl.make_inputs(cfg)
    o = torch.empty_like(inp["q"])
    bad = dict(inp, gb=inp["gb"][:, :16].contiguous())
    with pytest.raises(ValueError, match="gb"):
        bd.layer_fwd(p, bad, o=o, ws=_t((256,), torch.uint8))
    with pytest.raises(ValueError, match="idx_out"):
        bd.layer_fwd(p, inp, o=o, ws=_t((256,), torch.uint8), idx_out=_t((1, 32, cfg.topk), torch.int64))
    # a well-formed call reaches the pointer marshalling, which wants device tensors
    with pytest.raises(ValueError, match="GPU"):
        bd.layer_fwd(p, inp, o=o, ws=_t((256,), torch.uint8))
