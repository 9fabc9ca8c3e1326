#!/usr/bin/env python3
"""Throughput of the fused compressed-attention layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3|C2|C1|C4]

One step is one fused layer call (csa_fwd for CSA, hca_fwd for HCA) over one batch of
seeded synthetic inputs that are already resident in HBM: gated pooling + RMSNorm +
RoPE of the entries, rotation of the window latents, indexer scores and top-k (CSA),
sparse multi-query attention with de-rotation.  W untimed steps, then exactly K timed
steps bracketed by device synchronisation.  Per-kernel durations come from HIP events
recorded between the kernel launches of every timed step (the library records
caller-owned events; one event set per step, read after the timed region).

Prints one JSON line.  value = tokens/s of the whole job (B*S per step); TFLOP/s
counts algorithmic FLOPs of causally visible pairs only.  `roofline` describes the
kernel with the largest time per step; `cpu_baseline` times the fp64 oracle on a
bounded sample of query rows of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "CSA layer fwd tokens/s + TFLOP/s at S=64K (1 GPU); % of bf16 MFMA peak"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_work(cfg, wl):
    """Algorithmic work per step of each kernel: (amount, unit, bound)."""
    f = wl.layer_flops(cfg)
    es = 2 if cfg.dtype == wl.BF16 else 4
    B, S, D = cfg.B, cfg.S, cfg.D
    n_proj = 4 if cfg.kind == "csa" else 2
    work = {
        # read every projection once per token, write one entry per `ratio` tokens
        "compress": (B * S * n_proj * D * es + B * (S // cfg.ratio) * D * es, "bytes", "hbm"),
        # read and write every raw latent once
        "window_rope": (2 * B * S * D * es, "bytes", "hbm"),
        "attention": (f["attention"], "flops", "mfma"),
        # attention backward, query side: QK, dP = dU.K^T and dz.K per (query, key), 6*H*D
        "bwd_dq": (1.5 * f["attention"], "flops", "mfma"),
        # key side: QK and dP again, then the two contractions over heads that form each
        # key's gradient, 8*H*D per (query, key) (the inverse-index sums are HBM work on
        # top, counted in the same timed group)
        "bwd_dkv": (2.0 * f["attention"], "flops", "mfma"),
    }
    if cfg.kind == "csa":
        work["indexer"] = (f["indexer"], "flops", "mfma")
        # fused indexer + selection: the indexer's FLOPs (the selection reads no scores)
        work["index_topk"] = (f["indexer"], "flops", "mfma")
        # distillation target: one QK product per (query, selected entry) pair
        work["kl_target"] = (2 * cfg.H * cfg.D * wl.layer_flops(cfg)["selected_pairs"], "flops", "mfma")
        # indexer key prologue: read and write every indexer key once
        work["index_keys"] = (2 * B * (S // cfg.ratio) * cfg.idx_dim * es, "bytes", "hbm")
        # read every visible score once, write K indices + n_visible per row
        work["topk"] = (4 * f["visible_pairs"] + B * S * (4 * cfg.topk + 4), "bytes", "hbm")
    return work


def roofline_entry(amount, unit, bound, ms, peak_tflops=PEAK_BF16_TFLOPS):
    """peak_tflops: the MFMA peak of the contraction's own dtype."""
    if unit == "flops":
        achieved = amount / (ms * 1e-3) / 1e12
        return {"bound": bound, "achieved": round(achieved, 2), "peak": peak_tflops,
                "unit": "TFLOP/s", "frac": round(achieved / peak_tflops, 4)}
    achieved = amount / (ms * 1e-3) / 1e9
    return {"bound": bound, "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4)}


def dtype_label(index_fp8: bool) -> str:
    """The arithmetic type of the step: bf16 operands with fp32 accumulation, and with
    the FP8 indexer the indexer's QK on E4M3 codes."""
    return "bf16, indexer QK fp8 (e4m3)" if index_fp8 else "bf16"


# Library kernel -> (rocprofv3 kernel-name fragment, source files it is built from).
KERNEL_SOURCES = {
    "compress": ("compress_kernel", ["compress.hip"]),
    "window_rope": ("window_rope_kernel", ["compress.hip"]),
    "indexer": ("index_scores_kernel", ["indexer.hip"]),
    "index_topk": ("index_topk_kernel", ["indexer.hip"]),
    "topk": ("topk_kernel", ["topk.hip"]),
    "attention": ("sparse_mqa", ["sparse_mqa.hip"]),
    "kl_target": ("kl_target", ["kl_target.hip"]),
    "bwd_dq": ("mqa_bwd_dq", ["mqa_bwd.hip", "mqa_bwd.hpp"]),
    "bwd_dkv": ("mqa_bwd_dkv", ["mqa_bwd_dkv.hip", "mqa_bwd_dkv.hpp", "validate.hpp"]),
}
COMMON_SOURCES = ["common.hpp", "launch.hpp"]
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def kernel_source_sha(kernel: str) -> str:
    """sha256 over the sources a library kernel is compiled from: counters taken on
    another version of the kernel are not reported for this one."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "compressed_sparse_attention_hca_amd", "csrc")
    for f in KERNEL_SOURCES[kernel][1] + COMMON_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _counter_rows(d: str):
    """(kernel name, counter name, value) from every rocprofv3 counter CSV under d."""
    import csv
    import glob
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                yield r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"]), r.get("Dispatch_Id", "")


def summarize_counters(fetch_dir: str, write_dir: str, copy_mb: int, workload: str) -> dict:
    """Per-launch HBM bytes of each library kernel from one FETCH_SIZE run and one
    WRITE_SIZE run of this script under rocprofv3 (counters in KiB per dispatch).  Each
    counter is scaled by what it reads for the plain copy kernel of `copy_mb` MiB that
    the run performs first (--calib-copy-mb): factor = copied bytes / counter bytes."""
    out = {"workload": workload, "copy_bytes": copy_mb << 20, "kernels": {}}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        copies = []
        for name, cname, val, _ in _counter_rows(d):
            if cname != counter:
                continue
            if COPY_KERNEL in name:
                copies.append(val)
                continue
            # longest fragment first: "topk_kernel" is also part of "index_topk_kernel"
            for k, (frag, _) in sorted(KERNEL_SOURCES.items(), key=lambda kv: -len(kv[1][0])):
                if "csa" in name and frag in name:
                    per.setdefault(k, []).append(val)
                    break
        if not copies:
            raise SystemExit(f"no {COPY_KERNEL} dispatch under {d}: run with --calib-copy-mb")
        # the calibration copies are the largest copy dispatches of the run
        ref = max(copies)
        factor = (copy_mb << 20) / (ref * 1024.0)
        out[counter.lower() + "_factor"] = round(factor, 4)
        for k, vals in per.items():
            e = out["kernels"].setdefault(k, {})
            e[counter.lower() + "_kib_per_launch"] = sum(vals) / len(vals)
            e["launches"] = len(vals)
    for k, e in out["kernels"].items():
        if "fetch_size_kib_per_launch" in e and "write_size_kib_per_launch" in e:
            e["bytes_per_launch"] = round(1024.0 * (e["fetch_size_kib_per_launch"] * out["fetch_size_factor"]
                                                    + e["write_size_kib_per_launch"] * out["write_size_factor"]))
        e["source_sha"] = kernel_source_sha(k)
    return out


def traffic_for(kernel: str, path: str):
    """Counter-derived HBM bytes per launch of `kernel`, or None when there are none or
    they were taken on a different version of the kernel's sources."""
    if not path or not os.path.exists(path):
        return None
    with open(path) as fh:
        tj = json.load(fh)
    e = tj.get("kernels", {}).get(kernel)
    if not e or "bytes_per_launch" not in e or e.get("source_sha") != kernel_source_sha(kernel):
        return None
    return e["bytes_per_launch"]


class RowStore:
    """Host float64 rows of a [B,S,...] device tensor for the sampled (b, t) only."""

    def __init__(self, t, rows):
        import torch
        self.rows = {k: t[k].to(torch.float32).cpu().double().numpy() for k in rows}

    def __getitem__(self, key):
        return self.rows[key]


def cpu_baseline(cfg, inp, budget_s: float):
    """Time the fp64 oracle (as it stands) on the host: the full compression of batch
    0 plus a sample of query rows spread over the sequence; extrapolate to the
    layer and report tokens/s."""
    import numpy as np
    import torch
    from oracle import csa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        blas_threads = os.cpu_count()

    host = {}
    for k in ("va", "ga", "vb", "gb", "kv_raw", "k_idx"):
        if k in inp:
            host[k] = {0: inp[k][0].to(torch.float32).cpu().double().numpy()}
    host["bias"] = inp["bias"].cpu().double().numpy()
    sinks = inp["sinks"].cpu().double().numpy() if inp.get("sinks") is not None else None
    S = cfg.S

    class B0:  # batch-0 view with the shapes layer_rows indexes
        def __init__(self, arr):
            self.arr = arr

        def __getitem__(self, k):
            return self.arr[k]

    t_start = time.perf_counter()
    kv_c = O.compress(host["va"][0], host["ga"][0], host["vb"][0] if "vb" in host else None,
                      host["gb"][0] if "gb" in host else None, host["bias"], cfg.ratio,
                      cfg.kind == "csa", cfg.rope_dim, cfg.rope_theta, cfg.rms_eps, cfg.pos0)
    t_comp = time.perf_counter() - t_start

    # rows: a seeded random order of up to 16384 evenly spaced rows, so every prefix is
    # spread over the sequence; rows are added 32 at a time until the budget is used
    n_cand = min(S, 16384)
    order = np.random.default_rng(0).permutation(np.linspace(0, S - 1, n_cand).astype(int))
    sample, t_rows = [], 0.0
    for i in range(0, len(order), 32):
        rows = [(0, int(t)) for t in order[i:i + 32]]
        store = {"q": RowStore(inp["q"], rows), "kv_raw": B0(host["kv_raw"])}
        if cfg.kind == "csa":
            store.update({"q_idx": RowStore(inp["q_idx"], rows), "w_idx": RowStore(inp["w_idx"], rows),
                          "k_idx": B0(host["k_idx"])})
        t0 = time.perf_counter()
        O.layer_rows(cfg, store, rows, kv_c=[kv_c], sinks=sinks)
        t_rows += time.perf_counter() - t0
        sample += rows
        if t_comp + t_rows > budget_s:
            break
    per_row = t_rows / len(sample)
    t_full = cfg.B * (t_comp + S * per_row)
    return {"value": round(cfg.B * S / t_full, 3), "unit": "tokens/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": (f"batch 0: full entry compression ({t_comp:.1f} s) + {len(sample)} query rows "
                       f"evenly spaced over t in [0,{S}) ({t_rows:.1f} s, {per_row * 1e3:.1f} ms/row); "
                       f"layer time extrapolated as B*(compress + S*mean row)"),
            "seconds": round(t_comp + t_rows, 2)}


def stack_configs(index_fp8: bool = False):
    """The 43-layer stack's layer configs; with index_fp8 every CSA layer's indexer QK
    runs on E4M3 operands."""
    from compressed_sparse_attention_hca_amd import workloads as wl
    layers = wl.stack_layers()
    if index_fp8:
        layers = [c.replace(index_fp8=True) if c.kind == wl.CSA else c for c in layers]
    return layers


def stack_line(args, layers, ms_step: float, ms_per_kind: dict) -> dict:
    """The JSON line of the 43-layer stack from its measured step time and the summed
    per-kind layer times (ms per step)."""
    from compressed_sparse_attention_hca_amd import workloads as wl
    flops = sum(wl.layer_flops(c)["total"] for c in layers)
    B, S = layers[0].B, layers[0].S
    tflops = flops / (ms_step * 1e-3) / 1e12
    counts = {kd: sum(1 for c in layers if c.kind == kd) for kd in ms_per_kind}
    fp8 = any(c.index_fp8 for c in layers)
    return {
        "metric": "43-layer V4-Flash attention stack fwd tokens/s (B=4, S=8192, 1 GPU)",
        "value": round(B * S / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_label(fp8),
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": "v4flash_stack43_bf16_B4_S8192" + ("+index_fp8" if fp8 else ""),
                   "B": B, "S": S, "layers": len(layers),
                   "csa": counts.get("csa", 0), "hca": counts.get("hca", 0), "swa": counts.get("swa", 0),
                   "index_fp8": fp8},
        "layer_tokens_per_s": round(len(layers) * B * S / (ms_step * 1e-3), 1),
        "tflops": round(tflops, 2), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": flops,
        "ms_per_kind": {kd: round(v, 3) for kd, v in ms_per_kind.items()},
        "ms_per_layer_of_kind": {kd: round(v / counts[kd], 3) for kd, v in ms_per_kind.items()},
    }


def run_stack(args, dev) -> dict:
    """The 43-layer training-shape stack (B=4, S=8192): every layer's seeded inputs are
    generated once and stay resident (about 110 GB); a step runs all 43 layers in order
    through their entry points (window-only attention, csa_fwd, hca_fwd), each into the
    same output buffer.  tokens/s = B*S per step."""
    import torch
    from compressed_sparse_attention_hca_amd import binding as bd
    from compressed_sparse_attention_hca_amd import workloads as wl

    layers = stack_configs(args.index_fp8)
    log(f"[bench] 43-layer stack: generating inputs on the GPU")
    inps = [wl.make_inputs(c, dev) for c in layers]
    params = [bd.params(c) for c in layers]
    ops = {"csa": bd.OP_CSA_FWD, "hca": bd.OP_HCA_FWD, "swa": bd.OP_SPARSE_MQA}
    ws_bytes = max(bd.workspace_bytes(p, ops[c.kind]) for p, c in zip(params, layers))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    o = torch.empty_like(inps[0]["q"])

    def layer(k):
        c, p, inp = layers[k], params[k], inps[k]
        if c.kind == "swa":
            bd.sparse_mqa_fwd(p, inp["q"], None, inp["kv_raw"], o=o, ws=ws)
        else:
            bd.layer_fwd(p, inp, o=o, ws=ws)

    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        for k in range(len(layers)):
            layer(k)
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(layers) + 1)] for _ in range(args.steps)]
    t0 = time.perf_counter()
    for s in range(args.steps):
        ev[s][0].record()
        for k in range(len(layers)):
            layer(k)
            ev[s][k + 1].record()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    per_kind = {}
    for s in range(args.steps):
        for k, c in enumerate(layers):
            per_kind[c.kind] = per_kind.get(c.kind, 0.0) + ev[s][k].elapsed_time(ev[s][k + 1]) / args.steps
    return stack_line(args, layers, ms_step, per_kind)


def layer_line(args, cfg, ms_step: float, tot: dict, launches: dict, traffic_path, with_kl: bool,
               with_dq: bool, with_dkv: bool = False) -> dict:
    """The JSON line of one fused layer from its measured step time and the per-kernel
    times (ms per step) and launch counts."""
    from compressed_sparse_attention_hca_amd import workloads as wl
    work = kernel_work(cfg, wl)
    kernels = {}
    for k, v in tot.items():
        amt, unit, bound = work[k]
        fp8_qk = cfg.index_fp8 and k in ("index_topk", "indexer")
        e = roofline_entry(amt, unit, bound, v, PEAK_FP8_TFLOPS if fp8_qk else PEAK_BF16_TFLOPS)
        e.update({"ms_per_step": round(v, 4), "launches_per_step": launches[k],
                  "avg_launch_ms": round(v / launches[k], 4)})
        kernels[k] = e
    dom = max(tot, key=tot.get)
    traffic = traffic_for(dom, traffic_path)
    d = kernels[dom]
    amt, unit, bound = work[dom]
    roof = {"kernel": dom, "bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"],
            "unit": d["unit"], "frac": d["frac"], "traffic": traffic,
            "work_per_step": amt, "work_unit": unit, "launches_per_step": launches[dom],
            "avg_launch_ms": d["avg_launch_ms"]}

    f = wl.layer_flops(cfg)
    if with_kl:  # the step also forms the distillation target
        f = dict(f, total=f["total"] + work["kl_target"][0])
    if with_dq:  # and the attention backward's query side
        f = dict(f, total=f["total"] + work["bwd_dq"][0])
    if with_dkv:  # and its key side
        f = dict(f, total=f["total"] + work["bwd_dkv"][0])
    tokens = cfg.B * cfg.S
    value = tokens / (ms_step * 1e-3)
    tflops = f["total"] / (ms_step * 1e-3) / 1e12
    return {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_label(cfg.index_fp8),
        "data": "synthetic (seeded, resident in HBM)",
        "config": {"workload": cfg.name + ("+kl_target" if with_kl else "") +
                   ("+bwd" if with_dkv else ("+bwd_dq" if with_dq else "")),
                   "kind": cfg.kind, "B": cfg.B, "S": cfg.S, "H": cfg.H,
                   "D": cfg.D, "rope_dim": cfg.rope_dim, "ratio": cfg.ratio, "window": cfg.window,
                   "topk": cfg.topk, "idx_heads": cfg.idx_heads, "idx_dim": cfg.idx_dim,
                   "sink": bool(args.sink), "index_prologue": bool(cfg.index_prologue),
                   "index_fp8": bool(cfg.index_fp8)},
        "tflops": round(tflops, 2), "pct_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": f["total"],
        "page_convention_attention_tflops": round(
            wl.page_convention_attention_flops(cfg) / (tot.get("attention", ms_step) * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "roofline": roof,
        "cpu_baseline": None,
    }


def make_parser():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="C3", choices=["C1", "C2", "C3", "C4"],
                    help="C3 (default): the CSA layer at S=65536; C4: the 43-layer stack")
    ap.add_argument("--sink", action="store_true",
                    help="give every head a softmax-sink logit (seeded N(0, 2^2), fp32)")
    ap.add_argument("--index-prologue", action="store_true",
                    help="CSA: indexer prologue on (RoPE + Hadamard of q_I and k_I, temperature on w)")
    ap.add_argument("--index-fp8", action="store_true",
                    help="CSA: FP8 (E4M3, per-row scales) indexer operands")
    ap.add_argument("--bwd-dq", action="store_true",
                    help="each step also runs the attention backward's query side "
                         "(csa_sparse_mqa_bwd_dq) on the step's output and a seeded dL/do")
    ap.add_argument("--bwd", action="store_true",
                    help="also run the whole attention backward in each step: the forward keeps "
                         "lse, then csa_sparse_mqa_bwd_dq and csa_sparse_mqa_bwd_dkv on a seeded dL/do")
    ap.add_argument("--kl-target", action="store_true",
                    help="CSA: each step also forms the indexer distillation target (csa_kl_target)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--traffic", default=None,
                    help="JSON of per-kernel HBM bytes from rocprofv3 counters (default: "
                         "profiles/traffic_<workload>.json)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write the traffic JSON from a FETCH_SIZE run and a WRITE_SIZE run of "
                         "this script under rocprofv3 --pmc, then exit (no GPU use)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="before the steps, copy a buffer of this many MiB twice (a plain copy "
                         "kernel of known size, to scale the FETCH_SIZE / WRITE_SIZE counters)")
    return ap


def main():
    args = make_parser().parse_args()

    traffic_path = args.traffic or os.path.join(ROOT, "profiles", f"traffic_{args.workload}.json")
    if args.summarize_counters:
        s = summarize_counters(*args.summarize_counters, args.calib_copy_mb or 1024, args.workload)
        with open(traffic_path, "w") as fh:
            json.dump(s, fh, indent=1)
        print(json.dumps(s))
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: runs on one GPU only; the layer's multi-GPU sharding is a "
              "design note, not built. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from compressed_sparse_attention_hca_amd import binding as bd
    from compressed_sparse_attention_hca_amd import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.workload == "C4":
        print(json.dumps(run_stack(args, dev)), flush=True)
        return
    cfg = wl.CONFIGS[args.workload]
    if args.index_prologue:
        cfg = cfg.replace(index_prologue=True)
    if args.index_fp8:
        cfg = cfg.replace(index_fp8=True)
    log(f"[bench] workload {cfg.name}: generating inputs on the GPU")
    inp = wl.make_inputs(cfg, dev)
    if args.sink:
        g = torch.Generator().manual_seed(17)
        inp["sinks"] = (torch.randn(cfg.H, generator=g) * 2.0).to(dev)
    p = bd.params(cfg)
    op = bd.OP_CSA_FWD if cfg.kind == "csa" else bd.OP_HCA_FWD
    ws = bd.workspace(p, op, dev)
    o = torch.empty_like(inp["q"])
    traces = [bd.LayerTrace(p) for _ in range(args.steps)]
    kl = None
    if args.kl_target and cfg.kind == "csa":
        n = cfg.S // cfg.ratio
        kl = {"kv_c_out": torch.empty((cfg.B, n, cfg.D), dtype=inp["q"].dtype, device=dev),
              "idx_out": torch.empty((cfg.B, cfg.S, cfg.topk), dtype=torch.int32, device=dev),
              "target": torch.empty((cfg.B, cfg.S, cfg.topk), dtype=torch.float32, device=dev),
              "ev": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(args.steps)]}

    def kl_step(k=None):
        if kl is None:
            return
        if k is not None:
            kl["ev"][k][0].record()
        bd.kl_target(p, inp["q"], kl["kv_c_out"], kl["idx_out"], kl["target"])
        if k is not None:
            kl["ev"][k][1].record()
    dq = None
    if args.bwd:
        args.bwd_dq = True
    if args.bwd_dq:
        n = cfg.S // cfg.ratio
        g = torch.Generator(device=dev).manual_seed(cfg.seed + 23)
        dq = {"kv_c_out": kl["kv_c_out"] if kl else (None if cfg.kind == "swa" else
                                                     torch.empty((cfg.B, n, cfg.D), dtype=inp["q"].dtype, device=dev)),
              "idx_out": kl["idx_out"] if kl else (torch.empty((cfg.B, cfg.S, cfg.topk), dtype=torch.int32, device=dev)
                                                    if cfg.kind == "csa" else None),
              "d_o": torch.randn(inp["q"].shape, generator=g, device=dev).to(inp["q"].dtype),
              "dq": torch.empty_like(inp["q"]),
              "ws": bd.workspace(p, bd.OP_SPARSE_MQA, dev),
              "ev": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                     for _ in range(args.steps)]}

    dkv = None
    if args.bwd:
        n = cfg.S // cfg.ratio
        sk = inp.get("sinks")
        dkv = {"lse": torch.empty((cfg.B, cfg.S, cfg.H), dtype=torch.float32, device=dev),
               "dkv_c": None if cfg.kind == "swa" else torch.empty((cfg.B, n, cfg.D), dtype=torch.float32, device=dev),
               "dkv_raw": torch.empty((cfg.B, cfg.S, cfg.D), dtype=torch.float32, device=dev),
               "dsinks": None if sk is None else torch.empty((cfg.H,), dtype=torch.float32, device=dev),
               "ws": bd.workspace(p, bd.OP_SPARSE_MQA_BWD, dev),
               "ev": [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(args.steps)]}

    def dq_step(k=None):
        if dq is None:
            return
        if k is not None:
            dq["ev"][k][0].record()
        bd.sparse_mqa_bwd_dq(p, inp["q"], dq["kv_c_out"], inp["kv_raw"], dq["idx_out"], o, dq["d_o"],
                             dq=dq["dq"], ws=dq["ws"], sinks=inp.get("sinks"))
        if k is not None:
            dq["ev"][k][1].record()
        if dkv is None:
            return
        if k is not None:
            dkv["ev"][k][0].record()
        bd.sparse_mqa_bwd_dkv(p, inp["q"], dq["kv_c_out"], inp["kv_raw"], dq["idx_out"], o, dkv["lse"], dq["d_o"],
                              sinks=inp.get("sinks"), dkv_c=dkv["dkv_c"], dkv_raw=dkv["dkv_raw"],
                              dsinks=dkv["dsinks"], ws=dkv["ws"])
        if k is not None:
            dkv["ev"][k][1].record()
    layer_out = {}
    for src in (kl, dq):
        if src is not None:
            layer_out = {k: src[k] for k in ("kv_c_out", "idx_out") if src[k] is not None}
    if dkv is not None:
        layer_out["lse_out"] = dkv["lse"]
    if args.calib_copy_mb:
        n = args.calib_copy_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        del src, dst
    torch.cuda.synchronize()

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        bd.layer_fwd(p, inp, o=o, ws=ws, **layer_out)
        kl_step()
        dq_step()
    torch.cuda.synchronize()
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for k in range(args.steps):
        bd.layer_fwd_traced(p, inp, traces[k], o=o, ws=ws, **layer_out)
        kl_step(k)
        dq_step(k)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / args.steps

    # per-kernel time per step, averaged over the timed steps
    tot, launches = {}, {}
    for tr in traces:
        ms, nl = tr.kernel_ms()
        for k, v in ms.items():
            tot[k] = tot.get(k, 0.0) + v / args.steps
            launches[k] = nl[k]
    if kl is not None:
        tot["kl_target"] = sum(a.elapsed_time(b) for a, b in kl["ev"]) / args.steps
        launches["kl_target"] = 1
    if dq is not None:  # window rotation + dQ kernel, timed together on the step's stream
        tot["bwd_dq"] = sum(a.elapsed_time(b) for a, b in dq["ev"]) / args.steps
        launches["bwd_dq"] = 1
    if dkv is not None:  # window rotation, per-pair kernel and the sums, timed together
        tot["bwd_dkv"] = sum(a.elapsed_time(b) for a, b in dkv["ev"]) / args.steps
        launches["bwd_dkv"] = 1
    out = layer_line(args, cfg, ms_step, tot, launches, traffic_path, kl is not None, dq is not None,
                     dkv is not None)
    if not args.no_cpu_baseline:
        log(f"[bench] oracle CPU baseline (~{args.cpu_budget:.0f} s)")
        out["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
