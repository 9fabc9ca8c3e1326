"""bench.py's JSON lines, built on the CPU from stubbed timings: the fused layer (plain
and with the FP8 indexer) and the 43-layer stack (plain and with the FP8 indexer).
No GPU is touched; only the line-building functions run."""
import json

import pytest

import bench
from compressed_sparse_attention_hca_amd import workloads as wl

CONTRACT_KEYS = {"metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                 "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config"}


def _args(*extra):
    return bench.make_parser().parse_args(["--steps", "7", "--warmup", "2", *extra])


def test_layer_line_bf16_from_stubbed_timings():
    args = _args()
    cfg = wl.C3
    tot = {"compress": 0.1, "window_rope": 0.05, "index_topk": 7.5, "attention": 6.5}
    launches = {k: 1 for k in tot}
    line = bench.layer_line(args, cfg, 14.2, tot, launches, None, False, False)
    json.dumps(line)  # serialisable
    assert CONTRACT_KEYS <= set(line)
    assert line["dtype"] == "bf16"
    assert line["steps"] == 7 and line["warmup"] == 2 and line["n_gpus"] == 1
    assert line["value"] == pytest.approx(cfg.B * cfg.S / 14.2e-3, rel=1e-6)
    f = wl.layer_flops(cfg)["total"]
    assert line["tflops"] == pytest.approx(f / 14.2e-3 / 1e12, rel=1e-4)
    assert line["roofline"]["kernel"] == "index_topk"
    assert line["roofline"]["peak"] == bench.PEAK_BF16_TFLOPS
    assert line["kernels"]["attention"]["peak"] == bench.PEAK_BF16_TFLOPS
    assert line["config"]["workload"] == cfg.name and line["config"]["index_fp8"] is False


def test_layer_line_fp8_indexer_names_its_dtype_and_peak():
    args = _args("--index-fp8")
    cfg = wl.C3.replace(index_fp8=True)
    tot = {"compress": 0.1, "window_rope": 0.05, "index_keys": 0.01, "index_topk": 6.4, "attention": 6.6}
    launches = {k: 1 for k in tot}
    line = bench.layer_line(args, cfg, 13.2, tot, launches, None, False, False)
    assert line["dtype"] != "bf16" and "fp8" in line["dtype"]
    assert line["kernels"]["index_topk"]["peak"] == bench.PEAK_FP8_TFLOPS
    assert line["kernels"]["attention"]["peak"] == bench.PEAK_BF16_TFLOPS
    assert line["config"]["index_fp8"] is True


def test_stack_line_from_stubbed_timings():
    args = _args("--workload", "C4")
    layers = bench.stack_configs(args.index_fp8)
    assert len(layers) == 43
    per_kind = {"swa": 2 * 1.3, "csa": 21 * 3.9, "hca": 20 * 1.6}
    ms = sum(per_kind.values()) + 0.2
    line = bench.stack_line(args, layers, ms, per_kind)
    json.dumps(line)
    assert CONTRACT_KEYS <= set(line)
    assert line["dtype"] == "bf16"
    assert line["config"]["csa"] == 21 and line["config"]["hca"] == 20 and line["config"]["swa"] == 2
    assert line["ms_per_layer_of_kind"]["csa"] == pytest.approx(3.9, abs=1e-3)
    assert line["value"] == pytest.approx(4 * 8192 / (ms * 1e-3), rel=1e-6)
    flops = sum(wl.layer_flops(c)["total"] for c in layers)
    assert line["flops_per_step"] == flops


def test_stack_line_with_fp8_indexer():
    args = _args("--workload", "C4", "--index-fp8")
    layers = bench.stack_configs(args.index_fp8)
    assert sum(c.index_fp8 for c in layers) == 21
    assert all(c.index_fp8 == (c.kind == wl.CSA) for c in layers)
    per_kind = {"swa": 2.6, "csa": 70.0, "hca": 32.0}
    line = bench.stack_line(args, layers, 105.0, per_kind)
    assert "fp8" in line["dtype"]
    assert line["config"]["index_fp8"] is True


def test_more_than_one_gpu_is_refused(monkeypatch, capsys):
    monkeypatch.setattr("sys.argv", ["bench.py", "--gpus", "2"])
    with pytest.raises(SystemExit) as e:
        bench.main()
    assert e.value.code == 2
    assert "one GPU" in capsys.readouterr().err


def test_layer_line_with_the_attention_backward():
    """--bwd: the step runs the forward, dQ and the key side; the workload says so and
    the step's FLOPs include both backward parts."""
    args = _args("--bwd", "--workload", "C1")
    cfg = wl.C1
    tot = {"compress": 0.01, "window_rope": 0.01, "index_topk": 0.5, "attention": 0.4,
           "bwd_dq": 0.85, "bwd_dkv": 2.1}
    launches = {k: 1 for k in tot}
    line = bench.layer_line(args, cfg, 3.9, tot, launches, None, False, True, True)
    json.dumps(line)
    assert line["config"]["workload"] == cfg.name + "+bwd"
    work = bench.kernel_work(cfg, wl)
    f = wl.layer_flops(cfg)["total"] + work["bwd_dq"][0] + work["bwd_dkv"][0]
    assert line["flops_per_step"] == f
    assert line["roofline"]["kernel"] == "bwd_dkv"
    assert work["bwd_dkv"][0] == 2.0 * wl.layer_flops(cfg)["attention"]
