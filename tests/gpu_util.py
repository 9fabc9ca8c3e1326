"""Helpers for the GPU parity tests: lazy host views of device inputs, row sampling,
and the acceptance checks (selection admissibility and output tolerance)."""
from __future__ import annotations

import numpy as np
import torch

from compressed_sparse_attention_hca_amd import workloads as wl


class Lazy:
    """Index a device tensor and get a float64 numpy copy of just that slice."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, key):
        return self.t[key].detach().to(torch.float32).cpu().to(torch.float64).numpy()

    def __array__(self, dtype=None, copy=None):
        a = self.t.detach().to(torch.float32).cpu().to(torch.float64).numpy()
        return a if dtype is None else a.astype(dtype)


def lazy_inputs(inp: dict) -> dict:
    return {k: Lazy(v) for k, v in inp.items()}


def full_np(inp: dict) -> dict:
    return {k: v.detach().to(torch.float32).cpu().to(torch.float64).numpy() for k, v in inp.items()}


def sample_rows(cfg: wl.LayerConfig, n_random: int = 24, seed: int = 0):
    """Edge rows (first tokens, group boundaries, window and top-k edges, the end) plus
    evenly spread and random rows; as (b, t) pairs over every batch."""
    S, r, W, K = cfg.S, cfg.ratio, cfg.window, max(cfg.topk, 1)
    ts = {0, 1, 2, r - 2, r - 1, r, r + 1, 2 * r - 1, W - 2, W - 1, W, W + 1,
          K * r - 2, K * r - 1, K * r, K * r + 3, S // 2, S // 2 + 1, S - r - 1, S - r, S - 2, S - 1}
    ts |= {int(x) for x in np.linspace(0, S - 1, 9)}
    rng = np.random.default_rng(seed)
    ts |= {int(x) for x in rng.integers(0, S, n_random)}
    ts = sorted(t for t in ts if 0 <= t < S)
    return [(b, t) for b in range(cfg.B) for t in ts]


def tol(cfg: wl.LayerConfig) -> float:
    return 1e-5 if cfg.dtype == wl.F32 else 1e-2


def assert_close_rel(got: np.ndarray, want: np.ndarray, rel: float, what: str):
    scale = float(np.max(np.abs(want))) if want.size else 0.0
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= rel * scale + 1e-30, f"{what}: max err {err:.3e} > {rel:g} * max {scale:.3e}"
    return err, scale


def check_selection(gpu_row: np.ndarray, n_t: int, K: int, ora_scores: np.ndarray, ora_sel: np.ndarray,
                    rel: float = 1e-3):
    """|Sel_gpu| = |Sel_ora| = min(K, n_t); entries in the symmetric difference have an
    oracle score within rel * |I_k| of the oracle's k-th score I_k (1e-3 unless a test
    derives another bound); ascending order and -1 padding.  Returns the number of
    swapped entries."""
    m = min(K, n_t)
    sel = gpu_row[:m]
    assert np.all(gpu_row[m:] == -1), "padding must be -1"
    assert np.all(np.diff(sel) > 0), "selection must be strictly ascending"
    assert sel.size == 0 or (sel[0] >= 0 and sel[-1] < n_t), "index outside visible entries"
    a, b = set(sel.tolist()), set(ora_sel.tolist())
    diff = a ^ b
    if diff:
        kth = np.sort(ora_scores)[::-1][m - 1]
        for s in diff:
            assert abs(ora_scores[s] - kth) <= rel * abs(kth), (s, ora_scores[s], kth)
    return len(diff) // 2
