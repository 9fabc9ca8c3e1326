"""The fused indexer's streaming selection at sizes where its prune path runs.

csa_index_topk (top-k <= 512) keeps a per-query candidate buffer in LDS and prunes it
with a radix pass once a query holds more than about a thousand candidates, so only
queries with more visible entries than that exercise the prune, the admission bound
that follows it and the final exact select.  These tests check the selection of
  - every row of a CSA layer at S = 16384 (n_t up to 4096),
  - 4096 evenly spaced rows of the S = 65536 layer (n_t up to 16384),
  - a layer built so that scores tie exactly, in large groups, at the k-th value: the
    keys are drawn from a small pool of +-1 patterns and the queries from {-1, 0, 1},
    with head weights 0.5 or 1, so every score is an exact multiple of 0.5 on both
    sides and the selection must equal the oracle's bit for bit (ties at the k-th
    score go to the smaller entry index, "fix(deepseek-v4): correct V4-Flash
    attention math", Part 1 item 5, the selection kept in [B, S, K]).
The oracle scores come from oracle.indexer_scores_block (fp64), in row blocks.
"""
import numpy as np
import pytest
import torch

from compressed_sparse_attention_hca_amd import workloads as wl
from oracle import csa_oracle as O
from gpu_util import check_selection

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DEV = "cuda"


@pytest.fixture(scope="module")
def bd():
    from compressed_sparse_attention_hca_amd import binding
    return binding


def _np(t):
    return t.detach().to(torch.float32).cpu().double().numpy()


def _check_rows(cfg, q_idx, w_idx, k_idx, idx, nv, rows, block, exact=False):
    """Selection of every row in `rows` (batch 0) against the oracle; returns the
    number of admissible near-tie swaps (exact: none allowed, sets must be equal)."""
    ki = _np(k_idx[0])
    swaps = 0
    rows = list(rows)
    for i in range(0, len(rows), block):
        ts = rows[i:i + block]
        tt = torch.tensor(ts, device=q_idx.device)
        q = _np(q_idx[0].index_select(0, tt))
        w = _np(w_idx[0].index_select(0, tt))
        n_list = [O.visible_entries(t, cfg.ratio) for t in ts]
        scores = O.indexer_scores_block(q, w, ki, n_list)
        for t, n, sc in zip(ts, n_list, scores):
            assert nv[0, t] == n, (t, nv[0, t], n)
            want = O.topk_row(sc, cfg.topk)
            if exact:
                m = min(cfg.topk, n)
                got = idx[0, t]
                assert np.all(got[m:] == -1), t
                assert np.array_equal(got[:m], want), (t, np.setdiff1d(got[:m], want)[:8])
            else:
                swaps += check_selection(idx[0, t], n, cfg.topk, sc, want)
    return swaps


def test_prune_every_row_S16384(bd):
    cfg = wl.C1.replace(S=16384, name="csa_S16384", seed=2100)
    inp = wl.make_inputs(cfg, DEV)
    idx, nv = bd.index_topk(bd.params(cfg), inp["q_idx"], inp["w_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    idx, nv = idx.cpu().numpy(), nv.cpu().numpy()
    assert O.visible_entries(cfg.S - 1, cfg.ratio) > 1100  # the prune path is reached
    swaps = _check_rows(cfg, inp["q_idx"], inp["w_idx"], inp["k_idx"], idx, nv, range(cfg.S), 64)
    assert swaps <= cfg.S // 100, swaps


def test_prune_rows_C3(bd):
    cfg = wl.C3
    inp = wl.make_inputs(cfg, DEV)
    idx, nv = bd.index_topk(bd.params(cfg), inp["q_idx"], inp["w_idx"], inp["k_idx"])
    torch.cuda.synchronize()
    idx, nv = idx.cpu().numpy(), nv.cpu().numpy()
    rows = set(np.linspace(0, cfg.S - 1, 4096).astype(int).tolist())
    rows |= {4 * 1056 - 1, 4 * 1056, 4 * 1056 + 3, 4 * 2048 - 1, cfg.S - 2}  # around the first prunes
    swaps = _check_rows(cfg, inp["q_idx"], inp["w_idx"], inp["k_idx"], idx, nv, sorted(rows), 32)
    assert swaps <= len(rows) // 100, swaps


def test_prune_exact_ties_S16384(bd):
    cfg = wl.C1.replace(S=16384, name="csa_S16384_ties", seed=2200)
    g = torch.Generator().manual_seed(cfg.seed)
    S, n, HI, DI = cfg.S, cfg.S // cfg.ratio, cfg.idx_heads, cfg.idx_dim
    pool = torch.randint(0, 2, (24, DI), generator=g).float() * 2 - 1          # 24 +-1 patterns
    k = pool[torch.randint(0, pool.shape[0], (n,), generator=g)]               # [n, DI]
    q = torch.randint(-1, 2, (S, HI, DI), generator=g).float()                 # {-1, 0, 1}
    w = torch.randint(1, 3, (S, HI), generator=g).float() * 0.5                # {0.5, 1}
    q_idx = q.to(torch.bfloat16).reshape(1, S, HI, DI).to(DEV)
    k_idx = k.to(torch.bfloat16).reshape(1, n, DI).to(DEV)
    w_idx = w.reshape(1, S, HI).contiguous().to(DEV)
    idx, nv = bd.index_topk(bd.params(cfg), q_idx, w_idx, k_idx)
    torch.cuda.synchronize()
    idx, nv = idx.cpu().numpy(), nv.cpu().numpy()
    rows = list(range(0, S, 3)) + [S - 1]
    # the case is what it claims: the k-th score of late rows sits inside a tie group
    sc = O.indexer_scores_block(_np(q_idx[0, -1:]), _np(w_idx[0, -1:]), _np(k_idx[0]), [n])[0]
    kth = np.sort(sc)[::-1][cfg.topk - 1]
    assert np.sum(sc == kth) > 8 and np.sum(sc > kth) < cfg.topk
    _check_rows(cfg, q_idx, w_idx, k_idx, idx, nv, rows, 64, exact=True)
