"""GPU parity of fl_select_active (the next active-token set) with the CPU
oracle, through the C ABI."""
import numpy as np
import pytest

import workloads
from oracle import active

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _run(cfg, D, r, cand, k, h_prev, h_cur, all_positions=False):
    import torch
    import sparse_attn_residual_amd as fl
    import tests.gpu_harness as gh
    B = len(h_prev)
    hp = torch.stack([gh.upload(x, cfg) for x in h_prev])
    hc = torch.stack([gh.upload(x, cfg) for x in h_cur])
    n_prev = cfg.S if all_positions else len(cand[0])
    rows_prev = None if all_positions else torch.from_numpy(np.stack(cand).astype(np.int32)).cuda()
    rows_out = torch.empty(B, k, dtype=torch.int32, device="cuda")
    score = torch.empty(B, n_prev, dtype=torch.float32, device="cuda")
    fl.fl_select_active(B, cfg.S, D, hp, hc, gh.fl_dtype(cfg), n_prev, rows_prev, k, rows_out, score)
    torch.cuda.synchronize()
    return rows_out.cpu().numpy(), score.cpu().numpy()


def _check(cfg, D, r, ks, all_first=False, tol=1e-5):
    """Chained selections over loops r, r+1, ...: each GPU selection equals
    the oracle's up to near ties of the scores, and the sets nest."""
    import tests.gpu_harness as gh
    cand = [workloads.active_rows(cfg, b)[r - 2] for b in range(cfg.B)]
    for step, k in enumerate(ks):
        rr = r + step
        hs = [workloads.gen_hidden(cfg, b, D, rr, cand[b]) for b in range(cfg.B)]
        allp = all_first and step == 0
        sel, score = _run(cfg, D, rr, cand, k, [h[0] for h in hs], [h[1] for h in hs], all_positions=allp)
        nxt = []
        for b in range(cfg.B):
            s_or = active.change_scores(hs[b][0][cand[b]], hs[b][1][cand[b]])
            assert np.allclose(score[b], s_or, rtol=tol, atol=0), (rr, b, np.max(np.abs(score[b] - s_or)))
            want = active.select_active(hs[b][0], hs[b][1], cand[b], k)
            ok, nd = gh.near_tie_ok(sel[b], want, s_or, cand[b], tol * gh.kth_key(s_or, k))
            assert ok, (rr, b, nd)
            assert np.all(np.diff(sel[b]) > 0) and np.isin(sel[b], cand[b]).all()
            nxt.append(sel[b])
        cand = nxt


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_active_chain_small(dtype):
    cfg = workloads.custom(name="active-small", dtype=dtype, B=2, H=1, d=64, S=3000, R=4, act=(1, 0.6, 0.3, 0.1),
                           seed=3)
    _say("active chain", dtype, cfg.S)
    # loop 2 ranks every position (rows_prev NULL), then loops 3 and 4 nest
    _check(cfg, 256, 2, [1800, 900, 300], all_first=True)


def test_active_keep_all_and_ragged():
    """k == n_prev copies the candidates; D not a multiple of 512 and a
    candidate count that is not a multiple of the wave count."""
    cfg = workloads.custom(name="active-edge", dtype="bf16", B=3, H=1, d=64, S=1001, R=3, act=(1, 0.507, 0.2),
                           seed=4)
    _say("active edge", cfg.S)
    cand = [workloads.active_rows(cfg, b)[1] for b in range(cfg.B)]
    n = len(cand[0])
    hs = [workloads.gen_hidden(cfg, b, 72, 3, cand[b]) for b in range(cfg.B)]
    sel, _ = _run(cfg, 72, 3, cand, n, [h[0] for h in hs], [h[1] for h in hs])
    for b in range(cfg.B):
        assert np.array_equal(sel[b], cand[b])
    _check(cfg, 72, 3, [151])


def test_active_full_shape():
    """The 32K workload's shape: S = 32768, hidden size 2048 (16 heads x 128),
    bf16, budgets of the active fractions 30/15/8 %."""
    cfg = workloads.CONFIGS[2]
    _say("active full shape", cfg.name)
    _check(cfg, cfg.H * cfg.d, 2, [cfg.n[1], cfg.n[2], cfg.n[3]], all_first=True)
