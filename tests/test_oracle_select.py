"""Pins of the oracle's column ranking: exhaustive subset search, a rank-count
formulation, and the closed form of the loop-2 column mass."""
import itertools

import numpy as np
import pytest

from oracle import prefill
import workloads


def _best_subset(c, cand, K):
    """Exhaustive: the K-subset whose sorted (−c, j) key list is smallest."""
    best = None
    for sub in itertools.combinations(range(len(cand)), K):
        key = sorted((-c[t], cand[t]) for t in sub)
        if best is None or key < best[0]:
            best = (key, sorted(cand[t] for t in sub))
    return np.array(best[1], np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_topk_exhaustive_small(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 12))
    cand = np.sort(rng.choice(40, n, replace=False)).astype(np.int32)
    c = rng.integers(0, 4, n).astype(np.float64) / 4   # many exact ties
    for K in range(1, n + 1):
        assert np.array_equal(prefill.topk(c, cand, K), _best_subset(c, cand, K))


def test_topk_rank_count():
    """j is selected iff fewer than K candidates beat it under (c desc, j asc)."""
    rng = np.random.default_rng(7)
    n, K = 1500, 137
    cand = np.sort(rng.choice(5000, n, replace=False)).astype(np.int32)
    c = np.round(rng.random(n) * 50) / 50
    beats = (c[None, :] > c[:, None]) | ((c[None, :] == c[:, None]) & (cand[None, :] < cand[:, None]))
    chosen = cand[beats.sum(axis=1) < K]
    assert np.array_equal(prefill.topk(c, cand, K), chosen)


def test_loop2_mass_sums_to_active_rows():
    """At r = 2 every loop-1 row is a full distribution, so sum_j c_j = n_2."""
    cfg = workloads.custom(dtype="f32", H=1, d=64, S=200, R=2, act=(1.0, 0.35), col="0.2", bits=(8, 4))
    rows, sl = workloads.gen_batch(cfg)
    s = sl[(0, 0)]
    out = prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype=cfg.dtype)
    mass = out["mass"][1]
    assert abs(mass.sum() - len(s.rows[1])) < 1e-9 * len(s.rows[1])
    assert np.all(mass >= 0)
    # columns after the last active row get no mass
    assert np.all(mass[np.arange(cfg.S) > s.rows[1].max()] == 0)
