"""Pins of the active-set selection oracle (oracle/active.py): a hand-worked
example, the scale invariance of a relative change, tokens that did not move,
nesting, and agreement with an exhaustive subset search."""
import itertools

import numpy as np
import pytest

from oracle import active


def test_hand_example():
    """Three tokens in 2-D: relative changes 0.5, 0 and 1/sqrt(2)."""
    h_prev = np.array([[2.0, 0.0], [1.0, 1.0], [0.0, 3.0]])
    h_cur = np.array([[2.0, 1.0], [1.0, 1.0], [3.0, 3.0]])
    assert np.allclose(active.change_scores(h_prev, h_cur), [0.5, 0.0, 1.0])
    # cand 0..2, keep 2: tokens 2 (1.0) and 0 (0.5), ascending
    assert np.array_equal(active.select_active(h_prev, h_cur, np.arange(3), 2), [0, 2])
    assert np.array_equal(active.select_active(h_prev, h_cur, np.arange(3), 1), [2])


def test_scale_invariance_and_zero_states():
    rng = np.random.default_rng(1)
    p = rng.standard_normal((50, 16))
    c = p + 0.1 * rng.standard_normal((50, 16))
    s1 = active.change_scores(p, c)
    s2 = active.change_scores(7.5 * p, 7.5 * c)
    assert np.allclose(s1, s2, rtol=1e-12)
    z = np.zeros((3, 4))
    assert list(active.change_scores(z, z)) == [0.0, 0.0, 0.0]
    moved = z.copy()
    moved[1, 2] = 1e-30
    assert list(active.change_scores(z, moved)) == [0.0, np.inf, 0.0]


def test_unmoved_tokens_rank_last_and_sets_nest():
    """Tokens outside the previous set reuse their state (delta 0); chained
    selections nest."""
    rng = np.random.default_rng(2)
    S, D = 300, 32
    h0 = rng.standard_normal((S, D))
    cand = np.arange(S, dtype=np.int32)
    h = h0
    for k in (200, 120, 50):
        step = np.zeros_like(h)
        step[cand] = rng.random((cand.size, 1)) * rng.standard_normal((cand.size, D))
        h_next = h + step
        sel = active.select_active(h, h_next, cand, k)
        assert sel.size == k and np.all(np.diff(sel) > 0) and np.isin(sel, cand).all()
        # a candidate that did not move is never chosen over one that did
        frozen = cand[(step[cand] == 0).all(axis=1)]
        assert not np.isin(frozen, sel).any() or np.isin(np.setdiff1d(cand, frozen), sel).all()
        cand, h = sel, h_next


@pytest.mark.parametrize("seed", range(5))
def test_exhaustive_small(seed):
    rng = np.random.default_rng(seed + 10)
    S, D = 9, 3
    p = rng.integers(-2, 3, (S, D)).astype(float)
    c = p + rng.integers(-1, 2, (S, D))   # many exact ties, some zero rows
    cand = np.sort(rng.choice(S, 7, replace=False)).astype(np.int32)
    s = active.change_scores(p[cand], c[cand])
    for k in range(1, 8):
        best = min(itertools.combinations(range(7), k), key=lambda sub: sorted((-s[t], cand[t]) for t in sub))
        assert np.array_equal(active.select_active(p, c, cand, k), np.sort(cand[list(best)]))
