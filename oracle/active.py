"""Cross-loop token-sparse updates: the next loop's active set.

TEST INFRASTRUCTURE ONLY (see the package header).

After the dense early loops each loop keeps, among the tokens it updated,
the ones whose hidden state still moves the most (p1 §4.1 and §D.1: later
loops recompute only nested active-token sets with a budget k(r); the
guide's §3 summary: tokens are ranked by their normalized hidden-state
change and a top-k subset is kept, so the sets nest).

Reading taken where the pages stop: the normalized change of token i is the
relative L2 change of its hidden state across the loop just run,
delta_i = ||h_cur_i - h_prev_i|| / ||h_prev_i||, in float64; a token whose
state did not move has delta 0, and one that moved from a zero state has
delta +inf.  Candidates are the previous active set; the budget keeps the
k largest deltas, ties to the lower position, and the set is returned in
ascending position order (the same rule as the column selection).
"""
from __future__ import annotations

import numpy as np

from . import prefill


def change_scores(h_prev: np.ndarray, h_cur: np.ndarray) -> np.ndarray:
    """delta_i for rows i of [n, D] hidden states (float64)."""
    p = np.asarray(h_prev, np.float64)
    c = np.asarray(h_cur, np.float64)
    num = np.sqrt(((c - p) ** 2).sum(axis=1))
    den = np.sqrt((p ** 2).sum(axis=1))
    out = np.zeros(p.shape[0])
    nz = den > 0
    out[nz] = num[nz] / den[nz]
    out[~nz & (num > 0)] = np.inf
    return out


def select_active(h_prev: np.ndarray, h_cur: np.ndarray, cand: np.ndarray, k: int) -> np.ndarray:
    """The next active set: the k candidates with the largest delta (ties to
    the lower position), ascending.  h_prev, h_cur: [S, D] per position."""
    cand = np.asarray(cand, np.int32)
    s = change_scores(h_prev[cand], h_cur[cand])
    return prefill.topk(s, cand, k)
