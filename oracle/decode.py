"""One decode step of loop-r attention over the packed cache (one layer, b, h).

The pages: decode is bandwidth bound and its cost is reading the cache
(guide §1, Cell 1); the engine's attention kernels read the packed anchor and
residual streams directly and fuse the sparse decode selection (p1 App. G).
The new token attends every cached token (its own K/V is already cached) and
is active at every loop.

  r = 1:  s^1_j = tau q^1.k^1_j for all T tokens; O^1, lse^1, M^1 = 1, U^1 = 0;
          the logits s^1 are kept.
  r >= 2: S_r = top-K_r of the candidates S_{r-1} ranked by the stored loop
          r-1 logits (index ascending on ties; p1 §4.2: ranked using the
          preceding loop; for one row the logit orders exactly like its mass);
          P^(r-1)_j = M^(r-1) exp(s^(r-1)_j - lse^(r-1));
          M^r = sum_{S_r} P^(r-1)_j;  U^r = O^(r-1) - sum_{S_r} P^(r-1)_j v^(r-1)_j;
          s^r_j = tau q^r.k^r_j on S_r;  O^r = U^r + M^r softmax(s^r) v^r.

Operands: the decode path has no matrix-core step, so it attends the fp32
reconstructions themselves (k_hat, v_hat, exact fp32 values) with the query
as given.  All arithmetic below is float64.
"""
from __future__ import annotations

import numpy as np

from .prefill import softmax_scale, topk


def decode_slice(krec: list, vrec: list, qs: list, K_budget: int, sel_force=None):
    """krec[r-1], vrec[r-1]: reconstructions X_hat^(r) of every cached token
    (float32 [T, d]); qs[r-1]: loop-r query [d].  Returns per-loop dicts."""
    T, d = krec[0].shape
    tau = softmax_scale(d)
    q = np.asarray(qs[0], np.float64)
    k = krec[0].astype(np.float64)
    v = vrec[0].astype(np.float64)
    s = tau * (k @ q)
    m = s.max()
    e = np.exp(s - m)
    l = e.sum()
    O = (e / l) @ v
    lse = m + np.log(l)
    M = 1.0
    U = np.zeros(d)
    sel = np.arange(T, dtype=np.int32)
    logits = s
    out = [dict(O=O, lse=lse, M=M, U=U, sel=sel, logits=logits)]
    for r in range(1, len(qs)):
        K = min(K_budget, sel.shape[0])
        if sel_force is not None and (r + 1) in sel_force:
            new = np.asarray(sel_force[r + 1], np.int32)
        else:
            new = topk(logits, sel, K)
        pos = np.searchsorted(sel, new)
        assert np.array_equal(sel[pos], new)
        P = M * np.exp(logits[pos] - lse)
        vprev = vrec[r - 1][new].astype(np.float64)
        Mn = P.sum()
        U = O - P @ vprev
        qr = np.asarray(qs[r], np.float64)
        sr = tau * (krec[r][new].astype(np.float64) @ qr)
        m = sr.max()
        e = np.exp(sr - m)
        l = e.sum()
        O = U + Mn * ((e / l) @ vrec[r][new].astype(np.float64))
        lse = m + np.log(l)
        M = Mn
        sel = new
        logits = sr
        out.append(dict(O=O, lse=lse, M=M, U=U, sel=sel, logits=logits))
    return out
