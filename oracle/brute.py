"""Full-matrix bookkeeping form of the loop recurrences (tiny sizes only).

Keeps the explicit probability table P[i, j] of every row and the loop
rho[i, j] whose values last produced each entry, and forms every output as
O^r_i = sum_j P^r_ij v~^(rho(i,j))_j.  This restates the method without the
cached-mass / reused-part bookkeeping of ``prefill``: loop-aware sparse
attention recomputes the selected columns of the active rows and rescales them
by the mass those columns held in the previous loop's distribution, while
every other entry keeps its previous value (p1 §4.2 and §D.2; guide §3).
"""
from __future__ import annotations

import numpy as np

from .prefill import identity_chain, operands, softmax_scale, topk
from .quant import quantize_chain


def brute_slice(rows, q, k, v, *, K_budget, bits, dtype, quantize=True):
    R = len(q)
    S, d = k[0].shape
    tau = softmax_scale(d)
    if quantize:
        _, krec = quantize_chain(k, rows, bits)
        _, vrec = quantize_chain(v, rows, bits)
    else:
        krec, vrec = identity_chain(k, rows), identity_chain(v, rows)
    kt = [operands(x, dtype) for x in krec]
    vt = [operands(x, dtype) for x in vrec]
    P = np.zeros((S, S))
    rho = np.zeros((S, S), dtype=np.int64)
    qcur = np.zeros((S, d))
    qcur[rows[0]] = q[0]
    for i in range(S):
        s = np.array([tau * float(qcur[i] @ kt[0][j]) for j in range(i + 1)])
        e = np.exp(s - s.max())
        P[i, :i + 1] = e / e.sum()
    outs = [np.stack([sum(P[i, j] * vt[rho[i, j]][j] for j in range(i + 1)) for i in range(S)])]
    Ms = [np.ones(S)]
    sel = np.arange(S)
    sels = [sel]
    for r in range(1, R):
        A = rows[r]
        c = np.array([sum(P[i, j] for i in A if i >= j) for j in sel])
        sel = topk(c, sel, min(K_budget, len(sel))).astype(np.int64)
        qcur[A] = q[r]
        Mr = Ms[-1].copy()
        for i in A:
            J = [j for j in sel if j <= i]
            Mi = sum(P[i, j] for j in J)
            Mr[i] = Mi
            if not J:
                continue
            s = np.array([tau * float(qcur[i] @ kt[r][j]) for j in J])
            e = np.exp(s - s.max())
            p = e / e.sum()
            for t, j in enumerate(J):
                P[i, j] = Mi * p[t]
                rho[i, j] = r
        outs.append(np.stack([sum(P[i, j] * vt[rho[i, j]][j] for j in range(i + 1)) for i in range(S)]))
        Ms.append(Mr)
        sels.append(sel)
    return dict(O=outs, M=Ms, sel=sels, P=P)
