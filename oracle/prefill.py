"""Loop-r attention of one (b, h) slice over the cross-loop cache (prefill).

Follows the FlashLoop pages step by step, in float64:
  * loop 1 is dense causal attention of every row over the reconstructed
    base (the workload definition; p1 §D.1 makes the first loops dense and
    the later ones sparse);
  * loop r >= 2 recomputes only the active rows A_r (p1 §4.1, §D.1), only
    against the top-K key columns ranked by loop r-1's attention statistics
    (p1 §4.2 and §D.2; guide §3), and rescales the softmax over those columns
    by the share of loop r-1's distribution those columns held, keeping every
    other column's contribution from loop r-1's output (p1 §4.2; guide §3
    describes the update as a low-rank fix of the previous output, the
    paper's eq. 3, whose formula the pages do not print).

Reading of the unprinted eq. 3: with
J_i = {j in S_r : j <= i} and P^(r-1) the probabilities that loop r-1 left,
  M^r_i = sum_{J_i} P^(r-1)_ij                         (cached mass)
  U^r_i = O^(r-1)_i - sum_{J_i} P^(r-1)_ij v~^(r-1)_j  (reused part)
  O^r_i = U^r_i + M^r_i * sum_{J_i} softmax_{J_i}(tau q^r_i . k~^r_j) v~^r_j
and P^r_ij = M^r_i * softmax_{J_i}(...)_j on J_i, P^(r-1)_ij elsewhere.
Column ranking: c_j = sum_{i in A_r, i >= j} P^(r-1)_ij over the candidates
S_{r-1} (the selected sets nest, p1 §4.2 and §D.2), top K by (c desc, j asc).

Operands: k~ = k_hat and v~ = v_hat (the fp32 reconstructions) for fp32
inputs; for bf16 inputs they are rounded to bf16 (the matrix cores consume
bf16), queries are used as given.  tau = 1/sqrt(d) rounded once to fp32.
"""
from __future__ import annotations

import numpy as np

from .paper_format import quantize_chain_paper
from .quant import bf16_rne, quantize_chain

ROW_BLOCK = 1024


def softmax_scale(d: int) -> float:
    return float(np.float32(1.0 / np.sqrt(np.float64(d))))


def operands(recon: np.ndarray, dtype: str) -> np.ndarray:
    """Attention operand of a reconstruction (float64)."""
    if dtype == "bf16":
        return bf16_rne(recon).astype(np.float64)
    return recon.astype(np.float64)


def dense_causal(q: np.ndarray, k: np.ndarray, v: np.ndarray, tau: float):
    """Loop 1: O_i = sum_{j<=i} softmax_j(tau q_i.k_j) v_j and lse_i, all rows."""
    S = q.shape[0]
    O = np.zeros((S, v.shape[1]))
    lse = np.zeros(S)
    for i0 in range(0, S, ROW_BLOCK):
        i1 = min(S, i0 + ROW_BLOCK)
        s = tau * (q[i0:i1] @ k[:i1].T)
        ii = np.arange(i0, i1)[:, None]
        s[np.arange(i1)[None, :] > ii] = -np.inf
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(axis=1, keepdims=True)
        O[i0:i1] = (e / l) @ v[:i1]
        lse[i0:i1] = (m + np.log(l))[:, 0]
    return O, lse


class LoopState:
    """Per-row state after a loop: O, lse, M, U (position indexed), plus what
    is needed to re-form that loop's probabilities: its queries, operands and
    selected set."""

    def __init__(self, S, d):
        self.O = np.zeros((S, d))
        self.U = np.zeros((S, d))
        self.M = np.ones(S)
        self.lse = np.zeros(S)

    def copy(self):
        c = LoopState.__new__(LoopState)
        c.O, c.U, c.M, c.lse = self.O.copy(), self.U.copy(), self.M.copy(), self.lse.copy()
        return c


def loop_probs(rows_i, cols, qfull, kt, lse, M, tau):
    """P^(r-1)_ij for rows rows_i and candidate columns cols (float64).

    P^(r-1)_ij = M_i exp(tau q_i.k~_j - lse_i) for j <= i, zero for j > i.
    Rows with M_i == 0 (no column was left to them in loop r-1) give zeros."""
    s = tau * (qfull[rows_i] @ kt[cols].T)
    s[cols[None, :] > rows_i[:, None]] = -np.inf
    live = M[rows_i] > 0
    P = np.zeros_like(s)
    z = s[live] - lse[rows_i][live][:, None]
    P[live] = M[rows_i][live][:, None] * np.exp(z)
    return P


def column_mass(rows_r, cand, qfull_prev, kt_prev, st_prev: LoopState, tau):
    """c_j = sum_{i in A_r, i >= j} P^(r-1)_ij for j in cand (float64)."""
    c = np.zeros(cand.shape[0])
    for i0 in range(0, rows_r.shape[0], ROW_BLOCK):
        ri = rows_r[i0:i0 + ROW_BLOCK]
        c += loop_probs(ri, cand, qfull_prev, kt_prev, st_prev.lse, st_prev.M, tau).sum(axis=0)
    return c


def topk(mass: np.ndarray, cand: np.ndarray, K: int) -> np.ndarray:
    """The K candidates first under (mass desc, index asc), ascending by index."""
    order = np.lexsort((cand, -np.asarray(mass, np.float64)))
    return np.sort(cand[order[:K]]).astype(np.int32)


def cached_mass_and_reuse(rows_r, sel, qfull_prev, kt_prev, vt_prev, st: LoopState, tau):
    """M^r_i = sum_{J_i} P^(r-1)_ij and U^r_i = O^(r-1)_i - sum_{J_i} P^(r-1)_ij v~^(r-1)_j."""
    for i0 in range(0, rows_r.shape[0], ROW_BLOCK):
        ri = rows_r[i0:i0 + ROW_BLOCK]
        P = loop_probs(ri, sel, qfull_prev, kt_prev, st.lse, st.M, tau)
        Mi = P.sum(axis=1)
        C = P @ vt_prev[sel]
        st.U[ri] = st.O[ri] - C
        st.M[ri] = Mi


def sparse_update(rows_r, sel, qfull, kt, vt, st: LoopState, tau):
    """O^r_i = U^r_i + M^r_i sum_{J_i} softmax(tau q^r_i.k~^r_j) v~^r_j; lse^r_i.

    Rows whose J_i is empty keep O and get lse = -inf."""
    for i0 in range(0, rows_r.shape[0], ROW_BLOCK):
        ri = rows_r[i0:i0 + ROW_BLOCK]
        s = tau * (qfull[ri] @ kt[sel].T)
        s[sel[None, :] > ri[:, None]] = -np.inf
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        e = np.zeros_like(s)
        e[has] = np.exp(s[has] - m[has])
        l = e.sum(axis=1, keepdims=True)
        rh = ri[has]
        pv = (e[has] / l[has]) @ vt[sel]
        st.O[rh] = st.U[rh] + st.M[rh][:, None] * pv
        st.lse[rh] = (m[has] + np.log(l[has]))[:, 0]
        st.lse[ri[~has]] = -np.inf


def selected_log_mass(rows_r, sel, qfull_prev, kt_prev, tau):
    """L^r_i = log sum_{J_i} exp(tau q^(r-1)_i . k~^(r-1)_j), the loop r-1
    logits of the selected columns as one log-sum-exp (-inf when J_i is
    empty).  Only the exact mixed-logit combine uses it."""
    L = np.full(rows_r.shape[0], -np.inf)
    for i0 in range(0, rows_r.shape[0], ROW_BLOCK):
        ri = rows_r[i0:i0 + ROW_BLOCK]
        s = tau * (qfull_prev[ri] @ kt_prev[sel].T)
        s[sel[None, :] > ri[:, None]] = -np.inf
        m = s.max(axis=1)
        has = np.isfinite(m)
        L[i0:i0 + ROW_BLOCK][has] = m[has] + np.log(np.exp(s[has] - m[has][:, None]).sum(axis=1))
    return L


def sparse_update_mixed(rows_r, sel, qfull, kt, vt, st: LoopState, Lsel, tau):
    """Exact mixed-logit combine, the ablation of the mass-rescaled one: a
    single softmax over loop r's logits on J_i and the logits loop r-1's
    distribution held everywhere else (p1 §4.2 names the renormalization this
    avoids; the pages do not print it).  With Z_i the normalizer of loop r-1's
    distribution over all columns, Z_i = exp(L^r_i) / M^r_i, and
    b_i = log sum_{J_i} exp(tau q^r_i . k~^r_j), A_i = softmax_{J_i}(...) v~^r:
      O^r_i = (U^r_i Z_i + e^{b_i} A_i) / ((1 - M^r_i) Z_i + e^{b_i})
            = (U^r_i + M^r_i rho_i A_i) / (1 - M^r_i + M^r_i rho_i),  rho_i = e^{b_i - L^r_i}.
    The state keeps O = U + M A with M = M^r rho / D, U = U^r / D (D the
    denominator) and lse = b, so loop r's probabilities P^r = M e^{x - lse}
    on J_i are those of the combined softmax.  Rows whose J_i is empty keep O
    (lse = -inf); rows with M^r_i = 0 combine as in the mass-rescaled rule.
    Returns D per row of rows_r (1 where the mass-rescaled rule applies): the
    reused part enters O divided by it, so errors in U^r grow by 1/D."""
    denom = np.ones(rows_r.shape[0])
    for i0 in range(0, rows_r.shape[0], ROW_BLOCK):
        ri = rows_r[i0:i0 + ROW_BLOCK]
        Li = Lsel[i0:i0 + ROW_BLOCK]
        s = tau * (qfull[ri] @ kt[sel].T)
        s[sel[None, :] > ri[:, None]] = -np.inf
        m = s.max(axis=1, keepdims=True)
        has = np.isfinite(m[:, 0])
        e = np.zeros_like(s)
        e[has] = np.exp(s[has] - m[has])
        l = e.sum(axis=1, keepdims=True)
        b = np.full(ri.shape[0], -np.inf)
        b[has] = (m[has] + np.log(l[has]))[:, 0]
        for t in np.nonzero(has)[0]:
            i = ri[t]
            A = (e[t] / l[t, 0]) @ vt[sel]
            Mi = st.M[i]
            if Mi > 0 and np.isfinite(Li[t]):
                g = np.log(Mi) + b[t] - Li[t]          # log(M rho)
                denom[i0 + t] = 1.0 - Mi + np.exp(g)
                if g > 0:
                    D = (1.0 - Mi) * np.exp(-g) + 1.0
                    st.O[i] = (st.U[i] * np.exp(-g) + A) / D
                    st.U[i] = st.U[i] * np.exp(-g) / D
                    st.M[i] = 1.0 / D
                else:
                    D = 1.0 - Mi + np.exp(g)
                    st.O[i] = (st.U[i] + np.exp(g) * A) / D
                    st.U[i] = st.U[i] / D
                    st.M[i] = np.exp(g) / D
            else:
                st.O[i] = st.U[i] + Mi * A
        st.lse[ri] = b
    return denom


def _full_rows(S, rows, x):
    """Scatter a compact per-loop tensor to position-indexed rows (others 0)."""
    out = np.zeros((S, x.shape[1]))
    out[rows] = x
    return out


def identity_chain(x: list, rows: list):
    """Reconstructions when quantization is switched off (a special case used
    by the tests): X_hat^(r) = X^(r) on A_r, X_hat^(r-1) elsewhere."""
    cur = np.asarray(x[0], np.float32).copy()
    out = [cur.copy()]
    for r in range(1, len(x)):
        cur[rows[r]] = x[r]
        out.append(cur.copy())
    return out


def prefill_slice(rows, q, k, v, *, K_budget, bits, dtype, sel_force=None, stop_after=None,
                  quantize=True, combine="mass", fmt="workload"):
    """Run every loop of one (b, h) slice.

    rows[r-1], q[r-1], k[r-1], v[r-1]: loop-r active rows and compact inputs
    (loop 1 covers every row).  sel_force: optional {r: sel} that replaces the
    oracle's own selection at loop r (teacher forcing after near ties).
    combine: "mass" (the method's mass-rescaled update) or "mixed" (the exact
    mixed-logit ablation).  fmt: "workload" (int8 base, 4/2-bit residuals,
    32-dim groups) or "paper" (paper_format: INT4 g64, per-channel keys,
    bf16 tail; `bits` unused).  Returns a dict of per-loop results (index r-1)."""
    R = len(q)
    S, d = k[0].shape
    tau = softmax_scale(d)
    if quantize and fmt == "paper":
        ks, krec = quantize_chain_paper(k, rows, "k")
        vs, vrec = quantize_chain_paper(v, rows, "v")
    elif quantize:
        ks, krec = quantize_chain(k, rows, bits)
        vs, vrec = quantize_chain(v, rows, bits)
    else:
        ks = vs = None
        krec, vrec = identity_chain(k, rows), identity_chain(v, rows)
    kt = [operands(x, dtype) for x in krec]
    vt = [operands(x, dtype) for x in vrec]
    qf = [_full_rows(S, rows[r], q[r].astype(np.float64)) for r in range(R)]

    st = LoopState(S, d)
    O, lse = dense_causal(qf[0], kt[0], vt[0], tau)
    st.O, st.lse = O, lse
    sel = np.arange(S, dtype=np.int32)
    out = dict(k_streams=ks, v_streams=vs, k_recon=krec, v_recon=vrec,
               state=[st.copy()], sel=[sel], mass=[None])
    last = R if stop_after is None else stop_after
    for r in range(1, last):
        rr = rows[r].astype(np.int64)
        cand = sel
        mass = column_mass(rr, cand, qf[r - 1], kt[r - 1], st, tau)
        K = min(K_budget, cand.shape[0])
        if sel_force is not None and (r + 1) in sel_force:
            sel = np.asarray(sel_force[r + 1], dtype=np.int32)
        else:
            sel = topk(mass, cand, K)
        sl = sel.astype(np.int64)
        Lsel = selected_log_mass(rr, sl, qf[r - 1], kt[r - 1], tau) if combine == "mixed" else None
        cached_mass_and_reuse(rr, sl, qf[r - 1], kt[r - 1], vt[r - 1], st, tau)
        if combine == "mixed":
            D = sparse_update_mixed(rr, sl, qf[r], kt[r], vt[r], st, Lsel, tau)
            out.setdefault("lsel", [None] * R)[r] = Lsel
            out.setdefault("denom", [None] * R)[r] = D
        else:
            sparse_update(rr, sl, qf[r], kt[r], vt[r], st, tau)
        out["state"].append(st.copy())
        out["sel"].append(sel)
        out["mass"].append(mass)
    return out
