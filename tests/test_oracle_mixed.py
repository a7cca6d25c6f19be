"""Pins of the oracle's exact mixed-logit combine (the ablation of the
mass-rescaled update).  By its definition, chained over nested loops, every
row's output is one softmax over each column's most recently recomputed logit
with that loop's value; the brute force below forms exactly that, with no
cached mass, reused part or log-sum-exp bookkeeping."""
import numpy as np
import pytest

from oracle import prefill


def _nested(rng, S, R, act, keep):
    rows = [np.arange(S)]
    for r in range(1, R):
        rows.append(np.sort(rng.choice(rows[-1], int(act[r] * S), replace=False)))
    sels = [np.arange(S)]
    for r in range(1, R):
        sels.append(np.sort(rng.choice(sels[-1], int(keep[r] * S), replace=False)).astype(np.int32))
    return rows, sels


def _latest_logit_softmax(rows, sels, q, k, v, r, tau):
    """O^r_i for i in A_r: softmax over j <= i of tau q^t_i . k^t_j with
    v^t_j, t = the last loop <= r that selected column j; k^t_j, v^t_j are
    the values of the last loop <= t in which token j was active."""
    q, k, v = ([np.asarray(a, np.float64) for a in x] for x in (q, k, v))

    def at(x, t, j):  # token j's value at loop t (inactive tokens keep theirs)
        u = max(u for u in range(t + 1) if j in set(rows[u].tolist()))
        return x[u][np.searchsorted(rows[u], j)]

    out = {}
    for i in rows[r]:
        logits, vals = [], []
        for j in range(i + 1):
            t = max(u for u in range(r + 1) if j in set(sels[u].tolist()))
            qi = q[t][np.searchsorted(rows[t], i)]
            logits.append(tau * qi @ at(k, t, j))
            vals.append(at(v, t, j))
        logits = np.array(logits)
        w = np.exp(logits - logits.max())
        out[i] = (w / w.sum()) @ np.array(vals)
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_mixed_chain_is_latest_logit_softmax(seed):
    rng = np.random.default_rng(seed)
    S, d, R = 36, 8, 4
    rows, sels = _nested(rng, S, R, act=(1, 0.7, 0.5, 0.3), keep=(1, 0.6, 0.4, 0.25))
    q = [(rng.standard_normal((len(rows[r]), d)) * 1.5).astype(np.float32) for r in range(R)]
    k = [(rng.standard_normal((len(rows[r]), d)) * 1.5).astype(np.float32) for r in range(R)]
    v = [rng.standard_normal((len(rows[r]), d)).astype(np.float32) for r in range(R)]
    out = prefill.prefill_slice(rows, q, k, v, K_budget=S, bits=(8, 4, 4, 4), dtype="f32", quantize=False,
                                sel_force={r + 1: sels[r] for r in range(1, R)}, combine="mixed")
    tau = prefill.softmax_scale(d)
    for r in range(1, R):
        want = _latest_logit_softmax(rows, sels, q, k, v, r, tau)
        st = out["state"][r]
        for i, o in want.items():
            assert np.max(np.abs(st.O[i] - o)) < 1e-12, (r + 1, i)
        # the state's own invariant: O = U + M A with P^r = M e^{x - lse} on J_i
        assert np.all(st.M[rows[r]] >= 0) and np.all(st.M[rows[r]] <= 1 + 1e-12)


def test_mixed_differs_from_mass_rescaled():
    """The two combines agree only in special cases (all columns selected,
    unchanged logits); on a generic chain they differ, so the pin above can
    tell one from the other."""
    rng = np.random.default_rng(7)
    S, d, R = 36, 8, 3
    rows, sels = _nested(rng, S, R, act=(1, 0.7, 0.5), keep=(1, 0.5, 0.3))
    q = [(rng.standard_normal((len(rows[r]), d)) * 1.5).astype(np.float32) for r in range(R)]
    k = [(rng.standard_normal((len(rows[r]), d)) * 1.5).astype(np.float32) for r in range(R)]
    v = [rng.standard_normal((len(rows[r]), d)).astype(np.float32) for r in range(R)]
    kw = dict(K_budget=S, bits=(8, 4, 4), dtype="f32", quantize=False, sel_force={r + 1: sels[r] for r in range(1, R)})
    a = prefill.prefill_slice(rows, q, k, v, combine="mass", **kw)
    b = prefill.prefill_slice(rows, q, k, v, combine="mixed", **kw)
    assert np.max(np.abs(a["state"][2].O - b["state"][2].O)) > 1e-3


def test_mixed_with_every_column_is_dense():
    """Every column selected at every loop: both combines give loop r's dense
    causal attention."""
    rng = np.random.default_rng(3)
    S, d, R = 30, 8, 3
    rows = [np.arange(S)] * R
    q = [rng.standard_normal((S, d)).astype(np.float32) for _ in range(R)]
    k = [rng.standard_normal((S, d)).astype(np.float32) for _ in range(R)]
    v = [rng.standard_normal((S, d)).astype(np.float32) for _ in range(R)]
    for comb in ("mass", "mixed"):
        out = prefill.prefill_slice(rows, q, k, v, K_budget=S, bits=(8, 4, 4), dtype="f32", quantize=False,
                                    combine=comb)
        for r in range(R):
            O, _ = prefill.dense_causal(*(np.asarray(a[r], np.float64) for a in (q, k, v)), prefill.softmax_scale(d))
            assert np.max(np.abs(out["state"][r].O - O)) < 1e-12, (comb, r)
