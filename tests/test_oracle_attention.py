"""Pins of the oracle's loop attention: the textbook causal softmax when
nothing is sparse or quantized, invariants of the recurrence, the full-matrix
brute force, and decode == the last prefill row."""
import numpy as np
import pytest
import torch

from oracle import brute, decode, prefill, quant
import workloads


def _textbook(q, k, v):
    """torch's CPU scaled-dot-product attention in float64, causal."""
    t = lambda a: torch.from_numpy(np.asarray(a, np.float64))[None, None]
    # torch's default scale 1/sqrt(d) is exact for d = 64, so it pins tau too
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    return o[0, 0].numpy()


def _run(cfg, **kw):
    rows, sl = workloads.gen_batch(cfg)
    s = sl[(0, 0)]
    return s, prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype=cfg.dtype, **kw)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_dense_unquantized_equals_textbook_every_loop(dtype):
    cfg = workloads.custom(dtype=dtype, H=1, d=64, S=160, R=4, act=(1, 1, 1, 1), col="1.0", bits=(8, 4, 4, 4))
    s, out = _run(cfg, quantize=False)
    for r in range(4):
        kr = out["k_recon"][r]
        vr = out["v_recon"][r]
        kk = quant.bf16_rne(kr) if dtype == "bf16" else kr
        vv = quant.bf16_rne(vr) if dtype == "bf16" else vr
        want = _textbook(s.q[r], kk, vv)
        st = out["state"][r]
        assert np.max(np.abs(st.O - want)) < 1e-12
        assert np.allclose(st.M, 1.0, atol=1e-12)
        # lse against a direct log-sum-exp
        sc = prefill.softmax_scale(64) * (s.q[r].astype(np.float64) @ kk.astype(np.float64).T)
        sc[np.triu_indices(cfg.S, 1)] = -np.inf
        assert np.allclose(st.lse, np.logaddexp.reduce(sc, axis=1), atol=1e-12)


def test_zero_deltas_keep_output():
    """Unchanged q, k, v: the rescaled sparse softmax equals P restricted to
    the selection, so O^r = O^(r-1) for any selection."""
    cfg = workloads.custom(dtype="f32", H=1, d=32, S=120, R=4, act=(1, 0.5, 0.3, 0.2), col="0.15", bits=(8, 4, 4, 4), gamma=0.0)
    s, out = _run(cfg, quantize=False)
    for r in range(1, 4):
        assert np.max(np.abs(out["state"][r].O - out["state"][0].O)) < 1e-12


def test_empty_selection_rows_unchanged():
    cfg = workloads.custom(dtype="f32", H=1, d=32, S=100, R=2, act=(1, 0.5), col="0.05", bits=(8, 4))
    rows, sl = workloads.gen_batch(cfg)
    s = sl[(0, 0)]
    sel = np.array([95, 96, 97, 98, 99], np.int32)   # no active row below 95 sees any column
    out = prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype="f32", sel_force={2: sel})
    st0, st1 = out["state"]
    low = s.rows[1][s.rows[1] < 95]
    assert np.array_equal(st1.O[low], st0.O[low])
    assert np.all(st1.M[low] == 0) and np.all(np.isneginf(st1.lse[low]))
    others = np.setdiff1d(np.arange(100), s.rows[1])
    assert np.array_equal(st1.O[others], st0.O[others])


@pytest.mark.parametrize("seed,dtype,quantize,act,col", [
    (0, "f32", True, (1, 0.6, 0.4, 0.2), "0.3"),
    (1, "bf16", True, (1, 0.5, 0.5, 0.25), "0.2"),
    (2, "f32", False, (1, 0.7, 0.3, 0.1), "0.5"),
    (3, "f32", True, (1, 1.0, 0.5, 0.5), "0.1"),
])
def test_bruteforce_bookkeeping(seed, dtype, quantize, act, col):
    """Streaming O/U/M recurrences == explicit probability tables."""
    cfg = workloads.custom(dtype=dtype, H=1, d=32, S=48, R=4, act=act, col=col, bits=(8, 4, 2, 4), seed=seed,
                           lognormal=0.5)
    rows, sl = workloads.gen_batch(cfg)
    s = sl[(0, 0)]
    out = prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype=dtype, quantize=quantize)
    ref = brute.brute_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype=dtype, quantize=quantize)
    for r in range(4):
        assert np.array_equal(out["sel"][r], ref["sel"][r])
        assert np.max(np.abs(out["state"][r].O - ref["O"][r])) < 1e-12
        assert np.max(np.abs(out["state"][r].M - ref["M"][r])) < 1e-12
    # every row of the final table is a distribution
    assert np.allclose(ref["P"].sum(axis=1), 1.0, atol=1e-12)


def test_decode_equals_last_prefill_row():
    T, d, R = 256, 64, 4
    cfg = workloads.custom(dtype="f32", H=1, d=d, S=T, R=R, act=(1, 0.5, 0.25, 0.125), col="0.2", bits=(8, 4, 4, 2))
    rows, sl = workloads.gen_batch(cfg)
    s = sl[(0, 0)]
    # only the last token is active after loop 1: then the prefill's column mass
    # is that one row's probability and ranks like its logits
    last = np.array([T - 1], np.int32)
    rws = [s.rows[0]] + [last] * (R - 1)
    rng = np.random.default_rng(9)
    q = [s.q[0]] + [s.q[0][-1:] + 0.1 * r * rng.standard_normal((1, d)).astype(np.float32) for r in range(1, R)]
    k = [s.k[0]] + [s.k[0][-1:] + 0.1 * rng.standard_normal((1, d)).astype(np.float32) for _ in range(1, R)]
    v = [s.v[0]] + [s.v[0][-1:] + 0.1 * rng.standard_normal((1, d)).astype(np.float32) for _ in range(1, R)]
    pre = prefill.prefill_slice(rws, q, k, v, K_budget=cfg.K, bits=cfg.bits, dtype="f32")
    dec = decode.decode_slice(pre["k_recon"], pre["v_recon"], [q[0][-1]] + [x[0] for x in q[1:]], cfg.K)
    for r in range(R):
        st = pre["state"][r]
        assert np.array_equal(dec[r]["sel"], pre["sel"][r])
        assert np.max(np.abs(dec[r]["O"] - st.O[T - 1])) < 1e-12
        assert abs(dec[r]["lse"] - st.lse[T - 1]) < 1e-12
        assert abs(dec[r]["M"] - st.M[T - 1]) < 1e-12


def test_decode_equals_prefill_row_rich_cache():
    """A cache whose tokens are active at many loops (long residual chains):
    with the selection shared, the decode step equals prefill row T-1."""
    T, d, R = 192, 64, 4
    cfg = workloads.custom(dtype="f32", H=1, d=d, S=T, R=R, act=(1, 0.6, 0.4, 0.3), col="0.25", bits=(8, 4, 2, 4),
                           lognormal=0.5, seed=4)
    rows, sl = workloads.gen_batch(cfg)
    s = sl[(0, 0)]
    rws = [np.union1d(r, [T - 1]).astype(np.int32) for r in s.rows]   # the decode token stays active
    rng = np.random.default_rng(3)
    def chain(x0):
        out = [x0.copy()]
        cur = x0.copy()
        for r in range(1, R):
            cur[rws[r]] += np.float32(0.5 ** (r + 1)) * rng.standard_normal((len(rws[r]), d)).astype(np.float32)
            out.append(cur[rws[r]].copy())
        return out
    q, k, v = chain(s.q[0]), chain(s.k[0]), chain(s.v[0])
    pre = prefill.prefill_slice(rws, q, k, v, K_budget=cfg.K, bits=cfg.bits, dtype="f32")
    qd = [q[0][-1]] + [x[-1] for x in q[1:]]
    dec = decode.decode_slice(pre["k_recon"], pre["v_recon"], qd, cfg.K,
                              sel_force={r + 1: pre["sel"][r] for r in range(1, R)})
    for r in range(R):
        st = pre["state"][r]
        assert np.max(np.abs(dec[r]["O"] - st.O[T - 1])) < 1e-12, r
        assert np.max(np.abs(dec[r]["U"] - st.U[T - 1])) < 1e-12, r
        assert abs(dec[r]["lse"] - st.lse[T - 1]) < 1e-12
        assert abs(dec[r]["M"] - st.M[T - 1]) < 1e-12
