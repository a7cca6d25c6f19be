"""Pins of the oracle's paper-format quantizer (INT4 asymmetric, group 64,
keys per channel along tokens, values per token, 64-token BF16 tail): the
half-step bound, exact cases, the group geometry, the tail and the chain."""
import numpy as np
import pytest

from oracle import paper_format as pf
from oracle.quant import bf16_rne


def _chain(S=300, d=128, seed=0, frac=(1.0, 0.5, 0.25)):
    rng = np.random.default_rng(seed)
    rows = [np.arange(S)]
    for f in frac[1:]:
        rows.append(np.sort(rng.choice(rows[-1], int(f * S), replace=False)))
    x = [(rng.standard_normal((S, d)) * np.exp(rng.standard_normal((S, 1)))).astype(np.float32)]
    for r in range(1, len(frac)):
        x.append((rng.standard_normal((len(rows[r]), d)) * 0.3).astype(np.float32))
    return rows, x


def _full(rows, x, r, prev):
    cur = prev.copy()
    cur[rows[r]] = x[r]
    return cur


@pytest.mark.parametrize("kind", ["k", "v"])
def test_half_step_bound_and_tail(kind):
    rows, x = _chain()
    S, d = x[0].shape
    Sq = S - pf.TAIL
    st, rec = pf.quantize_chain_paper(x, rows, kind)
    exact = x[0].copy()
    for r in range(len(x)):
        if r:
            exact = _full(rows, x, r, exact)
        s = st[r]["scale"].astype(np.float32)
        body = np.arange(Sq) if r == 0 else st[r]["rows"]
        # step of every quantized element: per channel of a 64-token block (keys)
        # or per 64-dim group of a token (values)
        if kind == "k":
            step = s[np.arange(len(body)) // pf.GROUP]
        else:
            step = np.repeat(s, pf.GROUP, axis=1)
        err = np.abs(rec[r][body] - exact[body])
        # within half a step (the fp32 rounding of the chain adds a few ulps)
        assert np.all(err <= step / 2 + 4e-7 * (1 + np.abs(exact[body]))), (r, float(np.max(err - step / 2)))
        tail = np.arange(Sq, S) if r == 0 else st[r]["tail_rows"]
        assert np.array_equal(rec[r][tail], bf16_rne(exact[tail]))
        assert np.all(st[r]["codes"] <= 15) if "codes" in st[r] else True


def test_exact_integers_and_constants():
    """A group holding 0..15 quantizes with z = 0, s = 1 and no error; a
    constant fp16-representable group gets s = 0, codes 0 and x_hat = z."""
    S, d = 64 + pf.TAIL, 128
    x = np.zeros((S, d), np.float32)
    x[:64, :] = (np.arange(64) % 16)[:, None]          # keys: every channel sees 0..15
    x[:64, 5] = 0.75                                  # one constant channel
    st, rec = pf.quantize_chain_paper([x], [np.arange(S)], "k")
    assert np.array_equal(rec[0][:64], x[:64])
    assert st[0]["scale"][0, 5] == 0 and np.all(st[0]["codes"][:, 5] == 0)
    assert float(st[0]["zero"][0, 5]) == 0.75
    v = np.tile(np.arange(16, dtype=np.float32), 8)[None].repeat(S, 0)   # values: 0..15 in every group
    st, rec = pf.quantize_chain_paper([v], [np.arange(S)], "v")
    assert np.array_equal(rec[0][:S - pf.TAIL], v[:S - pf.TAIL])


def test_group_geometry():
    """Scaling one channel inside one 64-token key block changes that
    (block, channel) scale only; scaling one token's values changes only that
    token's value scales."""
    rows, x = _chain(S=64 * 3 + pf.TAIL, frac=(1.0,))
    st0, _ = pf.quantize_chain_paper(x, rows, "k")
    y = x[0].copy()
    y[70:80, 9] *= 50
    st1, _ = pf.quantize_chain_paper([y], rows, "k")
    diff = st0[0]["scale"] != st1[0]["scale"]
    assert diff.sum() == 1 and diff[1, 9]
    st0, _ = pf.quantize_chain_paper(x, rows, "v")
    y = x[0].copy()
    y[100, 64:] *= 50
    st1, _ = pf.quantize_chain_paper([y], rows, "v")
    diff = st0[0]["scale"] != st1[0]["scale"]
    assert diff.sum() == 1 and diff[100, 1]


def test_chain_keeps_inactive_and_short_sequences():
    """Tokens outside A_r keep x_hat^(r-1); a sequence no longer than the
    tail is stored entirely in bf16."""
    rows, x = _chain()
    for kind in "kv":
        _, rec = pf.quantize_chain_paper(x, rows, kind)
        for r in range(1, len(x)):
            off = np.setdiff1d(np.arange(x[0].shape[0]), rows[r])
            assert np.array_equal(rec[r][off], rec[r - 1][off])
    short = [x[0][:40]]
    _, rec = pf.quantize_chain_paper(short, [np.arange(40)], "k")
    assert np.array_equal(rec[0], bf16_rne(short[0]))
