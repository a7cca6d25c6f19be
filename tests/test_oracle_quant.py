"""Pins of the oracle's quantizer and record layout against brute force,
the half-step bound, special groups and a hand-worked packing example."""
import os

import numpy as np
import pytest

from oracle import quant, records

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# every finite fp16 value, as exact float64 numbers, sorted
_ALL_F16 = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
_ALL_F16 = np.unique(_ALL_F16[np.isfinite(_ALL_F16)].astype(np.float64))


def _smallest_f16_at_least(y):
    return _ALL_F16[np.searchsorted(_ALL_F16, y, side="left")]


def _largest_f16_at_most(y):
    return _ALL_F16[np.searchsorted(_ALL_F16, y, side="right") - 1]


def _groups(rng, n, scale):
    x = rng.standard_normal((n, 32)).astype(np.float32) * np.float32(scale)
    return x


@pytest.mark.parametrize("scale", [1e-6, 3e-3, 1.0, 250.0, 1.5e4])
def test_directed_fp16_rounding_bruteforce(scale):
    rng = np.random.default_rng(1)
    y = (rng.standard_normal(4000) * scale).astype(np.float32)
    up = quant.fp16_up(np.abs(y)).astype(np.float64)
    dn = quant.fp16_down(y).astype(np.float64)
    assert np.array_equal(up, _smallest_f16_at_least(np.abs(y).astype(np.float64)))
    assert np.array_equal(dn, _largest_f16_at_most(y.astype(np.float64)))


@pytest.mark.parametrize("scale", [1e-5, 0.02, 1.0, 40.0, 3e4])
def test_base_codes_are_nearest(scale):
    rng = np.random.default_rng(2)
    x = _groups(rng, 300, scale)
    c, s16, rec = quant.quant_base(x)
    s = s16.astype(np.float64)[:, 0]
    a = np.abs(x).max(axis=1).astype(np.float64)
    # scale: the smallest fp16 at or above fp32(a / 127)
    y = (np.abs(x).max(axis=1) / np.float32(127)).astype(np.float64)
    assert np.array_equal(s, _smallest_f16_at_least(y))
    assert np.all(s * 127 >= a * (1 - 2 ** -23))
    # codes: brute force over all 255 codes, nearest (ties: either neighbour)
    allc = np.arange(-127, 128, dtype=np.float64)
    err = np.abs(x[:, :, None].astype(np.float64) - allc[None, None, :] * s[:, None, None])
    best = err.min(axis=2)
    mine = np.abs(x.astype(np.float64) - c.astype(np.float64) * s[:, None])
    assert np.all(mine <= best + 2 ** -22 * np.maximum(np.abs(x), 1e-30))
    assert np.array_equal(rec, (c.astype(np.float32) * s16.astype(np.float32)[:, 0:1]))


@pytest.mark.parametrize("bits", [2, 4])
@pytest.mark.parametrize("scale", [1e-4, 0.1, 1.0, 77.0])
def test_residual_codes_are_nearest(bits, scale):
    rng = np.random.default_rng(3 + bits)
    prev = _groups(rng, 200, 1.0)
    x = (prev + _groups(rng, 200, scale)).astype(np.float32)
    c, s16, z16, rec = quant.quant_residual(x, prev, bits)
    delta = (x - prev).astype(np.float32)
    Q = 2 ** bits - 1
    z = z16[:, 0].astype(np.float64)
    s = s16[:, 0].astype(np.float64)
    assert np.array_equal(z, _largest_f16_at_most(delta.min(axis=1).astype(np.float64)))
    w = (delta.max(axis=1) - z16[:, 0].astype(np.float32)).astype(np.float32)
    assert np.array_equal(s, _smallest_f16_at_least((w / np.float32(Q)).astype(np.float64)))
    allc = np.arange(Q + 1, dtype=np.float64)
    err = np.abs(delta[:, :, None].astype(np.float64) - (z[:, None, None] + allc[None, None, :] * s[:, None, None]))
    best = err.min(axis=2)
    mine = np.abs(delta.astype(np.float64) - (z[:, None] + c.astype(np.float64) * s[:, None]))
    assert np.all(mine <= best + 2 ** -21 * np.maximum(np.abs(delta), np.abs(z)[:, None]) + 1e-30)
    # single-rounding dequantization and the fp32 chain sum
    dhat = (c.astype(np.float64) * s[:, None] + z[:, None]).astype(np.float32)
    assert np.array_equal(rec, (prev + dhat).astype(np.float32))


def _ulp32(x):
    x = np.abs(np.asarray(x, np.float32))
    return (np.nextafter(x, np.float32(np.inf)) - x).astype(np.float64)


@pytest.mark.parametrize("bits", [(8, 4, 4, 4), (8, 4, 4, 2), (8, 4, 4, 4, 2, 2, 2, 2)])
def test_half_step_bound_every_loop(bits):
    """|x - x_hat| <= s/2 + 4 ulp at every loop for the active rows."""
    rng = np.random.default_rng(11)
    S, d, R = 96, 64, len(bits)
    rows = [np.arange(S)]
    for r in range(1, R):
        rows.append(np.sort(rng.choice(rows[-1], max(1, len(rows[-1]) * 2 // 3), replace=False)))
    x = [rng.standard_normal((S, d)).astype(np.float32) * 3]
    full = x[0].copy()
    for r in range(1, R):
        full[rows[r]] += (0.6 ** r) * rng.standard_normal((len(rows[r]), d)).astype(np.float32)
        x.append(full[rows[r]].copy())
    streams, recon = quant.quantize_chain(x, rows, list(bits))
    for r in range(R):
        xr = x[r]
        xh = recon[r][rows[r]]
        s = streams[r]["scale"].astype(np.float64)
        step = np.repeat(s, 32, axis=-1) / 2
        tol = step + 4 * _ulp32(np.maximum(np.abs(xr), np.abs(xh)))
        assert np.all(np.abs(xr.astype(np.float64) - xh.astype(np.float64)) <= tol), r
        if r:
            inactive = np.setdiff1d(np.arange(S), rows[r])
            assert np.array_equal(recon[r][inactive], recon[r - 1][inactive])


def test_special_groups():
    z = np.zeros((3, 32), np.float32)
    c, s, rec = quant.quant_base(z)
    assert not c.any() and not s.astype(np.float32).any() and not rec.any()
    ints = np.arange(-127, 129, dtype=np.float32)[:256].reshape(8, 32)
    ints[ints > 127] = 127
    ints[:, 0] = 127
    c, s, rec = quant.quant_base(ints)
    assert np.all(s.astype(np.float32) == 1) and np.array_equal(c.astype(np.float32), ints)
    # constant residual group of an fp16 value: zero = value, scale 0, exact
    prev = np.full((2, 32), 1.5, np.float32)
    for val in (np.float32(0.375), np.float32(-2.0), np.float32(6.103515625e-05)):
        xg = (prev + val).astype(np.float32)
        c, s16, z16, rec = quant.quant_residual(xg, prev, 4)
        assert not c.any() and not s16.astype(np.float32).any()
        assert np.all(z16.astype(np.float32) == (xg - prev)) and np.array_equal(rec, xg)


def test_packing_worked_example():
    lines = [l.strip() for l in open(os.path.join(GOLDEN, "packing_worked_example.txt")) if l.strip() and not l.startswith("#")]
    pairs = [(lines[i], lines[i + 1]) for i in range(0, len(lines), 2)]
    for lc, lb in pairs:
        bits = int(lc.split()[0].split("=")[1])
        codes = np.array([int(t) for t in lc.split("codes=")[1].split(",")], np.uint8)
        want = np.array([int(t, 16) for t in lb.split("bytes=")[1].split(",")], np.uint8)
        got = records.pack_codes(codes, bits)
        assert np.array_equal(got, want)
        assert np.array_equal(records.unpack_codes(got, bits), codes)


@pytest.mark.parametrize("d,bits", [(64, 4), (64, 2), (128, 4), (128, 2)])
def test_record_roundtrip(d, bits):
    rng = np.random.default_rng(5)
    n = 17
    kc = rng.integers(-127, 128, (n, d)).astype(np.int8)
    vc = rng.integers(-127, 128, (n, d)).astype(np.int8)
    ks = rng.standard_normal((n, d // 32)).astype(np.float16)
    vs = rng.standard_normal((n, d // 32)).astype(np.float16)
    rec = records.pack_base(kc, ks, vc, vs)
    assert rec.shape[-1] == records.base_record_bytes(d) and rec.shape[-1] % 16 == 0
    out = records.unpack_base(rec, d)
    for a, b in zip(out, (kc, ks, vc, vs)):
        assert np.array_equal(a.view(np.uint8), np.asarray(b).view(np.uint8))
    Q = 2 ** bits
    parts = [rng.integers(0, Q, (n, d)).astype(np.uint8)] + [rng.standard_normal((n, d // 32)).astype(np.float16) for _ in range(2)]
    parts += [rng.integers(0, Q, (n, d)).astype(np.uint8)] + [rng.standard_normal((n, d // 32)).astype(np.float16) for _ in range(2)]
    rec = records.pack_residual(*parts, bits=bits)
    assert rec.shape[-1] == records.residual_record_bytes(d, bits) and rec.shape[-1] % 16 == 0
    out = records.unpack_residual(rec, d, bits)
    for a, b in zip(out, parts):
        assert np.array_equal(np.asarray(a).view(np.uint8), np.asarray(b).view(np.uint8))
    if d == 128:
        assert records.base_record_bytes(d) == 272
        assert records.residual_record_bytes(d, bits) == {4: 160, 2: 96}[bits]


def _bf16_probe_values():
    """float32 inputs for the bf16 rounding pins: random bit patterns of
    every exponent, exact halfway cases with even and odd kept bits, values
    next to halfway, the overflow edge, subnormals, signed zeros, infinities."""
    rng = np.random.default_rng(17)
    u = rng.integers(0, 1 << 32, 200000, dtype=np.uint64).astype(np.uint32)
    kept = rng.integers(0, 1 << 16, 20000, dtype=np.uint64).astype(np.uint32) << 16
    ties = kept | np.uint32(0x8000)
    below = kept | np.uint32(0x7FFF)
    above = kept | np.uint32(0x8001)
    edge = np.array([0x7F7F0000, 0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0xFF7F8000, 0xFF7F7FFF,
                     0x7F7E8000, 0x00008000, 0x00018000, 0x00007FFF, 0x0000FFFF, 0x80008000, 0x80018000,
                     0x00000000, 0x80000000, 0x7F800000, 0xFF800000, 0x3F808000, 0x3F818000, 0x3F80FFFF],
                    dtype=np.uint32)
    allu = np.concatenate([u, ties, below, above, edge])
    f = allu.view(np.float32)
    return f[~np.isnan(f)]


def test_bf16_rne_matches_torch_cast():
    """The oracle's bf16 rounding equals torch's CPU float32 -> bfloat16 cast
    (round to nearest, ties to even), bit for bit, on every probe value."""
    import torch
    x = _bf16_probe_values()
    got = quant.bf16_rne(x)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # NaN stays NaN (of either sign and any payload)
    nan = np.array([0x7FC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFFFFFF], dtype=np.uint32).view(np.float32)
    assert np.all(np.isnan(quant.bf16_rne(nan)))


def test_bf16_rne_is_nearest_even_bruteforce():
    """Independent of any library: the result is one of the two bf16 values
    around x (the truncation and its successor away from zero); it is the
    nearer one in exact float64 distance, and on an exact tie the one whose
    lowest kept bit is 0.  Past the largest finite bf16 value, x rounds to
    infinity when it lies at or beyond the halfway point to 2^128."""
    x = _bf16_probe_values()
    x = x[np.isfinite(x)]
    got = quant.bf16_rne(x).astype(np.float64)
    u = x.view(np.uint32)
    lo_u = u & np.uint32(0xFFFF0000)
    hi_u = lo_u + np.uint32(0x10000)           # next bf16 away from zero (may be infinity)
    lo = lo_u.view(np.float32).astype(np.float64)
    hi = hi_u.view(np.float32).astype(np.float64)
    xf = x.astype(np.float64)
    # distance to the successor: 2^128 stands in for infinity's position
    sign = np.sign(xf)
    hi_pos = np.where(np.isinf(hi), sign * 2.0 ** 128, hi)
    dlo, dhi = np.abs(xf - lo), np.abs(hi_pos - xf)
    lo_even = ((lo_u >> 16) & 1) == 0
    want = np.where(dlo < dhi, lo, np.where(dhi < dlo, hi, np.where(lo_even, lo, hi)))
    assert np.array_equal(got, want)
