"""Quantizers of the cross-loop KV cache (p1 §4.3 and §D.3; guide §3).

The pages store a quantized loop-1 base and, for every later loop, quantized
residuals of the active tokens taken against the *reconstructed* previous
loop (p1 §4.3; guide §3 writes the stored residual as X^(r) - X_hat^(r-1),
for active tokens only).  A token that is not active keeps its previous K/V
and stores nothing (p1 §4.3).

Storage format (the workload definitions fix it; the paper's own INT4/g64
setting of p1 App. E is a different format): groups of 32 consecutive
dimensions of one (token, head) row;
  * base: int8 symmetric codes in [-127, 127] and one fp16 scale per group;
  * residual: b-bit asymmetric codes in [0, 2^b - 1] (b = 4 or 2), one fp16
    scale and one fp16 zero (a float offset) per group.

Readings where the pages are silent:
  * scale = fp16 rounded *up* of (range / levels), zero = fp16 rounded *down*
    of the group minimum, so every element stays within half a step;
  * codes: fp32 divide (IEEE, round to nearest even), round half to even,
    clamp; no fused multiply-add in the code computation;
  * dequantized residual = one fused multiply-add c*s + z rounded once to
    fp32; the chain is added in fp32, base first, loops ascending.
"""
from __future__ import annotations

import numpy as np

GROUP = 32


def fp16_up(y: np.ndarray) -> np.ndarray:
    """Round float32 values to fp16 toward +infinity (result as float16)."""
    y = np.asarray(y, dtype=np.float32)
    h = y.astype(np.float16)                 # numpy casts with round-to-nearest-even
    low = h.astype(np.float32) < y
    if np.any(low):
        h = h.copy()
        h[low] = np.nextafter(h[low], np.float16(np.inf))
    return h


def fp16_down(y: np.ndarray) -> np.ndarray:
    """Round float32 values to fp16 toward -infinity (result as float16)."""
    y = np.asarray(y, dtype=np.float32)
    h = y.astype(np.float16)
    high = h.astype(np.float32) > y
    if np.any(high):
        h = h.copy()
        h[high] = np.nextafter(h[high], np.float16(-np.inf))
    return h


def _groups(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    assert x.shape[-1] % GROUP == 0
    return x.reshape(*x.shape[:-1], x.shape[-1] // GROUP, GROUP)


def quant_base(x: np.ndarray):
    """Loop-1 base quantizer (p1 §4.3 "quantized first-loop base").

    x: float32 [..., d].  Returns (codes int8 [..., d], scale float16 [..., d/32],
    recon float32 [..., d]).  Per group: a = max|x|; s = fp16_up(a / 127);
    c = clamp(rint(x / s), -127, 127), or 0 when s == 0; recon = c * s (exact).
    """
    g = _groups(x)
    a = np.max(np.abs(g), axis=-1)
    s16 = fp16_up(a / np.float32(127.0))
    s = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint(g / np.where(s == 0, np.float32(1), s))
    c = np.where(s == 0, 0, np.clip(q, -127, 127)).astype(np.int8)
    recon = (c.astype(np.float32) * s).reshape(x.shape)
    return c.reshape(x.shape), s16, recon


def quant_residual(x: np.ndarray, prev: np.ndarray, bits: int):
    """Residual quantizer of loop r >= 2 for the active rows (p1 §4.3, §D.3).

    x: loop-r values, prev: the reconstructed loop r-1 values of the same rows
    (both float32 [..., d]).  delta = x - prev (fp32); per group lo = min,
    hi = max; z = fp16_down(lo); s = fp16_up((hi - z) / (2^b - 1));
    c = clamp(rint((delta - z) / s), 0, 2^b - 1), or 0 when s == 0;
    dhat = fma(c, s, z) rounded once to fp32; recon = prev + dhat (fp32).
    Returns (codes uint8 [..., d], scale f16 [..., d/32], zero f16 [..., d/32],
    recon float32 [..., d]).
    """
    assert bits in (2, 4)
    levels = np.float32(2 ** bits - 1)
    delta = (np.asarray(x, np.float32) - np.asarray(prev, np.float32)).astype(np.float32)
    g = _groups(delta)
    lo = np.min(g, axis=-1)
    hi = np.max(g, axis=-1)
    z16 = fp16_down(lo)
    z = z16.astype(np.float32)
    w = (hi - z).astype(np.float32)
    s16 = fp16_up(w / levels)
    s = s16.astype(np.float32)
    sb, zb = s[..., None], z[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((g - zb) / np.where(sb == 0, np.float32(1), sb))
    c = np.where(sb == 0, 0, np.clip(q, 0, levels)).astype(np.uint8)
    # c has <= 8 significant bits and s, z are fp16 values: the float64 product
    # and sum are exact, so one cast to float32 is the single fma rounding.
    dhat = (c.astype(np.float64) * sb.astype(np.float64) + zb.astype(np.float64)).astype(np.float32)
    recon = (np.asarray(prev, np.float32) + dhat.reshape(delta.shape)).astype(np.float32)
    return c.reshape(delta.shape), s16, z16, recon


def quantize_chain(k: list, rows: list, bits: list):
    """Quantize one (b, h) tensor chain of all loops.

    k[r-1]: loop-r input for rows[r-1] (loop 1: every row).  Returns
    (streams, recon) where streams[r-1] holds the stored codes of loop r and
    recon[r-1] is the reconstruction X_hat^(r) of every row (float32 [S, d]).
    Tokens outside A_r keep X_hat^(r-1) (p1 §4.3: inactive tokens reuse their
    K/V states).
    """
    c, s, rec = quant_base(k[0])
    streams = [dict(codes=c, scale=s)]
    recon = [rec]
    for r in range(1, len(k)):
        rr = rows[r]
        cur = recon[-1].copy()
        c, s, z, new = quant_residual(k[r], cur[rr], bits[r])
        cur[rr] = new
        streams.append(dict(codes=c, scale=s, zero=z))
        recon.append(cur)
    return streams, recon


def bf16_rne(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16, round to nearest, ties to the even
    significand (IEEE 754 roundTiesToEven), returned as float32.

    bf16 keeps the upper 16 bits of a float32.  Adding 0x7FFF plus the lowest
    kept bit before truncating moves every value above the halfway point up,
    every value below it down, and a value exactly halfway to the neighbour
    whose lowest kept bit is 0.  A carry out of the significand raises the
    exponent, which is the right result, including overflow to infinity past
    the largest bf16 value.  NaN stays NaN (the carry could otherwise turn a
    NaN payload into infinity)."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    out = u.astype(np.uint32).view(np.float32)
    nan = np.isnan(f)
    if np.any(nan):
        out = np.where(nan, np.float32(np.nan), out).astype(np.float32)
    return out
