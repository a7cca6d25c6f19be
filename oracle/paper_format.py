"""The paper's own cache format (p1 App. E, and the guide's summary of the
method): INT4 asymmetric group-wise quantization with group size 64 for the
loop-1 base and for every residual; post-RoPE keys quantized per channel,
values per token; the 64 most recent tokens kept in BF16.  Test
infrastructure, like the rest of the oracle.

Readings where the pages are silent:
  * the 4-bit asymmetric quantizer of one group: z = fp16 rounded down of the
    group minimum, s = fp16 rounded up of ((max - z) / 15) (fp32 divide),
    c = clamp(rint((x - z) / s), 0, 15), or 0 when s == 0; x_hat = fma(c, s, z)
    rounded once to fp32 (the directed roundings keep every element within
    half a step, as in the workload format);
  * the base quantizes x^(1) itself; loop r >= 2 quantizes the residual
    delta = x^(r) - x_hat^(r-1) of its active tokens, and x_hat^(r) =
    x_hat^(r-1) + (dequantized delta) in fp32; inactive tokens keep theirs;
  * a value group is 64 consecutive dims of one token; a key group is one
    channel over 64 consecutive tokens: positions [0, S - 64) in blocks of 64
    from position 0 for the base (the last block may hold fewer), and, for a
    residual, the active tokens outside the tail in position order, in blocks
    of 64 of that order;
  * the tail is the last min(64, S) positions; a tail token's K and V are
    stored as bf16 (round to nearest even) of its values at every loop where
    it is active, so there x_hat^(r) = bf16(x^(r)).
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_rne, fp16_down, fp16_up

GROUP = 64
TAIL = 64
LEVELS = np.float32(15.0)


def asym4(g: np.ndarray):
    """Quantize groups laid out on the last axis (float32 [..., n]).
    Returns (codes uint8, scale f16 [...], zero f16 [...], dequantized f32)."""
    g = np.asarray(g, np.float32)
    z16 = fp16_down(np.min(g, axis=-1))
    z = z16.astype(np.float32)
    s16 = fp16_up((np.max(g, axis=-1) - z).astype(np.float32) / LEVELS)
    s = s16.astype(np.float32)
    sb, zb = s[..., None], z[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        q = np.rint((g - zb) / np.where(sb == 0, np.float32(1), sb))
    c = np.where(sb == 0, 0, np.clip(q, 0, LEVELS)).astype(np.uint8)
    # 4-bit codes times fp16 scales plus fp16 zeros are exact in float64:
    # one cast is the single rounding of the fused multiply-add
    deq = (c.astype(np.float64) * sb.astype(np.float64) + zb.astype(np.float64)).astype(np.float32)
    return c, s16, z16, deq


def quant_values(x: np.ndarray):
    """Per-token value groups (64 dims).  x: float32 [n, d]."""
    n, d = x.shape
    c, s, z, deq = asym4(np.asarray(x, np.float32).reshape(n, d // GROUP, GROUP))
    return c.reshape(n, d), s, z, deq.reshape(n, d)


def quant_keys(x: np.ndarray):
    """Per-channel key groups: one channel over 64 consecutive rows of x
    (float32 [n, d]; the last block may hold fewer rows).  Returns codes
    [n, d], scale and zero [ceil(n / 64), d], dequantized [n, d]."""
    n, d = x.shape
    nb = -(-n // GROUP)
    codes = np.zeros((n, d), np.uint8)
    deq = np.zeros((n, d), np.float32)
    scale = np.zeros((nb, d), np.float16)
    zero = np.zeros((nb, d), np.float16)
    for blk in range(nb):
        t0, t1 = blk * GROUP, min(n, (blk + 1) * GROUP)
        c, s, z, q = asym4(np.asarray(x[t0:t1], np.float32).T)   # [d, rows]: a channel per group
        codes[t0:t1], deq[t0:t1] = c.T, q.T
        scale[blk], zero[blk] = s, z
    return codes, scale, zero, deq


def quantize_chain_paper(x: list, rows: list, kind: str):
    """Quantize the K (kind "k") or V (kind "v") chain of one (b, h) slice of
    all loops in the paper's format.  x[r-1]: loop-r values of rows[r-1]
    (loop 1: every position).  Returns (streams, recon): streams[r-1] holds
    what loop r stores, recon[r-1] the reconstruction x_hat^(r) of every
    position (float32 [S, d])."""
    S, d = x[0].shape
    Sq = max(0, S - TAIL)                 # quantized positions; [Sq, S) is the tail
    quant = quant_keys if kind == "k" else quant_values
    x1 = np.asarray(x[0], np.float32)
    cur = np.zeros((S, d), np.float32)
    st = {}
    if Sq:
        c, s, z, deq = quant(x1[:Sq])
        cur[:Sq] = deq
        st.update(codes=c, scale=s, zero=z)
    cur[Sq:] = bf16_rne(x1[Sq:])
    st["tail"] = cur[Sq:].copy()
    streams, recon = [st], [cur.copy()]
    for r in range(1, len(x)):
        rr = np.asarray(rows[r], np.int64)
        xr = np.asarray(x[r], np.float32)
        body = rr < Sq                     # active tokens outside the tail, position order
        st = dict(rows=rr[body], tail_rows=rr[~body])
        if body.any():
            delta = (xr[body] - cur[rr[body]]).astype(np.float32)
            c, s, z, deq = quant(delta)
            cur[rr[body]] = (cur[rr[body]] + deq).astype(np.float32)
            st.update(codes=c, scale=s, zero=z)
        cur[rr[~body]] = bf16_rne(xr[~body])
        st["tail"] = cur[rr[~body]].copy()
        streams.append(st)
        recon.append(cur.copy())
    return streams, recon
