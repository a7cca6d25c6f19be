"""Algorithmic work and byte counts of the hot path (host-side bookkeeping).

The cost model follows the guide's Cell 1 (flozi-tech guide §1): one BF16
(K, V) pair per loop per layer, so bytes per (token, loop) =
layers * 2 * kv_heads * head_dim * 2, and decode arithmetic intensity =
2 * params * loops / cache bytes against a roofline ridge of peak FLOP/s over
bandwidth.  Prefill work counts only causally valid (query, key) pairs, from
the index lists of the run: 4*d FLOPs per pair for QK^T plus PV, 2*d plus one
exp per pair for the column-mass pass.  Decode bytes count the packed records
a step must read.
"""
from __future__ import annotations

import numpy as np

GIB = 1024 ** 3
MI355X_HBM_GBS = 8000.0          # vendor peak, GB/s
MI355X_BF16_TFLOPS = 2500.0      # dense MFMA, TFLOP/s


def bytes_per_token_loop(layers: int, kv_heads: int, head_dim: int, elem_bytes: int = 2) -> int:
    return layers * 2 * kv_heads * head_dim * elem_bytes


def loop_cache_bytes(layers, loops, tokens, kv_heads, head_dim, elem_bytes=2) -> int:
    return bytes_per_token_loop(layers, kv_heads, head_dim, elem_bytes) * tokens * loops


def ridge_flop_per_byte(tflops: float, gbs: float) -> float:
    return tflops * 1e12 / (gbs * 1e9)


def decode_intensity(params: float, loops: int, cache_bytes: float) -> float:
    """FLOPs per cache byte of one decode step that re-reads every loop's KV."""
    return 2.0 * params * loops / cache_bytes


def causal_pairs_dense(S: int) -> int:
    return S * (S + 1) // 2


def sparse_pairs(rows: np.ndarray, sel: np.ndarray) -> int:
    """sum over rows i of |{j in sel : j <= i}| (rows, sel ascending)."""
    return int(np.searchsorted(np.asarray(sel), np.asarray(rows), side="right").sum())


def base_record_bytes(d: int) -> int:
    """Algorithmic bytes of one base record: K and V codes plus fp16 scales."""
    return 2 * d + 4 * (d // 32)


def residual_record_bytes(d: int, bits: int) -> int:
    return 2 * (d * bits // 8) + 8 * (d // 32)


def resq_bytes(d: int, bits, n_rows: int, kv_heads: int, elem_bytes: int = 2) -> int:
    """Algorithmic HBM bytes of one fl_kv_resq call at loop r = len(bits): per
    active (row, KV head) the loop's K and V rows are read, the records of
    loops 1..r-1 the residual is taken against are read, and one record is
    written.  bits = (bits_1, ..., bits_r)."""
    r = len(bits)
    chain = base_record_bytes(d) + sum(residual_record_bytes(d, b) for b in bits[1:r - 1]) if r > 1 else 0
    write = base_record_bytes(d) if r == 1 else residual_record_bytes(d, bits[r - 1])
    return n_rows * kv_heads * (2 * d * elem_bytes + chain + write)


def prefill_work(cfg, rows_per_b, sels, masses_ran) -> dict:
    """Exact pair counts and FLOPs of one prefill step.

    rows_per_b[b][r-1]: A_r; sels[r-1]: int array [B][H][K_r] (None at r = 1);
    masses_ran[r-1]: whether the mass pass ran at loop r."""
    B, H, d = cfg.B, cfg.H, cfg.d
    out = dict(dense_pairs=B * H * causal_pairs_dense(cfg.S), loops=[])
    for r in range(2, cfg.R + 1):
        sp = mp = 0
        for b in range(B):
            A = rows_per_b[b][r - 1]
            for h in range(H):
                sp += sparse_pairs(A, sels[r - 1][b, h])
                if masses_ran[r - 1]:
                    cand = np.arange(cfg.S) if r == 2 else sels[r - 2][b, h]
                    mp += sparse_pairs(A, cand)
        out["loops"].append(dict(r=r, sparse_pairs=sp, mass_pairs=mp, um_pairs=sp if masses_ran[r - 1] else 0))
    flops = 4 * d * out["dense_pairs"]
    for lp in out["loops"]:
        flops += 4 * d * lp["sparse_pairs"] + 4 * d * lp["um_pairs"] + 2 * d * lp["mass_pairs"]
    out["flops"] = flops
    out["dense_flops"] = 4 * d * out["dense_pairs"]
    out["sparse_flops"] = sum(4 * d * lp["sparse_pairs"] for lp in out["loops"])
    return out
