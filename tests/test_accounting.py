"""Byte and FLOP accounting against the numbers the guide's Cell 1 prints."""
import os

import numpy as np

from sparse_attn_residual_amd import accounting as acc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "guide_cell1.txt")


def _golden():
    vals = {}
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#"):
            k, v = line.split("=")
            vals[k] = float(v)
    return vals


def test_cell1_bytes_per_token_loop():
    g = _golden()
    # Ouro-2.6B shape: 48 layers, 16 KV heads of 128 dims, BF16
    per = acc.bytes_per_token_loop(48, 16, 128)
    assert per == g["bytes_per_token_loop"]
    total = acc.loop_cache_bytes(48, int(g["loops"]), int(g["context_tokens"]), 16, 128)
    assert total == g["kv_gib"] * acc.GIB
    assert total / (g["context_tokens"] * g["loops"]) == g["bytes_per_token_loop"]


def test_cell1_roofline_numbers():
    g = _golden()
    ridge = acc.ridge_flop_per_byte(312.0, 1555.0)
    assert round(ridge) == g["ridge_flop_per_byte"]
    inten = acc.decode_intensity(2.6e9, 4, 48 * acc.GIB)
    assert round(inten, 2) == g["decode_intensity_flop_per_byte"]
    assert round(ridge / inten) == g["below_ridge_factor"]


def test_pair_counts_bruteforce():
    rng = np.random.default_rng(0)
    S = 300
    rows = np.sort(rng.choice(S, 70, replace=False))
    sel = np.sort(rng.choice(S, 40, replace=False))
    brute = sum(1 for i in rows for j in sel if j <= i)
    assert acc.sparse_pairs(rows, sel) == brute
    assert acc.causal_pairs_dense(7) == sum(i + 1 for i in range(7))


def test_record_bytes_match_layout():
    import sparse_attn_residual_amd as fl
    for d in (64, 128):
        assert fl.fl_base_record_bytes(d) == (acc.base_record_bytes(d) + 15) // 16 * 16
        for b in (2, 4):
            assert fl.fl_residual_record_bytes(d, b) == (acc.residual_record_bytes(d, b) + 15) // 16 * 16


def test_resq_bytes_hand_count():
    """fl_kv_resq bytes at d = 128, bf16 inputs, per active (row, KV head):
    K and V in (2 x 128 x 2 = 512 B), the earlier loops' records read (base
    272 B, 4-bit residual 160 B), one record out (2-bit residual 96 B)."""
    from sparse_attn_residual_amd import accounting as acc
    assert acc.resq_bytes(128, (8,), 32768, 16) == 32768 * 16 * (512 + 272)
    assert acc.resq_bytes(128, (8, 4), 9830, 16) == 9830 * 16 * (512 + 272 + 160)
    assert acc.resq_bytes(128, (8, 4, 4), 4915, 16) == 4915 * 16 * (512 + 272 + 160 + 160)
    assert acc.resq_bytes(128, (8, 4, 4, 2), 2621, 16) == 2621 * 16 * (512 + 272 + 160 + 160 + 96)
