"""Byte layout of the packed cache records, written from its specification.

The pages keep the cache as packed low-bit streams that the attention kernels
read without first expanding them (p1 App. G).
The record layout below is this implementation's own; the oracle writes and
reads it from the specification only (it never calls the library's code).

One record per (token, head):
  base record (loop 1), d dims, G = d / 32 groups:
    [0, d)            K codes, int8 two's complement, dim order
    [d, 2d)           V codes, int8
    [2d, 2d+2G)       K scales, fp16 little endian, group order
    [2d+2G, 2d+4G)    V scales
    zero padding up to a multiple of 16 bytes
  residual record (loop r >= 2, active tokens only), b bits, C = d*b/8:
    [0, C)            K codes packed; 4-bit: element 2k in the low nibble of
                      byte k, 2k+1 in the high nibble; 2-bit: element 4k+t in
                      bits 2t..2t+1 of byte k
    [C, 2C)           V codes packed
    [2C, 2C+2G)       K scales fp16      [2C+2G, 2C+4G)  K zeros fp16
    [2C+4G, 2C+6G)    V scales fp16      [2C+6G, 2C+8G)  V zeros fp16
    zero padding up to a multiple of 16 bytes
"""
from __future__ import annotations

import numpy as np


def _pad16(n: int) -> int:
    return (n + 15) // 16 * 16


def base_record_bytes(d: int) -> int:
    return _pad16(2 * d + 4 * (d // 32))


def residual_record_bytes(d: int, bits: int) -> int:
    return _pad16(2 * (d * bits // 8) + 8 * (d // 32))


def pack_codes(codes: np.ndarray, bits: int) -> np.ndarray:
    """codes uint8 [..., d] in [0, 2^bits) -> packed bytes [..., d*bits/8]."""
    c = np.asarray(codes, dtype=np.uint8)
    per = 8 // bits
    c = c.reshape(*c.shape[:-1], c.shape[-1] // per, per).astype(np.uint16)
    out = np.zeros(c.shape[:-1], dtype=np.uint16)
    for t in range(per):
        out |= c[..., t] << (bits * t)
    return out.astype(np.uint8)


def unpack_codes(packed: np.ndarray, bits: int) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    per = 8 // bits
    mask = (1 << bits) - 1
    parts = [(p >> (bits * t)) & mask for t in range(per)]
    return np.stack(parts, axis=-1).reshape(*p.shape[:-1], p.shape[-1] * per).astype(np.uint8)


def _f16_bytes(x: np.ndarray) -> np.ndarray:
    h = np.ascontiguousarray(np.asarray(x, dtype=np.float16))
    return h.view(np.uint8).reshape(*h.shape[:-1], h.shape[-1] * 2)


def _bytes_f16(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    return b.view(np.float16).reshape(*b.shape[:-1], b.shape[-1] // 2)


def pack_base(kc, ks, vc, vs) -> np.ndarray:
    """[..., d] int8 codes and [..., G] fp16 scales of K and V -> [..., rec] uint8."""
    d = kc.shape[-1]
    rec = np.zeros((*kc.shape[:-1], base_record_bytes(d)), dtype=np.uint8)
    G = d // 32
    rec[..., 0:d] = np.asarray(kc, np.int8).view(np.uint8)
    rec[..., d:2 * d] = np.asarray(vc, np.int8).view(np.uint8)
    rec[..., 2 * d:2 * d + 2 * G] = _f16_bytes(ks)
    rec[..., 2 * d + 2 * G:2 * d + 4 * G] = _f16_bytes(vs)
    return rec


def unpack_base(rec: np.ndarray, d: int):
    G = d // 32
    rec = np.asarray(rec, dtype=np.uint8)
    kc = np.ascontiguousarray(rec[..., 0:d]).view(np.int8)
    vc = np.ascontiguousarray(rec[..., d:2 * d]).view(np.int8)
    ks = _bytes_f16(rec[..., 2 * d:2 * d + 2 * G])
    vs = _bytes_f16(rec[..., 2 * d + 2 * G:2 * d + 4 * G])
    return kc, ks, vc, vs


def pack_residual(kc, ks, kz, vc, vs, vz, bits: int) -> np.ndarray:
    d = kc.shape[-1]
    G = d // 32
    C = d * bits // 8
    rec = np.zeros((*kc.shape[:-1], residual_record_bytes(d, bits)), dtype=np.uint8)
    rec[..., 0:C] = pack_codes(kc, bits)
    rec[..., C:2 * C] = pack_codes(vc, bits)
    o = 2 * C
    for arr in (ks, kz, vs, vz):
        rec[..., o:o + 2 * G] = _f16_bytes(arr)
        o += 2 * G
    return rec


def unpack_residual(rec: np.ndarray, d: int, bits: int):
    G = d // 32
    C = d * bits // 8
    rec = np.asarray(rec, dtype=np.uint8)
    kc = unpack_codes(rec[..., 0:C], bits)
    vc = unpack_codes(rec[..., C:2 * C], bits)
    o = 2 * C
    meta = []
    for _ in range(4):
        meta.append(_bytes_f16(rec[..., o:o + 2 * G]))
        o += 2 * G
    ks, kz, vs, vz = meta
    return kc, ks, kz, vc, vs, vz
