"""Seeded synthetic workloads for the FlashLoop loop-attention hot path.

This module is the only code shared by the CPU oracle's tests and the HIP
path's tests and benchmark.  It draws random numbers and nothing else: it
holds none of the method's arithmetic (no quantization, no attention, no
selection).  Every array it returns is an *input* of the method.

Shapes follow the synthetic stand-ins for the workloads on the FlashLoop pages
(paperlayer.ai abstract page, §1 and §5.1; flozi-tech guide, Cell 1): Ouro-like
16 heads x 128 dims, 8K/16K/32K contexts, R = 4 or 8 loops.  The structure
follows the pages' observations: nested active-token sets spread through the
context (§3.1, §4.1), geometrically shrinking adjacent-loop updates (§3.3), and
heavy-tailed rows that concentrate attention (§3.2).

Recipe (one stream per (seed, tensor, b, h), numpy PCG64 seeded through
SeedSequence, so any (b, h) slice can be regenerated alone):
  * loop 1: X^1 = cast(lam_i * N(0, 1)) for X in {Q, K, V} (lam_i = 1 unless
    the config asks for lognormal rows; then one lam per (b, h, row), drawn
    separately for Q and K; V is never scaled);
  * loop r >= 2: A_r = sorted(choice(A_{r-1}, n_r, replace=False)) per
    sequence b, shared by every head; active rows get
    X^r_i = cast(X^{r-1}_i + lam_i * gamma^r * N(0, 1)); inactive rows keep
    X^{r-1}_i and are not part of the loop-r input;
  * cast = round-to-nearest-even to the config dtype (fp32 or bf16); bf16
    values are returned widened to float32 (exactly).
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

# tensor ids of the per-slice random streams
_T_Q, _T_K, _T_V = 1, 2, 3
_T_LAM_Q, _T_LAM_K = 4, 5
_T_ROWS = 6
_T_DQ, _T_DK, _T_DV = 10, 30, 50   # + loop index r
_T_DEC_Q, _T_DEC_LAM, _T_DEC_DQ = 70, 71, 80
_T_HID, _T_HID_EPS, _T_HID_DIR = 90, 91, 92   # + loop index r for the last two


def frac_count(f: str | float, n: int) -> int:
    """floor(f * n), at least 1, computed exactly from the decimal fraction."""
    return max(1, math.floor(Fraction(str(f)) * n))


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  Loop-indexed lists have index 0 = loop 1."""
    name: str
    dtype: str                 # "f32" or "bf16"
    B: int
    H: int
    d: int
    S: int                     # context length (prefill) or cached tokens T (decode)
    R: int
    act: tuple                 # active-row fraction per loop (act[0] == 1)
    col: str                   # column budget fraction (as a decimal string)
    bits: tuple                # 8 for loop 1, residual bits afterwards
    gamma: float               # per-loop delta scale gamma^r
    lognormal: float | None = None   # sigma of the per-row lognormal scale
    L: int = 1                 # stacked layers (decode only)
    decode: bool = False
    seed: int = 0
    Hkv: int = 0               # key/value heads (0: H); query head h reads KV head h // (H // Hkv)
    ragged: tuple = ()         # per-sequence factors m_b: |A_r| of sequence b = max(1, floor(m_b * n_r)), r >= 2

    @property
    def kv_heads(self) -> int:
        return self.H if self.Hkv == 0 else self.Hkv

    @property
    def G(self) -> int:
        """Query heads per KV head."""
        return self.H // self.kv_heads

    @property
    def n(self) -> list[int]:
        """n_r for r = 1..R (index 0 = loop 1)."""
        return [self.S if r == 0 else frac_count(self.act[r], self.S) for r in range(self.R)]

    @property
    def K(self) -> int:
        """Column budget per head for the sparse loops."""
        return frac_count(self.col, self.S)

    def counts(self, b: int) -> list[int]:
        """|A_r| of sequence b for r = 1..R (n when the batch is not ragged)."""
        if not self.ragged:
            return self.n
        m = Fraction(str(self.ragged[b]))
        return [self.S if r == 0 else max(1, math.floor(m * self.n[r])) for r in range(self.R)]

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


def _halving(R):
    return tuple(1.0 if r == 0 else 2.0 ** (-r) for r in range(R))


CONFIGS: dict[int, Config] = {
    0: Config("tiny-fp32-s512", "f32", 1, 2, 64, 512, 4, (1.0, 0.5, 0.25, 0.125), "0.25",
              (8, 4, 4, 4), 0.5),
    1: Config("ouro1.4b-prefill-s8192", "bf16", 1, 16, 128, 8192, 4, (1.0, 0.4, 0.2, 0.1), "0.10",
              (8, 4, 4, 4), 0.5),
    2: Config("ouro2.6b-prefill-s32768", "bf16", 1, 16, 128, 32768, 4, (1.0, 0.3, 0.15, 0.08), "0.10",
              (8, 4, 4, 2), 0.5, lognormal=0.5),
    3: Config("ouro2.6b-decode-t32768-l48", "bf16", 16, 16, 128, 32768, 4, (1.0, 0.3, 0.15, 0.08), "0.10",
              (8, 4, 4, 2), 0.5, lognormal=0.5, L=48, decode=True),
    4: Config("deep-loop-s16384-r8", "bf16", 1, 16, 128, 16384, 8, _halving(8), "0.05",
              (8, 4, 4, 4, 2, 2, 2, 2), 0.7),
}


def _rng(cfg: Config, *ids) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg.seed, *ids])))


def cast(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the config dtype (RNE) and return them as float32."""
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f32":
        return x
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def active_rows(cfg: Config, b: int) -> list[np.ndarray]:
    """Nested active sets A_1 ⊇ A_2 ⊇ ... for sequence b (int32, ascending)."""
    rng = _rng(cfg, _T_ROWS, b)
    rows = [np.arange(cfg.S, dtype=np.int32)]
    cnt = cfg.counts(b)
    for r in range(1, cfg.R):
        prev = rows[-1]
        pick = rng.choice(prev.shape[0], cnt[r], replace=False)
        rows.append(np.sort(prev[pick]).astype(np.int32))
    return rows


@dataclass
class Slice:
    """Inputs of one (b, h) slice: per-loop compact tensors in rows order."""
    rows: list            # rows[r-1]: int32 [n_r]
    q: list               # q[r-1]: float32 [n_r, d]
    k: list
    v: list


def _chain(cfg: Config, rows, tid_base, tid_delta, lam, b, h):
    S, d = cfg.S, cfg.d
    g = _rng(cfg, tid_base, b, h)
    x = cast(lam[:, None] * g.standard_normal((S, d), dtype=np.float32), cfg.dtype)
    out = [x]
    full = x.copy()
    for r in range(1, cfg.R):
        rr = rows[r]
        g = _rng(cfg, tid_delta + r + 1, b, h)
        step = np.float32(cfg.gamma ** (r + 1))
        delta = g.standard_normal((rr.shape[0], d), dtype=np.float32)
        xr = cast(full[rr] + (lam[rr, None] * step) * delta, cfg.dtype)
        full[rr] = xr
        out.append(xr)
    return out


def _lam(cfg: Config, tid, b, h):
    if cfg.lognormal is None:
        return np.ones(cfg.S, dtype=np.float32)
    return _rng(cfg, tid, b, h).lognormal(0.0, cfg.lognormal, cfg.S).astype(np.float32)


def gen_slice(cfg: Config, b: int, h: int, rows=None, with_q: bool = True) -> Slice:
    """All loop inputs of one (b, h) slice.  Loop-1 tensors cover every row.
    with_q=False skips the queries (a decode cache needs keys and values only)."""
    if rows is None:
        rows = active_rows(cfg, b)
    hk = h // cfg.G   # keys and values come from the query head's KV head
    lam_q = _lam(cfg, _T_LAM_Q, b, h)
    lam_k = _lam(cfg, _T_LAM_K, b, hk)
    ones = np.ones(cfg.S, dtype=np.float32)
    q = _chain(cfg, rows, _T_Q, _T_DQ, lam_q, b, h) if with_q else None
    k = _chain(cfg, rows, _T_K, _T_DK, lam_k, b, hk)
    v = _chain(cfg, rows, _T_V, _T_DV, ones, b, hk)
    return Slice(rows=rows, q=q, k=k, v=v)


def gen_batch(cfg: Config, heads=None, batches=None, threads: int | None = None, with_q: bool = True):
    """Slices for every (b, h) requested: returns (rows[b], {(b, h): Slice})."""
    heads = range(cfg.H) if heads is None else heads
    batches = range(cfg.B) if batches is None else batches
    rows = {b: active_rows(cfg, b) for b in batches}
    keys = [(b, h) for b in batches for h in heads]
    with ThreadPoolExecutor(max_workers=threads or min(16, len(keys))) as ex:
        res = list(ex.map(lambda bh: gen_slice(cfg, bh[0], bh[1], rows[bh[0]], with_q), keys))
    return rows, dict(zip(keys, res))


def stack_loop(cfg: Config, slices: dict, r: int, what: str, batches=None, heads=None) -> np.ndarray:
    """[B][H][n_r][d] float32 tensor of loop r (1-based) for q; for k/v the
    heads default to the KV heads ([B][Hkv][n_r][d], taken from the first
    query head of each group)."""
    batches = range(cfg.B) if batches is None else batches
    if heads is None:
        heads = range(cfg.H) if what == "q" else range(0, cfg.H, cfg.G)
    n = cfg.S if r == 1 else cfg.n[r - 1]   # capacity: ragged sequences are zero-padded
    out = np.zeros((len(batches), len(heads), n, cfg.d), np.float32)
    for bi, b in enumerate(batches):
        for hi, h in enumerate(heads):
            x = getattr(slices[(b, h)], what)[r - 1]
            out[bi, hi, :x.shape[0]] = x
    return out


def decode_queries(cfg: Config, layers=None, batches=None, heads=None) -> list[np.ndarray]:
    """Decode queries q^r [L][B][H][d] for r = 1..R (float32, dtype-exact).

    q^1 = cast(lam * N(0,1)), q^r = cast(q^{r-1} + lam * 0.5^r * N(0,1)) with one
    lognormal lam per (layer, b, h)."""
    layers = range(cfg.L) if layers is None else layers
    batches = range(cfg.B) if batches is None else batches
    heads = range(cfg.H) if heads is None else heads
    out = [np.zeros((len(layers), len(batches), len(heads), cfg.d), np.float32) for _ in range(cfg.R)]
    for li, l in enumerate(layers):
        for bi, b in enumerate(batches):
            for hi, h in enumerate(heads):
                lam = np.float32(1.0)
                if cfg.lognormal is not None:
                    lam = np.float32(_rng(cfg, _T_DEC_LAM, l, b, h).lognormal(0.0, cfg.lognormal))
                x = cast(lam * _rng(cfg, _T_DEC_Q, l, b, h).standard_normal(cfg.d, dtype=np.float32), cfg.dtype)
                out[0][li, bi, hi] = x
                for r in range(1, cfg.R):
                    step = np.float32(0.5 ** (r + 1))
                    dq = _rng(cfg, _T_DEC_DQ + r + 1, l, b, h).standard_normal(cfg.d, dtype=np.float32)
                    x = cast(x + (lam * step) * dq, cfg.dtype)
                    out[r][li, bi, hi] = x
    return out


def custom(name="custom", dtype="f32", B=1, H=1, d=64, S=64, R=4, act=(1.0, 0.5, 0.25, 0.125), col="0.25",
           bits=(8, 4, 4, 4), gamma=0.5, lognormal=None, seed=0, L=1, decode=False, Hkv=0, ragged=()) -> Config:
    """A small ad-hoc configuration (tests: ragged tails, edge cases)."""
    return Config(name, dtype, B, H, d, S, R, tuple(act), str(col), tuple(bits), gamma, lognormal, L, decode, seed,
                  Hkv, tuple(str(x) for x in ragged))


def gen_hidden(cfg: Config, b: int, D: int, r: int, moving) -> tuple[np.ndarray, np.ndarray]:
    """Synthetic hidden states of sequence b before and after loop r-1,
    [S, D] float32 rounded to the config dtype.  Tokens in `moving` (the
    active set of loop r-1) move by a relative step of lognormal size (median
    2 %, sigma 0.8) in a random direction; the others keep their state, as
    inactive tokens reuse theirs.  Row magnitudes are lognormal (sigma 0.5)."""
    S = cfg.S
    rng = _rng(cfg, _T_HID, b)
    h = rng.standard_normal((S, D)).astype(np.float32)
    h *= np.exp(0.5 * rng.standard_normal((S, 1))).astype(np.float32)
    h_prev = cast(h, cfg.dtype)
    moving = np.asarray(moving, np.int64)
    eps = 0.02 * np.exp(0.8 * _rng(cfg, _T_HID_EPS + 100 * r, b).standard_normal(moving.size))
    u = _rng(cfg, _T_HID_DIR + 100 * r, b).standard_normal((moving.size, D))
    u /= np.linalg.norm(u, axis=1, keepdims=True)
    step = (eps * np.linalg.norm(h_prev[moving].astype(np.float64), axis=1))[:, None] * u
    h_cur = h_prev.copy()
    h_cur[moving] = cast((h_prev[moving] + step).astype(np.float32), cfg.dtype)
    return h_prev, h_cur
