"""GPU parity of the paper's own cache format (fl_cache.fmt = FL_FMT_PAPER):
the quantized streams bit for bit against the oracle's codes, scales, zeros
and bf16 tail, then the prefill path over them."""
import numpy as np
import pytest

import workloads
from oracle import paper_format as pf

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _nibbles(b):
    return np.stack([b & 15, b >> 4], axis=-1).reshape(*b.shape[:-1], b.shape[-1] * 2)


def unpack_stream(buf, m):
    """One stream's bytes -> codes, scales and zeros of keys and values, and
    the bf16 tail as float32 (the layout the cache header documents)."""
    nb = -(-m // 64)
    rec = buf[:m * 144].reshape(m, 144)
    km = buf[m * 144:m * 144 + nb * 512].view(np.float16).reshape(nb, 2, 128)
    tail = buf[m * 144 + nb * 512:m * 144 + nb * 512 + 64 * 512].view(np.uint16).reshape(64, 2, 128)
    tail = (tail.astype(np.uint32) << 16).view(np.float32)
    vm = rec[:, 128:136].copy().view(np.float16).reshape(m, 2, 2)
    return dict(kc=_nibbles(rec[:, :64]), vc=_nibbles(rec[:, 64:128]), ks=km[:, 0], kz=km[:, 1],
                vs=vm[:, :, 0], vz=vm[:, :, 1], tail=tail)


def build_paper_cache(cfg, rows, slices):
    import torch
    import sparse_attn_residual_amd as fl
    import tests.gpu_harness as gh
    cache = fl.CacheBuffers(1, cfg.B, cfg.H, cfg.S, cfg.d, cfg.R, cfg.n, cfg.bits, gh.rows_list(cfg, rows),
                            Hkv=cfg.kv_heads, counts=gh.counts_list(cfg), fmt=fl.FL_FMT_PAPER)
    for r in range(1, cfg.R + 1):
        k = gh.upload(workloads.stack_loop(cfg, slices, r, "k"), cfg)
        v = gh.upload(workloads.stack_loop(cfg, slices, r, "v"), cfg)
        fl.fl_kv_resq(cache.fl, r, k, v, gh.fl_dtype(cfg))
    torch.cuda.synchronize()
    return cache


def check_streams(cfg, cache, rows, slices):
    Sq = max(0, cfg.S - pf.TAIL)
    for r in range(1, cfg.R + 1):
        got = cache.streams(r).cpu().numpy()
        m = Sq if r == 1 else cfg.n[r - 1]
        for b in range(cfg.B):
            for hk in range(cfg.kv_heads):
                s = slices[(b, hk * cfg.G)]
                g = unpack_stream(got[0, b, hk], m)
                for kind, cc, sc, zc in (("k", "kc", "ks", "kz"), ("v", "vc", "vs", "vz")):
                    st, _ = pf.quantize_chain_paper(getattr(s, kind), s.rows, kind)
                    o = st[r - 1]
                    n_body = Sq if r == 1 else len(o["rows"])
                    if n_body:
                        assert np.array_equal(g[cc][:n_body], o["codes"]), (r, b, hk, kind, "codes")
                        nsc = o["scale"].shape[0]
                        assert np.array_equal(g[sc][:nsc].view(np.uint16), o["scale"].view(np.uint16)), (r, b, hk, kind)
                        assert np.array_equal(g[zc][:nsc].view(np.uint16), o["zero"].view(np.uint16)), (r, b, hk, kind)
                    tpos = np.arange(Sq, cfg.S) if r == 1 else o["tail_rows"]
                    kv = 0 if kind == "k" else 1
                    assert np.array_equal(g["tail"][tpos - Sq, kv], o["tail"]), (r, b, hk, kind, "tail")


@pytest.mark.parametrize("dtype,S,Hkv,ragged", [("f32", 1000, 2, ()), ("bf16", 1000, 4, ()), ("bf16", 700, 2, (1, 0.6)),
                                                ("f32", 50, 2, ())])
def test_paper_streams_bitexact(dtype, S, Hkv, ragged):
    cfg = workloads.custom(name="paper-streams", dtype=dtype, B=2, H=4, d=128, S=S, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.25", bits=(8, 4, 4, 4), lognormal=0.5, seed=51, Hkv=Hkv, ragged=ragged)
    _say("paper streams", cfg)
    rows, slices = workloads.gen_batch(cfg)
    cache = build_paper_cache(cfg, rows, slices)
    check_streams(cfg, cache, rows, slices)
