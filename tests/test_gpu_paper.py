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


def _paper_prefill_case(cfg, budgets, heads):
    """All loops of one layer over paper-format streams on the GPU; the oracle
    runs on the given heads with the GPU's selections forced (which must match
    its own up to near ties) and its own paper-format reconstructions."""
    import tests.gpu_harness as gh
    from oracle import prefill
    import sparse_attn_residual_amd as fl
    f32 = cfg.dtype == "f32"
    rows, slices = workloads.gen_batch(cfg)
    gpu = gh.run_prefill(cfg, rows, slices, K_budget=budgets, fmt=fl.FL_FMT_PAPER)
    tol = 1e-5 if f32 else 2e-3
    for b in range(cfg.B):
        for h in heads:
            s = slices[(b, h)]
            force = {r + 1: gpu["sel"][r][b, h] for r in range(1, cfg.R)}
            o = prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype=cfg.dtype,
                                      sel_force=force, fmt="paper")
            cand = np.arange(cfg.S)
            for r in range(cfg.R):
                if r >= 1:
                    m = o["mass"][r]
                    K = budgets[r - 1] if isinstance(budgets, list) else cfg.K
                    own = prefill.topk(m, cand, min(K, len(cand)))
                    ok, nd = gh.near_tie_ok(gpu["sel"][r][b, h], own, m, cand,
                                            (1e-5 if f32 else 2e-3) * gh.kth_key(m, K))
                    assert ok, (b, h, r + 1, nd)
                    cand = gpu["sel"][r][b, h]
                g, st = gpu["state"][r], o["state"][r]
                O = g["O"][b, h]
                if f32:
                    assert np.max(np.abs(O - st.O)) <= tol, (b, h, r + 1, np.max(np.abs(O - st.O)))
                else:
                    err = np.linalg.norm(O - st.O) / np.linalg.norm(st.O)
                    assert err <= tol, (b, h, r + 1, err)
    return gpu, rows, slices


@pytest.mark.parametrize("dtype,d,Hkv", [("f32", 128, 2), ("bf16", 128, 4)])
def test_paper_prefill(dtype, d, Hkv):
    """All loops of one layer over paper-format streams (pruning budgets):
    selections up to near ties, outputs within tolerance of the oracle run on
    the oracle's own paper-format reconstructions; the streams bit-exact."""
    f32 = dtype == "f32"
    cfg = workloads.custom(name="paper-prefill", dtype=dtype, B=2, H=4, d=d, S=1200, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.30", bits=(8, 4, 4, 4), lognormal=None if f32 else 0.5, seed=53, Hkv=Hkv)
    _say("paper prefill", cfg)
    gpu, rows, slices = _paper_prefill_case(cfg, [360, 180, 90], heads=(0, cfg.H - 1))
    check_streams(cfg, gpu["cache"], rows, slices)


def test_paper_prefill_full_size():
    """The 32K workload in the paper's cache format, in the launch
    configuration the benchmark times; oracle on two heads."""
    cfg = workloads.CONFIGS[2]
    _say("paper prefill full size", cfg.name)
    _paper_prefill_case(cfg, cfg.K, heads=(0, cfg.H - 1))


def _paper_decode_case(cfg):
    """Decode over paper-format streams (tail tokens included) against the
    oracle's decode step on the paper-format reconstructions, every head."""
    import tests.gpu_harness as gh
    import sparse_attn_residual_amd as fl
    from oracle import decode, prefill
    rows, slices = workloads.gen_batch(cfg)
    cache = gh.build_decode_cache(cfg, rows, slices, fmt=fl.FL_FMT_PAPER)
    qs = workloads.decode_queries(cfg)
    gpu = gh.run_decode(cfg, cache, qs)
    rel = cfg.dtype != "f32"
    tol = 2e-3 if rel else 1e-5
    for b in range(cfg.B):
        for h in range(cfg.H):
            s = slices[(b, h)]
            _, krec = pf.quantize_chain_paper(s.k, s.rows, "k")
            _, vrec = pf.quantize_chain_paper(s.v, s.rows, "v")
            for l in range(cfg.L):
                force = {r + 1: gpu[r]["sel"][l, b, h] for r in range(1, cfg.R)}
                orc = decode.decode_slice(krec, vrec, [q[l, b, h] for q in qs], cfg.K, sel_force=force)
                cand = np.arange(cfg.S)
                for r in range(cfg.R):
                    if r >= 1:
                        key = orc[r - 1]["logits"]
                        own = prefill.topk(key, cand, min(cfg.K, len(cand)))
                        ok, nd = gh.near_tie_ok(gpu[r]["sel"][l, b, h], own, key, cand, gh.LOGIT_TIE)
                        assert ok, (l, b, h, r + 1, nd)
                        cand = gpu[r]["sel"][l, b, h]
                    O, o = gpu[r]["O"][l, b, h], orc[r]["O"]
                    err = np.linalg.norm(O - o) / np.linalg.norm(o) if rel else np.max(np.abs(O - o))
                    assert err <= tol, (l, b, h, r + 1, err)


@pytest.mark.parametrize("dtype,Hkv", [("f32", 2), ("bf16", 4)])
def test_paper_decode(dtype, Hkv):
    """Decode over paper-format streams with grouped KV heads, two layers."""
    cfg = workloads.custom(name="paper-decode", dtype=dtype, B=2, H=4, d=128, S=900, R=4, act=(1, 0.3, 0.15, 0.08),
                           col="0.10", bits=(8, 4, 4, 4), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=55,
                           Hkv=Hkv)
    _say("paper decode", cfg)
    _paper_decode_case(cfg)


def test_paper_decode_full_shape():
    """The 48-layer decode workload's per-head shape (T = 32768, K = 3276,
    R = 4) in the paper's cache format, two heads of one layer and sequence."""
    import dataclasses
    cfg = dataclasses.replace(workloads.CONFIGS[3], name="paper-decode-full-shape", B=1, H=2, L=1)
    _say("paper decode full shape", cfg)
    _paper_decode_case(cfg)
