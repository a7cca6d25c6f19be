"""Checkpoint and resume: the loop state is everything a later loop reads (the
packed cache with its row and slot maps, O, U, M, lse, the previous loop's
selection and, for decode, the stored logits).  Stopping after loop r,
copying that state to the host, restoring it into freshly allocated device
buffers and running the remaining loops gives the same bits as running all
loops without a stop."""
import numpy as np
import pytest
import torch

import workloads
import tests.gpu_harness as gh

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _host(t):
    return None if t is None else t.detach().cpu().numpy().copy()


def _fill(dst, src):
    if dst is not None:
        dst.copy_(torch.from_numpy(src).to(dst.device))


def _new_cache(cfg, rows_l, fmt=0, L=1):
    import sparse_attn_residual_amd as fl
    return fl.CacheBuffers(L, cfg.B, cfg.H, cfg.S, cfg.d, cfg.R, cfg.n, cfg.bits, rows_l, Hkv=cfg.kv_heads,
                           counts=gh.counts_list(cfg), fmt=fmt)


def _cache_to_host(c):
    return dict(base=_host(c.base), res=[_host(x) for x in c.res], rows=[_host(x) for x in c.rows],
                slot=[_host(x) for x in c.slot], cnt=[_host(x) for x in c.cnt])


def _cache_from_host(c, h):
    _fill(c.base, h["base"])
    for key in ("res", "rows", "slot", "cnt"):
        for dst, src in zip(getattr(c, key), h[key]):
            if src is not None:
                _fill(dst, src)


def _prefill_loops(cfg, slices, cache, st, qs, budgets, r0, r1, sel_prev, K_prev):
    """Loops r0..r1 of one layer (the steps of gpu_harness.run_prefill)."""
    import sparse_attn_residual_amd as fl
    dt = gh.fl_dtype(cfg)
    out = {}
    for r in range(r0, r1 + 1):
        k = gh.upload(workloads.stack_loop(cfg, slices, r, "k"), cfg)
        v = gh.upload(workloads.stack_loop(cfg, slices, r, "v"), cfg)
        fl.fl_kv_resq(cache.fl, r, k, v, dt)
        sel, K, mass = None, 0, None
        if r >= 2:
            K = min(budgets[r - 2], K_prev)
            sel = torch.empty(cfg.B, cfg.H, K, dtype=torch.int32, device=gh.DEV)
            mass = torch.empty(cfg.B, cfg.H, K_prev, dtype=torch.float32, device=gh.DEV)
            nws = fl.fl_workspace_bytes(fl.FL_WS_COLSEL, cache.fl, r, K_prev, K)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=gh.DEV)
            fl.fl_colsel(cache.fl, r, qs[r - 2], dt, st.fl, K_prev, sel_prev, K, None, mass, sel, ws, nws)
        nws = fl.fl_workspace_bytes(fl.FL_WS_ATTN, cache.fl, r, K, K)
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=gh.DEV)
        fl.fl_loop_attn(cache.fl, r, qs[r - 1], dt, K, sel, st.fl, ws, nws)
        torch.cuda.synchronize()
        out[r] = dict(state={k2: v2.cpu().numpy() for k2, v2 in st.snapshot().items()},
                      sel=None if sel is None else sel.cpu().numpy(), mass=None if mass is None else mass.cpu().numpy())
        if r >= 2:
            sel_prev, K_prev = sel, K
    return out, sel_prev, K_prev


@pytest.mark.parametrize("dtype,cut,mixed", [("bf16", 1, False), ("bf16", 2, False), ("bf16", 3, True),
                                             ("f32", 2, False)])
def test_prefill_resume_bit_identical(dtype, cut, mixed):
    import sparse_attn_residual_amd as fl
    cfg = workloads.custom(name="prefill-resume", dtype=dtype, B=2, H=2, d=128 if dtype == "bf16" else 64, S=1300,
                           R=4, act=(1, 0.5, 0.3, 0.15), col="0.30", bits=(8, 4, 2, 4),
                           lognormal=0.5 if dtype == "bf16" else None, seed=41, ragged=(1, 0.7))
    budgets = [390, 200, 90]
    _say("prefill resume", dtype, "cut after loop", cut, "mixed" if mixed else "", cfg)
    rows, slices = workloads.gen_batch(cfg, heads=None)
    rows_l = gh.rows_list(cfg, rows)
    qs = [gh.upload(workloads.stack_loop(cfg, slices, r, "q"), cfg) for r in range(1, cfg.R + 1)]
    # uninterrupted
    cache = _new_cache(cfg, rows_l)
    st = fl.PrefillState(cfg.B, cfg.H, cfg.S, cfg.d, mixed=mixed)
    full, _, _ = _prefill_loops(cfg, slices, cache, st, qs, budgets, 1, cfg.R, None, cfg.S)
    del cache, st
    # stopped after loop `cut`, state copied out, restored into new buffers
    cache = _new_cache(cfg, rows_l)
    st = fl.PrefillState(cfg.B, cfg.H, cfg.S, cfg.d, mixed=mixed)
    _, sel_prev, K_prev = _prefill_loops(cfg, slices, cache, st, qs, budgets, 1, cut, None, cfg.S)
    hc = _cache_to_host(cache)
    hs = {k: _host(v) for k, v in st.snapshot().items()}
    hsel = _host(sel_prev)
    cache2 = _new_cache(cfg, rows_l)      # allocated while the first still lives: other addresses
    st2 = fl.PrefillState(cfg.B, cfg.H, cfg.S, cfg.d, mixed=mixed)
    del cache, st, sel_prev
    torch.cuda.synchronize()
    _cache_from_host(cache2, hc)
    for k, v in hs.items():
        _fill(getattr(st2, k), v)
    sel2 = None if hsel is None else torch.from_numpy(hsel).to(gh.DEV)
    rest, _, _ = _prefill_loops(cfg, slices, cache2, st2, qs, budgets, cut + 1, cfg.R, sel2, K_prev)
    for r in range(cut + 1, cfg.R + 1):
        for k in full[r]["state"]:
            assert np.array_equal(full[r]["state"][k], rest[r]["state"][k]), (r, k)
        if r >= 2:
            assert np.array_equal(full[r]["sel"], rest[r]["sel"]), (r, "sel")
            assert np.array_equal(full[r]["mass"], rest[r]["mass"]), (r, "mass")


@pytest.mark.parametrize("cut", [1, 2])
def test_decode_resume_bit_identical(cut):
    import sparse_attn_residual_amd as fl
    cfg = workloads.custom(name="decode-resume", dtype="bf16", B=2, H=2, d=128, S=1000, R=4, act=(1, 0.3, 0.15, 0.08),
                           col="0.10", bits=(8, 4, 4, 2), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=43)
    _say("decode resume", "cut after loop", cut, cfg)
    rows, slices = workloads.gen_batch(cfg)
    qs = workloads.decode_queries(cfg)
    cache = gh.build_decode_cache(cfg, rows, slices)
    full = gh.run_decode(cfg, cache, qs)
    dt = gh.fl_dtype(cfg)
    T = cfg.S

    def loops(cache_, st_, r0, r1, K_prev):
        snaps = {}
        for r in range(r0, r1 + 1):
            q = gh.upload(qs[r - 1], cfg)
            K = T if r == 1 else min(cfg.K, K_prev)
            fl.fl_loop_decode(cache_.fl, r, q, dt, K_prev, K, st_.fl)
            torch.cuda.synchronize()
            snaps[r] = dict(O=_host(st_.O), U=_host(st_.U), M=_host(st_.M), lse=_host(st_.lse),
                            logits=_host(st_.logits[..., :K]), sel=_host(st_.sel[..., :K]) if r > 1 else None)
            K_prev = K
        return snaps, K_prev

    st = fl.DecodeState(cfg.L, cfg.B, cfg.H, cfg.S, cfg.d)
    cache.fl.T = T
    _, K_prev = loops(cache, st, 1, cut, T)
    hc = _cache_to_host(cache)
    hs = {k: _host(getattr(st, k)) for k in ("O", "U", "M", "lse", "logits", "sel")}
    rows_l = gh.rows_list(cfg, rows)
    cache2 = _new_cache(cfg, rows_l, L=cfg.L)
    st2 = fl.DecodeState(cfg.L, cfg.B, cfg.H, cfg.S, cfg.d)
    del st
    _cache_from_host(cache2, hc)
    for k, v in hs.items():
        _fill(getattr(st2, k), v)
    cache2.fl.T = T
    rest, _ = loops(cache2, st2, cut + 1, cfg.R, K_prev)
    for r in range(cut + 1, cfg.R + 1):
        g = full[r - 1]
        for k in ("O", "U", "M", "lse", "logits"):
            assert np.array_equal(g[k], rest[r][k]), (r, k)
        assert np.array_equal(g["sel"], rest[r]["sel"]), (r, "sel")
