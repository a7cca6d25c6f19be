"""GPU parity of fl_loop_decode with the CPU oracle's decode step."""
import numpy as np
import pytest

import workloads
from oracle import decode, prefill, quant

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _decode_case(cfg, tol, rel):
    import tests.gpu_harness as gh
    rows, slices = workloads.gen_batch(cfg)
    cache = gh.build_decode_cache(cfg, rows, slices)
    qs = workloads.decode_queries(cfg)
    gpu = gh.run_decode(cfg, cache, qs)
    for b in range(cfg.B):
        for h in range(cfg.H):
            s = slices[(b, h)]
            _, krec = quant.quantize_chain(s.k, s.rows, list(cfg.bits))
            _, vrec = quant.quantize_chain(s.v, s.rows, list(cfg.bits))
            for l in range(cfg.L):
                force = {r + 1: gpu[r]["sel"][l, b, h] for r in range(1, cfg.R)}
                orc = decode.decode_slice(krec, vrec, [q[l, b, h] for q in qs], cfg.K, sel_force=force)
                cand = np.arange(cfg.S)
                # loop 2's selection from the GPU's own loop-1 logits: bit-exact
                exact = prefill.topk(gpu[0]["logits"][l, b, h].astype(np.float64), cand, min(cfg.K, cfg.S))
                assert np.array_equal(gpu[1]["sel"][l, b, h], exact), (l, b, h, "loop-2 selection from its logits")
                for r in range(cfg.R):
                    g = {k: gpu[r][k][l, b, h] for k in ("O", "U", "M", "lse")}
                    o = orc[r]
                    if r >= 1:
                        key = orc[r - 1]["logits"]
                        own = prefill.topk(key, cand, min(cfg.K, len(cand)))
                        ok, nd = gh.near_tie_ok(gpu[r]["sel"][l, b, h], own, key, cand, gh.LOGIT_TIE)
                        assert ok, (l, b, h, r + 1, nd)
                        cand = gpu[r]["sel"][l, b, h]
                    lg = gpu[r]["logits"][l, b, h]
                    assert np.max(np.abs(lg - o["logits"])) <= 1e-4 * max(1.0, np.max(np.abs(o["logits"])))
                    if rel:
                        err = np.linalg.norm(g["O"] - o["O"]) / np.linalg.norm(o["O"])
                        assert err <= tol, (l, b, h, r + 1, err)
                    else:
                        assert np.max(np.abs(g["O"] - o["O"])) <= tol, (l, b, h, r + 1)
                    assert abs(g["lse"] - o["lse"]) <= tol, (l, b, h, r + 1, "lse")
                    assert abs(g["M"] - o["M"]) <= tol, (l, b, h, r + 1, "M")
                    assert np.max(np.abs(g["U"] - o["U"])) <= tol * max(1.0, np.max(np.abs(o["O"])))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_small(dtype):
    cfg = workloads.custom(name="decode-small", dtype=dtype, B=2, H=2, d=128, S=1000, R=4, act=(1, 0.3, 0.15, 0.08),
                           col="0.10", bits=(8, 4, 4, 2), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=1)
    _say("decode", dtype, cfg)
    _decode_case(cfg, 1e-5, rel=False)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("S,act,col", [
    (64, (1, "0.02", "0.02", "0.02"), "0.02"),   # one tile of context, one residual row, one selected column
    (65, (1, "0.5", "0.25", "0.02"), "0.02"),    # a tile and one position of context, one selected column
    (130, (1, 1, 1, 1), "1"),                    # every position selected at every loop
    (1, (1, 1, 1, 1), "1"),                      # a single token
])
def test_decode_degenerate(dtype, S, act, col):
    """Degenerate decode problems: a context of one token, one tile or one
    tile and one position, a selection of one column (K_r = 1), residual
    chains of a single token, and loops that keep every position."""
    cfg = workloads.custom(name="decode-degenerate", dtype=dtype, B=2, H=2, d=128, S=S, R=4, act=act, col=col,
                           bits=(8, 4, 4, 2), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=42)
    _say("decode degenerate", dtype, S, cfg.n, cfg.K)
    if dtype == "f32":
        _decode_case(cfg, 1e-5, rel=False)
    else:
        _decode_case(cfg, 2e-3, rel=True)


def test_decode_pruned_every_loop():
    """Budgets that shrink every loop exercise the reuse update at r >= 3."""
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="decode-prune", dtype="f32", B=1, H=2, d=128, S=777, R=4, act=(1, 0.5, 0.3, 0.2),
                           col="0.3", bits=(8, 4, 2, 4), lognormal=0.5, L=1, decode=True, seed=2)
    _say("decode prune", cfg)
    rows, slices = workloads.gen_batch(cfg)
    cache = gh.build_decode_cache(cfg, rows, slices)
    qs = workloads.decode_queries(cfg)
    budgets = [None, 233, 120, 61]
    import sparse_attn_residual_amd as fl
    import torch
    st = fl.DecodeState(cfg.L, cfg.B, cfg.H, cfg.S, cfg.d)
    K_prev = cfg.S
    snaps = []
    for r in range(1, cfg.R + 1):
        K = cfg.S if r == 1 else budgets[r - 1]
        fl.fl_loop_decode(cache.fl, r, gh.upload(qs[r - 1], cfg), fl.FL_F32, K_prev, K, st.fl)
        torch.cuda.synchronize()
        snaps.append(dict(O=st.O.cpu().numpy(), M=st.M.cpu().numpy(), sel=st.sel[..., :K].cpu().numpy()))
        K_prev = K
    for h in range(cfg.H):
        s = slices[(0, h)]
        _, krec = quant.quantize_chain(s.k, s.rows, list(cfg.bits))
        _, vrec = quant.quantize_chain(s.v, s.rows, list(cfg.bits))
        T = cfg.S
        # the oracle with the same per-loop budgets
        force = {r + 1: snaps[r]["sel"][0, 0, h] for r in range(1, cfg.R)}
        orc = decode.decode_slice(krec, vrec, [q[0, 0, h] for q in qs], 10 ** 9, sel_force=force)
        for r in range(cfg.R):
            assert np.max(np.abs(snaps[r]["O"][0, 0, h] - orc[r]["O"])) <= 1e-5, (h, r + 1)
            assert abs(snaps[r]["M"][0, 0, h] - orc[r]["M"]) <= 1e-5


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_deep_loops(dtype):
    """Seven loops: residual loops past the batched slot lookups, and a
    selection spanning many 64-token chunks with a ragged last one."""
    cfg = workloads.custom(name="decode-deep", dtype=dtype, B=1, H=2, d=128, S=1500, R=7,
                           act=(1, 0.6, 0.45, 0.3, 0.2, 0.12, 0.07), col="0.47", bits=(8, 4, 2, 4, 2, 4, 2),
                           gamma=0.5, lognormal=0.5, L=1, decode=True, seed=4)
    _say("decode deep", dtype, cfg)
    _decode_case(cfg, 1e-5 if dtype == "f32" else 2e-3, rel=dtype != "f32")


def test_decode_full_shape():
    """The 48-layer decode workload's per-head shape (T = 32768, K = 3276,
    R = 4, bits 8/4/4/2) on two heads of one layer and sequence."""
    import dataclasses
    cfg = dataclasses.replace(workloads.CONFIGS[3], name="decode-full-shape", B=1, H=2, L=1)
    _say("decode full shape", cfg)
    _decode_case(cfg, 2e-3, rel=True)


@pytest.mark.parametrize("dtype,H,Hkv", [("f32", 4, 2), ("bf16", 6, 2), ("bf16", 8, 2), ("f32", 8, 1)])
def test_decode_gqa(dtype, H, Hkv):
    """Grouped-query attention: each query head reads its KV head's packed
    records and selects its own columns."""
    cfg = workloads.custom(name="decode-gqa", dtype=dtype, B=2, H=H, d=128, S=900, R=4, act=(1, 0.3, 0.15, 0.08),
                           col="0.10", bits=(8, 4, 4, 2), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=6, Hkv=Hkv)
    _say("decode gqa", dtype, cfg)
    _decode_case(cfg, 1e-5 if dtype == "f32" else 2e-3, rel=dtype != "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_ragged_counts(dtype):
    """Sequences with different active-row counts share one cache (n_r is the
    capacity, per-sequence counts bound the residual streams)."""
    cfg = workloads.custom(name="decode-ragged", dtype=dtype, B=3, H=2, d=128, S=800, R=4, act=(1, 0.4, 0.2, 0.1),
                           col="0.10", bits=(8, 4, 2, 4), gamma=0.5, lognormal=0.5, L=1, decode=True, seed=8,
                           ragged=(0.3, 1, 0.65))
    _say("decode ragged", dtype, cfg)
    _decode_case(cfg, 1e-5 if dtype == "f32" else 2e-3, rel=dtype != "f32")


def _check_decode(cfg, gpu, slices, qs, T, tol, rel, K_budget=None):
    """Decode outputs of every (layer, b, h) against the oracle over the first
    T cached tokens, teacher-forced with the GPU's selections, which must
    match the oracle's own up to near ties of the logits."""
    import tests.gpu_harness as gh
    K_budget = cfg.K if K_budget is None else K_budget
    for b in range(cfg.B):
        for h in range(cfg.H):
            s = slices[(b, h)]
            _, krec = quant.quantize_chain(s.k, s.rows, list(cfg.bits))
            _, vrec = quant.quantize_chain(s.v, s.rows, list(cfg.bits))
            krec, vrec = [x[:T] for x in krec], [x[:T] for x in vrec]
            for l in range(cfg.L):
                force = {r + 1: gpu[r]["sel"][l, b, h] for r in range(1, cfg.R)}
                orc = decode.decode_slice(krec, vrec, [q[l, b, h] for q in qs], K_budget, sel_force=force)
                cand = np.arange(T)
                for r in range(cfg.R):
                    if r >= 1:
                        key = orc[r - 1]["logits"]
                        own = prefill.topk(key, cand, min(K_budget, len(cand)))
                        ok, nd = gh.near_tie_ok(gpu[r]["sel"][l, b, h], own, key, cand, gh.LOGIT_TIE)
                        assert ok, (l, b, h, r + 1, nd)
                        cand = gpu[r]["sel"][l, b, h]
                    O, o = gpu[r]["O"][l, b, h], orc[r]["O"]
                    err = np.linalg.norm(O - o) / np.linalg.norm(o) if rel else np.max(np.abs(O - o))
                    assert err <= tol, (l, b, h, r + 1, err)
                    assert abs(gpu[r]["lse"][l, b, h] - orc[r]["lse"]) <= tol * max(1.0, abs(orc[r]["lse"]))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_partial_context(dtype):
    """A cache with room for S positions decoding over its first T < S
    (fl_cache.T): the dense loop, the top-K and the sparse loops see only
    positions below T."""
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="decode-partial", dtype=dtype, B=2, H=2, d=128, S=700, R=4, act=(1, 0.4, 0.2, 0.1),
                           col="0.10", bits=(8, 4, 2, 4), gamma=0.5, lognormal=0.5, L=1, decode=True, seed=14)
    T = 513
    _say("decode partial context", dtype, T, cfg)
    rows, slices = workloads.gen_batch(cfg)
    cache = gh.build_decode_cache(cfg, rows, slices)
    qs = workloads.decode_queries(cfg)
    gpu = gh.run_decode(cfg, cache, qs, T=T)
    _check_decode(cfg, gpu, slices, qs, T, 1e-5 if dtype == "f32" else 2e-3, rel=dtype != "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_append(dtype):
    """The token being decoded, appended loop by loop with fl_kv_append to a
    cache of the earlier tokens, gives byte for byte the cache fl_kv_resq
    builds for all tokens (base, residual records, rows, slots, counts), and
    decoding over it matches the oracle.  Grouped heads, two layers."""
    import torch
    import sparse_attn_residual_amd as fl
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="decode-append", dtype=dtype, B=2, H=4, d=128, S=640, R=4, act=(1, 0.4, 0.2, 0.1),
                           col="0.10", bits=(8, 4, 2, 4), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=12, Hkv=2)
    S, R, B, L = cfg.S, cfg.R, cfg.B, cfg.L
    _say("decode append", dtype, cfg)
    last = np.array([S - 1], np.int32)
    rows_full = {b: [np.union1d(x, last).astype(np.int32) for x in workloads.active_rows(cfg, b)] for b in range(B)}
    slices = {(b, h): workloads.gen_slice(cfg, b, h, rows_full[b]) for b in range(B) for h in range(cfg.H)}
    cnt_full = [np.array([len(rows_full[b][r]) for b in range(B)], np.int32) for r in range(R)]
    cap = [int(c.max()) for c in cnt_full]

    def padded(rws):
        return [np.stack([np.concatenate([rws[b][r], np.full(cap[r] - len(rws[b][r]), rws[b][r][-1], np.int32)])
                          for b in range(B)]) for r in range(R)]

    def stack(r, what):
        out = np.zeros((B, cfg.kv_heads, cap[r - 1] if r > 1 else S, cfg.d), np.float32)
        for b in range(B):
            for hk in range(cfg.kv_heads):
                x = getattr(slices[(b, hk * cfg.G)], what)[r - 1]
                out[b, hk, :x.shape[0]] = x
        return out

    def build(rws, counts, drop_last):
        cache = fl.CacheBuffers(L, B, cfg.H, S, cfg.d, R, cap, cfg.bits, padded(rws), Hkv=cfg.kv_heads, counts=counts)
        for layer in range(L):
            view = cache.layer_view(layer)
            for r in range(1, R + 1):
                k, v = stack(r, "k"), stack(r, "v")
                if drop_last and r == 1:
                    k[:, :, S - 1] = 0.0
                    v[:, :, S - 1] = 0.0
                fl.fl_kv_resq(view, r, gh.upload(k, cfg), gh.upload(v, cfg), gh.fl_dtype(cfg))
        torch.cuda.synchronize()
        return cache

    full = build(rows_full, cnt_full, False)
    rows_pre = {b: [rows_full[b][0]] + [x[:-1] for x in rows_full[b][1:]] for b in range(B)}
    cnt_pre = [cnt_full[0]] + [c - 1 for c in cnt_full[1:]]
    app = build(rows_pre, cnt_pre, True)
    for r in range(1, R + 1):
        x = {w: np.zeros((L, B, cfg.kv_heads, cfg.d), np.float32) for w in ("k", "v")}
        for w in ("k", "v"):
            st = stack(r, w)
            for b in range(B):
                t = S - 1 if r == 1 else cnt_full[r - 1][b] - 1
                x[w][:, b] = st[b, :, t][None]
        fl.fl_kv_append(app.fl, r, S - 1, gh.upload(x["k"], cfg), gh.upload(x["v"], cfg), gh.fl_dtype(cfg))
    torch.cuda.synchronize()
    assert np.array_equal(app.base.cpu().numpy(), full.base.cpu().numpy())
    for r in range(2, R + 1):
        assert np.array_equal(app.cnt[r - 1].cpu().numpy(), full.cnt[r - 1].cpu().numpy()), r
        ra, rf = app.res_records(r).cpu().numpy(), full.res_records(r).cpu().numpy()
        sa, sf = app.rows[r - 1].cpu().numpy(), full.rows[r - 1].cpu().numpy()
        for b in range(B):
            c = cnt_full[r - 1][b]
            assert np.array_equal(ra[:, b, :, :c], rf[:, b, :, :c]), (r, b)
            assert np.array_equal(sa[b, :c], sf[b, :c]), (r, b)
        assert np.array_equal(app.slot[r - 1].cpu().numpy(), full.slot[r - 1].cpu().numpy()), r
    qs = workloads.decode_queries(cfg)
    ga = gh.run_decode(cfg, app, qs)
    gf = gh.run_decode(cfg, full, qs)
    for r in range(R):
        for key in ("O", "lse", "M"):
            assert np.array_equal(ga[r][key], gf[r][key]), (r + 1, key)
    _check_decode(cfg, ga, slices, qs, S, 1e-5 if dtype == "f32" else 2e-3, rel=dtype != "f32")


def _full_launch_cache_and_queries():
    """The 48-layer decode workload exactly as the benchmark times it: the
    cache quantized sequence by sequence through fl_kv_resq, layer 0 copied to
    every layer, and the per-layer queries."""
    import tests.gpu_harness as gh
    cfg = workloads.CONFIGS[3]
    cache = gh.build_decode_cache_per_sequence(cfg)
    qs = workloads.decode_queries(cfg)
    return cfg, cache, qs


def test_decode_full_launch_sampled():
    """The full 48-layer launch (L = 48, B = 16, H = 16, T = 32768: the
    12288-problem top-K and the decode grids the benchmark times) compared
    with the oracle on sampled (layer, sequence, head) slices, and repeated
    bit for bit."""
    import torch
    import tests.gpu_harness as gh
    cfg, cache, qs = _full_launch_cache_and_queries()
    _say("decode full launch", cfg.name)
    runs = [gh.run_decode_device(cfg, cache, qs) for _ in range(2)]
    for r in range(cfg.R):
        for key in ("O", "U", "M", "lse", "logits", "sel"):
            a, b = runs[0][r][key], runs[1][r][key]
            if a is None:
                continue
            assert torch.equal(a, b), (r + 1, key, "repeat run differs")
    picks = [(0, 0, 0), (47, 15, 15), (17, 3, 9), (30, 8, 4), (5, 12, 13), (41, 6, 2)]
    snaps = [{k: (v.cpu().numpy() if v is not None else None) for k, v in run.items()} for run in runs[0]]
    by_b = {}
    for l, b, h in picks:
        by_b.setdefault(b, []).append((l, h))
    for b, lh in sorted(by_b.items()):
        _, sl = workloads.gen_batch(cfg, batches=[b], heads=sorted({h for _, h in lh}), with_q=False)
        for l, h in lh:
            s = sl[(b, h)]
            _, krec = quant.quantize_chain(s.k, s.rows, list(cfg.bits))
            _, vrec = quant.quantize_chain(s.v, s.rows, list(cfg.bits))
            force = {r + 1: snaps[r]["sel"][l, b, h] for r in range(1, cfg.R)}
            orc = decode.decode_slice(krec, vrec, [q[l, b, h] for q in qs], cfg.K, sel_force=force)
            cand = np.arange(cfg.S)
            exact = prefill.topk(snaps[0]["logits"][l, b, h].astype(np.float64), cand, cfg.K)
            assert np.array_equal(snaps[1]["sel"][l, b, h], exact), (l, b, h, "loop-2 selection from its logits")
            for r in range(cfg.R):
                if r >= 1:
                    key = orc[r - 1]["logits"]
                    own = prefill.topk(key, cand, min(cfg.K, len(cand)))
                    ok, nd = gh.near_tie_ok(snaps[r]["sel"][l, b, h], own, key, cand, gh.LOGIT_TIE)
                    assert ok, (l, b, h, r + 1, nd)
                    cand = snaps[r]["sel"][l, b, h]
                O, o = snaps[r]["O"][l, b, h], orc[r]["O"]
                err = np.linalg.norm(O - o) / np.linalg.norm(o)
                print(f"[parity] decode l={l} b={b} h={h} loop={r + 1} O_rel={err:.2e} "
                      f"dlse={abs(snaps[r]['lse'][l, b, h] - orc[r]['lse']):.2e} "
                      f"dM={abs(snaps[r]['M'][l, b, h] - orc[r]['M']):.2e}", flush=True)
                assert err <= 2e-3, (l, b, h, r + 1, "O", err)
                assert abs(snaps[r]["lse"][l, b, h] - orc[r]["lse"]) <= 2e-3, (l, b, h, r + 1, "lse")
                assert abs(snaps[r]["M"][l, b, h] - orc[r]["M"]) <= 2e-3, (l, b, h, r + 1, "M")
                lg = snaps[r]["logits"][l, b, h]
                assert np.max(np.abs(lg - orc[r]["logits"])) <= 1e-4 * max(1.0, np.max(np.abs(orc[r]["logits"])))
    del cache, runs
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,T,ties", [("f32", 2500, False), ("bf16", 4096, True), ("f32", 2048, True)])
def test_decode_selection_from_loop1_histogram(dtype, T, ties):
    """Loop 2's selection starts from the histogram the dense loop leaves in
    the selection rows (caches of at least 2048 positions): over a partial
    context (T < S) and with logits made to tie (every loop-1 key repeated
    over four consecutive positions, so equal records give equal logits), it
    equals the oracle's top-K of the GPU's own loop-1 logits exactly (ties
    to the lower position), and the outputs match the oracle."""
    import torch
    import sparse_attn_residual_amd as fl
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="decode-hist", dtype=dtype, B=2, H=2, d=128, S=4096, R=3, act=(1, 0.4, 0.2),
                           col="0.10", bits=(8, 4, 2), gamma=0.5, lognormal=0.5, L=2, decode=True, seed=17)
    _say("decode selection from the loop-1 histogram", dtype, T, ties)
    rows, slices = workloads.gen_batch(cfg)
    if ties:
        for s in slices.values():
            s.k[0] = s.k[0][(np.arange(cfg.S) // 4) * 4].copy()
    cache = gh.build_decode_cache(cfg, rows, slices)
    qs = workloads.decode_queries(cfg)
    gpu = gh.run_decode(cfg, cache, qs, T=T)
    K = min(cfg.K, T)
    n_ties = 0
    for l in range(cfg.L):
        for b in range(cfg.B):
            for h in range(cfg.H):
                lg = gpu[0]["logits"][l, b, h][:T].astype(np.float64)
                exact = prefill.topk(lg, np.arange(T), K)
                assert np.array_equal(gpu[1]["sel"][l, b, h], exact), (l, b, h)
                kth = np.sort(lg)[::-1][K - 1]
                n_ties += int(np.sum(lg == kth) > 1)
    if ties:
        assert n_ties > 0, "the tie case produced no tie at the threshold"
    _check_decode(cfg, gpu, slices, qs, T, 1e-5 if dtype == "f32" else 2e-3, rel=dtype != "f32")


@pytest.mark.parametrize("pattern", ["plain", "groups", "equal"])
def test_decode_selection_full_problem(pattern):
    """Loop 2's selection on problems of exactly 32768 keys (the top-K kernel
    variant without per-key range masks): plain logits, logits tied in
    groups of four consecutive positions, and every logit equal (the whole
    problem in one bin down to the last level, the first K positions taken).
    The selection equals the oracle's top-K of the GPU's own loop-1 logits,
    ties to the lower position, and the outputs match the oracle."""
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="decode-full-problem", dtype="bf16", B=1, H=2, d=128, S=32768, R=2, act=(1, 0.3),
                           col="0.10", bits=(8, 4), gamma=0.5, lognormal=0.5, L=1, decode=True, seed=29)
    _say("decode selection on 32768-key problems", pattern)
    rows, slices = workloads.gen_batch(cfg)
    for sl in slices.values():
        if pattern == "groups":
            sl.k[0] = sl.k[0][(np.arange(cfg.S) // 4) * 4].copy()
        elif pattern == "equal":
            sl.k[0] = np.repeat(sl.k[0][:1], cfg.S, axis=0)
    cache = gh.build_decode_cache(cfg, rows, slices)
    qs = workloads.decode_queries(cfg)
    gpu = gh.run_decode(cfg, cache, qs)
    for h in range(cfg.H):
        lg = gpu[0]["logits"][0, 0, h].astype(np.float64)
        exact = prefill.topk(lg, np.arange(cfg.S), cfg.K)
        assert np.array_equal(gpu[1]["sel"][0, 0, h], exact), (pattern, h)
        if pattern == "equal":
            assert np.all(lg == lg[0]) and np.array_equal(exact, np.arange(cfg.K))
    _check_decode(cfg, gpu, slices, qs, cfg.S, 2e-3, rel=True)

