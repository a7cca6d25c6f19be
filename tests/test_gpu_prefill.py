"""GPU parity of the prefill path (fl_kv_resq, fl_colsel, fl_loop_attn) with
the CPU oracle, through the C ABI."""
import numpy as np
import pytest

import workloads
from oracle import prefill, records

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _oracle_slices(cfg, rows, slices, gpu, heads, combine="mass"):
    """Oracle per (b, h), teacher-forced with the GPU's selections."""
    res = {}
    for b in range(cfg.B):
        for h in heads:
            s = slices[(b, h)]
            force = {r + 1: gpu["sel"][r][b, h] for r in range(1, cfg.R)}
            res[(b, h)] = prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits,
                                                dtype=cfg.dtype, sel_force=force, combine=combine)
    return res


def _check_records(cfg, gpu, orc, heads):
    cache = gpu["cache"]
    base = cache.base_records().cpu().numpy()
    for b in range(cfg.B):
        for h in heads:
            o = orc[(b, h)]
            hk = h // cfg.G   # the streams are per KV head
            ks, vs = o["k_streams"], o["v_streams"]
            want = records.pack_base(ks[0]["codes"], ks[0]["scale"], vs[0]["codes"], vs[0]["scale"])
            assert np.array_equal(base[0, b, hk], want), (b, h, "base")
            for r in range(2, cfg.R + 1):
                got = cache.res_records(r).cpu().numpy()[0, b, hk]
                k, v = ks[r - 1], vs[r - 1]
                want = records.pack_residual(k["codes"], k["scale"], k["zero"], v["codes"], v["scale"], v["zero"],
                                             cfg.bits[r - 1])
                got = got[:want.shape[0]]   # a ragged sequence fills the first |A_r| records
                assert np.array_equal(got, want), (b, h, r)


def _kth_mass(mass, K):
    """The K-th largest candidate mass (the selection threshold)."""
    K = min(K, mass.shape[0])
    return float(np.partition(np.asarray(mass, np.float64), mass.shape[0] - K)[mass.shape[0] - K])


def _row_errors(g, ref):
    """Per-row 2-norm of the error and of the reference."""
    return np.linalg.norm(g - ref, axis=1), np.linalg.norm(ref, axis=1)


def _check_outputs(cfg, gpu, orc, heads, tol, rel, budgets=None):
    """Outputs of every loop against the oracle, teacher-forced.

    bf16 (rel): over the rows loop r recomputes (A_r; every row at loop 1):
    ||dO||_F / ||O||_F <= tol, and every recomputed row within tol of its own
    norm, floored at the median recomputed row's norm (rows whose output
    nearly cancels are held to the typical row's scale); U in the same class;
    lse to tol absolute (a relative error of the softmax normalizer); M to tol
    (M is a probability mass).  fp32: max-abs <= tol everywhere.  Both: rows
    outside A_r keep loop r-1's state bit for bit; the column mass within tol
    of max(c_j, c_K), c_K the K-th largest mass (the selection threshold)."""
    for b in range(cfg.B):
        act = workloads.active_rows(cfg, b)
        for h in heads:
            o = orc[(b, h)]
            for r in range(cfg.R):
                g = gpu["state"][r]
                st = o["state"][r]
                A = np.arange(cfg.S) if r == 0 else np.asarray(act[r], np.int64)
                Og, Oo = g["O"][b, h][A], st.O[A]
                lse_o, lse_g = st.lse[A], g["lse"][b, h][A]
                fin = np.isfinite(lse_o)
                assert np.array_equal(fin, np.isfinite(lse_g)), (b, h, r + 1, "lse finite")
                dlse = float(np.max(np.abs(lse_g[fin] - lse_o[fin]), initial=0.0))
                dM = float(np.max(np.abs(g["M"][b, h][A] - st.M[A])))
                if rel:
                    frob = np.linalg.norm(Og - Oo) / np.linalg.norm(Oo)
                    en, on = _row_errors(Og, Oo)
                    floor = np.median(on)
                    row = en / np.maximum(on, floor)
                    uf = np.linalg.norm(g["U"][b, h][A] - st.U[A]) / np.linalg.norm(Oo)
                    mabs = np.max(np.abs(Og - Oo)) / np.max(np.abs(Oo))
                    print(f"[parity] b={b} h={h} loop={r + 1} rows={A.size} O_frob={frob:.2e} O_row_max={row.max():.2e} "
                          f"O_row_p999={np.quantile(row, 0.999):.2e} maxabs/max|O|={mabs:.2e} U_frob={uf:.2e} "
                          f"dlse={dlse:.2e} dM={dM:.2e}", flush=True)
                    assert frob <= tol, (b, h, r + 1, "O", frob)
                    assert row.max() <= tol, (b, h, r + 1, "O per row", row.max(), int(np.argmax(row)))
                    assert uf <= tol, (b, h, r + 1, "U", uf)
                    assert dlse <= tol, (b, h, r + 1, "lse", dlse)
                    assert dM <= tol, (b, h, r + 1, "M", dM)
                else:
                    for key, ref in (("O", st.O), ("U", st.U)):
                        e = np.max(np.abs(g[key][b, h] - ref))
                        assert e <= tol, (b, h, r + 1, key, e)
                    assert dlse <= tol, (b, h, r + 1, "lse", dlse)
                    assert np.max(np.abs(g["M"][b, h] - st.M)) <= tol, (b, h, r + 1, "M")
                if r >= 1:
                    # rows outside A_r are never touched: loop r-1's state stays
                    out = np.ones(cfg.S, bool)
                    out[A] = False
                    prev = gpu["state"][r - 1]
                    for key in ("O", "U", "M", "lse"):
                        assert np.array_equal(g[key][b, h][out], prev[key][b, h][out]), (b, h, r + 1, key, "untouched")
                    m_or = o["mass"][r]
                    m_g = gpu["mass"][r][b, h]
                    K = (budgets[r - 1] if budgets else cfg.K)
                    thr = _kth_mass(m_or, K)
                    # relative to max(c_j, c_K); where both are zero (a row set
                    # that sees none of the candidates) only an exact zero agrees
                    den = np.maximum(np.abs(m_or), thr)
                    dif = np.abs(m_g - m_or)
                    em = float(np.max(np.where(den > 0, dif / np.where(den > 0, den, 1.0),
                                               np.where(dif > 0, np.inf, 0.0)), initial=0.0))
                    print(f"[parity] b={b} h={h} loop={r + 1} mass_err/max(c,c_K)={em:.2e} c_K={thr:.3e}", flush=True)
                    assert em <= tol, (b, h, r + 1, "mass", em)


@pytest.mark.parametrize("cfgid", [0])
def test_prefill_fp32_parity(cfgid):
    import tests.gpu_harness as gh
    cfg = workloads.CONFIGS[cfgid]
    _say("prefill parity", cfg.name)
    rows, slices = workloads.gen_batch(cfg)
    gpu = gh.run_prefill(cfg, rows, slices)
    heads = list(range(cfg.H))
    orc = _oracle_slices(cfg, rows, slices, gpu, heads)
    _check_records(cfg, gpu, orc, heads)
    # teacher forcing is only allowed over near ties
    for b in range(cfg.B):
        for h in heads:
            s = slices[(b, h)]
            cand = np.arange(cfg.S)
            for r in range(1, cfg.R):
                m = orc[(b, h)]["mass"][r]
                own = prefill.topk(m, cand, min(cfg.K, len(cand)))
                ok, ndiff = gh.near_tie_ok(gpu["sel"][r][b, h], own, m, cand, 1e-5 * _kth_mass(m, cfg.K))
                assert ok, (b, h, r + 1, ndiff)
                cand = gpu["sel"][r][b, h]
    _check_outputs(cfg, gpu, orc, heads, 1e-5, rel=False)


def test_topk_bitexact_with_mass_in():
    """Given the same fp32 masses, the GPU selection equals the oracle's."""
    import tests.gpu_harness as gh
    cfg = workloads.custom(dtype="f32", B=2, H=3, d=64, S=700, R=2, act=(1, 0.4), col="0.13", bits=(8, 4))
    _say("topk mass_in", cfg)
    rows, slices = workloads.gen_batch(cfg)
    rng = np.random.default_rng(0)
    # masses with many exact ties (quantized values) exercise the tie rule
    mass = (np.round(rng.random((cfg.B, cfg.H, cfg.S)) * 64) / 64).astype(np.float32)
    gpu = gh.run_prefill(cfg, rows, slices, mass_in={2: mass})
    for b in range(cfg.B):
        for h in range(cfg.H):
            want = prefill.topk(mass[b, h].astype(np.float64), np.arange(cfg.S), cfg.K)
            assert np.array_equal(gpu["sel"][1][b, h], want), (b, h)


@pytest.mark.parametrize("bits,d", [((8, 2, 4, 2), 64), ((8, 4, 2, 4, 2), 64)])
def test_prefill_fp32_ragged(bits, d):
    """Sizes that leave ragged tails everywhere, 2- and 4-bit residuals."""
    import tests.gpu_harness as gh
    R = len(bits)
    act = tuple([1.0, 0.55, 0.4, 0.23, 0.11][:R])
    cfg = workloads.custom(dtype="f32", B=2, H=2, d=d, S=333, R=R, act=act, col="0.17", bits=bits, lognormal=0.5,
                           seed=3)
    _say("prefill ragged", cfg)
    rows, slices = workloads.gen_batch(cfg)
    gpu = gh.run_prefill(cfg, rows, slices)
    heads = list(range(cfg.H))
    orc = _oracle_slices(cfg, rows, slices, gpu, heads)
    _check_records(cfg, gpu, orc, heads)
    _check_outputs(cfg, gpu, orc, heads, 1e-5, rel=False)


def test_prefill_deterministic():
    import tests.gpu_harness as gh
    cfg = workloads.CONFIGS[0]
    _say("determinism", cfg.name)
    rows, slices = workloads.gen_batch(cfg)
    a = gh.run_prefill(cfg, rows, slices)
    b = gh.run_prefill(cfg, rows, slices)
    for r in range(cfg.R):
        for k in ("O", "U", "M", "lse"):
            assert np.array_equal(a["state"][r][k], b["state"][r][k]), (r, k)
    for r in range(1, cfg.R):
        assert np.array_equal(a["sel"][r], b["sel"][r])
        assert np.array_equal(a["mass"][r], b["mass"][r])


def test_prefill_mfma_deterministic_full_size():
    """The 32K workload twice through the matrix-core kernels (every loop, in
    the launch configuration the benchmark times): states, selections and
    masses are equal bit for bit."""
    import tests.gpu_harness as gh
    cfg = workloads.CONFIGS[2]
    _say("determinism full size", cfg.name)
    rows, slices = workloads.gen_batch(cfg)
    a = gh.run_prefill(cfg, rows, slices)
    b = gh.run_prefill(cfg, rows, slices)
    for r in range(cfg.R):
        for k in ("O", "U", "M", "lse"):
            assert np.array_equal(a["state"][r][k], b["state"][r][k]), (r + 1, k)
    for r in range(1, cfg.R):
        assert np.array_equal(a["sel"][r], b["sel"][r]), r + 1
        assert np.array_equal(a["mass"][r], b["mass"][r]), r + 1


def _bf16_case(cfg, heads, sel_eps=2e-3, budgets=None, tol=2e-3, rel=True, combine="mass", check=True):
    """budgets: optional per-loop K (loop r uses budgets[r-2]); the oracle is
    teacher-forced with the GPU's selections, which must match its own up to
    near ties of the masses."""
    import tests.gpu_harness as gh
    rows, slices = workloads.gen_batch(cfg, heads=None)
    gpu = gh.run_prefill(cfg, rows, slices, K_budget=list(budgets) if budgets else None, mixed=combine == "mixed")
    orc = _oracle_slices(cfg, rows, slices, gpu, heads, combine=combine)
    _check_records(cfg, gpu, orc, heads)
    for b in range(cfg.B):
        for h in heads:
            cand = np.arange(cfg.S)
            for r in range(1, cfg.R):
                m = orc[(b, h)]["mass"][r]
                K = budgets[r - 1] if budgets else cfg.K
                own = prefill.topk(m, cand, min(K, len(cand)))
                ok, ndiff = gh.near_tie_ok(gpu["sel"][r][b, h], own, m, cand, sel_eps * _kth_mass(m, K))
                assert ok, (b, h, r + 1, ndiff)
                cand = gpu["sel"][r][b, h]
    if check:
        _check_outputs(cfg, gpu, orc, heads, tol, rel=rel, budgets=budgets)
    return gpu, orc


@pytest.mark.parametrize("S,bits,col", [(777, (8, 4, 4, 2), "0.10"), (1300, (8, 2, 4, 4), "0.33")])
def test_prefill_bf16_mfma_small(S, bits, col):
    cfg = workloads.custom(name="bf16-small", dtype="bf16", B=2, H=2, d=128, S=S, R=4, act=(1, 0.3, 0.15, 0.08),
                           col=col, bits=bits, lognormal=0.5, seed=5)
    _say("prefill bf16 mfma", cfg)
    _bf16_case(cfg, heads=[0, 1])


@pytest.mark.parametrize("cfgid,heads", [(1, [0, 11]), (2, [0, 15]), (4, [3])])
def test_prefill_bf16_full_size(cfgid, heads):
    """Full-size workloads (all heads on the GPU, the launch configuration the
    benchmark times for the 32K one), oracle on sampled heads."""
    cfg = workloads.CONFIGS[cfgid]
    _say("prefill full size", cfg.name, heads)
    _bf16_case(cfg, heads=heads)


@pytest.mark.parametrize("act", [(1, 0.5, 0.1253, 0.125), (1, 0.50025, 0.2505, 0.12525)])
def test_prefill_split_boundaries(act):
    """Sparse launches on both sides of the column-split thresholds (16 heads,
    S = 4096): loops of 2048, 513 and 512 active rows (two splits exactly at
    their limit, two splits, four exactly at theirs) and of 2049, 1026 and 513
    (no split one row past the limit, two, two); with a pruning schedule the
    cached-mass passes take the same launch rule."""
    cfg = workloads.custom(name="split-bounds", dtype="bf16", B=1, H=16, d=128, S=4096, R=4, act=act, col="0.10",
                           bits=(8, 4, 4, 2), lognormal=0.5, seed=51)
    _say("prefill split boundaries", cfg.n, cfg)
    _bf16_case(cfg, heads=[0, 15], budgets=[409, 300, 200])


def test_prefill_bf16_mfma_wide():
    """Enough heads that the 384-row block kernels run: the 48-row one in
    the dense loop and the twelve-wave one in loop 2, with ragged row blocks
    and a ragged last tile; loops 3 and 4 take the four-wave kernel."""
    cfg = workloads.custom(name="bf16-wide", dtype="bf16", B=4, H=64, d=128, S=1000, R=4, act=(1, 0.9, 0.6, 0.3),
                           col="0.25", bits=(8, 4, 2, 4), lognormal=0.5, seed=7)
    _say("prefill bf16 wide", cfg)
    _bf16_case(cfg, heads=[0, 37, 63])


def _keys(pattern, shape, rng):
    x = rng.standard_normal(shape)
    if pattern == "ties8":
        x = np.round(x * 8) / 8
    elif pattern == "binary":
        x = (rng.random(shape) < 0.5).astype(np.float64)
    elif pattern == "equal":
        x = np.full(shape, 0.5)
    elif pattern == "lognormal-wide":
        x = np.exp(5.0 * x)
    elif pattern == "inf":
        x[..., ::97] = np.inf
        x[..., 5::89] = -np.inf
    elif pattern == "signed-zero":
        x = np.where(rng.random(shape) < 0.6, np.where(rng.random(shape) < 0.5, -0.0, 0.0), x)
    return x.astype(np.float32)


@pytest.mark.parametrize("S,col", [(9000, "0.10"), (32768, "0.10"), (32768, "0.0001")])
@pytest.mark.parametrize("pattern", ["normal", "ties8", "binary", "equal", "lognormal-wide", "inf", "signed-zero"])
def test_topk_key_patterns(S, col, pattern):
    """Selections from given keys equal the oracle's exactly: the value-binned
    first stage, its exact resolution of the threshold bin, and the radix
    fallback (non-finite keys, one over-full bin, all keys equal)."""
    import tests.gpu_harness as gh
    cfg = workloads.custom(dtype="f32", B=1, H=2, d=64, S=S, R=2, act=(1, 0.3), col=col, bits=(8, 4), seed=11)
    _say("topk keys", pattern, S, cfg.K)
    rows, slices = workloads.gen_batch(cfg)
    mass = _keys(pattern, (cfg.B, cfg.H, cfg.S), np.random.default_rng(S + len(pattern)))
    gpu = gh.run_prefill(cfg, rows, slices, mass_in={2: mass})
    for h in range(cfg.H):
        want = prefill.topk(mass[0, h].astype(np.float64), np.arange(cfg.S), cfg.K)
        assert np.array_equal(gpu["sel"][1][0, h], want), (pattern, h)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_prefill_pruned_every_loop(dtype, d):
    """Budgets that shrink every loop (K_r < K_{r-1}): the column mass over
    the previous selection's tiles, top-K with a candidate list, and the
    cached-mass pass at loops 3 and 4 against loop r-1's chains."""
    # fp32 inputs keep unit row norms: with lognormal norms the logits reach
    # about 48 here, and fp32 rounding of the logits alone (in any fp32
    # implementation) moves O by about 2.4e-5, above the 1e-5 bound
    cfg = workloads.custom(name="prefill-prune", dtype=dtype, B=2, H=3, d=d, S=1700, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.40", bits=(8, 4, 2, 4), lognormal=0.5 if dtype == "bf16" else None, seed=9)
    _say("prefill pruned", dtype, cfg)
    if dtype == "bf16":
        _bf16_case(cfg, heads=[0, 2], budgets=[680, 350, 140])
    else:
        _bf16_case(cfg, heads=[0, 1, 2], sel_eps=1e-5, budgets=[680, 350, 140], tol=1e-5, rel=False)


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128)])
def test_prefill_vector_path_other_dims(dtype, d):
    """bf16 at head dim 64 and fp32 at head dim 128 take the vector-ALU
    kernels (the matrix-core ones take bf16 at d = 128): every loop with
    pruning budgets against the oracle."""
    f32 = dtype == "f32"
    cfg = workloads.custom(name="prefill-vector", dtype=dtype, B=2, H=2, d=d, S=1100, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.40", bits=(8, 4, 2, 4), lognormal=None if f32 else 0.5, seed=41)
    _say("prefill vector path", dtype, d, cfg)
    _bf16_case(cfg, heads=[0, 1], sel_eps=1e-5 if f32 else 2e-3, budgets=[440, 220, 90], tol=1e-5 if f32 else 2e-3,
               rel=not f32)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
@pytest.mark.parametrize("S,act,col", [
    (64, (1, "0.02", "0.02", "0.02"), "0.02"),   # one tile; one active row and one selected column per loop
    (65, (1, "0.5", "0.25", "0.02"), "0.02"),    # a tile and one position; one selected column
    (130, (1, 1, 1, 1), "1"),                    # every row and every column at every loop
    (1, (1, 1, 1, 1), "1"),                      # a single token
])
def test_prefill_degenerate(dtype, d, S, act, col):
    """Degenerate sizes of the method: a single active row (n_r = 1), a
    single selected column (K_r = 1, so most rows have no selected column at
    or before them and keep loop r-1's state), a sequence of one token, one
    tile or one tile and one position, and loops that keep every row and
    column (the cached mass is one and the reused part zero)."""
    f32 = dtype == "f32"
    cfg = workloads.custom(name="degenerate", dtype=dtype, B=2, H=2, d=d, S=S, R=4, act=act, col=col,
                           bits=(8, 4, 4, 2), lognormal=0.5, seed=41)
    _say("prefill degenerate", cfg.name, dtype, d, S, cfg.n, cfg.K)
    _bf16_case(cfg, heads=[0, 1], sel_eps=1e-5 if f32 else 2e-3, tol=1e-5 if f32 else 2e-3, rel=not f32)


def test_prefill_pruned_full_size():
    """The 32K-token workload with a budget that shrinks every loop
    (3277 -> 2000 -> 1000 columns), all heads on the GPU, oracle on two."""
    cfg = workloads.CONFIGS[2]
    _say("prefill pruned full size", cfg.name)
    _bf16_case(cfg, heads=[0, 15], budgets=[cfg.K, 2000, 1000])


def test_prefill_dense_second_loop():
    """Loops 1 and 2 dense (every candidate column kept at loop 2), then a
    pruned loop 3: with J_i all of i's causal columns the cached mass is one
    and the reused part vanishes, so loop 2 is exact dense attention over the
    rows it recomputes."""
    cfg = workloads.custom(name="prefill-dense2", dtype="bf16", B=1, H=4, d=128, S=2500, R=3, act=(1, 0.6, 0.3),
                           col="0.20", bits=(8, 4, 4), lognormal=0.5, seed=13)
    _say("prefill dense loop 2", cfg)
    gpu, orc = _bf16_case(cfg, heads=[0, 3], budgets=[cfg.S, cfg.K])
    act = workloads.active_rows(cfg, 0)[1]
    for h in (0, 3):
        g = gpu["state"][1]
        assert np.max(np.abs(g["M"][0, h][act] - 1.0)) <= 1e-5
        U, O = g["U"][0, h][act], g["O"][0, h][act]
        assert np.linalg.norm(U) <= 2e-3 * np.linalg.norm(O), np.linalg.norm(U) / np.linalg.norm(O)


@pytest.mark.parametrize("dtype,d,budgets", [("f32", 64, (680, 350, 140)), ("f32", 64, (680, 680, 300)),
                                             ("bf16", 128, (680, 350, 140)), ("bf16", 128, (680, 680, 300))])
def test_prefill_mixed_combine(dtype, d, budgets):
    """The exact mixed-logit combine (ablation): O, lse, M, U and the loop
    r-1 log-sum-exp over the selected columns, against the oracle's mixed
    rule; pruning loops and an unpruned loop (lsel copied from lse)."""
    cfg = workloads.custom(name="prefill-mixed", dtype=dtype, B=2, H=3, d=d, S=1700, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.40", bits=(8, 4, 2, 4), lognormal=0.5 if dtype == "bf16" else None, seed=21)
    _say("prefill mixed combine", dtype, budgets, cfg)
    f32 = dtype == "f32"
    tol = 1e-5 if f32 else 2e-3
    gpu, orc = _bf16_case(cfg, heads=[0, 2], sel_eps=1e-5 if f32 else 2e-3, budgets=list(budgets), tol=tol,
                          rel=not f32, combine="mixed", check=f32)
    rows = {b: workloads.active_rows(cfg, b) for b in range(cfg.B)}
    for b in range(cfg.B):
        for h in (0, 2):
            o = orc[(b, h)]
            w = np.ones(cfg.S)
            for r in range(1, cfg.R):
                g = gpu["state"][r]
                st = o["state"][r]
                U = g["U"][b, h]
                rr = rows[b][r]
                if f32:
                    assert np.max(np.abs(U - st.U)) <= tol, (b, h, r + 1, "U")
                else:
                    # The reused part U^r is formed by a cancellation (O^(r-1)
                    # minus the selected columns' share) with the bf16/fp16
                    # operands' error, which the mass-rescaled rule passes on
                    # unscaled; the mixed rule divides it by D_i (the oracle's
                    # denominator), and loop r inherits loop r-1's error through
                    # O^(r-1), so rows are compared with weights
                    # prod_{t <= r} max(1, 1/D^t_i).
                    w[rr] *= np.maximum(1.0, 1.0 / o["denom"][r])
                    for key, ref in (("O", st.O), ("U", st.U)):
                        e = np.linalg.norm((g[key][b, h] - ref) / w[:, None])
                        assert e <= tol * np.linalg.norm(st.O), (b, h, r + 1, key, e / np.linalg.norm(st.O))
                    assert np.max(np.abs(g["M"][b, h] - st.M) / w) <= 4 * tol, (b, h, r + 1, "M")
                    # Rows whose combine never divided by D < 1 carry no
                    # amplification: there the plain bar holds, over the rows
                    # and per row (floored at the median row norm).
                    good = rr[w[rr] == 1.0]
                    if good.size:
                        Og, Oo = g["O"][b, h][good], st.O[good]
                        frob = np.linalg.norm(Og - Oo) / np.linalg.norm(Oo)
                        en, on = _row_errors(Og, Oo)
                        row = en / np.maximum(on, np.median(on))
                        print(f"[parity] mixed b={b} h={h} loop={r + 1} unamplified rows={good.size}/{rr.size} "
                              f"O_frob={frob:.2e} O_row_max={row.max():.2e}", flush=True)
                        assert frob <= tol and row.max() <= tol, (b, h, r + 1, "O unamplified", frob, row.max())
                    fin = np.isfinite(st.lse)
                    assert np.array_equal(fin, np.isfinite(g["lse"][b, h]))
                    # lse is loop r's log-sum-exp over the selection: no division by D
                    assert np.max(np.abs(g["lse"][b, h][fin] - st.lse[fin])) <= tol, (b, h, r + 1, "lse")
                want, got = o["lsel"][r], g["lsel"][b, h][rr]
                fin = np.isfinite(want)
                assert np.array_equal(fin, np.isfinite(got)), (b, h, r + 1)
                err = np.max(np.abs(got[fin] - want[fin])) if fin.any() else 0.0
                # (fp32: relative to the log-sum-exp's size, the precision a float keeps)
                lim = tol * max(1.0, np.max(np.abs(want[fin]), initial=0.0)) if f32 else tol
                assert err <= lim, (b, h, r + 1, "lsel", err)


@pytest.mark.parametrize("dtype,d,H,Hkv", [("f32", 64, 4, 2), ("bf16", 128, 6, 2), ("bf16", 128, 4, 1)])
def test_prefill_gqa(dtype, d, H, Hkv):
    """Grouped-query attention: H query heads read Hkv key/value heads; the
    streams are per KV head, loop 1's tiles are built once per KV head, every
    other step is per query head (pruning budgets)."""
    f32 = dtype == "f32"
    cfg = workloads.custom(name="prefill-gqa", dtype=dtype, B=2, H=H, d=d, S=1300, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.30", bits=(8, 4, 2, 4), lognormal=None if f32 else 0.5, seed=31, Hkv=Hkv)
    _say("prefill gqa", cfg)
    heads = sorted({0, min(H // Hkv, H - 1), H - 1})
    _bf16_case(cfg, heads=heads, sel_eps=1e-5 if f32 else 2e-3, budgets=[390, 200, 90], tol=1e-5 if f32 else 2e-3,
               rel=not f32)


def test_prefill_gqa_full_size():
    """The 32K workload with 4 KV heads for its 16 query heads, in the launch
    configuration the benchmark times; oracle on one query head of each of two
    KV groups."""
    cfg = workloads.CONFIGS[2].with_(Hkv=4)
    _say("prefill gqa full size", cfg.name, cfg.kv_heads)
    _bf16_case(cfg, heads=[0, 7])


@pytest.mark.parametrize("dtype,d,ragged", [("f32", 64, (1, 0.55, 0.3)), ("bf16", 128, (0.4, 1, 0.7))])
def test_prefill_ragged_counts(dtype, d, ragged):
    """A batch whose sequences keep different numbers of active rows (a
    per-sequence count array; n_r is the capacity): records, selections and
    outputs per sequence against the oracle; pruning budgets."""
    f32 = dtype == "f32"
    cfg = workloads.custom(name="prefill-ragged", dtype=dtype, B=3, H=2, d=d, S=1100, R=4, act=(1, 0.5, 0.3, 0.15),
                           col="0.30", bits=(8, 4, 2, 4), lognormal=None if f32 else 0.5, seed=41, ragged=ragged)
    _say("prefill ragged", cfg, [cfg.counts(b) for b in range(cfg.B)])
    _bf16_case(cfg, heads=[0, 1], sel_eps=1e-5 if f32 else 2e-3, budgets=[330, 170, 80], tol=1e-5 if f32 else 2e-3,
               rel=not f32)


def test_fl_check_validator(monkeypatch):
    """FL_CHECK=1, the synchronous validator: valid index data gives results
    bit-identical to an unchecked run; rows that are unsorted or not nested,
    a count outside its bounds and an unsorted selection are refused with
    FL_EINVAL before anything is written.  Every corrupted array keeps its
    positions inside [0, S), so no access could leave its buffer even if the
    check were missing."""
    import torch
    import sparse_attn_residual_amd as fl
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="fl-check", dtype="bf16", B=2, H=2, d=128, S=777, R=4, act=(1, 0.3, 0.15, 0.08),
                           col="0.10", bits=(8, 4, 4, 2), lognormal=0.5, seed=5, ragged=(1, 0.6))
    _say("FL_CHECK validator", cfg)
    rows, slices = workloads.gen_batch(cfg)
    monkeypatch.delenv("FL_CHECK", raising=False)
    a = gh.run_prefill(cfg, rows, slices)
    monkeypatch.setenv("FL_CHECK", "1")
    b = gh.run_prefill(cfg, rows, slices)
    for r in range(cfg.R):
        for k in ("O", "U", "M", "lse"):
            assert np.array_equal(a["state"][r][k], b["state"][r][k]), (r + 1, k)
    cache = b["cache"]
    st = fl.PrefillState(cfg.B, cfg.H, cfg.S, cfg.d)
    for k in ("O", "U", "M", "lse"):
        getattr(st, k).copy_(torch.from_numpy(b["state"][3][k]).cuda())
    before = {k: v.clone() for k, v in st.snapshot().items()}
    K = cfg.K
    sel = torch.from_numpy(b["sel"][3]).cuda().contiguous()
    nws = fl.fl_workspace_bytes(fl.FL_WS_ATTN, cache.fl, 4, K, K)
    ws = torch.empty(max(nws, 16), dtype=torch.uint8, device="cuda")
    q4 = b["q"][3]

    def refused(call, what):
        with pytest.raises(fl.FlashLoopError) as ei:
            call()
        assert ei.value.status == 1 and "FL_CHECK" in str(ei.value), (what, str(ei.value))
        torch.cuda.synchronize()
        for k, v in st.snapshot().items():
            assert torch.equal(v, before[k]), (what, k)

    attn4 = lambda: fl.fl_loop_attn(cache.fl, 4, q4, fl.FL_BF16, K, sel, st.fl, ws, nws)  # noqa: E731
    # loop-4 rows of sequence 0 not ascending
    rw = cache.rows[3]
    keep = rw.clone()
    rw[0, 1], rw[0, 2] = keep[0, 2], keep[0, 1]
    refused(attn4, "unsorted rows")
    rw.copy_(keep)
    # loop-4 rows not inside loop 3's set (sorted, in range)
    in3 = set(cache.rows[2][0, :cfg.counts(0)[2]].tolist())
    outside = next(j for j in range(cfg.S) if j not in in3)
    vals = sorted(set(keep[0, :cfg.counts(0)[3]].tolist()[1:]) | {outside})
    rw[0, :len(vals)] = torch.tensor(vals, dtype=torch.int32, device="cuda")
    refused(attn4, "rows not nested")
    rw.copy_(keep)
    # a count of zero
    cnt = cache.cnt[3]
    keep_c = cnt.clone()
    cnt[1] = 0
    refused(attn4, "zero count")
    cnt.copy_(keep_c)
    # a loop-4 count above loop 3's
    cnt[1] = min(cfg.n[3], int(cache.cnt[2][1].item()) + 1)
    if int(cnt[1].item()) > int(cache.cnt[2][1].item()):
        refused(attn4, "count above the previous loop's")
    cnt.copy_(keep_c)
    # selection not ascending
    keep_s = sel.clone()
    sel[1, 0, 3], sel[1, 0, 4] = keep_s[1, 0, 4], keep_s[1, 0, 3]
    refused(attn4, "unsorted selection")
    sel.copy_(keep_s)
    # the untouched data passes again, and the refused calls wrote nothing
    attn4()
    torch.cuda.synchronize()
    assert torch.equal(st.O, torch.from_numpy(b["state"][3]["O"]).cuda())


@pytest.mark.parametrize("B,H", [(1, 2), (2, 128)])
def test_prefill_bf16_values_beyond_fp16(B, H):
    """Values whose bf16 reconstructions exceed fp16's range (|v~| up to
    ~6e5, inside the int8 base's fp16-scale range) take the matrix-core
    path's per-tile V shift.  Head 0 has every value's loop-1 part scaled by
    2^17, the other heads only the positions below 300, so tiles with and
    without a shift meet in one row; the loop-to-loop changes keep their size
    (a residual's fp16 zero bounds them by 65504).  Outputs are finite and
    within the bf16 bar of the oracle.  With 2 x 128 heads the dense loop runs
    on the 48-row kernel."""
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="bf16-large-v", dtype="bf16", B=B, H=H, d=128, S=900, R=4, act=(1, 0.4, 0.2, 0.1),
                           col="0.20", bits=(8, 4, 4, 2), lognormal=0.5, seed=29)
    _say("prefill bf16 large values", cfg)
    rows, slices = workloads.gen_batch(cfg)
    big = np.float32(2.0 ** 17)
    for (b, h), s in slices.items():
        v1 = s.v[0].copy()
        for r in range(cfg.R):
            pos = s.rows[r]
            sel = np.ones(pos.shape[0], bool) if h == 0 else pos < 300
            # loop r's value plus (2^17 - 1) times its loop-1 value, rounded to bf16
            s.v[r][sel] = workloads.cast(s.v[r][sel] + (big - 1) * v1[pos[sel]], "bf16")
    assert max(np.max(np.abs(s.v[0])) for s in slices.values()) > 65504
    gpu = gh.run_prefill(cfg, rows, slices)
    heads = [0, 1]
    orc = _oracle_slices(cfg, rows, slices, gpu, heads)
    _check_records(cfg, gpu, orc, heads)
    for r in range(cfg.R):
        assert np.all(np.isfinite(gpu["state"][r]["O"])), r + 1
    for h in heads:
        cand = np.arange(cfg.S)
        for r in range(1, cfg.R):
            m = orc[(0, h)]["mass"][r]
            own = prefill.topk(m, cand, min(cfg.K, len(cand)))
            ok, nd = gh_near_tie(gpu["sel"][r][0, h], own, m, cand, 2e-3 * _kth_mass(m, cfg.K))
            assert ok, (h, r + 1, nd)
            cand = gpu["sel"][r][0, h]
    _check_outputs(cfg, gpu, orc, heads, 2e-3, rel=True)


def gh_near_tie(*a):
    import tests.gpu_harness as gh
    return gh.near_tie_ok(*a)


def test_kernel_timer_records_launches():
    """The library's kernel timer: with it on, every launch of a prefill
    step is recorded (name and a positive duration) in launch order; off, no
    record is kept."""
    import sparse_attn_residual_amd as fl
    import tests.gpu_harness as gh
    cfg = workloads.custom(name="timer", dtype="bf16", B=1, H=2, d=128, S=640, R=2, act=(1, 0.3), col="0.10",
                           bits=(8, 4), lognormal=0.5, seed=2)
    rows, slices = workloads.gen_batch(cfg)
    fl.fl_timing_collect()
    fl.fl_timing_enable(True)
    try:
        gh.run_prefill(cfg, rows, slices)
        recs = fl.fl_timing_collect()
    finally:
        fl.fl_timing_enable(False)
    names = [n for n, _ in recs]
    _say("kernel timer", names)
    assert names[0].startswith("k_quant_base") and any(n.startswith("k_attn_mfma") for n in names), names
    assert any(n.startswith("k_mass_mfma") for n in names) and any(n.startswith("k_topk") for n in names), names
    assert all(t > 0 for _, t in recs), recs
    gh.run_prefill(cfg, rows, slices)
    assert fl.fl_timing_collect() == []


@pytest.mark.parametrize("cfgid", [None, 4])
def test_prefill_tile_sources_agree(monkeypatch, cfgid):
    """The sparse loops' attention from tile images built once per loop (the
    default) and from tiles each row block builds in LDS (FL_TILES=lds, the
    measured alternative) both match the oracle; a small case and the deep
    16K R = 8 workload.  Loop 1 and the selections do not depend on the
    source and agree bit for bit (the image path splits small launches'
    columns across waves, so its sparse-loop sums are ordered differently)."""
    import tests.gpu_harness as gh
    if cfgid is None:
        cfg = workloads.custom(name="tile-src", dtype="bf16", B=2, H=2, d=128, S=1300, R=4, act=(1, 0.3, 0.15, 0.08),
                               col="0.15", bits=(8, 4, 2, 4), lognormal=0.5, seed=33)
        heads = [0, 1]
    else:
        cfg = workloads.CONFIGS[cfgid]
        heads = [5]
    _say("tile sources", cfg.name)
    rows, slices = workloads.gen_batch(cfg, heads=None)
    runs = {}
    for src in ("images", "lds"):
        monkeypatch.setenv("FL_TILES", src)
        runs[src] = gh.run_prefill(cfg, rows, slices)
    monkeypatch.delenv("FL_TILES")
    a, b = runs["images"], runs["lds"]
    for k in ("O", "U", "M", "lse"):
        assert np.array_equal(a["state"][0][k], b["state"][0][k]), (1, k)
    for r in range(1, cfg.R):
        assert np.array_equal(a["sel"][r], b["sel"][r]), r + 1
    for run in (a, b):
        orc = _oracle_slices(cfg, rows, slices, run, heads)
        _check_outputs(cfg, run, orc, heads, 2e-3, rel=True)
