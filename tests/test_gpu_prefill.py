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


def _check_outputs(cfg, gpu, orc, heads, tol, rel):
    for b in range(cfg.B):
        for h in heads:
            o = orc[(b, h)]
            for r in range(cfg.R):
                g = gpu["state"][r]
                st = o["state"][r]
                O = g["O"][b, h]
                if rel:
                    err = np.linalg.norm(O - st.O) / np.linalg.norm(st.O)
                    assert err <= tol, (b, h, r + 1, "O", err)
                    fin = np.isfinite(st.lse)
                    assert np.array_equal(fin, np.isfinite(g["lse"][b, h]))
                    assert np.max(np.abs(g["lse"][b, h][fin] - st.lse[fin])) <= 8 * tol * max(1, np.max(np.abs(st.lse[fin])))
                    assert np.max(np.abs(g["M"][b, h] - st.M)) <= 4 * tol
                else:
                    assert np.max(np.abs(O - st.O)) <= tol, (b, h, r + 1, "O", np.max(np.abs(O - st.O)))
                    fin = np.isfinite(st.lse)
                    assert np.array_equal(fin, np.isfinite(g["lse"][b, h]))
                    assert np.max(np.abs(g["lse"][b, h][fin] - st.lse[fin])) <= tol
                    assert np.max(np.abs(g["M"][b, h] - st.M)) <= tol
                if r >= 1:
                    m_or = o["mass"][r]
                    m_g = gpu["mass"][r][b, h]
                    scale = np.max(m_or)
                    assert np.max(np.abs(m_g - m_or)) <= (tol if not rel else 4 * tol) * max(scale, 1.0), (b, h, r + 1)


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
                ok, ndiff = gh.near_tie_ok(gpu["sel"][r][b, h], own, m, cand, 1e-5)
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
                ok, ndiff = gh.near_tie_ok(gpu["sel"][r][b, h], own, m, cand, sel_eps)
                assert ok, (b, h, r + 1, ndiff)
                cand = gpu["sel"][r][b, h]
    if check:
        _check_outputs(cfg, gpu, orc, heads, tol, rel=rel)
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


def test_prefill_bf16_mfma_wide():
    """Enough heads that the twelve-wave (384-row block) kernel runs in the
    dense loop and in loop 2, with ragged row blocks; loops 3 and 4 take the
    four-wave kernel."""
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
                    fin = np.isfinite(st.lse)
                    assert np.array_equal(fin, np.isfinite(g["lse"][b, h]))
                    assert np.max(np.abs(g["lse"][b, h][fin] - st.lse[fin])) <= \
                        8 * tol * max(1, np.max(np.abs(st.lse[fin])))
                want, got = o["lsel"][r], g["lsel"][b, h][rr]
                fin = np.isfinite(want)
                assert np.array_equal(fin, np.isfinite(got)), (b, h, r + 1)
                err = np.max(np.abs(got[fin] - want[fin])) if fin.any() else 0.0
                assert err <= (tol if f32 else 8 * tol) * max(1.0, np.max(np.abs(want[fin]), initial=0.0)), \
                    (b, h, r + 1, "lsel", err)


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
