"""fl_loop_attn_noalloc, the allocation-free variant of fl_loop_attn (its
tile images live in a device array the library holds), against fl_loop_attn
with a caller workspace: two calls in a row, the second on a smaller input,
every loop's state equal bit for bit; and the refusal of a call that would
need more scratch than the array holds."""
import numpy as np
import pytest

import workloads

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _same(cfg, a, b):
    for r in range(cfg.R):
        for k in ("O", "U", "M", "lse"):
            assert np.array_equal(a["state"][r][k], b["state"][r][k]), (cfg.name, r + 1, k)


def test_noalloc_matches_workspace_entry_point():
    import tests.gpu_harness as gh
    big = workloads.custom(name="noalloc-big", dtype="bf16", B=2, H=4, d=128, S=1500, R=4, act=(1, 0.4, 0.2, 0.1),
                           col="0.15", bits=(8, 4, 4, 2), lognormal=0.5, seed=23)
    small = workloads.custom(name="noalloc-small", dtype="bf16", B=1, H=2, d=128, S=700, R=4,
                             act=(1, 0.3, 0.15, 0.08), col="0.10", bits=(8, 4, 2, 4), lognormal=0.5, seed=24)
    vec = workloads.custom(name="noalloc-f32", dtype="f32", B=1, H=2, d=64, S=600, R=3, act=(1, 0.5, 0.2),
                           col="0.20", bits=(8, 4, 2), seed=25)
    for cfg in (big, small, vec):
        _say("noalloc", cfg.name)
        rows, slices = workloads.gen_batch(cfg)
        got = gh.run_prefill(cfg, rows, slices, noalloc=True)
        want = gh.run_prefill(cfg, rows, slices)
        _same(cfg, got, want)


def test_noalloc_refuses_oversized_call():
    """A 32K, 16-head dense loop 1 needs 302 MB of tile images: refused with
    FL_EUNSUPPORTED before anything touches the device."""
    import sparse_attn_residual_amd as fl
    c = fl.FlCache()
    c.L, c.B, c.H, c.S, c.d, c.R = 1, 1, 16, 32768, 128, 1
    c.n[1], c.bits[1] = 32768, 8
    c.base = 0x10000
    s = fl.FlState(0x40000, 0x40000, 0x40000, 0x40000)
    with pytest.raises(fl.FlashLoopError) as ei:
        fl.fl_loop_attn_noalloc(c, 1, 0x40000, fl.FL_BF16, 0, None, s)
    assert ei.value.status == 2 and "FL_NOALLOC_SCRATCH_BYTES" in str(ei.value)
