"""Benchmark of the FlashLoop loop-attention hot path on one MI355X.

One step = one pass of the whole prefill hot path over one layer of the
32K-token, R = 4 workload (Ouro-2.6B shaped: 16 heads x 128 dims, bf16,
nested active rows 100/30/15/8 %, top 10 % of columns, int8 base + 4/4/2-bit
residuals): for every loop r, fl_kv_resq(r), then fl_colsel(r) (r >= 2), then
fl_loop_attn(r).  Inputs (queries, keys and values of every loop) are
resident in HBM before the timed region.  `value` is prefill tokens/s.

The same run also times one decode step of the 48-layer packed cache
(B = 16 sequences x 16 heads x 32K cached tokens, R = 4 launches of
fl_loop_decode) and reports its packed-KV GB/s against the HBM roofline, and
times the CPU oracle on a bounded sample of the prefill workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-decode] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PREFILL_CFG = 2
DECODE_CFG = 3
OTHER_PREFILL_CFGS = (1, 4)
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "bench_prefill_s32768_decode_t32768_l48_hbm_traffic.md")


def measured_traffic(key):
    """HBM bytes (read + written) per launch of one kernel, from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE profile scaled by its copy calibration;
    None when the kernel sources changed since that profile was taken."""
    import re
    try:
        with open(TRAFFIC_PROFILE) as f:
            text = f.read()
    except OSError:
        return None
    m = re.search(r"```json\n(\{.*\})\n```", text)
    if not m:
        return None
    prof = json.loads(m.group(1))
    from sparse_attn_residual_amd.build import source_digest
    if prof.get("source_sha256") != source_digest():
        return None
    k = prof.get("kernels", {}).get(key)
    return None if k is None else k["read_bytes"] + k["write_bytes"]


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def _upload(x, torch):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to("cuda").to(torch.bfloat16).contiguous()


class Timer:
    """HIP events on the stream the library launches on (torch's current)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = {}

    def wrap(self, key, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        self.pairs.setdefault(key, []).append((e0, e1))

    def reset(self):
        self.pairs = {}

    def mean_ms(self):
        return {k: float(np.mean([a.elapsed_time(b) for a, b in v])) for k, v in self.pairs.items()}


def prefill_bench(args, torch, fl, workloads, acc, cfg=None, pruned=True, fmt=0):
    cfg = workloads.CONFIGS[PREFILL_CFG] if cfg is None else cfg
    t0 = time.time()
    rows, slices = workloads.gen_batch(cfg)
    log(f"generated {cfg.name} inputs in {time.time() - t0:.1f}s")
    R, B, H, S, d = cfg.R, cfg.B, cfg.H, cfg.S, cfg.d
    q = [_upload(workloads.stack_loop(cfg, slices, r, "q"), torch) for r in range(1, R + 1)]
    k = [_upload(workloads.stack_loop(cfg, slices, r, "k"), torch) for r in range(1, R + 1)]
    v = [_upload(workloads.stack_loop(cfg, slices, r, "v"), torch) for r in range(1, R + 1)]
    del slices
    # per-sequence rows padded to the capacity with their last row (ragged batches)
    rows_l = [np.stack([np.concatenate([rows[b][r], np.full(cfg.n[r] - len(rows[b][r]), rows[b][r][-1], np.int32)])
                        for b in range(B)]) for r in range(R)]
    counts = [np.array([cfg.counts(b)[r] for b in range(B)], np.int32) for r in range(R)] if cfg.ragged else None
    cache = fl.CacheBuffers(1, B, H, S, d, R, cfg.n, cfg.bits, rows_l, Hkv=cfg.kv_heads, counts=counts, fmt=fmt)
    st = fl.PrefillState(B, H, S, d)
    res = measure_prefill(args, torch, fl, acc, cfg, rows, q, k, v, cache, st, [cfg.K] * (R - 1))
    if pruned:
        # nested pruning: the budget halves at every loop after the second
        res["pruned"] = measure_prefill(args, torch, fl, acc, cfg, rows, q, k, v, cache, st,
                                        [cfg.K >> (r - 2) for r in range(2, R + 1)])
    return res


def measure_prefill(args, torch, fl, acc, cfg, rows, q, k, v, cache, st, budgets):
    """Time args.steps prefill steps of one layer with column budgets
    budgets[r-2] for loops r >= 2 (each clipped to the previous loop's)."""
    R, B, H, S = cfg.R, cfg.B, cfg.H, cfg.S
    Ks = [S]
    for r in range(2, R + 1):
        Ks.append(min(budgets[r - 2], Ks[r - 2]))
    sel = [None] + [torch.empty(B, H, Ks[r], dtype=torch.int32, device="cuda") for r in range(1, R)]
    ws_bytes = fl.fl_workspace_bytes(fl.FL_WS_ATTN, cache.fl, 1, S, S)
    for r in range(2, R + 1):
        ws_bytes = max(ws_bytes, fl.fl_workspace_bytes(fl.FL_WS_COLSEL, cache.fl, r, Ks[r - 2], Ks[r - 1]),
                       fl.fl_workspace_bytes(fl.FL_WS_ATTN, cache.fl, r, Ks[r - 1], Ks[r - 1]))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    dt = fl.FL_BF16
    tm = Timer(torch)

    def step(timed):
        w = timed if callable(timed) else (tm.wrap if timed else (lambda key, fn: fn()))
        for r in range(1, R + 1):
            w(f"resq{r}", lambda r=r: fl.fl_kv_resq(cache.fl, r, k[r - 1], v[r - 1], dt))
            if r >= 2:
                cand = sel[r - 2] if r >= 3 else None
                w(f"colsel{r}", lambda r=r, cand=cand: fl.fl_colsel(
                    cache.fl, r, q[r - 2], dt, st.fl, Ks[r - 2], cand, Ks[r - 1], None, None, sel[r - 1], ws,
                    ws_bytes))
            w(f"attn{r}", lambda r=r: fl.fl_loop_attn(cache.fl, r, q[r - 1], dt, Ks[r - 1], sel[r - 1], st.fl, ws,
                                                     ws_bytes))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    # timed region: barrier + synchronize on both sides (one process); the
    # steps run with no events between their calls
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step(False)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    # per-call times: as many more steps with events around every call
    tm.reset()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    per = tm.mean_ms()
    log(f"prefill K={Ks[1:]}: {ms_step:.3f} ms/step (wall {1e3 * wall / args.steps:.3f}); per call (ms): "
        + ", ".join(f"{kk}={vv:.3f}" for kk, vv in per.items()))
    kern = kernel_times(fl, torch, step, args.steps)

    # algorithmic work from the index lists of the run
    sels = [None] + [s.cpu().numpy() for s in sel[1:]]
    masses_ran = [False] + [Ks[r] < Ks[r - 1] for r in range(1, R)]
    work = acc.prefill_work(cfg, rows, sels, masses_ran)
    dense_t = per["attn1"] * 1e-3
    dense_tf = work["dense_flops"] / dense_t / 1e12
    sparse_t = sum(per[f"attn{r}"] for r in range(2, R + 1)) * 1e-3
    sparse_tf = work["sparse_flops"] / sparse_t / 1e12
    total_tf = work["flops"] / (ms_step * 1e-3) / 1e12
    # the attention kernels alone (the tile builds excluded), from the kernel timer
    k_dense = attn_kernel_ms(kern, "attn1")
    k_sparse = sum(attn_kernel_ms(kern, f"attn{r}") for r in range(2, R + 1))
    return dict(cfg=cfg, ms_step=ms_step, per=per, work=work, dense_tf=dense_tf, sparse_tf=sparse_tf,
                total_tf=total_tf, Ks=Ks, kern=kern, dense_kernel_ms=k_dense,
                dense_kernel_tf=work["dense_flops"] / (k_dense * 1e-3) / 1e12,
                sparse_kernel_ms=k_sparse, sparse_kernel_tf=work["sparse_flops"] / (k_sparse * 1e-3) / 1e12)


def kernel_times(fl, torch, step, steps):
    """Per-kernel durations of each library call of a step: the library's
    kernel timer brackets every launch with HIP events on its stream.  Runs
    `steps` extra steps (the timed region above ran without the timer) and
    returns {call: [(kernel, mean ms), ...]} in launch order."""
    rec = {}
    fl.fl_timing_enable(True)
    try:
        for _ in range(steps):
            def wrap(key, fn):
                fn()
                rec.setdefault(key, []).append(fl.fl_timing_collect())
            step(wrap)
    finally:
        fl.fl_timing_enable(False)
        fl.fl_timing_collect()
    out = {}
    for key, runs in rec.items():
        n = min(len(r) for r in runs)
        out[key] = [(runs[0][i][0], float(np.mean([r[i][1] for r in runs]))) for i in range(n)]
    return out


def attn_kernel_ms(kern, key):
    """Time of the attention kernel of one fl_loop_attn call (its k_attn
    launches, without the tile build)."""
    return sum(t for name, t in kern.get(key, []) if name.startswith("k_attn_"))


def decode_bench(args, torch, fl, workloads, acc, cfg=None, fmt=0):
    cfg = workloads.CONFIGS[DECODE_CFG] if cfg is None else cfg
    L, B, H, S, d, R = cfg.L, cfg.B, cfg.H, cfg.S, cfg.d, cfg.R
    Hkv = cfg.kv_heads
    t0 = time.time()
    rows = {b: workloads.active_rows(cfg, b) for b in range(B)}
    rows_l = [np.stack([rows[b][r] for b in range(B)]) for r in range(R)]
    cache = fl.CacheBuffers(L, B, H, S, d, R, cfg.n, cfg.bits, rows_l, Hkv=Hkv, fmt=fmt)
    log(f"decode cache: {cache.nbytes() / 1e9:.1f} GB on device")
    for b in range(B):
        _, sl = workloads.gen_batch(cfg, batches=[b], with_q=False)
        view = cache.seq_view(0, b)
        for r in range(1, R + 1):
            kk = _upload(workloads.stack_loop(cfg, sl, r, "k", batches=[b]), torch)
            vv = _upload(workloads.stack_loop(cfg, sl, r, "v", batches=[b]), torch)
            fl.fl_kv_resq(view, r, kk, vv, fl.FL_BF16)
            torch.cuda.synchronize()
            del kk, vv
        del sl
        log(f"decode cache: sequence {b + 1}/{B} quantized ({time.time() - t0:.0f}s)")
    cache.replicate_layer0()
    qs = [_upload(x, torch) for x in workloads.decode_queries(cfg)]
    st = fl.DecodeState(L, B, H, S, d)
    Ks = [S] + [min(cfg.K, S)] * (R - 1)
    tm = Timer(torch)

    def step(timed):
        w = timed if callable(timed) else (tm.wrap if timed else (lambda key, fn: fn()))
        for r in range(1, R + 1):
            w(f"decode{r}", lambda r=r: fl.fl_loop_decode(cache.fl, r, qs[r - 1], fl.FL_BF16,
                                                          Ks[r - 2] if r >= 2 else S, Ks[r - 1], st.fl))

    for _ in range(max(1, args.warmup // 2)):
        step(False)
    torch.cuda.synchronize()
    steps = max(2, args.steps // 2)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step(False)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    # per-loop times: as many more steps with events around every call
    for _ in range(steps):
        step(True)
    torch.cuda.synchronize()
    per = tm.mean_ms()
    log(f"decode: {ms_step:.3f} ms/step; per loop (ms): " + ", ".join(f"{kk}={vv:.3f}" for kk, vv in per.items()))
    kern = kernel_times(fl, torch, step, 1)

    # algorithmic packed bytes of the step, from the selections of the run
    # (the dense loop reads every record of every KV head once)
    base_b = acc.base_record_bytes(d)
    res_b = [0] + [acc.residual_record_bytes(d, cfg.bits[r]) for r in range(1, R)]
    loop_bytes = [float(L * B * Hkv * S * base_b)]
    # S_2 = S_3 = S_4 with a constant budget: the last loop's selection,
    # checked on the host before it indexes anything
    sel = check_selection(st.sel[..., :Ks[-1]].cpu().numpy(), S, Ks[-1])
    cum = np.full((B, S), float(base_b))
    for r in range(2, R + 1):
        cum += (cache.slot[r - 1].cpu().numpy() >= 0) * float(res_b[r - 1])
        loop_bytes.append(float(sum(np.take_along_axis(cum[b][None, None, :], sel[:, b], axis=2).sum()
                                    for b in range(B))))
    total = sum(loop_bytes)
    logits_overhead = float(L * B * H * S * 4 * 2)
    dense_kms = sum(t for n, t in kern.get("decode1", []) if n.startswith("k_decode_dense")) or per["decode1"]
    return dict(cfg=cfg, ms_step=ms_step, per=per, kern=kern, dense_kernel_ms=dense_kms,
                dense_kernel_gbs=loop_bytes[0] / (dense_kms * 1e-3) / 1e9, loop_bytes=loop_bytes, bytes=total,
                cache_stream1_bytes=float(cache.base.numel()),
                gbs=total / (ms_step * 1e-3) / 1e9, dense_gbs=loop_bytes[0] / (per["decode1"] * 1e-3) / 1e9,
                logits_overhead=logits_overhead, cache_bytes=cache.nbytes())


def check_selection(sel, T, K):
    """sel [..., K] int32 from the device: every row must hold K positions in
    [0, T), strictly ascending.  Raises before the selection indexes anything."""
    if sel.shape[-1] != K:
        raise RuntimeError(f"decode selection has {sel.shape[-1]} entries per row, expected {K}")
    if sel.size and (sel.min() < 0 or sel.max() >= T):
        raise RuntimeError(f"decode selection holds positions outside [0, {T}): min {sel.min()}, max {sel.max()}")
    if K > 1 and not np.all(np.diff(sel, axis=-1) > 0):
        raise RuntimeError("decode selection is not strictly ascending")
    return sel.astype(np.int64)


def select_bench(args, torch, fl, workloads, acc):
    """Next active sets of the 32K workload (hidden size H*d = 2048, bf16):
    one fl_select_active call per loop 2..R, each ranking the previous active
    set.  Algorithmic bytes: both hidden states of every candidate."""
    cfg = workloads.CONFIGS[PREFILL_CFG]
    S, D = cfg.S, cfg.H * cfg.d
    rows = workloads.active_rows(cfg, 0)
    hp, hcs = None, []
    for r in range(2, cfg.R + 1):
        h_prev, h_cur = workloads.gen_hidden(cfg, 0, D, r, rows[r - 2])
        if hp is None:
            hp = _upload(h_prev, torch)
        hcs.append(_upload(h_cur, torch))
        del h_prev, h_cur
    cands = [None] + [torch.from_numpy(rows[r - 2]).cuda() for r in range(3, cfg.R + 1)]
    outs = [torch.empty(1, cfg.n[r - 1], dtype=torch.int32, device="cuda") for r in range(2, cfg.R + 1)]
    scores = [torch.empty(1, cfg.n[r - 2], dtype=torch.float32, device="cuda") for r in range(2, cfg.R + 1)]
    tm = Timer(torch)

    def step(timed):
        w = tm.wrap if timed else (lambda key, fn: fn())
        for i, r in enumerate(range(2, cfg.R + 1)):
            w(f"select{r}", lambda i=i, r=r: fl.fl_select_active(1, S, D, hp, hcs[i], fl.FL_BF16, cfg.n[r - 2],
                                                                  cands[i], cfg.n[r - 1], outs[i], scores[i]))

    for _ in range(max(1, args.warmup)):
        step(False)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    per = tm.mean_ms()
    loop_bytes = {f"select{r}": 2.0 * cfg.n[r - 2] * D * 2 for r in range(2, cfg.R + 1)}
    gbs = {k: loop_bytes[k] / (per[k] * 1e-3) / 1e9 for k in per}
    log("select: per loop (ms): " + ", ".join(f"{k}={v:.3f}" for k, v in per.items()))
    return dict(per=per, bytes=loop_bytes, gbs=gbs, D=D)


def measured_peaks(torch):
    """Achievable rate of the vendor library's bf16 GEMM on this GPU (torch
    .matmul -> hipBLASLt, 16384^3), measured in the same run; the MFMA
    roofline reports its fraction next to the vendor peak."""
    n = 16384
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        torch.matmul(a, b)
    torch.cuda.synchronize()
    reps = 10
    e0.record()
    for _ in range(reps):
        torch.matmul(a, b)
    e1.record()
    torch.cuda.synchronize()
    gemm = 2.0 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    # streaming HBM rate: the library's elementwise y = x + 1 over 4 GiB of
    # fp32 (bytes read plus written; its reductions stream more slowly)
    x = torch.ones(1 << 30, device="cuda", dtype=torch.float32)
    y = torch.empty_like(x)
    for _ in range(2):
        torch.add(x, 1.0, out=y)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(5):
        e0.record()
        torch.add(x, 1.0, out=y)
        e1.record()
        torch.cuda.synchronize()
        best = max(best, 2 * x.numel() * 4 / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del x, y
    torch.cuda.empty_cache()
    log(f"measured peak: library bf16 GEMM {gemm:.0f} TFLOP/s, streaming elementwise {best:.0f} GB/s")
    return dict(bf16_gemm_tflops=gemm, hbm_read_gbs=best)


def cpu_baseline(workloads, cfg_id=PREFILL_CFG):
    """The oracle as it stands on every head of one layer of a prefill
    workload, all loops, the heads spread over a pool of worker threads (one
    BLAS thread each; numpy releases the interpreter lock in its kernels)."""
    from concurrent.futures import ThreadPoolExecutor
    from oracle import prefill
    from threadpoolctl import threadpool_limits
    cfg = workloads.CONFIGS[cfg_id]
    heads = list(range(cfg.H))
    workers = max(1, min(len(heads), len(os.sched_getaffinity(0)), 16))
    rows, sl = workloads.gen_batch(cfg, heads=heads)

    def one(h):
        s = sl[(0, h)]
        prefill.prefill_slice(s.rows, s.q, s.k, s.v, K_budget=cfg.K, bits=cfg.bits, dtype=cfg.dtype)

    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, heads))
        t = time.perf_counter() - t0
    value = cfg.B * cfg.S / t
    log(f"cpu oracle {cfg.name}: {t:.1f}s for all {cfg.H} heads on {workers} threads")
    return dict(value=value, unit="tokens/s", cores=int(workers), kind="oracle",
                sample=f"{cfg.name}: all {cfg.H} heads of one layer, all {cfg.R} loops in float64 ({t:.1f}s), "
                       f"{workers} worker threads with one BLAS thread each", cpu_model=_cpu_model(), blas=_blas())


def cpu_decode_baseline(workloads, step_bytes):
    """The oracle's decode step (all R loops) on 64 (sequence, head) queries of
    the 48-layer workload over the cache records of four of its slices (the
    records are built first and not timed), the problems spread over a pool of
    worker threads (one BLAS thread each), extrapolated to every slice of the
    step."""
    import dataclasses
    from concurrent.futures import ThreadPoolExecutor
    from oracle import decode, quant
    from threadpoolctl import threadpool_limits
    cfg = workloads.CONFIGS[DECODE_CFG]
    nrec = 4
    small = dataclasses.replace(cfg, name=cfg.name + "-cpu-sample", B=1, H=nrec, L=1)
    rows, sl = workloads.gen_batch(small)
    recs = []
    for h in range(nrec):
        s = sl[(0, h)]
        recs.append((quant.quantize_chain(s.k, s.rows, list(small.bits))[1],
                     quant.quantize_chain(s.v, s.rows, list(small.bits))[1]))
    qcfg = dataclasses.replace(cfg, name=cfg.name + "-cpu-queries", B=4, H=16, L=1)
    qs = workloads.decode_queries(qcfg)
    probs = [(b, h) for b in range(qcfg.B) for h in range(qcfg.H)]
    workers = max(1, min(len(probs), len(os.sched_getaffinity(0)), 16))

    def one(bh):
        b, h = bh
        krec, vrec = recs[(b * qcfg.H + h) % nrec]
        decode.decode_slice(krec, vrec, [q[0, b, h] for q in qs], cfg.K)

    with threadpool_limits(1):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(one, probs))
        t = time.perf_counter() - t0
    slices = cfg.L * cfg.B * cfg.H
    step_s = t / len(probs) * slices
    log(f"cpu oracle decode: {len(probs)} problems in {t:.2f}s on {workers} threads")
    return dict(value=step_bytes / step_s / 1e9, unit="GB/s", kind="oracle", extrapolated=True, cores=int(workers),
                ms_per_step=step_s * 1e3,
                sample=f"{len(probs)} (sequence, head) decode queries over the cache records of {nrec} of the "
                       f"step's {slices} (layer, sequence, head) slices, all {cfg.R} loops in float64 ({t:.2f}s on "
                       f"{workers} worker threads with one BLAS thread each), extrapolated to the whole step",
                cpu_model=_cpu_model(), blas=_blas())


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _blas() -> str:
    try:
        from threadpoolctl import threadpool_info
        libs = [f"{p.get('internal_api')} {p.get('version')}" for p in threadpool_info() if p.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:
        return "unknown"


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--main-only", action="store_true",
                    help="only the 32K prefill and 48-layer decode workloads (no gqa, paper_format, ragged sections)")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only copy 1 GiB device to device three times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the hot path shards by heads and sequences with no exchange, and this "
              f"build measures one GPU's share (asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.calib_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes_read": 1 << 30, "calib_copy_bytes_written": 1 << 30, "copies": 3}))
        return
    import sparse_attn_residual_amd as fl
    from sparse_attn_residual_amd import accounting as acc
    import workloads

    peaks = measured_peaks(torch)
    pf = prefill_bench(args, torch, fl, workloads, acc)
    # the other prefill workloads: 8K (Ouro-1.4B shaped) and the deep 16K, R = 8 one
    others = {cid: prefill_bench(args, torch, fl, workloads, acc, cfg=workloads.CONFIGS[cid], pruned=False)
              for cid in OTHER_PREFILL_CFGS}
    sel = select_bench(args, torch, fl, workloads, acc)
    dec = None if args.no_decode else decode_bench(args, torch, fl, workloads, acc)
    torch.cuda.empty_cache()
    extra = not args.main_only
    # grouped-query attention (4 query heads per KV head) on the same shapes
    gqa_pf = gqa_dec = pap_pf = pap_dec = rag_pf = None
    if extra:
        gqa_pf = prefill_bench(args, torch, fl, workloads, acc, cfg=workloads.CONFIGS[PREFILL_CFG].with_(Hkv=4),
                               pruned=False)
        gqa_dec = None if args.no_decode else decode_bench(args, torch, fl, workloads, acc,
                                                           cfg=workloads.CONFIGS[DECODE_CFG].with_(Hkv=4))
        torch.cuda.empty_cache()
        # the paper's own cache format (INT4 g64, per-channel keys, bf16 tail) on the same shapes
        pap_pf = prefill_bench(args, torch, fl, workloads, acc, cfg=workloads.CONFIGS[PREFILL_CFG], pruned=False,
                               fmt=fl.FL_FMT_PAPER)
        pap_dec = None if args.no_decode else decode_bench(args, torch, fl, workloads, acc, fmt=fl.FL_FMT_PAPER)
        torch.cuda.empty_cache()
    # a ragged batch: two 32K sequences, the second keeping half as many active rows
    rag_cfg = workloads.CONFIGS[PREFILL_CFG].with_(B=2, ragged=("1", "0.5"))
    if extra:
        rag_pf = prefill_bench(args, torch, fl, workloads, acc, cfg=rag_cfg, pruned=False)
    cpu = None if args.no_cpu else cpu_baseline(workloads)
    cpu_others = {} if args.no_cpu else {cid: cpu_baseline(workloads, cid) for cid in OTHER_PREFILL_CFGS}

    cfg = pf["cfg"]
    tokens_s = cfg.B * cfg.S / (pf["ms_step"] * 1e-3)
    dense_flops = pf["work"]["dense_flops"]
    out = {
        "metric": "loop-attn prefill tokens/s @32K R=4; decode packed-KV GB/s vs HBM peak",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": pf["ms_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one layer, B={cfg.B}, H={cfg.H}, d={cfg.d}, S={cfg.S}, R={cfg.R}, "
                        f"active rows {cfg.n}, K={pf['Ks'][1]}, bits {list(cfg.bits)}",
            "per_call_ms": {k: round(v, 4) for k, v in pf["per"].items()},
            "prefill_flops": pf["work"]["flops"],
            "mfma_frac_whole_step": pf["total_tf"] / acc.MI355X_BF16_TFLOPS,
            "sparse_attn_tflops": pf["sparse_tf"],
            "sparse_attn_mfma_frac": pf["sparse_tf"] / acc.MI355X_BF16_TFLOPS,
            "sparse_attn_kernel_ms": pf["sparse_kernel_ms"],
            "sparse_attn_kernel_mfma_frac": pf["sparse_kernel_tf"] / acc.MI355X_BF16_TFLOPS,
            "kernel_ms": {k: [[n, round(t, 4)] for n, t in v] for k, v in pf["kern"].items()},
            "pruned_schedule": {
                "K": pf["pruned"]["Ks"][1:],
                "ms_per_step": pf["pruned"]["ms_step"],
                "tokens_per_s": cfg.B * cfg.S / (pf["pruned"]["ms_step"] * 1e-3),
                "per_call_ms": {k: round(v, 4) for k, v in pf["pruned"]["per"].items()},
            },
        },
        "roofline": {
            "kernel": "k_attn_dense48<8, 3> (the attention kernel of fl_loop_attn r=1: dense causal over the int8 base)",
            "bound": "mfma",
            "achieved": pf["dense_kernel_tf"],
            "peak": acc.MI355X_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": pf["dense_kernel_tf"] / acc.MI355X_BF16_TFLOPS,
            "measured_peak": peaks["bf16_gemm_tflops"],
            "measured_peak_kind": "hipBLASLt bf16 GEMM 16384^3 via torch.matmul, same run",
            "frac_of_measured": pf["dense_kernel_tf"] / peaks["bf16_gemm_tflops"],
            "traffic": measured_traffic("attn1"),
            "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
            "flops_per_launch": dense_flops,
            "avg_launch_ms": pf["dense_kernel_ms"],
            "timing": "HIP events around the kernel's launch on its stream (the library's kernel timer)",
            "call_ms": pf["per"]["attn1"],
            "call_frac": pf["dense_tf"] / acc.MI355X_BF16_TFLOPS,
        },
    }
    qb = [acc.resq_bytes(cfg.d, cfg.bits[:r], cfg.B * cfg.n[r - 1], cfg.kv_heads) for r in range(1, cfg.R + 1)]
    qt = [pf["per"][f"resq{r}"] for r in range(1, cfg.R + 1)]
    out["quantize"] = {
        "kernel": "k_quant_base (r = 1), k_quant_res (r >= 2): fl_kv_resq of the prefill workload",
        "algorithmic_bytes_per_loop": qb,
        "ms_per_loop": [round(t, 4) for t in qt],
        "gbs_per_loop": [b / (t * 1e6) for b, t in zip(qb, qt)],
        "frac_per_loop": [b / (t * 1e6) / acc.MI355X_HBM_GBS for b, t in zip(qb, qt)],
        "bound": "hbm",
        "peak_gbs": acc.MI355X_HBM_GBS,
        "bytes_note": "per active (row, KV head): K and V rows in, the records of the earlier loops the residual is "
                      "taken against, one record out",
    }
    out["select"] = {
        "workload": f"{cfg.name}: next active sets of loops 2..{cfg.R}, hidden size {sel['D']}, bf16 "
                    f"(fl_select_active, candidates {cfg.n[:-1]} -> {cfg.n[1:]})",
        "per_loop_ms": {k: round(v, 4) for k, v in sel["per"].items()},
        "roofline": {
            "kernel": "k_active_score + k_topk (fl_select_active, loop 2)",
            "bound": "hbm",
            "achieved": sel["gbs"]["select2"],
            "peak": acc.MI355X_HBM_GBS,
            "unit": "GB/s",
            "frac": sel["gbs"]["select2"] / acc.MI355X_HBM_GBS,
            "algorithmic_bytes": sel["bytes"]["select2"],
        },
    }
    if dec is not None:
        dcfg = dec["cfg"]
        out["decode"] = {
            "workload": f"{dcfg.name}: L={dcfg.L} stacked layers, B={dcfg.B}, H={dcfg.H}, T={dcfg.S}, R={dcfg.R}, "
                        f"K={min(dcfg.K, dcfg.S)}, bits {list(dcfg.bits)}",
            "ms_per_step": dec["ms_step"],
            "packed_kv_bytes_per_step": dec["bytes"],
            "value": dec["gbs"],
            "unit": "GB/s",
            "per_loop_ms": {k: round(v, 4) for k, v in dec["per"].items()},
            "loop_bytes": dec["loop_bytes"],
            "kernel_ms": {k: [[n, round(t, 4)] for n, t in v] for k, v in dec["kern"].items()},
            "logits_overhead_bytes": dec["logits_overhead"],
            "roofline": {
                "kernel": "k_decode_dense (fl_loop_decode r=1)",
                "bound": "hbm",
                "achieved": dec["dense_kernel_gbs"],
                "peak": acc.MI355X_HBM_GBS,
                "unit": "GB/s",
                "frac": dec["dense_kernel_gbs"] / acc.MI355X_HBM_GBS,
                "avg_launch_ms": dec["dense_kernel_ms"],
                "measured_peak": peaks["hbm_read_gbs"],
                "measured_peak_kind": "torch elementwise y = x + 1 over 4 GiB fp32 (read + written), same run",
                "frac_of_measured": dec["dense_kernel_gbs"] / peaks["hbm_read_gbs"],
                "traffic": measured_traffic("decode1"),
                "algorithmic_bytes": dec["loop_bytes"][0],
                "step_frac": dec["gbs"] / acc.MI355X_HBM_GBS,
            },
        }
        if not args.no_cpu:
            out["decode"]["cpu_oracle"] = cpu_decode_baseline(workloads, dec["bytes"])
    out["workloads"] = {}
    for cid, o in others.items():
        c = o["cfg"]
        out["workloads"][c.name] = {
            "workload": f"{c.name}: one layer, B={c.B}, H={c.H}, d={c.d}, S={c.S}, R={c.R}, active rows {c.n}, "
                        f"K={o['Ks'][1]}, bits {list(c.bits)}",
            "metric": "prefill tokens/s",
            "value": c.B * c.S / (o["ms_step"] * 1e-3),
            "unit": "tokens/s",
            "ms_per_step": o["ms_step"],
            "per_call_ms": {k: round(v, 4) for k, v in o["per"].items()},
            "prefill_flops": o["work"]["flops"],
            "mfma_frac_whole_step": o["total_tf"] / acc.MI355X_BF16_TFLOPS,
            "roofline": {
                "kernel": "dense loop-1 attention kernel", "bound": "mfma", "achieved": o["dense_kernel_tf"],
                "peak": acc.MI355X_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": o["dense_kernel_tf"] / acc.MI355X_BF16_TFLOPS, "avg_launch_ms": o["dense_kernel_ms"],
            },
            "sparse_attn_kernel_ms": o["sparse_kernel_ms"],
            "sparse_attn_kernel_mfma_frac": o["sparse_kernel_tf"] / acc.MI355X_BF16_TFLOPS,
            "sparse_attn_mfma_frac": o["sparse_tf"] / acc.MI355X_BF16_TFLOPS,
            "cpu_baseline": cpu_others.get(cid),
        }
    if extra:
        _extras(out, cfg, gqa_pf, gqa_dec, pap_pf, pap_dec, rag_cfg, rag_pf)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


def _extras(out, cfg, gqa_pf, gqa_dec, pap_pf, pap_dec, rag_cfg, rag_pf):
    """The gqa, paper_format and ragged sections of the JSON line."""
    out["gqa"] = {
        "workload": f"the two workloads above with Hkv = 4 key/value heads for H = {cfg.H} query heads",
        "prefill_ms_per_step": gqa_pf["ms_step"],
        "prefill_tokens_per_s": cfg.B * cfg.S / (gqa_pf["ms_step"] * 1e-3),
        "prefill_per_call_ms": {k: round(v, 4) for k, v in gqa_pf["per"].items()},
    }
    if gqa_dec is not None:
        out["gqa"].update({
            "decode_ms_per_step": gqa_dec["ms_step"],
            "decode_per_loop_ms": {k: round(v, 4) for k, v in gqa_dec["per"].items()},
            "decode_dense_unique_gbs": gqa_dec["dense_gbs"],
            "decode_dense_note": "loop 1 reads each KV head's records once for its 4 query heads; GB/s counts "
                                 "those unique bytes (the kernel is vector-ALU bound at this ratio)",
        })
    out["paper_format"] = {
        "workload": "the 32K prefill and 48-layer decode workloads above with the paper's own cache format (INT4 "
                    "asymmetric, group 64, keys per channel along tokens, values per token, 64-token bf16 tail)",
        "prefill_ms_per_step": pap_pf["ms_step"],
        "prefill_tokens_per_s": cfg.B * cfg.S / (pap_pf["ms_step"] * 1e-3),
        "prefill_per_call_ms": {k: round(v, 4) for k, v in pap_pf["per"].items()},
    }
    if pap_dec is not None:
        out["paper_format"].update({
            "decode_ms_per_step": pap_dec["ms_step"],
            "decode_per_loop_ms": {k: round(v, 4) for k, v in pap_dec["per"].items()},
            "decode_cache_bytes": pap_dec["cache_bytes"],
            "decode_dense_stream_gbs": pap_dec["cache_stream1_bytes"] / (pap_dec["per"]["decode1"] * 1e-3) / 1e9,
        })
    out["ragged"] = {
        "workload": f"{rag_cfg.name} with B = 2: active rows per loop {rag_cfg.counts(0)} and {rag_cfg.counts(1)}",
        "prefill_ms_per_step": rag_pf["ms_step"],
        "prefill_tokens_per_s": rag_cfg.B * rag_cfg.S / (rag_pf["ms_step"] * 1e-3),
        "prefill_per_call_ms": {k: round(v, 4) for k, v in rag_pf["per"].items()},
    }


if __name__ == "__main__":
    main()
