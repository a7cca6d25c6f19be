"""Shared driver of the GPU parity tests: runs the HIP path through the C ABI
binding on seeded workloads and collects what the oracle is compared with.
Inputs come from ``workloads`` only; no expected value comes from here."""
from __future__ import annotations

import numpy as np
import torch

import workloads

DEV = "cuda"


def tdtype(cfg):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def fl_dtype(cfg):
    import sparse_attn_residual_amd as fl
    return fl.FL_BF16 if cfg.dtype == "bf16" else fl.FL_F32


def upload(x: np.ndarray, cfg) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(tdtype(cfg)).contiguous()


def rows_list(cfg, rows):
    """rows[b][r] -> per-loop [B][n_r] arrays (ragged sequences padded to the
    capacity with their last row; the kernels read only the counted ones)."""
    out = []
    for r in range(cfg.R):
        n = cfg.n[r]
        out.append(np.stack([np.concatenate([rows[b][r], np.full(n - len(rows[b][r]), rows[b][r][-1], np.int32)])
                             for b in range(cfg.B)]))
    return out


def counts_list(cfg):
    """Per-loop [B] counts for a ragged batch, else None."""
    if not cfg.ragged:
        return None
    return [np.array([cfg.counts(b)[r] for b in range(cfg.B)], np.int32) for r in range(cfg.R)]


def run_prefill(cfg, rows, slices, *, mass_in=None, K_budget=None, mfma=None, mixed=False, fmt=0, noalloc=False):
    """All loops of one layer.  mass_in: optional {r: float32 [B][H][K_prev]}.
    K_budget: one budget for every loop, or a list (loop r uses K_budget[r-2]).
    mixed: the exact mixed-logit combine (the state carries lsel).
    noalloc: the attention of every loop through fl_loop_attn_noalloc.
    Returns dict with per-loop snapshots (index r-1), sel, mass and the cache."""
    import sparse_attn_residual_amd as fl
    K_budget = cfg.K if K_budget is None else K_budget
    R, B, H, S, d = cfg.R, cfg.B, cfg.H, cfg.S, cfg.d
    cache = fl.CacheBuffers(1, B, H, S, d, R, cfg.n, cfg.bits, rows_list(cfg, rows), Hkv=cfg.kv_heads,
                            counts=counts_list(cfg), fmt=fmt)
    st = fl.PrefillState(B, H, S, d, mixed=mixed)
    dt = fl_dtype(cfg)
    qs = [upload(workloads.stack_loop(cfg, slices, r, "q"), cfg) for r in range(1, R + 1)]
    out = dict(state=[], sel=[None], mass=[None], cache=cache, q=qs)
    K_prev = S
    sel_prev = None
    for r in range(1, R + 1):
        k = upload(workloads.stack_loop(cfg, slices, r, "k"), cfg)
        v = upload(workloads.stack_loop(cfg, slices, r, "v"), cfg)
        fl.fl_kv_resq(cache.fl, r, k, v, dt)
        sel = None
        K = 0
        if r >= 2:
            K = min(K_budget[r - 2] if isinstance(K_budget, (list, tuple)) else K_budget, K_prev)
            sel = torch.empty(B, H, K, dtype=torch.int32, device=DEV)
            mass = torch.empty(B, H, K_prev, dtype=torch.float32, device=DEV)
            mi = None
            if mass_in is not None and r in mass_in:
                mi = torch.from_numpy(np.ascontiguousarray(mass_in[r], np.float32)).to(DEV)
            nws = fl.fl_workspace_bytes(fl.FL_WS_COLSEL, cache.fl, r, K_prev, K)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
            fl.fl_colsel(cache.fl, r, qs[r - 2], dt, st.fl, K_prev, sel_prev, K, mi, mass, sel, ws, nws)
            out["sel"].append(sel.cpu().numpy())
            out["mass"].append(mass.cpu().numpy())
        if noalloc:
            fl.fl_loop_attn_noalloc(cache.fl, r, qs[r - 1], dt, K, sel, st.fl)
        else:
            nws = fl.fl_workspace_bytes(fl.FL_WS_ATTN, cache.fl, r, K, K)
            ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=DEV)
            fl.fl_loop_attn(cache.fl, r, qs[r - 1], dt, K, sel, st.fl, ws, nws)
        torch.cuda.synchronize()
        out["state"].append({k2: v2.cpu().numpy() for k2, v2 in st.snapshot().items()})
        if r >= 2:
            sel_prev, K_prev = sel, K
        del k, v
    return out


def near_tie_ok(sel_gpu, sel_orc, mass_orc, cand, gap_max):
    """Selections may differ only between candidates whose oracle keys lie
    within gap_max of each other (an absolute gap in the key's units: callers
    pass a fraction of the K-th candidate's mass, or a logit difference)."""
    a, b = set(sel_gpu.tolist()), set(sel_orc.tolist())
    if a == b:
        return True, 0
    pos = {int(j): t for t, j in enumerate(cand)}
    only_g = [mass_orc[pos[j]] for j in a - b]
    only_o = [mass_orc[pos[j]] for j in b - a]
    gap = max(only_o) - min(only_g)
    return gap <= gap_max, len(a - b)


def kth_key(keys, K):
    """The K-th largest key (the selection threshold)."""
    keys = np.asarray(keys, np.float64)
    K = min(K, keys.shape[0])
    return float(np.partition(keys, keys.shape[0] - K)[keys.shape[0] - K])


# Selections ranked by logits (decode): a logit gap g is a relative mass gap
# of e^g - 1 ~ g, so near ties are bounded in logit units.
LOGIT_TIE = 1e-4


def build_decode_cache(cfg, rows, slices, L=None, fmt=0):
    """Quantize layer 0 through fl_kv_resq, then copy it to every layer."""
    import sparse_attn_residual_amd as fl
    L = cfg.L if L is None else L
    cache = fl.CacheBuffers(L, cfg.B, cfg.H, cfg.S, cfg.d, cfg.R, cfg.n, cfg.bits, rows_list(cfg, rows),
                            Hkv=cfg.kv_heads, counts=counts_list(cfg), fmt=fmt)
    view = cache.layer_view(0)
    dt = fl_dtype(cfg)
    for r in range(1, cfg.R + 1):
        k = upload(workloads.stack_loop(cfg, slices, r, "k"), cfg)
        v = upload(workloads.stack_loop(cfg, slices, r, "v"), cfg)
        fl.fl_kv_resq(view, r, k, v, dt)
        torch.cuda.synchronize()
        del k, v
    if L > 1:
        cache.replicate_layer0()
    return cache


def run_decode(cfg, cache, queries, K_budget=None, T=None):
    """queries[r-1]: float32 [L][B][H][d].  T: tokens attended (the cache's
    first T positions; None: all S).  Returns per-loop snapshots."""
    import sparse_attn_residual_amd as fl
    K_budget = cfg.K if K_budget is None else K_budget
    T = cfg.S if T is None else T
    L = queries[0].shape[0]
    st = fl.DecodeState(L, cfg.B, cfg.H, cfg.S, cfg.d)
    dt = fl_dtype(cfg)
    out = []
    K_prev = T
    c = cache.fl
    c.T = T
    for r in range(1, cfg.R + 1):
        q = upload(queries[r - 1], cfg)
        K = T if r == 1 else min(K_budget, K_prev)
        fl.fl_loop_decode(c, r, q, dt, K_prev, K, st.fl)
        torch.cuda.synchronize()
        snap = dict(O=st.O.cpu().numpy(), U=st.U.cpu().numpy(), M=st.M.cpu().numpy(), lse=st.lse.cpu().numpy(),
                    logits=st.logits[..., :K].cpu().numpy(), sel=st.sel[..., :K].cpu().numpy() if r > 1 else None)
        out.append(snap)
        K_prev = K
    return out


def build_decode_cache_per_sequence(cfg, fmt=0):
    """The decode cache of every sequence of cfg (L layers), quantized one
    sequence at a time (bounded host memory) into layer 0, then copied to
    every layer."""
    import sparse_attn_residual_amd as fl
    rows = {b: workloads.active_rows(cfg, b) for b in range(cfg.B)}
    cache = fl.CacheBuffers(cfg.L, cfg.B, cfg.H, cfg.S, cfg.d, cfg.R, cfg.n, cfg.bits, rows_list(cfg, rows),
                            Hkv=cfg.kv_heads, counts=counts_list(cfg), fmt=fmt)
    dt = fl_dtype(cfg)
    for b in range(cfg.B):
        _, sl = workloads.gen_batch(cfg, batches=[b], with_q=False)
        view = cache.seq_view(0, b)
        for r in range(1, cfg.R + 1):
            k = upload(workloads.stack_loop(cfg, sl, r, "k", batches=[b]), cfg)
            v = upload(workloads.stack_loop(cfg, sl, r, "v", batches=[b]), cfg)
            fl.fl_kv_resq(view, r, k, v, dt)
            torch.cuda.synchronize()
            del k, v
        del sl
    if cfg.L > 1:
        cache.replicate_layer0()
    return cache


def run_decode_device(cfg, cache, queries, K_budget=None):
    """run_decode with the per-loop snapshots kept on the device (clones)."""
    import sparse_attn_residual_amd as fl
    K_budget = cfg.K if K_budget is None else K_budget
    T = cfg.S
    L = queries[0].shape[0]
    st = fl.DecodeState(L, cfg.B, cfg.H, cfg.S, cfg.d)
    dt = fl_dtype(cfg)
    out = []
    K_prev = T
    for r in range(1, cfg.R + 1):
        q = upload(queries[r - 1], cfg)
        K = T if r == 1 else min(K_budget, K_prev)
        fl.fl_loop_decode(cache.fl, r, q, dt, K_prev, K, st.fl)
        torch.cuda.synchronize()
        out.append(dict(O=st.O.clone(), U=st.U.clone(), M=st.M.clone(), lse=st.lse.clone(),
                        logits=st.logits[..., :K].clone(), sel=st.sel[..., :K].clone() if r > 1 else None))
        K_prev = K
    return out
