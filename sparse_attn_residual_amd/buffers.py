"""Device buffers for the C ABI structs, allocated with torch (memory only)."""
from __future__ import annotations

import numpy as np
import torch

from ._lib import (FL_FMT_WORKLOAD, FL_MAX_LOOPS, FlCache, FlDState, FlState, fl_base_record_bytes,
                   fl_residual_record_bytes, fl_stream_bytes)


def _dev_i32(x, device):
    return torch.as_tensor(np.ascontiguousarray(np.asarray(x, dtype=np.int32))).to(device)


class CacheBuffers:
    """A packed cross-loop cache of L layers and the FlCache struct pointing at it.

    rows[r-1]: int32 [B][n_r] active positions of loop r (loop 1 ignored).
    Hkv: key/value heads (None: H); the streams are [L][B][Hkv][...].
    counts: optional per-loop [B] int32 |A_r| of each sequence (ragged batch;
    n is then the capacity and rows[r-1][b] holds counts[r-1][b] positions).
    fmt: FL_FMT_WORKLOAD (per-token records) or FL_FMT_PAPER (the paper's
    streams; sizes from fl_stream_bytes)."""

    def __init__(self, L, B, H, S, d, R, n, bits, rows, device="cuda", Hkv=None, counts=None, fmt=FL_FMT_WORKLOAD):
        assert R <= FL_MAX_LOOPS and len(n) == R and len(bits) == R
        self.L, self.B, self.H, self.S, self.d, self.R = L, B, H, S, d, R
        self.Hkv = H if Hkv is None else Hkv   # heads of the streams
        self.n, self.bits = list(n), list(bits)
        self.fmt = fmt
        self.base_rb = fl_base_record_bytes(d)
        self.res_rb = [0] + [fl_residual_record_bytes(d, bits[r]) for r in range(1, R)]
        probe = self._probe(L)
        # bytes of one (layer, sequence, KV head) stream of each loop
        self.stream = [fl_stream_bytes(probe, r) for r in range(1, R + 1)]
        assert all(x > 0 for x in self.stream), self.stream
        self.base = torch.empty(L * B * self.Hkv * self.stream[0], dtype=torch.uint8, device=device)
        self.res = [None] + [torch.empty(L * B * self.Hkv * self.stream[r], dtype=torch.uint8, device=device)
                             for r in range(1, R)]
        self.rows = [None] + [_dev_i32(rows[r], device).reshape(B, n[r]) for r in range(1, R)]
        self.slot = [None] + [torch.full((B, S), -1, dtype=torch.int32, device=device) for _ in range(1, R)]
        self.cnt = [None] * R if counts is None else \
            [None] + [_dev_i32(counts[r], device).reshape(B) for r in range(1, R)]
        self.fl = self._struct(0, L)

    def _probe(self, L):
        c = FlCache()
        c.L, c.B, c.H, c.S, c.d, c.R, c.Hkv, c.fmt = L, self.B, self.H, self.S, self.d, self.R, self.Hkv, self.fmt
        for r in range(1, self.R + 1):
            c.n[r], c.bits[r] = self.n[r - 1], self.bits[r - 1]
        return c

    def _struct(self, layer, L):
        c = FlCache()
        c.L, c.B, c.H, c.S, c.d, c.R = L, self.B, self.H, self.S, self.d, self.R
        c.Hkv = self.Hkv
        c.fmt = self.fmt
        per_base = self.B * self.Hkv * self.stream[0]
        c.base = self.base.data_ptr() + layer * per_base
        for r in range(1, self.R + 1):
            c.n[r] = self.n[r - 1]
            c.bits[r] = self.bits[r - 1]
            if r >= 2:
                c.rows[r] = self.rows[r - 1].data_ptr()
                c.slot[r] = self.slot[r - 1].data_ptr()
                if self.cnt[r - 1] is not None:
                    c.cnt[r] = self.cnt[r - 1].data_ptr()
                per = self.B * self.Hkv * self.stream[r - 1]
                c.res[r] = self.res[r - 1].data_ptr() + layer * per
        return c

    def layer_view(self, layer: int) -> FlCache:
        """The same cache restricted to one layer (L = 1)."""
        return self._struct(layer, 1)

    def seq_view(self, layer: int, b: int) -> FlCache:
        """One layer and one sequence (L = B = 1): the records of (layer, b) are
        contiguous in the [L][B][Hkv][...] layout."""
        c = self._struct(layer, 1)
        c.B = 1
        c.base += b * self.Hkv * self.stream[0]
        for r in range(2, self.R + 1):
            c.rows[r] += b * self.n[r - 1] * 4
            c.slot[r] += b * self.S * 4
            if c.cnt[r]:
                c.cnt[r] += b * 4
            c.res[r] += b * self.Hkv * self.stream[r - 1]
        return c

    def replicate_layer0(self):
        """Copy layer 0's records into every other layer."""
        per_base = self.B * self.Hkv * self.stream[0]
        b = self.base.view(self.L, per_base)
        b[1:].copy_(b[0:1].expand(self.L - 1, per_base))
        for r in range(1, self.R):
            per = self.B * self.Hkv * self.stream[r]
            x = self.res[r].view(self.L, per)
            x[1:].copy_(x[0:1].expand(self.L - 1, per))

    def base_records(self) -> torch.Tensor:
        return self.base.view(self.L, self.B, self.Hkv, self.S, self.base_rb)

    def res_records(self, r: int) -> torch.Tensor:
        return self.res[r - 1].view(self.L, self.B, self.Hkv, self.n[r - 1], self.res_rb[r - 1])

    def streams(self, r: int) -> torch.Tensor:
        """Loop r's streams as [L][B][Hkv][bytes] (either format)."""
        x = self.base if r == 1 else self.res[r - 1]
        return x.view(self.L, self.B, self.Hkv, self.stream[r - 1])

    def nbytes(self) -> int:
        return self.base.numel() + sum(x.numel() for x in self.res[1:])


class PrefillState:
    """mixed=True adds the lsel buffer, which selects the exact mixed-logit
    combine (an ablation of the mass-rescaled one)."""

    def __init__(self, B, H, S, d, device="cuda", mixed=False):
        self.O = torch.zeros(B, H, S, d, dtype=torch.float32, device=device)
        self.U = torch.zeros(B, H, S, d, dtype=torch.float32, device=device)
        self.M = torch.ones(B, H, S, dtype=torch.float32, device=device)
        self.lse = torch.zeros(B, H, S, dtype=torch.float32, device=device)
        self.lsel = torch.full((B, H, S), float("-inf"), dtype=torch.float32, device=device) if mixed else None
        self.fl = FlState(self.O.data_ptr(), self.U.data_ptr(), self.M.data_ptr(), self.lse.data_ptr(),
                          self.lsel.data_ptr() if mixed else None)

    def snapshot(self):
        keys = ("O", "U", "M", "lse") + (("lsel",) if self.lsel is not None else ())
        return {k: getattr(self, k).clone() for k in keys}


class DecodeState:
    def __init__(self, L, B, H, S, d, device="cuda"):
        self.O = torch.zeros(L, B, H, d, dtype=torch.float32, device=device)
        self.U = torch.zeros(L, B, H, d, dtype=torch.float32, device=device)
        self.M = torch.ones(L, B, H, dtype=torch.float32, device=device)
        self.lse = torch.zeros(L, B, H, dtype=torch.float32, device=device)
        self.logits = torch.zeros(L, B, H, S, dtype=torch.float32, device=device)
        self.sel = torch.zeros(L, B, H, S, dtype=torch.int32, device=device)
        self.fl = FlDState(self.O.data_ptr(), self.U.data_ptr(), self.M.data_ptr(), self.lse.data_ptr(),
                           self.logits.data_ptr(), self.sel.data_ptr())
