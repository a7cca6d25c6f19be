"""ctypes view of include/flashloop.h.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

FL_MAX_LOOPS = 16
FL_MAX_S = 1 << 21
FL_F32, FL_BF16 = 0, 1
FL_WS_COLSEL, FL_WS_ATTN, FL_WS_DECODE = 1, 2, 3
FL_FMT_WORKLOAD, FL_FMT_PAPER = 0, 1
_N = FL_MAX_LOOPS + 1

_HERE = os.path.dirname(os.path.abspath(__file__))


def lib_path() -> str:
    return os.environ.get("FLASHLOOP_LIB", os.path.join(_HERE, "libflashloop.so"))


class FlashLoopError(RuntimeError):
    def __init__(self, fn, status, msg):
        super().__init__(f"{fn} failed with status {status}: {msg}")
        self.status = status


class FlCache(ctypes.Structure):
    _fields_ = [
        ("L", ctypes.c_int), ("B", ctypes.c_int), ("H", ctypes.c_int), ("S", ctypes.c_int),
        ("d", ctypes.c_int), ("R", ctypes.c_int),
        ("n", ctypes.c_int * _N), ("bits", ctypes.c_int * _N),
        ("rows", ctypes.c_void_p * _N), ("slot", ctypes.c_void_p * _N),
        ("base", ctypes.c_void_p), ("res", ctypes.c_void_p * _N),
        ("Hkv", ctypes.c_int),
        ("cnt", ctypes.c_void_p * _N),
        ("T", ctypes.c_int),
        ("fmt", ctypes.c_int),
    ]


class FlState(ctypes.Structure):
    _fields_ = [("O", ctypes.c_void_p), ("U", ctypes.c_void_p), ("M", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("lsel", ctypes.c_void_p)]


class FlDState(ctypes.Structure):
    _fields_ = [("O", ctypes.c_void_p), ("U", ctypes.c_void_p), ("M", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("logits", ctypes.c_void_p), ("sel", ctypes.c_void_p)]


def _load():
    # The library links libamdhip64.so.7 by SONAME.  torch ships its own HIP
    # runtime under that SONAME; importing torch first makes the dynamic
    # linker reuse it, so device memory and streams from torch and the
    # library's launches share one runtime.
    import torch  # noqa: F401
    path = lib_path()
    if not os.path.exists(path):
        raise ImportError(f"libflashloop.so not built ({path}); run __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    S = ctypes.c_size_t
    cp = ctypes.POINTER(FlCache)
    lib.fl_abi_version.restype = I
    lib.fl_last_error.restype = ctypes.c_char_p
    lib.fl_base_record_bytes.argtypes = [I]
    lib.fl_base_record_bytes.restype = S
    lib.fl_residual_record_bytes.argtypes = [I, I]
    lib.fl_residual_record_bytes.restype = S
    lib.fl_workspace_bytes.argtypes = [I, cp, I, I, I]
    lib.fl_workspace_bytes.restype = S
    lib.fl_kv_resq.argtypes = [cp, I, P, P, I, P]
    lib.fl_kv_resq.restype = I
    lib.fl_stream_bytes.argtypes = [cp, I]
    lib.fl_stream_bytes.restype = S
    lib.fl_kv_append.argtypes = [cp, I, I, P, P, I, P]
    lib.fl_kv_append.restype = I
    lib.fl_colsel.argtypes = [cp, I, P, I, ctypes.POINTER(FlState), I, P, I, P, P, P, P, S, P]
    lib.fl_colsel.restype = I
    lib.fl_loop_attn.argtypes = [cp, I, P, I, I, P, ctypes.POINTER(FlState), P, S, P]
    lib.fl_loop_attn.restype = I
    lib.fl_loop_attn_noalloc.argtypes = [cp, I, P, I, I, P, ctypes.POINTER(FlState), P]
    lib.fl_loop_attn_noalloc.restype = I
    lib.fl_loop_decode.argtypes = [cp, I, P, I, I, I, ctypes.POINTER(FlDState), P, S, P]
    lib.fl_loop_decode.restype = I
    lib.fl_timing_enable.argtypes = [I]
    lib.fl_timing_enable.restype = None
    lib.fl_timing_collect.argtypes = [P, P, I]
    lib.fl_timing_collect.restype = I
    lib.fl_select_active.argtypes = [I, I, I, P, P, I, I, P, I, P, P, P]
    lib.fl_select_active.restype = I
    return lib


_lib = _load()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn, status):
    if status != 0:
        raise FlashLoopError(fn, status, _lib.fl_last_error().decode())


def fl_abi_version() -> int:
    return _lib.fl_abi_version()


def fl_last_error() -> str:
    return _lib.fl_last_error().decode()


def fl_base_record_bytes(d: int) -> int:
    return _lib.fl_base_record_bytes(d)


def fl_residual_record_bytes(d: int, bits: int) -> int:
    return _lib.fl_residual_record_bytes(d, bits)


def fl_workspace_bytes(which: int, cache: FlCache, r: int, K_prev: int, K_r: int) -> int:
    return _lib.fl_workspace_bytes(which, ctypes.byref(cache), r, K_prev, K_r)


def fl_kv_resq(cache: FlCache, r: int, k, v, dtype: int, stream=None) -> None:
    _check("fl_kv_resq", _lib.fl_kv_resq(ctypes.byref(cache), r, _ptr(k), _ptr(v), dtype, _stream(stream)))


def fl_stream_bytes(cache: FlCache, r: int) -> int:
    return _lib.fl_stream_bytes(ctypes.byref(cache), r)


def fl_kv_append(cache: FlCache, r: int, pos: int, k, v, dtype: int, stream=None) -> None:
    _check("fl_kv_append", _lib.fl_kv_append(ctypes.byref(cache), r, pos, _ptr(k), _ptr(v), dtype, _stream(stream)))


def fl_colsel(cache: FlCache, r: int, q_prev, dtype: int, state: FlState, K_prev: int, cand, K_r: int,
              mass_in, mass_out, sel_out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    _check("fl_colsel", _lib.fl_colsel(ctypes.byref(cache), r, _ptr(q_prev), dtype, ctypes.byref(state), K_prev,
                                       _ptr(cand), K_r, _ptr(mass_in), _ptr(mass_out), _ptr(sel_out), _ptr(ws),
                                       ws_bytes, _stream(stream)))


def fl_loop_attn(cache: FlCache, r: int, q, dtype: int, K_r: int, sel, state: FlState, ws=None, ws_bytes: int = 0,
                 stream=None) -> None:
    _check("fl_loop_attn", _lib.fl_loop_attn(ctypes.byref(cache), r, _ptr(q), dtype, K_r, _ptr(sel),
                                             ctypes.byref(state), _ptr(ws), ws_bytes, _stream(stream)))


def fl_loop_attn_noalloc(cache: FlCache, r: int, q, dtype: int, K_r: int, sel, state: FlState, stream=None) -> None:
    _check("fl_loop_attn_noalloc", _lib.fl_loop_attn_noalloc(ctypes.byref(cache), r, _ptr(q), dtype, K_r, _ptr(sel),
                                                             ctypes.byref(state), _stream(stream)))


def fl_loop_decode(cache: FlCache, r: int, q, dtype: int, K_prev: int, K_r: int, state: FlDState, ws=None,
                   ws_bytes: int = 0, stream=None) -> None:
    _check("fl_loop_decode", _lib.fl_loop_decode(ctypes.byref(cache), r, _ptr(q), dtype, K_prev, K_r,
                                                 ctypes.byref(state), _ptr(ws), ws_bytes, _stream(stream)))


def fl_select_active(B: int, S: int, D: int, h_prev, h_cur, dtype: int, n_prev: int, rows_prev, k: int, rows_out,
                     score_out, stream=None) -> None:
    _check("fl_select_active", _lib.fl_select_active(B, S, D, _ptr(h_prev), _ptr(h_cur), dtype, n_prev,
                                                     _ptr(rows_prev), k, _ptr(rows_out), _ptr(score_out),
                                                     _stream(stream)))


FL_TIMING_NAME = 48


def fl_timing_enable(on: bool) -> None:
    _lib.fl_timing_enable(1 if on else 0)


def fl_timing_collect(max_records: int = 4096) -> list:
    """[(kernel name, ms), ...] of the launches recorded since the last
    collect on this thread, in launch order."""
    names = (ctypes.c_char * FL_TIMING_NAME * max_records)()
    ms = (ctypes.c_float * max_records)()
    n = _lib.fl_timing_collect(ctypes.addressof(names), ctypes.addressof(ms), max_records)
    return [(names[i].value.decode(), float(ms[i])) for i in range(n)]
