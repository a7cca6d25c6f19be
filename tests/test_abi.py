"""Host-side checks of the C ABI: exported symbols, struct layout, and the
validation layer (every call below fails validation, so nothing launches)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashloop.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(fl_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    import sparse_attn_residual_amd as fl
    lib = ctypes.CDLL(fl.lib_path())
    names = _declared()
    assert {"fl_kv_resq", "fl_colsel", "fl_loop_attn", "fl_loop_decode", "fl_select_active"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_layout_matches_c(tmp_path):
    import sparse_attn_residual_amd as fl
    prog = tmp_path / "layout.c"
    prog.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "flashloop.h"\n'
                    'int main(void){printf("%zu %zu %zu %zu %zu %zu %zu %zu\\n", sizeof(fl_cache),'
                    'offsetof(fl_cache,n), offsetof(fl_cache,rows), offsetof(fl_cache,slot),'
                    'offsetof(fl_cache,base), offsetof(fl_cache,res), sizeof(fl_state), sizeof(fl_dstate));return 0;}\n')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-I", os.path.dirname(HEADER), str(prog), "-o", str(exe)], check=True)
    got = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    C = fl.FlCache
    want = [ctypes.sizeof(C), C.n.offset, C.rows.offset, C.slot.offset, C.base.offset, C.res.offset,
            ctypes.sizeof(fl.FlState), ctypes.sizeof(fl.FlDState)]
    assert got == want


def _cache(**kw):
    import sparse_attn_residual_amd as fl
    c = fl.FlCache()
    c.L, c.B, c.H, c.S, c.d, c.R = 1, 1, 2, 64, 64, 2
    c.n[1], c.n[2] = 64, 32
    c.bits[1], c.bits[2] = 8, 4
    c.base = 0x10000
    c.rows[2] = c.slot[2] = 0x20000
    c.res[2] = 0x30000
    for k, v in kw.items():
        setattr(c, k, v)
    return c


def _status(fn, *args):
    import sparse_attn_residual_amd as fl
    lib = fl._lib._lib
    return getattr(lib, fn)(*args), fl.fl_last_error()


def test_validation_errors():
    import sparse_attn_residual_amd as fl
    EINVAL, EUNSUP = 1, 2
    ok_ptr = 0x40000
    st, msg = _status("fl_kv_resq", None, 1, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "cache is NULL" in msg
    st, msg = _status("fl_kv_resq", ctypes.byref(_cache(d=96)), 1, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EUNSUP and "head dim" in msg
    st, msg = _status("fl_kv_resq", ctypes.byref(_cache()), 3, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "outside" in msg
    bad = _cache()
    bad.bits[2] = 3
    st, msg = _status("fl_kv_resq", ctypes.byref(bad), 2, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EUNSUP and "bits" in msg
    st, msg = _status("fl_kv_resq", ctypes.byref(_cache()), 1, ok_ptr + 4, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "aligned" in msg
    st, msg = _status("fl_kv_resq", ctypes.byref(_cache()), 1, ok_ptr, ok_ptr, 7, None)
    assert st == EUNSUP and "dtype" in msg
    nest = _cache()
    nest.n[2] = 65
    st, msg = _status("fl_kv_resq", ctypes.byref(nest), 1, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "nested" in msg
    # appending: the position must lie in the cache, a residual row needs counts
    st, msg = _status("fl_kv_append", ctypes.byref(_cache()), 1, 64, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "pos" in msg
    st, msg = _status("fl_kv_append", ctypes.byref(_cache()), 2, 63, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "cnt" in msg
    st, msg = _status("fl_kv_append", ctypes.byref(_cache(T=65)), 1, 3, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "T =" in msg
    # a per-sequence count array must be 4-byte aligned
    rc = _cache()
    rc.cnt[2] = ok_ptr + 2
    st, msg = _status("fl_kv_resq", ctypes.byref(rc), 2, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "cnt" in msg
    # key/value heads must divide the query heads
    st, msg = _status("fl_kv_resq", ctypes.byref(_cache(Hkv=3)), 1, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EINVAL and "Hkv" in msg
    # sequences longer than FL_MAX_S tokens are refused before any launch
    long_c = _cache(S=fl.FL_MAX_S + 64)
    long_c.n[1] = long_c.S
    st, msg = _status("fl_kv_resq", ctypes.byref(long_c), 1, ok_ptr, ok_ptr, fl.FL_F32, None)
    assert st == EUNSUP and "FL_MAX_S" in msg
    s = fl.FlState(ok_ptr, ok_ptr, ok_ptr, ok_ptr)
    st, msg = _status("fl_colsel", ctypes.byref(_cache()), 2, ok_ptr, fl.FL_F32, ctypes.byref(s), 64, None, 65,
                      None, None, ok_ptr, None, 0, None)
    assert st == EINVAL and "K_r" in msg
    st, msg = _status("fl_colsel", ctypes.byref(_cache()), 2, ok_ptr, fl.FL_F32, ctypes.byref(s), 64, None, 10,
                      None, None, ok_ptr, None, 0, None)
    assert st == EINVAL and "workspace" in msg
    bad = fl.FlState(ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr + 2)
    st, msg = _status("fl_loop_attn", ctypes.byref(_cache()), 2, ok_ptr, fl.FL_F32, 10, ok_ptr, ctypes.byref(bad),
                      None, 0, None)
    assert st == EINVAL and "lsel" in msg
    st, msg = _status("fl_colsel", ctypes.byref(_cache()), 1, ok_ptr, fl.FL_F32, ctypes.byref(s), 64, None, 10,
                      None, None, ok_ptr, None, 0, None)
    assert st == EINVAL
    st, msg = _status("fl_loop_attn", ctypes.byref(_cache()), 2, ok_ptr, fl.FL_F32, 10, None, ctypes.byref(s),
                      None, 0, None)
    assert st == EINVAL and "sel" in msg
    # loop 1 (bf16, head dim 128) needs the tile images of every position
    # whatever K_r holds: a negative K_r must not shrink the requirement
    c1 = _cache(d=128)
    assert fl.fl_workspace_bytes(fl.FL_WS_ATTN, c1, 1, -1, -1) == 1 * 2 * 1 * 36864
    for kr in (-1, 0, 5):
        st, msg = _status("fl_loop_attn", ctypes.byref(c1), 1, ok_ptr, fl.FL_BF16, kr, None, ctypes.byref(s),
                          None, 0, None)
        assert st == EINVAL and "workspace" in msg, (kr, msg)
    ds = fl.FlDState(ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr, ok_ptr)
    st, msg = _status("fl_loop_decode", ctypes.byref(_cache()), 1, ok_ptr, fl.FL_F32, 64, 64, ctypes.byref(ds),
                      None, 0, None)
    assert st == EUNSUP and "decode" in msg   # head dim 64
    c128 = _cache(d=128)
    st, msg = _status("fl_loop_decode", ctypes.byref(c128), 2, ok_ptr, fl.FL_F32, 30, 10, ctypes.byref(ds),
                      None, 0, None)
    assert st == EINVAL and "K_prev" in msg
    assert fl.fl_workspace_bytes(fl.FL_WS_COLSEL, _cache(), 2, 64, 10) == 1 * 2 * 64 * 4
    # head dim 128: masses, the masses' 2048-bin histogram per head, then the
    # larger of the mass pass's 64-row images (18 KiB each) and the
    # cached-mass pass's 64-column tiles (36 KiB each)
    assert fl.fl_workspace_bytes(fl.FL_WS_COLSEL, c128, 2, 64, 10) == 512 + 2 * 2048 * 4 + 2 * 36864
    c128.n[2] = 64 * 5
    c128.S = c128.n[1] = 64 * 5
    assert fl.fl_workspace_bytes(fl.FL_WS_COLSEL, c128, 2, 320, 10) == 2 * 320 * 4 + 2 * 2048 * 4 + 2 * 5 * 18432
    # a pruning selection takes at most 32768 candidates
    big = _cache(S=40000)
    big.n[1], big.n[2] = 40000, 20000
    st, msg = _status("fl_colsel", ctypes.byref(big), 2, ok_ptr, fl.FL_F32, ctypes.byref(s), 40000, None, 10,
                      None, None, ok_ptr, ok_ptr, 1 << 40, None)
    assert st == EUNSUP and "candidates" in msg
    # active-set selection
    st, msg = _status("fl_select_active", 1, 64, 12, ok_ptr, ok_ptr, fl.FL_F32, 64, None, 10, ok_ptr, ok_ptr, None)
    assert st == EUNSUP and "hidden size" in msg
    st, msg = _status("fl_select_active", 1, 64, 16, ok_ptr, ok_ptr, fl.FL_F32, 32, None, 10, ok_ptr, ok_ptr, None)
    assert st == EINVAL and "rows_prev is NULL" in msg
    st, msg = _status("fl_select_active", 1, 64, 16, ok_ptr, ok_ptr, fl.FL_F32, 64, None, 65, ok_ptr, ok_ptr, None)
    assert st == EINVAL and "k = 65" in msg
    st, msg = _status("fl_select_active", 1, 64, 16, ok_ptr + 4, ok_ptr, fl.FL_F32, 64, None, 10, ok_ptr, ok_ptr,
                      None)
    assert st == EINVAL and "h_prev" in msg
    st, msg = _status("fl_select_active", 1, 40000, 16, ok_ptr, ok_ptr, fl.FL_F32, 40000, None, 10, ok_ptr, ok_ptr,
                      None)
    assert st == EUNSUP and "candidates" in msg


def test_binding_raises():
    import sparse_attn_residual_amd as fl
    with pytest.raises(fl.FlashLoopError) as ei:
        fl.fl_kv_resq(_cache(d=96), 1, 0x40000, 0x40000, fl.FL_F32, stream=0)
    assert ei.value.status == 2


def test_validation_layer_under_address_sanitizer(tmp_path):
    """abi.cpp's argument checks and the FL_CHECK index validator, built with
    AddressSanitizer against a host stand-in of the launch layer
    (tests/abi_host): every refused call launches nothing and returns
    FL_EINVAL with an FL_CHECK message; valid index data passes; no memory
    error is reported.  CPU only: host arrays play the device buffers."""
    here = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_host")
    csrc = os.path.join(ROOT, "sparse_attn_residual_amd", "csrc")
    exe = tmp_path / "abi_harness"
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    cmd = [hipcc, "-x", "hip", "--offload-host-only", "-std=c++17", "-O1", "-g",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer",
           "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "abi.cpp"), os.path.join(here, "stub_launch.cpp"), os.path.join(here, "harness.cpp"),
           "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0")
    env.pop("FL_CHECK", None)
    res = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "PASS" in res.stdout and "AddressSanitizer" not in res.stderr, res.stdout + res.stderr


def test_noalloc_refuses_oversized_call_on_host():
    """fl_loop_attn_noalloc checks its scratch need before touching a device:
    a 32K, 16-head dense loop 1 (302 MB of tile images) is refused with
    FL_EUNSUPPORTED, naming the array's size."""
    import sparse_attn_residual_amd as fl
    c = _cache(d=128, H=16, S=32768, R=1)
    c.n[1] = 32768
    s = fl.FlState(0x40000, 0x40000, 0x40000, 0x40000)
    st, msg = _status("fl_loop_attn_noalloc", ctypes.byref(c), 1, 0x40000, fl.FL_BF16, 0, None, ctypes.byref(s), None)
    assert st == 2 and "FL_NOALLOC_SCRATCH_BYTES" in msg, msg
