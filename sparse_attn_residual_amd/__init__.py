"""FlashLoop loop-attention hot path for MI355X (gfx950): Python binding.

The work happens in libflashloop.so (hand-written HIP kernels behind the C ABI
of include/flashloop.h).  This package only marshals arguments: torch tensors
are passed as device pointers and the current torch stream as the HIP stream.
There is no fallback: if the library is missing, importing the binding fails.
"""
from ._lib import (  # noqa: F401
    FL_BF16, FL_F32, FL_FMT_PAPER, FL_FMT_WORKLOAD, FL_MAX_LOOPS, FL_MAX_S, FL_WS_ATTN, FL_WS_COLSEL, FL_WS_DECODE,
    FlashLoopError, FlCache, FlDState, FlState,
    fl_abi_version, fl_base_record_bytes, fl_colsel, fl_kv_append, fl_kv_resq, fl_last_error, fl_loop_attn, fl_loop_attn_noalloc,
    fl_loop_decode, fl_residual_record_bytes, fl_select_active, fl_stream_bytes, fl_timing_collect, fl_timing_enable, fl_workspace_bytes, lib_path,
)
from .buffers import CacheBuffers, DecodeState, PrefillState  # noqa: F401
