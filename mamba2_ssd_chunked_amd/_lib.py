"""ctypes view of libssd.so (the C ABI in include/ssd.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  There is no CPU fallback; if the library cannot be loaded the
import of any op raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libssd.so")

SSD_F32 = 0
SSD_BF16 = 1
SSD_WS_FORWARD = 0
SSD_WS_BACKWARD = 1
SSD_WS_FORWARD_CONV = 2
SSD_MAX_SEGMENTS = 64
SSD_SCRATCH_BYTES = 64 << 20


class Problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int32), ("headdim", ctypes.c_int32),
                ("dstate", ctypes.c_int32), ("ngroups", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("conv_width", ctypes.c_int32),
                ("act_dtype", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


class Segment(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int64)]


_vp = ctypes.c_void_p
_PP = ctypes.POINTER(Problem)
_SP = ctypes.POINTER(Segment)
_i32 = ctypes.c_int32

# name -> (restype, argtypes)
SIGNATURES = {
    "ssd_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "ssd_abi_version": (ctypes.c_int32, []),
    "ssd_supported": (ctypes.c_int32, [_i32, _i32, _i32]),
    "ssd_workspace_bytes": (ctypes.c_size_t, [_PP, _SP, _i32, _i32]),
    "ssd_conv1d_fwd": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp]),
    "ssd_segment_fwd": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       ctypes.c_size_t, _vp]),
    "ssd_segment_states": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          ctypes.c_size_t, _vp]),
    "ssd_segment_output": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, ctypes.c_size_t, _vp,
                                          _vp]),
    "ssd_boundary_scan": (ctypes.c_int, [_PP, _i32, _vp, _vp, _i32, _vp, _vp, _vp]),
    "ssd_segment_bwd_summary": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, ctypes.c_size_t, _vp]),
    "ssd_segment_bwd": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp, _vp, ctypes.c_size_t, _vp, _vp, _vp, _vp, _vp,
                                       _vp, _vp]),
    "ssd_segment_bwd_pass": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp]),
    "ssd_segment_bwd_chunks": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                              _vp]),
    "ssd_conv1d_bwd": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                      ctypes.c_size_t, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "ssd_apply_init_state": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                            ctypes.c_size_t, _vp, _vp]),
    "ssd_segment_output_fused": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp,
                                                ctypes.c_size_t, _vp, _vp]),
    "ssd_segment_fwd_noalloc": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp]),
    "ssd_conv_segment_states": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                               _vp, ctypes.c_size_t, _vp]),
    "ssd_conv_segment_output": (ctypes.c_int, [_PP, _SP, _i32, _vp, _vp, _vp, _vp, _vp, _vp,
                                               ctypes.c_size_t, _vp, _vp]),
}

_lib = None
_lock = threading.Lock()


def load():
    """Load libssd.so, building it first if no build is present."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            from . import build as _build
            _build.build()
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
        return lib


class SSDError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = load().ssd_status_string(status).decode()
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status
