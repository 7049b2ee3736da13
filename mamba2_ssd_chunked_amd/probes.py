"""ctypes view of libssd_probe.so: the achievable-peak probes (a streaming copy
and a bf16 MFMA loop) that the roofline figures are also quoted against.
Measurement only; the SSD path does not use them."""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB_PATH = os.path.join(HERE, "libssd_probe.so")
SYMBOLS = ("ssd_probe_copy", "ssd_probe_mfma", "ssd_probe_mfma_flops")

_lib = None


def load():
    """Load libssd_probe.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(PROBE_LIB_PATH):
            raise RuntimeError(f"{PROBE_LIB_PATH} is missing: run __graft_entry__.build()")
        lib = ctypes.CDLL(PROBE_LIB_PATH)
        lib.ssd_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
        lib.ssd_probe_copy.restype = ctypes.c_int
        lib.ssd_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p]
        lib.ssd_probe_mfma.restype = ctypes.c_int
        lib.ssd_probe_mfma_flops.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32]
        lib.ssd_probe_mfma_flops.restype = ctypes.c_double
        _lib = lib
    return _lib


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise RuntimeError(f"{what} failed ({'bad arguments' if rc == -1 else 'launch error'})")


def probe_copy(src, dst, stream=None) -> None:
    """dst[:] = src[:] (byte copy of equal-sized, 16-byte aligned CUDA tensors whose
    size is a multiple of 4096 bytes)."""
    import torch
    nbytes = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nbytes and src.is_cuda and dst.is_cuda
    s = (stream or torch.cuda.current_stream()).cuda_stream
    _check(load().ssd_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, s), "ssd_probe_copy")


def probe_mfma(out, blocks: int, iters: int, shape: int = 16, stream=None) -> float:
    """Launch the MFMA loop (shape 16: 16x16x32 products, 32: 32x32x16) into out
    (float32 CUDA tensor of blocks*256); returns the flops of the launch."""
    import torch
    assert out.is_cuda and out.dtype == torch.float32 and out.numel() == blocks * 256
    s = (stream or torch.cuda.current_stream()).cuda_stream
    _check(load().ssd_probe_mfma(out.data_ptr(), blocks, iters, shape, s), "ssd_probe_mfma")
    return float(load().ssd_probe_mfma_flops(blocks, iters, shape))


def mfma_expected(iters: int, shape: int = 16) -> float:
    """Per-thread output of probe_mfma: over chains c, elements x (c + iters x K / 64^2)
    (16x16x32: 8 chains of 4 elements, K = 32; 32x32x16: 4 chains of 16, K = 16)."""
    chains, elems, k = (8, 4, 32) if shape == 16 else (4, 16, 16)
    return sum(elems * (c + iters * k / 4096.0) for c in range(chains))
