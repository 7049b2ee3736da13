"""Python binding of the C ABI, one function per entry point, same names.

Torch tensors provide device memory and the stream; this module only checks
that every tensor has the size, dtype, device and contiguity the call needs
(the C ABI receives raw pointers and cannot check sizes itself) and passes
pointers through.  All computation happens in libssd's HIP kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import (SSD_BF16, SSD_F32, SSD_WS_BACKWARD, SSD_WS_FORWARD, SSD_WS_FORWARD_CONV,
                   Problem, SSDError)

_TORCH_ACT = {SSD_F32: torch.float32, SSD_BF16: torch.bfloat16}


def make_problem(*, batch: int, seqlen: int, nheads: int, headdim: int, dstate: int,
                 ngroups: int, chunk: int, conv_width: int, act: str | int,
                 dt_min: float = 1e-3, dt_max: float = 0.1) -> Problem:
    if isinstance(act, str):
        act = {"f32": SSD_F32, "float32": SSD_F32, "bf16": SSD_BF16, "bfloat16": SSD_BF16}[act]
    return Problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk, conv_width, act,
                   dt_min, dt_max)


class Segments:
    """Segment table in causal order: [(memory start, length), ...]."""

    def __init__(self, segs: Sequence[Tuple[int, int]]):
        self.list = [(int(s), int(n)) for s, n in segs]
        self.n = len(self.list)
        arr = (_lib.Segment * max(1, self.n))()
        for i, (s, n) in enumerate(self.list):
            arr[i].start = s
            arr[i].len = n
        self.arr = arr

    def ptr(self):
        return ctypes.cast(self.arr, ctypes.POINTER(_lib.Segment))


def _segs(segs) -> Segments:
    return segs if isinstance(segs, Segments) else Segments(segs)


def _conv_dim(p: Problem) -> int:
    return p.nheads * p.headdim + 2 * p.ngroups * p.dstate


def _need(t: Optional[torch.Tensor], name: str, numel: int, dtype, optional: bool = False):
    if t is None:
        if optional:
            return None
        raise ValueError(f"{name} is required")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws):
    if ws is None or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(fn: str, rc: int):
    if rc != 0:
        raise SSDError(fn, rc)


def ssd_workspace_bytes(problem: Problem, segs, kind: int = SSD_WS_FORWARD) -> int:
    s = _segs(segs)
    return int(_lib.load().ssd_workspace_bytes(ctypes.byref(problem), s.ptr(), s.n, kind))


def summary_numel(problem: Problem, nseg: int) -> int:
    bh = problem.batch * problem.nheads
    return nseg * bh * problem.headdim * problem.dstate + nseg * bh


def ssd_conv1d_fwd(problem: Problem, segs, xBC, conv_w, seq_idx, xBC_conv, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C = problem.batch * problem.seqlen, _conv_dim(problem)
    args = (_need(xBC, "xBC", BL * C, act), _need(conv_w, "conv_w", C * problem.conv_width,
                                                    torch.float32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(xBC_conv, "xBC_conv", BL * C, act))
    _check("ssd_conv1d_fwd", _lib.load().ssd_conv1d_fwd(ctypes.byref(problem), s.ptr(), s.n,
                                                        *args, _stream(stream)))


def ssd_segment_fwd(problem: Problem, segs, xBC_conv, dt_raw, dt_bias, A_log, seq_idx, y_zero,
                    summary, ws, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads
    f32 = torch.float32
    args = (_need(xBC_conv, "xBC_conv", BL * C, act), _need(dt_raw, "dt_raw", BL * H, act),
            _need(dt_bias, "dt_bias", H, f32), _need(A_log, "A_log", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(y_zero, "y_zero", BL * H * problem.headdim, f32),
            _need(summary, "summary", summary_numel(problem, s.n), f32))
    if ws is None or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    _check("ssd_segment_fwd", _lib.load().ssd_segment_fwd(
        ctypes.byref(problem), s.ptr(), s.n, *args, ctypes.c_void_p(ws.data_ptr()), nbytes,
        _stream(stream)))


def ssd_segment_fwd_noalloc(problem: Problem, segs, xBC_conv, dt_raw, dt_bias, A_log, seq_idx,
                            y_zero, summary, stream=None):
    """ssd_segment_fwd with the workspace in the library's fixed device scratch
    (nothing is allocated; overlapping calls on one GPU race)."""
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads
    f32 = torch.float32
    args = (_need(xBC_conv, "xBC_conv", BL * C, act), _need(dt_raw, "dt_raw", BL * H, act),
            _need(dt_bias, "dt_bias", H, f32), _need(A_log, "A_log", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(y_zero, "y_zero", BL * H * problem.headdim, f32),
            _need(summary, "summary", summary_numel(problem, s.n), f32))
    _check("ssd_segment_fwd_noalloc", _lib.load().ssd_segment_fwd_noalloc(
        ctypes.byref(problem), s.ptr(), s.n, *args, _stream(stream)))


def ssd_segment_states(problem: Problem, segs, xBC_conv, dt_raw, dt_bias, A_log, seq_idx,
                       summary, ws, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads
    f32 = torch.float32
    args = (_need(xBC_conv, "xBC_conv", BL * C, act), _need(dt_raw, "dt_raw", BL * H, act),
            _need(dt_bias, "dt_bias", H, f32), _need(A_log, "A_log", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(summary, "summary", summary_numel(problem, s.n), f32))
    ws_p, nbytes = _ws(ws)
    _check("ssd_segment_states", _lib.load().ssd_segment_states(
        ctypes.byref(problem), s.ptr(), s.n, *args, ws_p, nbytes, _stream(stream)))


def ssd_segment_output(problem: Problem, segs, xBC_conv, seq_idx, ws, y_zero, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads
    xp = _need(xBC_conv, "xBC_conv", BL * C, act)
    sp = _need(seq_idx, "seq_idx", BL, torch.int32, optional=True)
    ws_p, nbytes = _ws(ws)
    yp = _need(y_zero, "y_zero", BL * H * problem.headdim, torch.float32)
    _check("ssd_segment_output", _lib.load().ssd_segment_output(
        ctypes.byref(problem), s.ptr(), s.n, xp, sp, ws_p, nbytes, yp, _stream(stream)))


def ssd_boundary_scan(problem: Problem, nseg: int, summary, init, reverse: bool, out,
                      final_state=None, stream=None):
    f32 = torch.float32
    st = problem.batch * problem.nheads * problem.headdim * problem.dstate
    args = (_need(summary, "summary", summary_numel(problem, nseg), f32),
            _need(init, "init", st, f32, optional=True))
    out_p = _need(out, "out", nseg * st, f32)
    fin_p = _need(final_state, "final_state", st, f32, optional=True)
    _check("ssd_boundary_scan", _lib.load().ssd_boundary_scan(
        ctypes.byref(problem), nseg, *args, 1 if reverse else 0, out_p, fin_p, _stream(stream)))


def ssd_apply_init_state(problem: Problem, segs, y_zero, xBC_conv, D, seq_idx, S_in, ws, y,
                         stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H, P = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads, problem.headdim
    f32 = torch.float32
    args = (_need(y_zero, "y_zero", BL * H * P, f32), _need(xBC_conv, "xBC_conv", BL * C, act),
            _need(D, "D", H, f32), _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(S_in, "S_in", s.n * problem.batch * H * P * problem.dstate, f32))
    if ws is None or not ws.is_cuda or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous device tensor")
    nbytes = ws.numel() * ws.element_size()
    y_p = _need(y, "y", BL * H * P, act)
    _check("ssd_apply_init_state", _lib.load().ssd_apply_init_state(
        ctypes.byref(problem), s.ptr(), s.n, *args, ctypes.c_void_p(ws.data_ptr()), nbytes, y_p,
        _stream(stream)))


def ssd_segment_output_fused(problem: Problem, segs, xBC_conv, D, seq_idx, S_in, ws, y,
                             stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H, P = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads, problem.headdim
    f32 = torch.float32
    args = (_need(xBC_conv, "xBC_conv", BL * C, act), _need(D, "D", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(S_in, "S_in", s.n * problem.batch * H * P * problem.dstate, f32))
    ws_p, nbytes = _ws(ws)
    y_p = _need(y, "y", BL * H * P, act)
    _check("ssd_segment_output_fused", _lib.load().ssd_segment_output_fused(
        ctypes.byref(problem), s.ptr(), s.n, *args, ws_p, nbytes, y_p, _stream(stream)))


def ssd_conv_segment_states(problem: Problem, segs, xBC, conv_w, dt_raw, dt_bias, A_log, seq_idx,
                            summary, ws, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads
    f32 = torch.float32
    args = (_need(xBC, "xBC", BL * C, act),
            _need(conv_w, "conv_w", C * problem.conv_width, f32),
            _need(dt_raw, "dt_raw", BL * H, act),
            _need(dt_bias, "dt_bias", H, f32), _need(A_log, "A_log", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(summary, "summary", summary_numel(problem, s.n), f32))
    ws_p, nbytes = _ws(ws)
    _check("ssd_conv_segment_states", _lib.load().ssd_conv_segment_states(
        ctypes.byref(problem), s.ptr(), s.n, *args, ws_p, nbytes, _stream(stream)))


def ssd_conv_segment_output(problem: Problem, segs, xBC, conv_w, D, seq_idx, S_in, ws, y,
                            stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H, P = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads, problem.headdim
    f32 = torch.float32
    args = (_need(xBC, "xBC", BL * C, act),
            _need(conv_w, "conv_w", C * problem.conv_width, f32), _need(D, "D", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(S_in, "S_in", s.n * problem.batch * H * P * problem.dstate, f32))
    ws_p, nbytes = _ws(ws)
    y_p = _need(y, "y", BL * H * P, act)
    _check("ssd_conv_segment_output", _lib.load().ssd_conv_segment_output(
        ctypes.byref(problem), s.ptr(), s.n, *args, ws_p, nbytes, y_p, _stream(stream)))


def ssd_segment_bwd_summary(problem: Problem, segs, xBC, conv_w, dt_raw, dt_bias, A_log, seq_idx,
                            dy, summary, ws, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H, P = problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads, problem.headdim
    f32 = torch.float32
    args = (_need(xBC, "xBC", BL * C, act),
            _need(conv_w, "conv_w", C * problem.conv_width, f32),
            _need(dt_raw, "dt_raw", BL * H, act), _need(dt_bias, "dt_bias", H, f32),
            _need(A_log, "A_log", H, f32),
            _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
            _need(dy, "dy", BL * H * P, act),
            _need(summary, "summary", summary_numel(problem, s.n), f32))
    ws_p, nbytes = _ws(ws)
    _check("ssd_segment_bwd_summary", _lib.load().ssd_segment_bwd_summary(
        ctypes.byref(problem), s.ptr(), s.n, *args, ws_p, nbytes, _stream(stream)))


def ssd_segment_bwd(problem: Problem, segs, xBC, conv_w, dt_raw, dt_bias, A_log, D, seq_idx, dy,
                    S_in, dS_out, ws, dxBC, ddt_raw, dconv_w, ddt_bias, dA_log, dD, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H, P, N = (problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads,
                      problem.headdim, problem.dstate)
    f32 = torch.float32
    W = problem.conv_width
    st = s.n * problem.batch * H * P * N
    ins = (_need(xBC, "xBC", BL * C, act), _need(conv_w, "conv_w", C * W, f32),
           _need(dt_raw, "dt_raw", BL * H, act), _need(dt_bias, "dt_bias", H, f32),
           _need(A_log, "A_log", H, f32), _need(D, "D", H, f32),
           _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
           _need(dy, "dy", BL * H * P, act), _need(S_in, "S_in", st, f32),
           _need(dS_out, "dS_out", st, f32))
    ws_p, nbytes = _ws(ws)
    outs = (_need(dxBC, "dxBC", BL * C, act), _need(ddt_raw, "ddt_raw", BL * H, act),
            _need(dconv_w, "dconv_w", C * W, f32), _need(ddt_bias, "ddt_bias", H, f32),
            _need(dA_log, "dA_log", H, f32), _need(dD, "dD", H, f32))
    _check("ssd_segment_bwd", _lib.load().ssd_segment_bwd(
        ctypes.byref(problem), s.ptr(), s.n, *ins, ws_p, nbytes, *outs, _stream(stream)))


def ssd_segment_bwd_pass(problem: Problem, segs, seq_idx, dy, S_in, dS_out, ws, stream=None):
    s = _segs(segs)
    st = s.n * problem.batch * problem.nheads * problem.headdim * problem.dstate
    f32 = torch.float32
    act = _TORCH_ACT[problem.act_dtype]
    BL = problem.batch * problem.seqlen
    ins = (_need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
           _need(dy, "dy", BL * problem.nheads * problem.headdim, act),
           _need(S_in, "S_in", st, f32), _need(dS_out, "dS_out", st, f32))
    ws_p, nbytes = _ws(ws)
    _check("ssd_segment_bwd_pass", _lib.load().ssd_segment_bwd_pass(
        ctypes.byref(problem), s.ptr(), s.n, *ins, ws_p, nbytes, _stream(stream)))


def ssd_segment_bwd_chunks(problem: Problem, segs, D, seq_idx, dy, ws, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, H, P = problem.batch * problem.seqlen, problem.nheads, problem.headdim
    ins = (_need(D, "D", H, torch.float32),
           _need(seq_idx, "seq_idx", BL, torch.int32, optional=True),
           _need(dy, "dy", BL * H * P, act))
    ws_p, nbytes = _ws(ws)
    _check("ssd_segment_bwd_chunks", _lib.load().ssd_segment_bwd_chunks(
        ctypes.byref(problem), s.ptr(), s.n, *ins, ws_p, nbytes, _stream(stream)))


def ssd_conv1d_bwd(problem: Problem, segs, xBC, conv_w, dt_raw, dt_bias, A_log, seq_idx, ws, dxBC,
                   ddt_raw, dconv_w, ddt_bias, dA_log, dD, stream=None):
    s = _segs(segs)
    act = _TORCH_ACT[problem.act_dtype]
    BL, C, H, W = (problem.batch * problem.seqlen, _conv_dim(problem), problem.nheads,
                   problem.conv_width)
    f32 = torch.float32
    ins = (_need(xBC, "xBC", BL * C, act), _need(conv_w, "conv_w", C * W, f32),
           _need(dt_raw, "dt_raw", BL * H, act), _need(dt_bias, "dt_bias", H, f32),
           _need(A_log, "A_log", H, f32),
           _need(seq_idx, "seq_idx", BL, torch.int32, optional=True))
    ws_p, nbytes = _ws(ws)
    outs = (_need(dxBC, "dxBC", BL * C, act), _need(ddt_raw, "ddt_raw", BL * H, act),
            _need(dconv_w, "dconv_w", C * W, f32), _need(ddt_bias, "ddt_bias", H, f32),
            _need(dA_log, "dA_log", H, f32), _need(dD, "dD", H, f32))
    _check("ssd_conv1d_bwd", _lib.load().ssd_conv1d_bwd(
        ctypes.byref(problem), s.ptr(), s.n, *ins, ws_p, nbytes, *outs, _stream(stream)))


# ---------------------------------------------------------------------------
# Convenience: buffers for one forward pass and the four calls in order.


@dataclass
class ForwardBuffers:
    xBC_conv: torch.Tensor
    y_zero: torch.Tensor
    summary: torch.Tensor
    S_in: torch.Tensor
    ws: torch.Tensor
    y: torch.Tensor
    final_state: torch.Tensor  # [b][H][P][N] float32, the state after each row's last token

    @staticmethod
    def allocate(problem: Problem, segs, device) -> "ForwardBuffers":
        s = _segs(segs)
        act = _TORCH_ACT[problem.act_dtype]
        b, L, H, P, N = (problem.batch, problem.seqlen, problem.nheads, problem.headdim,
                         problem.dstate)
        C = _conv_dim(problem)
        wsb = ssd_workspace_bytes(problem, s, SSD_WS_FORWARD)
        if wsb == 0:
            raise SSDError("ssd_workspace_bytes", -2)
        # room for the conv-fused forward too, where it is compiled (width 4)
        wsb = max(wsb, ssd_workspace_bytes(problem, s, SSD_WS_FORWARD_CONV))
        return ForwardBuffers(
            xBC_conv=torch.empty((b, L, C), dtype=act, device=device),
            y_zero=torch.empty((b, L, H, P), dtype=torch.float32, device=device),
            summary=torch.empty(summary_numel(problem, s.n), dtype=torch.float32, device=device),
            S_in=torch.empty((s.n, b, H, P, N), dtype=torch.float32, device=device),
            ws=torch.empty(wsb, dtype=torch.uint8, device=device),
            y=torch.empty((b, L, H, P), dtype=act, device=device),
            final_state=torch.empty((b, H, P, N), dtype=torch.float32, device=device))


def forward(problem: Problem, segs, xBC, conv_w, dt_raw, dt_bias, A_log, D, seq_idx=None,
            init=None, bufs: Optional[ForwardBuffers] = None, stream=None,
            fused: bool = True, want_final: bool = False,
            conv_fused: bool = False) -> ForwardBuffers:
    """The forward path; returns the buffers.

    conv_fused=True: conv-fused segment states -> boundary scan -> conv-fused
                 output pass (the conv runs inside the two phases; y only,
                 bufs.xBC_conv and bufs.y_zero are left untouched).
    fused=True : conv1d -> segment states -> boundary scan -> fused output pass
                 (y only; bufs.y_zero is left untouched).
    fused=False: conv1d -> segment-local SSD (states and y_zero) -> boundary scan
                 -> correction pass.
    init       : optional [b][H][P][N] float32 state before each row's first token.
    want_final : also write bufs.final_state (the boundary scan's final state).
    """
    s = _segs(segs)
    if bufs is None:
        bufs = ForwardBuffers.allocate(problem, s, xBC.device)
    if conv_fused:
        ssd_conv_segment_states(problem, s, xBC, conv_w, dt_raw, dt_bias, A_log, seq_idx,
                                bufs.summary, bufs.ws, stream)
        ssd_boundary_scan(problem, s.n, bufs.summary, init, False, bufs.S_in,
                          bufs.final_state if want_final else None, stream)
        ssd_conv_segment_output(problem, s, xBC, conv_w, D, seq_idx, bufs.S_in, bufs.ws, bufs.y,
                                stream)
        return bufs
    ssd_conv1d_fwd(problem, s, xBC, conv_w, seq_idx, bufs.xBC_conv, stream)
    if fused:
        ssd_segment_states(problem, s, bufs.xBC_conv, dt_raw, dt_bias, A_log, seq_idx,
                           bufs.summary, bufs.ws, stream)
        ssd_boundary_scan(problem, s.n, bufs.summary, init, False, bufs.S_in,
                          bufs.final_state if want_final else None, stream)
        ssd_segment_output_fused(problem, s, bufs.xBC_conv, D, seq_idx, bufs.S_in, bufs.ws,
                                 bufs.y, stream)
        return bufs
    ssd_segment_fwd(problem, s, bufs.xBC_conv, dt_raw, dt_bias, A_log, seq_idx, bufs.y_zero,
                    bufs.summary, bufs.ws, stream)
    ssd_boundary_scan(problem, s.n, bufs.summary, init, False, bufs.S_in,
                      bufs.final_state if want_final else None, stream)
    ssd_apply_init_state(problem, s, bufs.y_zero, bufs.xBC_conv, D, seq_idx, bufs.S_in, bufs.ws,
                         bufs.y, stream)
    return bufs


@dataclass
class BackwardBuffers:
    summary: torch.Tensor
    dS_out: torch.Tensor
    ws: torch.Tensor
    dxBC: torch.Tensor
    ddt_raw: torch.Tensor
    dconv_w: torch.Tensor
    ddt_bias: torch.Tensor
    dA_log: torch.Tensor
    dD: torch.Tensor
    dinit: torch.Tensor  # [b][H][P][N] float32, gradient of the initial state

    @staticmethod
    def allocate(problem: Problem, segs, device) -> "BackwardBuffers":
        s = _segs(segs)
        act = _TORCH_ACT[problem.act_dtype]
        b, L, H, P, N = (problem.batch, problem.seqlen, problem.nheads, problem.headdim,
                         problem.dstate)
        C, W = _conv_dim(problem), problem.conv_width
        wsb = ssd_workspace_bytes(problem, s, SSD_WS_BACKWARD)
        if wsb == 0:
            raise SSDError("ssd_workspace_bytes", -3)
        f32 = torch.float32
        return BackwardBuffers(
            summary=torch.empty(summary_numel(problem, s.n), dtype=f32, device=device),
            dS_out=torch.empty((s.n, b, H, P, N), dtype=f32, device=device),
            ws=torch.empty(wsb, dtype=torch.uint8, device=device),
            dxBC=torch.empty((b, L, C), dtype=act, device=device),
            ddt_raw=torch.empty((b, L, H), dtype=act, device=device),
            dconv_w=torch.empty((C, W), dtype=f32, device=device),
            ddt_bias=torch.empty(H, dtype=f32, device=device),
            dA_log=torch.empty(H, dtype=f32, device=device),
            dD=torch.empty(H, dtype=f32, device=device),
            dinit=torch.empty((b, H, P, N), dtype=f32, device=device))


def backward(problem: Problem, segs, xBC, conv_w, dt_raw, dt_bias, A_log, D, dy, S_in,
             seq_idx=None, bufs: Optional[BackwardBuffers] = None, stream=None,
             dfinal=None, want_dinit: bool = False) -> BackwardBuffers:
    """Summary phase -> reverse boundary scan -> segment phase; returns the buffers.

    ``S_in`` is the forward boundary scan's output (ForwardBuffers.S_in).
    dfinal     : optional [b][H][P][N] float32 gradient of the final state (the
                 reverse scan starts from it).
    want_dinit : also write bufs.dinit, the gradient of the forward's initial state.
    """
    s = _segs(segs)
    if bufs is None:
        bufs = BackwardBuffers.allocate(problem, s, xBC.device)
    ssd_segment_bwd_summary(problem, s, xBC, conv_w, dt_raw, dt_bias, A_log, seq_idx, dy,
                            bufs.summary, bufs.ws, stream)
    ssd_boundary_scan(problem, s.n, bufs.summary, dfinal, True, bufs.dS_out,
                      bufs.dinit if want_dinit else None, stream)
    ssd_segment_bwd(problem, s, xBC, conv_w, dt_raw, dt_bias, A_log, D, seq_idx, dy, S_in,
                    bufs.dS_out, bufs.ws, bufs.dxBC, bufs.ddt_raw, bufs.dconv_w, bufs.ddt_bias,
                    bufs.dA_log, bufs.dD, stream)
    return bufs
