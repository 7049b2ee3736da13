"""Every shape the library accepts, run on the GPU against the oracle.

The support table (activation dtype, headdim, dstate, chunk) is read from the
library itself (ssd_workspace_bytes accepts or refuses each combination; the CPU
test test_abi_cpu.py pins that table), and every accepted combination runs a
small forward, and a forward + backward where the backward accepts it, with a
packed-sequence reset inside a segment.  Every conv width 1..8 runs at two
shapes.  Tolerances as everywhere: float32 max relative error 1e-4 (floored at
the RMS), bf16 relative RMS error 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_workloads as W
from ssd_testlib import assert_close, device_inputs, log, problem_of, to_np

pytestmark = pytest.mark.gpu

GRADS = ["dxBC", "dconv_w", "ddt_raw", "ddt_bias", "dA_log", "dD"]


def _accepted():
    import mamba2_ssd_chunked_amd as ssd
    out = []
    for act in ("f32", "bf16"):
        for P in (16, 32, 64, 128):
            for N in (16, 32, 64, 128):
                for Q in (64, 128, 256):
                    p = ssd.make_problem(batch=1, seqlen=4 * Q, nheads=4, headdim=P, dstate=N,
                                         ngroups=2, chunk=Q, conv_width=4, act=act)
                    segs = [(0, 2 * Q), (2 * Q, 2 * Q)]
                    if ssd.ssd_workspace_bytes(p, segs, ssd.SSD_WS_FORWARD):
                        bwd = ssd.ssd_workspace_bytes(p, segs, ssd.SSD_WS_BACKWARD) > 0
                        out.append((act, P, N, Q, bwd))
    return out


SHAPES = _accepted()


def _workload(act, P, N, Q, W_=4, seed=0):
    L = 4 * Q
    # a reset inside the first segment and one inside the second
    lengths = [Q // 2 + 3, 2 * Q, L - (Q // 2 + 3) - 2 * Q]
    return W.make_workload(f"shape_{act}_{P}_{N}_{Q}_w{W_}", batch=1, seqlen=L, nheads=4,
                           headdim=P, dstate=N, ngroups=2, chunk=Q, conv_width=W_, act=act,
                           seed=900 + seed, seg_lens=[2 * Q, 2 * Q], lengths=lengths,
                           with_dy=True)


def _run(wl, bwd):
    import mamba2_ssd_chunked_amd as ssd
    p = problem_of(wl)
    x = device_inputs(wl)
    fb = ssd.forward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                     x["A_log"], x["D"], x["seq_idx"])
    bb = None
    if bwd:
        bb = ssd.backward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                          x["A_log"], x["D"], x["dy"], fb.S_in, seq_idx=x["seq_idx"])
    torch.cuda.synchronize()
    ref = oracle.backward(wl)
    assert_close(to_np(fb.y), ref["y"], wl.act, "y")
    if bb is None:
        return
    got = dict(dxBC=to_np(bb.dxBC), dconv_w=to_np(bb.dconv_w), ddt_raw=to_np(bb.ddt_raw),
               ddt_bias=to_np(bb.ddt_bias), dA_log=to_np(bb.dA_log), dD=to_np(bb.dD))
    for name in GRADS:
        assert_close(got[name], ref[name], wl.act, name)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s[0]}-P{s[1]}-N{s[2]}-Q{s[3]}"
                         + ("-bwd" if s[4] else "-fwd"))
def test_every_accepted_shape(shape):
    act, P, N, Q, bwd = shape
    wl = _workload(act, P, N, Q, seed=P + N + Q)
    log(f"[shape] act={act} P={P} N={N} Q={Q} backward={bwd}")
    _run(wl, bwd)


@pytest.mark.parametrize("width", range(1, 9))
@pytest.mark.parametrize("act,P,N,Q", [("f32", 16, 16, 64), ("bf16", 64, 128, 128)])
def test_every_conv_width(width, act, P, N, Q):
    wl = _workload(act, P, N, Q, W_=width, seed=width)
    log(f"[conv width] W={width} act={act} P={P} N={N} Q={Q}")
    _run(wl, True)
