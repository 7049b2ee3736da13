"""Initial state in, final state out, and their gradients, through the C ABI, against
the CPU oracle; and the whole forward + backward replayed from a captured HIP graph,
bitwise equal to the eager run.

The initial state is the state before each row's first token (it feeds the row's first
packed sequence); the final state is the state after the row's last token in causal
order.  Their gradients: ``dinit`` = dL/d(initial state) for L = <dy, y> + <dfinal,
final state>, ``dfinal`` given.  The oracle's recurrence takes ``init`` and returns the
final state and dL/d(init) for dfinal = 0; the dfinal path is pinned by central
differences of the oracle's final state.
"""
import copy

import numpy as np
import pytest
import torch

import oracle
import ssd_workloads as W
from ssd_testlib import (assert_close, device_inputs, log, oracle_v, problem_of, to_np)
from test_gpu_backward import GRADS, _bwd_small, gpu_grads

pytestmark = pytest.mark.gpu

CASES = ["tiny_f32", "slow_tiny_f32", "f32_virtual", "bf16_small", "bf16_thd", "bf16_q64"]


def _state(wl, seed, scale=0.5):
    rng = np.random.default_rng(seed)
    return (scale * rng.standard_normal((wl.batch, wl.nheads, wl.headdim, wl.dstate))
            ).astype(np.float32)


def _kw(wl):
    return dict(nheads=wl.nheads, headdim=wl.headdim, dstate=wl.dstate, ngroups=wl.ngroups,
                dt_min=wl.dt_min, dt_max=wl.dt_max, seq_idx=wl.causal_seq_idx())


def _run(wl, init, dfinal=None, fused=True):
    import mamba2_ssd_chunked_amd as ssd
    p = problem_of(wl)
    x = device_inputs(wl)
    dev = x["xBC"].device
    ini = torch.from_numpy(init).to(dev)
    fb = ssd.forward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                     x["A_log"], x["D"], x["seq_idx"], init=ini, fused=fused, want_final=True)
    bb = None
    if "dy" in x:
        dfin = None if dfinal is None else torch.from_numpy(dfinal).to(dev)
        bb = ssd.backward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                          x["A_log"], x["D"], x["dy"], fb.S_in, seq_idx=x["seq_idx"],
                          dfinal=dfin, want_dinit=True)
    torch.cuda.synchronize()
    return fb, bb


@pytest.mark.parametrize("case", CASES)
def test_forward_initial_and_final_state(case):
    wl = _bwd_small(case)
    log(f"[state io] forward {wl.name}")
    init = _state(wl, 11)
    v = oracle_v(wl)
    y_o, fin_o = oracle.ssd_fwd(v, wl.to_causal(wl.dt_raw), wl.dt_bias, wl.A_log, wl.D,
                                init=init.astype(np.float64), want_final=True, **_kw(wl))
    for fused in (True, False):
        fb, _ = _run(wl, init, fused=fused)
        assert_close(wl.to_causal(to_np(fb.y)), y_o, wl.act, f"y with init (fused={fused})")
        assert_close(to_np(fb.final_state), fin_o, wl.act, f"final state (fused={fused})")


@pytest.mark.parametrize("case", CASES)
def test_backward_with_initial_state(case):
    """All gradients and dL/d(init) when the forward starts from a nonzero state."""
    wl = _bwd_small(case)
    log(f"[state io] backward {wl.name}")
    init = _state(wl, 12)
    fb, bb = _run(wl, init)
    xBC = wl.to_causal(wl.xBC)
    seq = wl.causal_seq_idx()
    _, v = oracle.conv_silu(xBC, wl.conv_w, seq)
    g = oracle.ssd_bwd(v, wl.to_causal(wl.dt_raw), wl.dt_bias, wl.A_log, wl.D,
                       wl.to_causal(wl.dy), init=init.astype(np.float64), want_dinit=True,
                       **_kw(wl))
    dxBC, dw = oracle.conv_silu_bwd(xBC, wl.conv_w, g["dv"], seq)
    ref = dict(dxBC=dxBC, dconv_w=dw, ddt_raw=g["ddt_raw"], ddt_bias=g["ddt_bias"],
               dA_log=g["dA_log"], dD=g["dD"])
    got = gpu_grads(wl, bb)
    for name in GRADS:
        assert_close(got[name], ref[name], wl.act, f"{name} with init")
    assert_close(to_np(bb.dinit), g["dinit"], wl.act, "dinit")


def test_final_state_gradient_finite_differences():
    """L = <dfinal, final state> (dy = 0): sampled gradients against central differences
    of the float64 oracle's final state, for the inputs and the initial state."""
    wl = copy.copy(_bwd_small("tiny_f32"))
    wl.dy = np.zeros_like(wl.dy)
    log("[state io] final-state gradient, finite differences")
    init = _state(wl, 13)
    dfinal = _state(wl, 14, scale=1.0)
    _, bb = _run(wl, init, dfinal=dfinal)
    got = gpu_grads(wl, bb)
    got["dinit"] = to_np(bb.dinit)

    def loss(w2, ini):
        _, v = oracle.conv_silu(w2.to_causal(w2.xBC), w2.conv_w, w2.causal_seq_idx())
        _, fin = oracle.ssd_fwd(v, w2.to_causal(w2.dt_raw), w2.dt_bias, w2.A_log, w2.D,
                                init=ini.astype(np.float64), want_final=True, **_kw(w2))
        return float((fin * dfinal).sum())

    rng = np.random.default_rng(15)
    eps = 1e-3
    for name, field in [("dxBC", "xBC"), ("dconv_w", "conv_w"), ("ddt_raw", "dt_raw"),
                        ("ddt_bias", "dt_bias"), ("dA_log", "A_log"), ("dinit", None)]:
        base = init if field is None else getattr(wl, field)
        idx = rng.choice(base.size, size=min(8, base.size), replace=False)
        scale = np.sqrt(np.mean(got[name] ** 2)) + 1e-12
        for fi in idx:
            plus = base.copy().reshape(-1)
            minus = base.copy().reshape(-1)
            plus[fi] = np.float32(plus[fi] + eps)
            minus[fi] = np.float32(minus[fi] - eps)
            h = float(plus[fi]) - float(minus[fi])
            if field is None:
                lp, lm = loss(wl, plus.reshape(base.shape)), loss(wl, minus.reshape(base.shape))
            else:
                wp, wm = copy.copy(wl), copy.copy(wl)
                setattr(wp, field, plus.reshape(base.shape))
                setattr(wm, field, minus.reshape(base.shape))
                lp, lm = loss(wp, init), loss(wm, init)
            fd = (lp - lm) / h
            an = got[name].reshape(-1)[fi]
            assert abs(fd - an) <= 1e-3 * max(abs(fd), scale), (name, int(fi), fd, an)
    # dD does not reach the state: exactly zero
    assert np.all(got["dD"] == 0.0)


def test_graph_replay_is_bitwise():
    """Forward (with initial and final state) and backward captured in one HIP graph;
    every replay, with eager work and synchronisation between replays, gives outputs
    bit-identical to the eager run, and after new values are written into the
    captured input buffers the replay's outputs follow them."""
    import mamba2_ssd_chunked_amd as ssd
    wl = _bwd_small("bf16_thd")
    log(f"[state io] graph replay {wl.name}")
    p = problem_of(wl)
    x = device_inputs(wl)
    dev = x["xBC"].device
    init = torch.from_numpy(_state(wl, 16)).to(dev)
    dfinal = torch.from_numpy(_state(wl, 17)).to(dev)

    def run(fb, bb):
        ssd.forward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                    x["A_log"], x["D"], x["seq_idx"], init=init, bufs=fb, want_final=True)
        ssd.backward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                     x["A_log"], x["D"], x["dy"], fb.S_in, seq_idx=x["seq_idx"], bufs=bb,
                     dfinal=dfinal, want_dinit=True)

    def outputs(fb, bb):
        return [fb.y, fb.final_state, bb.dxBC, bb.ddt_raw, bb.dconv_w, bb.ddt_bias, bb.dA_log,
                bb.dD, bb.dinit]

    fe, be = ssd.ForwardBuffers.allocate(p, wl.segments, dev), ssd.BackwardBuffers.allocate(
        p, wl.segments, dev)
    run(fe, be)
    torch.cuda.synchronize()
    eager = [t.clone() for t in outputs(fe, be)]

    fg, bg = ssd.ForwardBuffers.allocate(p, wl.segments, dev), ssd.BackwardBuffers.allocate(
        p, wl.segments, dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run(fg, bg)  # warm-up on the capture side stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(fg, bg)
    for rep in range(3):
        for t in outputs(fg, bg):
            t.zero_()
        graph.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outputs(fg, bg), eager)):
            assert torch.equal(a, b), (rep, i)
        run(fe, be)  # eager work between replays
        torch.cuda.synchronize()
    # new values in the captured input buffers: the replay reads them (its outputs
    # follow the eager run on the new inputs and differ from the old ones)
    with torch.no_grad():
        x["xBC"].mul_(-0.75).add_(0.125)
        x["dy"].mul_(1.5)
    run(fe, be)
    torch.cuda.synchronize()
    fresh = [t.clone() for t in outputs(fe, be)]
    graph.replay()
    torch.cuda.synchronize()
    for i, (a, b, c) in enumerate(zip(outputs(fg, bg), fresh, eager)):
        assert torch.equal(a, b), ("new inputs", i)
        assert not torch.equal(a, c), ("unchanged after new inputs", i)
