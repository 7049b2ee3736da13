"""Shared helpers for the GPU parity tests: device transfer, runs, error metrics.

Expected values always come from the CPU oracle (``oracle``) or from plain
float64 loops written here; nothing expected is ever taken from the device.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import ssd_workloads as W


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rms(a) -> float:
    a = np.asarray(a, np.float64)
    return float(np.sqrt(np.mean(a * a)))


def err_fp32(g, o) -> float:
    """max_i |g_i - o_i| / max(|o_i|, rms(o)): elementwise relative error floored at the RMS."""
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.max(np.abs(g - o) / np.maximum(np.abs(o), rms(o))))


def err_rel_rms(g, o) -> float:
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return rms(g - o) / rms(o)


TOL_FP32 = 1e-4   # max relative error for float32 inputs
TOL_BF16 = 2e-2   # relative RMS error for bf16 inputs (FP32 state)


def assert_close(g, o, act: str, what: str = "", tol_scale: float = 1.0):
    if act == "f32":
        e = err_fp32(g, o)
        log(f"  {what}: max-rel err {e:.3e} (tol {TOL_FP32 * tol_scale:.1e})")
        assert e <= TOL_FP32 * tol_scale, (what, e)
    else:
        e = err_rel_rms(g, o)
        log(f"  {what}: rel-RMS err {e:.3e} (tol {TOL_BF16 * tol_scale:.1e}), "
            f"max/rms {np.max(np.abs(np.asarray(g, np.float64) - o)) / rms(o):.3e}")
        assert e <= TOL_BF16 * tol_scale, (what, e)


def problem_of(wl):
    import mamba2_ssd_chunked_amd as ssd
    return ssd.make_problem(batch=wl.batch, seqlen=wl.seqlen, nheads=wl.nheads,
                            headdim=wl.headdim, dstate=wl.dstate, ngroups=wl.ngroups,
                            chunk=wl.chunk, conv_width=wl.conv_width, act=wl.act,
                            dt_min=wl.dt_min, dt_max=wl.dt_max)


def device_inputs(wl, device="cuda"):
    act = torch.bfloat16 if wl.act == "bf16" else torch.float32
    f32 = torch.float32
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)
    d = dict(xBC=t(wl.xBC, act), conv_w=t(wl.conv_w, f32), dt_raw=t(wl.dt_raw, act),
             dt_bias=t(wl.dt_bias, f32), A_log=t(wl.A_log, f32), D=t(wl.D, f32),
             seq_idx=None if wl.seq_idx is None else t(wl.seq_idx, torch.int32))
    if wl.dy is not None:
        d["dy"] = t(wl.dy, act)
    return d


def run_forward(wl, inputs=None, init=None, fused=True, conv_fused=False):
    """The forward path through the C ABI.  fused=True runs the states-first order
    (segment states, boundary scan, fused output pass); fused=False runs the
    zero-state output (y_zero) and the separate correction pass; conv_fused=True
    runs the states-first order with the conv inside the two phases."""
    import mamba2_ssd_chunked_amd as ssd
    p = problem_of(wl)
    x = inputs or device_inputs(wl)
    bufs = ssd.forward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                       x["A_log"], x["D"], x["seq_idx"], init=init, fused=fused,
                       conv_fused=conv_fused)
    torch.cuda.synchronize()
    return p, x, bufs


def to_np(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


# --------------------------------------------------------------------------- oracle views


def oracle_v(wl):
    """Post-conv activations in causal order, float64 (oracle)."""
    _, v = oracle.conv_silu(wl.to_causal(wl.xBC), wl.conv_w, wl.causal_seq_idx())
    return v


def causal_ranges(wl):
    """Causal token range [a, b) of every segment, in causal order."""
    out = []
    pos = 0
    for _, n in wl.segments:
        out.append((pos, pos + n))
        pos += n
    return out


def oracle_segment(wl, v, k, init=None, D_zero=True):
    """Oracle run of causal segment k alone, from ``init`` (zero if None).

    Returns (y [b, len, H, P], final [b, H, P, N]).  If the segment's first token
    starts a new packed sequence, the initial state cannot reach it, so the
    run starts from zero (that is what the recurrence does at a reset).
    """
    a, b = causal_ranges(wl)[k]
    seq = wl.causal_seq_idx()
    s = None if seq is None else seq[:, a:b]
    dt_raw = wl.to_causal(wl.dt_raw)[:, a:b]
    D = np.zeros_like(wl.D) if D_zero else wl.D
    ini = None
    if init is not None:
        ini = np.array(init, np.float64, copy=True)
        if seq is not None and a > 0:
            for r in range(wl.batch):
                if seq[r, a] != seq[r, a - 1]:
                    ini[r] = 0.0
    return oracle.ssd_fwd(v[:, a:b], dt_raw, wl.dt_bias, wl.A_log, D, nheads=wl.nheads,
                          headdim=wl.headdim, dstate=wl.dstate, ngroups=wl.ngroups,
                          dt_min=wl.dt_min, dt_max=wl.dt_max, seq_idx=s, init=ini,
                          want_final=True)
