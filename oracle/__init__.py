"""CPU oracle (float64) for the Mamba2 causal conv1d + SSD mixer core.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``mamba2_ssd_chunked_amd``) never imports it, and the two share no code:
this package loads its own C library (``ssd_oracle.c``) with its own ctypes
declarations.

Every function runs the plain token-by-token recurrence over the whole,
unsegmented sequence in causal order (see the header of ``ssd_oracle.c`` for
the definitions and the passages they follow).  Nothing here chunks, segments,
scans or passes states; segment-level quantities used by invariant tests are
obtained by running this same recurrence on sub-ranges with an initial state.

Pins: every function here is pinned by ``tests/test_oracle_pins.py`` against a
brute-force quadratic form, closed forms, a worked fixture under
``tests/golden/``, torch's conv1d, finite differences and invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_fp = ctypes.POINTER(ctypes.c_float)
_ip = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, IEEE float64, no fast-math)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    lib.oracle_conv_silu.argtypes = [_i64, _i64, _i64, _i64, _fp, _fp, _ip, _dp, _dp]
    lib.oracle_conv_silu.restype = None
    lib.oracle_conv_silu_bwd.argtypes = [_i64, _i64, _i64, _i64, _fp, _fp, _ip, _dp, _dp, _dp]
    lib.oracle_conv_silu_bwd.restype = None
    lib.oracle_ssd_fwd.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _dp, _fp, _fp, _fp, _fp,
                                   ctypes.c_double, ctypes.c_double, _ip, _dp, _dp, _dp]
    lib.oracle_ssd_fwd.restype = None
    lib.oracle_ssd_bwd.argtypes = [_i64, _i64, _i64, _i64, _i64, _i64, _dp, _fp, _fp, _fp, _fp,
                                   ctypes.c_double, ctypes.c_double, _ip, _dp, _fp,
                                   _dp, _dp, _dp, _dp, _dp, _dp]
    lib.oracle_ssd_bwd.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    return int(_load().oracle_num_threads())


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a, t):
    return None if a is None else a.ctypes.data_as(t)


def _seq(seq_idx):
    return None if seq_idx is None else np.ascontiguousarray(seq_idx, dtype=np.int32)


def conv_silu(xBC: np.ndarray, conv_w: np.ndarray, seq_idx: Optional[np.ndarray] = None):
    """Causal depthwise conv + SiLU.  xBC [b, L, C] -> (u, v) float64 [b, L, C]."""
    xBC = _f32(xBC)
    w = _f32(conv_w)
    b, L, C = xBC.shape
    W = w.shape[1]
    si = _seq(seq_idx)
    u = np.empty((b, L, C), np.float64)
    v = np.empty((b, L, C), np.float64)
    _load().oracle_conv_silu(b, L, C, W, _ptr(xBC, _fp), _ptr(w, _fp), _ptr(si, _ip),
                             _ptr(u, _dp), _ptr(v, _dp))
    return u, v


def conv_silu_bwd(xBC, conv_w, dv, seq_idx=None):
    """Adjoint of conv_silu: returns (dxBC [b, L, C], dconv_w [C, W]) in float64."""
    xBC = _f32(xBC)
    w = _f32(conv_w)
    dv = _f64(dv)
    b, L, C = xBC.shape
    W = w.shape[1]
    si = _seq(seq_idx)
    dx = np.empty((b, L, C), np.float64)
    dw = np.empty((C, W), np.float64)
    _load().oracle_conv_silu_bwd(b, L, C, W, _ptr(xBC, _fp), _ptr(w, _fp), _ptr(si, _ip),
                                 _ptr(dv, _dp), _ptr(dx, _dp), _ptr(dw, _dp))
    return dx, dw


def ssd_fwd(v, dt_raw, dt_bias, A_log, D, *, nheads, headdim, dstate, ngroups,
            dt_min=1e-3, dt_max=0.1, seq_idx=None, init=None, want_final=False):
    """Token-by-token SSD.  v [b, L, C] float64 (post-conv) -> y [b, L, H, P]."""
    v = _f64(v)
    b, L, C = v.shape
    H, P, N, G = nheads, headdim, dstate, ngroups
    assert C == H * P + 2 * G * N and H % G == 0
    dt_raw = _f32(dt_raw)
    y = np.empty((b, L, H, P), np.float64)
    fin = np.empty((b, H, P, N), np.float64) if want_final else None
    ini = None if init is None else _f64(init)
    si = _seq(seq_idx)
    _load().oracle_ssd_fwd(b, L, H, P, N, G, _ptr(v, _dp), _ptr(dt_raw, _fp),
                           _ptr(_f32(dt_bias), _fp), _ptr(_f32(A_log), _fp), _ptr(_f32(D), _fp),
                           float(np.float32(dt_min)), float(np.float32(dt_max)),
                           _ptr(si, _ip), _ptr(ini, _dp), _ptr(y, _dp), _ptr(fin, _dp))
    return (y, fin) if want_final else y


def ssd_bwd(v, dt_raw, dt_bias, A_log, D, dy, *, nheads, headdim, dstate, ngroups,
            dt_min=1e-3, dt_max=0.1, seq_idx=None, init=None, want_dinit=False):
    """Adjoint of ssd_fwd.  Returns dict with dv, ddt_raw, ddt_bias, dA_log, dD (+ dinit)."""
    v = _f64(v)
    b, L, C = v.shape
    H, P, N, G = nheads, headdim, dstate, ngroups
    dt_raw = _f32(dt_raw)
    dy = _f32(dy)
    dv = np.empty((b, L, C), np.float64)
    ddt = np.empty((b, L, H), np.float64)
    ddb = np.empty(H, np.float64)
    dal = np.empty(H, np.float64)
    dd = np.empty(H, np.float64)
    dinit = np.empty((b, H, P, N), np.float64) if want_dinit else None
    ini = None if init is None else _f64(init)
    si = _seq(seq_idx)
    _load().oracle_ssd_bwd(b, L, H, P, N, G, _ptr(v, _dp), _ptr(dt_raw, _fp),
                           _ptr(_f32(dt_bias), _fp), _ptr(_f32(A_log), _fp), _ptr(_f32(D), _fp),
                           float(np.float32(dt_min)), float(np.float32(dt_max)),
                           _ptr(si, _ip), _ptr(ini, _dp), _ptr(dy, _fp),
                           _ptr(dv, _dp), _ptr(ddt, _dp), _ptr(ddb, _dp), _ptr(dal, _dp),
                           _ptr(dd, _dp), _ptr(dinit, _dp))
    out = dict(dv=dv, ddt_raw=ddt, ddt_bias=ddb, dA_log=dal, dD=dd)
    if want_dinit:
        out["dinit"] = dinit
    return out


# ---------------------------------------------------------------------------
# Whole-path helpers on a workload (causal order in, causal order out).


def _select_heads(wl, heads: Sequence[int]):
    """Channel subset of xBC / conv_w holding the given heads and their groups.

    Running the recurrence on this reduced problem gives exactly the same
    outputs for those heads: heads never interact except through the shared
    B and C channels of their group, which are kept.
    """
    H, P, N, G = wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    hpg = H // G
    heads = list(heads)
    groups = sorted({h // hpg for h in heads})
    # Reduced problem: each selected group keeps only the selected heads; every
    # group must keep the same head count, so select per group evenly.
    per_group = {g: [h for h in heads if h // hpg == g] for g in groups}
    k = max(len(v) for v in per_group.values())
    assert all(len(v) == k for v in per_group.values()), "select the same head count per group"
    new_heads = [h for g in groups for h in per_group[g]]
    ch = []
    for h in new_heads:
        ch.extend(range(h * P, (h + 1) * P))
    for g in groups:
        ch.extend(range(H * P + g * N, H * P + (g + 1) * N))
    for g in groups:
        ch.extend(range(H * P + G * N + g * N, H * P + G * N + (g + 1) * N))
    return new_heads, groups, np.asarray(ch, dtype=np.int64)


def forward(wl, heads: Optional[Sequence[int]] = None, rows: Optional[Sequence[int]] = None):
    """y for a workload, in causal token order, float64 [b', L, H', P].

    ``heads`` / ``rows`` restrict the computation to a subset (exactly the same
    values as the full run for those heads and rows).
    """
    xBC = wl.to_causal(wl.xBC)
    dt_raw = wl.to_causal(wl.dt_raw)
    seq = wl.causal_seq_idx()
    H, P, N, G = wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    conv_w, dt_bias, A_log, D = wl.conv_w, wl.dt_bias, wl.A_log, wl.D
    if rows is not None:
        rows = list(rows)
        xBC, dt_raw = xBC[rows], dt_raw[rows]
        seq = None if seq is None else seq[rows]
    if heads is not None:
        new_heads, groups, ch = _select_heads(wl, heads)
        xBC = xBC[:, :, ch]
        conv_w = conv_w[ch]
        dt_raw = dt_raw[:, :, new_heads]
        dt_bias, A_log, D = dt_bias[new_heads], A_log[new_heads], D[new_heads]
        H, G = len(new_heads), len(groups)
    _, v = conv_silu(xBC, conv_w, seq)
    return ssd_fwd(v, dt_raw, dt_bias, A_log, D, nheads=H, headdim=P, dstate=N, ngroups=G,
                   dt_min=wl.dt_min, dt_max=wl.dt_max, seq_idx=seq)


def backward(wl, heads: Optional[Sequence[int]] = None):
    """All gradients for a workload with ``dy``; causal token order, float64.

    Returns dict: y, dxBC [b, L, C], dconv_w [C, W], ddt_raw [b, L, H],
    ddt_bias, dA_log, dD [H].

    ``heads`` restricts the problem to those heads and their groups' B and C
    channels.  The gradients that belong to a head alone are then exactly those
    of the full problem: dxBC and dconv_w of the head's x channels (returned as
    [b, L, H' * P] and [H' * P, W]), ddt_raw [b, L, H'], ddt_bias, dA_log and
    dD [H'].  B and C channel gradients sum over every head of a group: they are
    returned only when ``heads`` holds every head of each group it touches, and
    then dxBC and dconv_w also cover those groups' B and C channels.  The key
    ``channels`` lists the channel of the full problem behind each returned one.
    """
    xBC = wl.to_causal(wl.xBC)
    dt_raw = wl.to_causal(wl.dt_raw)
    dy = wl.to_causal(wl.dy)
    seq = wl.causal_seq_idx()
    H, P, G = wl.nheads, wl.headdim, wl.ngroups
    conv_w, dt_bias, A_log, D = wl.conv_w, wl.dt_bias, wl.A_log, wl.D
    if heads is not None:
        new_heads, groups, ch = _select_heads(wl, heads)
        xBC = xBC[:, :, ch]
        conv_w = conv_w[ch]
        dt_raw = dt_raw[:, :, new_heads]
        dy = dy[:, :, new_heads]
        dt_bias, A_log, D = dt_bias[new_heads], A_log[new_heads], D[new_heads]
        H, G = len(new_heads), len(groups)
    kw = dict(nheads=H, headdim=P, dstate=wl.dstate, ngroups=G,
              dt_min=wl.dt_min, dt_max=wl.dt_max, seq_idx=seq)
    _, v = conv_silu(xBC, conv_w, seq)
    y = ssd_fwd(v, dt_raw, dt_bias, A_log, D, **kw)
    g = ssd_bwd(v, dt_raw, dt_bias, A_log, D, dy, **kw)
    dxBC, dw = conv_silu_bwd(xBC, conv_w, g["dv"], seq)
    channels = np.arange(wl.conv_dim)
    if heads is not None:
        hpg = wl.nheads // wl.ngroups
        whole = all(sum(1 for h in new_heads if h // hpg == gg) == hpg for gg in groups)
        keep = dxBC.shape[2] if whole else H * P
        dxBC, dw, channels = dxBC[:, :, :keep], dw[:keep], ch[:keep]
    return dict(y=y, dxBC=dxBC, dconv_w=dw, ddt_raw=g["ddt_raw"], ddt_bias=g["ddt_bias"],
                dA_log=g["dA_log"], dD=g["dD"], channels=channels)
