"""C ABI checks that need no GPU: exports, host-side validation, workspace sizes.

Every call here is made with arguments that fail validation, so the library
returns an error before touching the device.
"""
import ctypes
import os
import re

import pytest

import mamba2_ssd_chunked_amd as ssd
from mamba2_ssd_chunked_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(ssd_\w+)\s*\(", text))
    return names


def test_every_declared_symbol_is_exported():
    lib = _lib.load()
    names = _declared()
    assert {"ssd_conv1d_fwd", "ssd_segment_fwd", "ssd_boundary_scan",
            "ssd_apply_init_state"} <= names
    for n in sorted(names):
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES, f"{n} has no ctypes signature"


def test_struct_layout_matches_header():
    assert ctypes.sizeof(_lib.Problem) == 56
    assert ctypes.sizeof(_lib.Segment) == 16


def _p(**kw):
    base = dict(batch=2, seqlen=8192, nheads=32, headdim=64, dstate=128, ngroups=1, chunk=256,
                conv_width=4, act="bf16")
    base.update(kw)
    return ssd.make_problem(**base)


SEGS8 = [(i * 1024, 1024) for i in range(8)]
FAKE = ctypes.c_void_p(0x100000)       # never dereferenced: every call below fails validation
MISALIGNED = ctypes.c_void_p(0x100004)


def _conv(p, segs, xbc=FAKE, w=FAKE, seq=None, out=FAKE):
    s = ssd.Segments(segs)
    return _lib.load().ssd_conv1d_fwd(ctypes.byref(p) if p is not None else None, s.ptr(), s.n,
                                      xbc, w, seq, out, None)


def test_workspace_bytes():
    p = _p()
    b, H, L, nc, P, N = 2, 32, 8192, 32, 64, 128
    al = lambda x: (x + 255) // 256 * 256
    want = al(al(al(b * H * L * 4) + b * H * L * 4) + b * H * nc * 4)
    want = al(want + b * nc * H * P * N * 2)
    qt = 256 // 16
    want = al(want + b * nc * 1 * (qt * (qt + 1) // 2) * 256 * 2)  # causal Gram tiles per group
    assert ssd.ssd_workspace_bytes(p, SEGS8) == want
    assert ssd.ssd_workspace_bytes(p, SEGS8, kind=7) == 0
    assert ssd.ssd_workspace_bytes(_p(chunk=100), SEGS8) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(nheads=30, ngroups=4), -2),
    (dict(chunk=96), -3),
    (dict(conv_width=9), -3),
    (dict(headdim=48), -3),
    (dict(act=5), -3),
    (dict(seqlen=8000), -2),
    (dict(batch=0), -2),
])
def test_problem_validation(kw, code):
    assert _conv(_p(**kw), SEGS8) == code


def test_null_and_alignment():
    assert _lib.load().ssd_conv1d_fwd(None, ssd.Segments(SEGS8).ptr(), 8, FAKE, FAKE, None, FAKE,
                                      None) == -1
    assert _conv(_p(), SEGS8, xbc=None) == -1
    assert _conv(_p(), SEGS8, out=MISALIGNED) == -4
    assert _conv(_p(), SEGS8, seq=MISALIGNED) == -4


@pytest.mark.parametrize("segs", [
    [(i * 1024, 1024) for i in range(7)],                        # does not cover
    [(0, 1024)] * 8,                                             # overlapping
    [(i * 1024 + 128, 1024) for i in range(8)],                  # out of range
    [(0, 1000), (1000, 7192)],                                   # not chunk aligned
    [(i * 128, 128) for i in range(64)] + [(8192, 0)],           # too many segments / empty
])
def test_segment_validation(segs):
    assert _conv(_p(), segs) == -7


def test_workspace_too_small_enqueues_nothing():
    p = _p()
    s = ssd.Segments(SEGS8)
    lib = _lib.load()
    need = ssd.ssd_workspace_bytes(p, SEGS8)
    rc = lib.ssd_segment_fwd(ctypes.byref(p), s.ptr(), s.n, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                             FAKE, FAKE, need - 1, None)
    assert rc == -5
    rc = lib.ssd_apply_init_state(ctypes.byref(p), s.ptr(), s.n, FAKE, FAKE, FAKE, None, FAKE,
                                  None, need, FAKE, None)
    assert rc == -5


def test_boundary_scan_validation():
    lib = _lib.load()
    p = _p()
    assert lib.ssd_boundary_scan(ctypes.byref(p), 0, FAKE, None, 0, FAKE, None, None) == -7
    assert lib.ssd_boundary_scan(ctypes.byref(p), 65, FAKE, None, 0, FAKE, None, None) == -7
    assert lib.ssd_boundary_scan(ctypes.byref(p), 8, FAKE, None, 2, FAKE, None, None) == -2
    assert lib.ssd_boundary_scan(ctypes.byref(p), 8, None, None, 0, FAKE, None, None) == -1
    assert lib.ssd_boundary_scan(ctypes.byref(p), 8, FAKE, MISALIGNED, 0, FAKE, None, None) == -4


def test_status_strings_and_support():
    lib = _lib.load()
    for code in range(-8, 1):
        assert lib.ssd_status_string(code)
    assert lib.ssd_supported(64, 128, 1) == 1
    assert lib.ssd_supported(16, 16, 0) == 1
    assert lib.ssd_supported(16, 16, 1) == 0
    assert lib.ssd_abi_version() >= 1


def test_binding_rejects_wrong_sizes_before_the_library():
    import torch
    p = _p(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, chunk=64, act="f32")
    x = torch.zeros(10)
    with pytest.raises(ValueError):
        ssd.ssd_conv1d_fwd(p, [(0, 256)], x, x, None, x)


# Every (activation, headdim, dstate, chunk) the library accepts, forward and
# backward.  tests/test_gpu_shapes.py runs each accepted combination on the GPU
# against the oracle, so a shape cannot be accepted without being exercised.
FWD_SHAPES = {(a, p, n, q) for a, p, n in [("f32", 16, 16), ("f32", 32, 32), ("f32", 64, 64),
                                           ("f32", 64, 128), ("bf16", 32, 64), ("bf16", 64, 64),
                                           ("bf16", 64, 128)]
              for q in (64, 128, 256)}
BWD_SHAPES = {s for s in FWD_SHAPES if s[0] == "bf16" or s[3] != 256}


def accepted_shapes():
    """(forward set, backward set) of the combinations ssd_workspace_bytes accepts, over a
    grid wider than the compiled one."""
    fwd, bwd = set(), set()
    for act in ("f32", "bf16"):
        for P in (8, 16, 32, 48, 64, 128, 256):
            for N in (8, 16, 32, 64, 96, 128, 256):
                for Q in (32, 64, 128, 256, 512):
                    p = _p(batch=1, seqlen=2 * 512, nheads=2, headdim=P, dstate=N, chunk=Q,
                           act=act)
                    segs = [(0, 1024)]
                    if ssd.ssd_workspace_bytes(p, segs, ssd.SSD_WS_FORWARD):
                        fwd.add((act, P, N, Q))
                    if ssd.ssd_workspace_bytes(p, segs, ssd.SSD_WS_BACKWARD):
                        bwd.add((act, P, N, Q))
    return fwd, bwd


def test_support_table_is_the_tested_one():
    fwd, bwd = accepted_shapes()
    assert fwd == FWD_SHAPES
    assert bwd == BWD_SHAPES
    lib = _lib.load()
    for act, P, N, Q in FWD_SHAPES:
        assert lib.ssd_supported(P, N, 0 if act == "f32" else 1) == 1
    assert lib.ssd_supported(128, 128, 1) == 0


def test_backward_refuses_unsupported_shape_before_launching():
    p = _p(batch=1, seqlen=1024, nheads=2, headdim=64, dstate=128, chunk=256, act="f32")
    s = ssd.Segments([(0, 1024)])
    lib = _lib.load()
    rc = lib.ssd_segment_bwd_summary(ctypes.byref(p), s.ptr(), s.n, FAKE, FAKE, FAKE, FAKE, FAKE,
                                     None, FAKE, FAKE, FAKE, 1 << 30, None)
    assert rc == -3


def test_over_long_row_is_refused_before_launching():
    """A row of 2^23 tokens needs 2^17 conv workgroups along the grid's y dimension
    (beyond 65535): validation refuses it, for the conv alone and for the multi-kernel
    backward summary, before anything is launched (no GPU here, so a launch would fail
    with SSD_ERR_HIP instead)."""
    L = 1 << 23
    p = _p(batch=1, seqlen=L, nheads=2, headdim=64, dstate=128, chunk=256)
    segs = [(0, L)]
    assert _conv(p, segs) == -2
    assert ssd.ssd_workspace_bytes(p, segs, ssd.SSD_WS_BACKWARD) == 0
    s = ssd.Segments(segs)
    rc = _lib.load().ssd_segment_bwd_summary(ctypes.byref(p), s.ptr(), s.n, FAKE, FAKE, FAKE, FAKE,
                                             FAKE, None, FAKE, FAKE, FAKE, 1 << 40, None)
    assert rc == -2
    # the longest row the conv grid takes is accepted by validation
    ok = _p(batch=1, seqlen=65535 * 64 // 256 * 256, nheads=2, headdim=64, dstate=128, chunk=256)
    assert ssd.ssd_workspace_bytes(ok, [(0, ok.seqlen)], ssd.SSD_WS_FORWARD) > 0


def test_chunk_rows_beyond_31_bit_offsets_are_refused():
    """chunk x C x sizeof(activation) must stay below 2^31 bytes: 65535 heads of
    headdim 64 (C = 4194496 channels) at bf16 pass with 128-token chunks and are
    refused with 256-token chunks."""
    kw = dict(batch=1, seqlen=256, nheads=65535, headdim=64, dstate=128, ngroups=1)
    assert ssd.ssd_workspace_bytes(_p(chunk=128, **kw), [(0, 256)], ssd.SSD_WS_FORWARD) > 0
    assert _conv(_p(chunk=256, **kw), [(0, 256)]) == -2


def test_grid_overflow_is_refused():
    """batch x heads x P x N beyond 2^32 work-items of the boundary scan's grid."""
    p = _p(batch=4096, seqlen=256, nheads=4096, headdim=64, dstate=128, chunk=256)
    assert _conv(p, [(0, 256)]) == -2


def test_forward_workspace_holds_span_regions_for_long_segments():
    """The packed 32768-token batch (4 segments of 32 chunks, 32 heads walked two per
    workgroup) has too few walk workgroups per segment-long walk: the walk splits each
    segment into spans until 256 workgroups (one per CU) exist or a span would drop
    below 1024 tokens: 16 spans of 8 chunks.  The forward workspace then holds the span summaries
    and the states entering the spans (FP32, [32][1][32][64*128] each, the summaries
    with their block decays)."""
    p = _p(batch=1, seqlen=32768, nheads=32, headdim=64, dstate=128, chunk=256)
    segs = [(i * 8192, 8192) for i in range(4)]
    al = lambda x: (x + 255) // 256 * 256
    b, H, L, nc, P, N = 1, 32, 32768, 128, 64, 128
    base = al(al(al(b * H * L * 4) + b * H * L * 4) + b * H * nc * 4)
    base = al(base + b * nc * H * P * N * 2)
    qt = 256 // 16
    base = al(base + b * nc * (qt * (qt + 1) // 2) * 256 * 2)
    nsp = 16
    want = al(al(base + nsp * b * H * (P * N + 1) * 4) + nsp * b * H * P * N * 4)
    assert ssd.ssd_workspace_bytes(p, segs) == want
    # the mixer shard's segments are walked whole: no span regions
    assert ssd.ssd_workspace_bytes(_p(), SEGS8) < want


def test_conv_fused_forward_workspace_and_refusals():
    """The conv-fused forward's workspace is the forward one plus the convolved B
    and C channels ([b][L][2 G N] bf16); it is compiled for conv width 4 only, and
    both of its calls refuse other widths, missing pointers and a short workspace
    before launching anything."""
    p = _p()
    b, L, G, N = 2, 8192, 1, 128
    base = ssd.ssd_workspace_bytes(p, SEGS8)
    want = base + (b * L * 2 * G * N * 2 + 255) // 256 * 256
    assert ssd.ssd_workspace_bytes(p, SEGS8, ssd.SSD_WS_FORWARD_CONV) == want
    assert ssd.ssd_workspace_bytes(_p(conv_width=3), SEGS8, ssd.SSD_WS_FORWARD_CONV) == 0
    lib = _lib.load()
    s = ssd.Segments(SEGS8)
    st = lambda pp, xbc=FAKE, ws_bytes=want: lib.ssd_conv_segment_states(
        ctypes.byref(pp), s.ptr(), s.n, xbc, FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, ws_bytes,
        None)
    out = lambda pp, w=FAKE, ws_bytes=want: lib.ssd_conv_segment_output(
        ctypes.byref(pp), s.ptr(), s.n, FAKE, w, FAKE, None, FAKE, FAKE, ws_bytes, FAKE, None)
    assert st(_p(conv_width=3)) == -3 and out(_p(conv_width=5)) == -3
    assert st(p, xbc=None) == -1 and out(p, w=None) == -1
    assert st(p, ws_bytes=want - 1) == -5 and out(p, ws_bytes=base) == -5
    assert st(p, xbc=MISALIGNED) == -4
