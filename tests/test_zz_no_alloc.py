"""The entry point that allocates nothing (ssd_segment_fwd_noalloc) against the
one it is a variant of (ssd_segment_fwd with a caller-allocated workspace), on
two calls in a row, the second with a smaller input: y_zero and the summary
must be bit-identical (same kernels, same inputs, the workspace only moves).
Also: a problem whose workspace exceeds the fixed scratch is refused with
SSD_ERR_SCRATCH.
"""
import pytest
import torch

import ssd_workloads as W
from ssd_testlib import device_inputs, log, problem_of

pytestmark = pytest.mark.gpu


def _both(wl):
    import mamba2_ssd_chunked_amd as ssd
    p = problem_of(wl)
    x = device_inputs(wl)
    s = ssd.Segments(wl.segments)
    ws_bytes = ssd.ssd_workspace_bytes(p, s, ssd.SSD_WS_FORWARD)
    log(f"[no alloc] {wl.name}: forward workspace {ws_bytes} bytes "
        f"(scratch {ssd._lib.SSD_SCRATCH_BYTES})")
    assert 0 < ws_bytes <= ssd._lib.SSD_SCRATCH_BYTES
    dev = x["xBC"].device
    b, L, H, P = wl.batch, wl.seqlen, wl.nheads, wl.headdim
    xc = torch.empty((b, L, wl.conv_dim), dtype=x["xBC"].dtype, device=dev)
    ssd.ssd_conv1d_fwd(p, s, x["xBC"], x["conv_w"], x["seq_idx"], xc)
    nsum = ssd.summary_numel(p, s.n)
    y_ref = torch.empty((b, L, H, P), dtype=torch.float32, device=dev)
    sum_ref = torch.empty(nsum, dtype=torch.float32, device=dev)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ssd.ssd_segment_fwd(p, s, xc, x["dt_raw"], x["dt_bias"], x["A_log"], x["seq_idx"], y_ref,
                        sum_ref, ws)
    # the outputs of the allocation-free call start as NaN: every element is written
    y_na = torch.full_like(y_ref, float("nan"))
    sum_na = torch.full_like(sum_ref, float("nan"))
    ssd.ssd_segment_fwd_noalloc(p, s, xc, x["dt_raw"], x["dt_bias"], x["A_log"], x["seq_idx"],
                                y_na, sum_na)
    torch.cuda.synchronize()
    assert torch.equal(y_na, y_ref)
    assert torch.equal(sum_na, sum_ref)


def test_no_alloc_matches_allocating_entry_point_twice():
    # first the mixer shard (2 x 8192 tokens, 32 heads, packed sequences, 8 segments),
    # then a smaller problem of another shape: the second call reuses the scratch
    # the first one left behind
    big = W.make_workload("noalloc_big", batch=2, seqlen=8192, nheads=32, headdim=64, dstate=128,
                          ngroups=1, chunk=256, act="bf16", nseg=8, seed=1201,
                          packed=(500, 3000))
    small = W.make_workload("noalloc_small", batch=1, seqlen=1024, nheads=4, headdim=64,
                            dstate=64, ngroups=2, chunk=64, act="bf16", seed=1202,
                            seg_lens=[64, 320, 640], packed=(40, 300))
    _both(big)
    _both(small)


def test_no_alloc_refuses_problem_beyond_scratch():
    import mamba2_ssd_chunked_amd as ssd
    wl = W.config("packed_thd_bf16")  # 32768 tokens x 32 heads: about 80 MB of workspace
    p = problem_of(wl)
    s = ssd.Segments(wl.segments)
    assert ssd.ssd_workspace_bytes(p, s, ssd.SSD_WS_FORWARD) > ssd._lib.SSD_SCRATCH_BYTES
    x = device_inputs(wl)
    dev = x["xBC"].device
    y = torch.empty((1, wl.seqlen, wl.nheads, wl.headdim), dtype=torch.float32, device=dev)
    summ = torch.empty(ssd.summary_numel(p, s.n), dtype=torch.float32, device=dev)
    with pytest.raises(ssd.SSDError) as e:
        ssd.ssd_segment_fwd_noalloc(p, s, x["xBC"], x["dt_raw"], x["dt_bias"], x["A_log"],
                                    x["seq_idx"], y, summ)
    assert e.value.status == -8
