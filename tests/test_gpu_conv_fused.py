"""GPU parity of the conv-fused forward (ssd_conv_segment_states, the boundary
scan, ssd_conv_segment_output) against the CPU oracle, through the C ABI.

The fused calls convolve the x channels inside the state walk and the output
pass, reading the raw input and each segment's halo (the causal predecessor's
last tokens) themselves.  Their conv arithmetic is the conv pass's, operation
for operation, so besides matching the oracle within the usual tolerances
(float32: max relative error 1e-4; bf16: relative RMS error 2e-2) y and the
summaries must equal those of the unfused states-first path bit for bit.  The
cases cover packed sequences that start inside a conv window (including a
one-token sequence), the virtual front/back layout (halo from a segment stored
elsewhere), one-chunk segments, spans, and the full-size workloads.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_workloads as W
from ssd_testlib import (assert_close, causal_ranges, device_inputs, log, oracle_segment, oracle_v,
                         run_forward, to_np)
from test_gpu_forward import SMALL, _small

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", params=SMALL)
def fused_run(request):
    wl = _small(request.param)
    log(f"[conv-fused] case {wl.name}: b={wl.batch} L={wl.seqlen} H={wl.nheads} P={wl.headdim} "
        f"N={wl.dstate} Q={wl.chunk} act={wl.act} segs={len(wl.segments)} layout={wl.layout} "
        f"packed={wl.seq_idx is not None}")
    p, x, bufs = run_forward(wl, conv_fused=True)
    return wl, p, x, bufs


def test_conv_fused_against_oracle(fused_run):
    wl, _, _, bufs = fused_run
    assert_close(wl.to_causal(to_np(bufs.y)), oracle.forward(wl), wl.act, "y (conv-fused)")


def test_conv_fused_equals_unfused_bitwise(fused_run):
    wl, _, x, bufs = fused_run
    _, _, ref = run_forward(wl, inputs=x, fused=True)
    assert torch.equal(bufs.summary, ref.summary)
    assert torch.equal(bufs.S_in, ref.S_in)
    assert torch.equal(bufs.y, ref.y)


def test_conv_fused_output_random_states(fused_run):
    """The conv-fused output pass from random S_in equals the oracle run of each
    segment from that S_in."""
    import mamba2_ssd_chunked_amd as ssd
    wl, p, x, bufs = fused_run
    S, b, H, P, N = len(wl.segments), wl.batch, wl.nheads, wl.headdim, wl.dstate
    rng = np.random.default_rng(79)
    S_in = rng.standard_normal((S, b, H, P, N)).astype(np.float32)
    y = torch.empty_like(bufs.y)
    ssd.ssd_conv_segment_output(p, wl.segments, x["xBC"], x["conv_w"], x["D"], x["seq_idx"],
                                torch.from_numpy(S_in).cuda(), bufs.ws, y)
    torch.cuda.synchronize()
    g = wl.to_causal(to_np(y))
    v = oracle_v(wl)
    for k, (a, e) in enumerate(causal_ranges(wl)):
        yk, _ = oracle_segment(wl, v, k, init=S_in[k].astype(np.float64), D_zero=False)
        assert_close(g[:, a:e], yk, wl.act, f"y conv-fused (S_in random)[{k}]")


@pytest.mark.parametrize("cfg", ["mixer_shard_bf16", "packed_thd_bf16"])
def test_conv_fused_full_config(cfg):
    wl = W.config(cfg)
    log(f"[conv-fused full] {cfg}")
    _, x, bufs = run_forward(wl, conv_fused=True)
    assert_close(wl.to_causal(to_np(bufs.y)), oracle.forward(wl), wl.act, f"y {cfg}")
    _, _, ref = run_forward(wl, inputs=x, fused=True)
    assert torch.equal(bufs.y, ref.y)


@pytest.mark.parametrize("cfg", ["long_context_bf16", "long_context_virtual_bf16"])
def test_conv_fused_long_context_all_heads(cfg):
    """131072 tokens, 64 heads in 8 groups: every head against the oracle, one
    group at a time, and bitwise equal to the unfused path."""
    wl = W.config(cfg)
    log(f"[conv-fused full] {cfg} all heads")
    _, x, bufs = run_forward(wl, conv_fused=True)
    _, _, ref = run_forward(wl, inputs=x, fused=True)
    assert torch.equal(bufs.y, ref.y)
    del ref
    hpg = wl.nheads // wl.ngroups
    for g in range(wl.ngroups):
        heads = list(range(g * hpg, (g + 1) * hpg))
        got = wl.to_causal(to_np(bufs.y[:, :, g * hpg:(g + 1) * hpg]))
        o = oracle.forward(wl, heads=heads)
        assert_close(got, o, wl.act, f"y {cfg} group {g}")
