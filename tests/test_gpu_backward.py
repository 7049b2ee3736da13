"""GPU parity of the backward path against the CPU oracle's analytic gradients.

Also: the backward summary (dL/dS_in of each segment's own outputs) against the
oracle's initial-state gradient per segment, central finite differences of the
oracle forward on the tiny float32 workload, the full mixer shard, determinism, and bitwise isolation
of packed sequences.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_workloads as W
from ssd_testlib import (assert_close, causal_ranges, device_inputs, log, oracle_v, problem_of,
                         to_np)

pytestmark = pytest.mark.gpu

GRADS = ["dxBC", "dconv_w", "ddt_raw", "ddt_bias", "dA_log", "dD"]


def _bwd_small(name):
    mk = W.make_workload
    kw = dict(with_dy=True)
    if name == "tiny_f32":
        return mk("tiny_f32", batch=1, seqlen=256, nheads=2, headdim=16, dstate=16,
                  ngroups=1, chunk=64, act="f32", nseg=2, seed=1000, **kw)
    if name == "slow_tiny_f32":
        return mk("slow_tiny_f32", batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, ngroups=1,
                  chunk=64, act="f32", nseg=2, seed=2000, slow_decay=True, **kw)
    if name == "f32_head_thd":
        # float32 backward at P = 64 needs N <= 64 to fit the chunk kernel's LDS
        return mk(name, batch=2, seqlen=512, nheads=4, headdim=64, dstate=64, ngroups=2,
                  chunk=64, act="f32", seed=301, seg_lens=[128, 256, 128],
                  lengths=[37, 150, 1, 200, 124], **kw)
    if name == "f32_virtual":
        return mk(name, batch=1, seqlen=512, nheads=2, headdim=32, dstate=32, ngroups=1,
                  chunk=64, act="f32", seed=302, nseg=4, layout="virtual", slow_decay=True, **kw)
    if name == "bf16_small":
        return mk(name, batch=2, seqlen=2048, nheads=4, headdim=64, dstate=128, ngroups=1,
                  chunk=256, act="bf16", seed=303, nseg=4, **kw)
    if name == "bf16_virtual":
        return mk(name, batch=1, seqlen=2048, nheads=4, headdim=64, dstate=128, ngroups=2,
                  chunk=256, act="bf16", seed=304, nseg=4, layout="virtual", slow_decay=True, **kw)
    if name == "bf16_thd":
        return mk(name, batch=1, seqlen=4096, nheads=4, headdim=64, dstate=128, ngroups=1,
                  chunk=256, act="bf16", seed=305, nseg=4, packed=(100, 1500), **kw)
    if name == "bf16_q64":
        return mk(name, batch=1, seqlen=1024, nheads=4, headdim=64, dstate=64, ngroups=2,
                  chunk=64, act="bf16", seed=306, seg_lens=[64, 320, 640], slow_decay=True, **kw)
    if name == "bf16_q128":
        return mk(name, batch=2, seqlen=1024, nheads=2, headdim=32, dstate=64, ngroups=1,
                  chunk=128, act="bf16", seed=307, nseg=2, packed=(60, 300), **kw)
    if name == "bf16_blocks":
        # 16 heads in one group: two head blocks of 8 per group, summed per group
        return mk(name, batch=1, seqlen=1024, nheads=16, headdim=64, dstate=128, ngroups=1,
                  chunk=256, act="bf16", seed=308, nseg=2, packed=(100, 700), **kw)
    if name == "bf16_odd_hpg":
        # three heads per group: one head per walk block, head blocks of three
        return mk(name, batch=1, seqlen=1024, nheads=6, headdim=64, dstate=128, ngroups=2,
                  chunk=256, act="bf16", seed=310, nseg=2, packed=(90, 600), **kw)
    raise KeyError(name)


SMALL = ["tiny_f32", "slow_tiny_f32", "f32_head_thd", "f32_virtual", "bf16_small", "bf16_virtual", "bf16_thd",
         "bf16_q64", "bf16_q128", "bf16_blocks", "bf16_odd_hpg"]


def run_fwd_bwd(wl, inputs=None):
    import mamba2_ssd_chunked_amd as ssd
    p = problem_of(wl)
    x = inputs or device_inputs(wl)
    fb = ssd.forward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                     x["A_log"], x["D"], x["seq_idx"])
    bb = ssd.backward(p, wl.segments, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                      x["A_log"], x["D"], x["dy"], fb.S_in, seq_idx=x["seq_idx"])
    torch.cuda.synchronize()
    return p, x, fb, bb


def gpu_grads(wl, bb):
    return dict(dxBC=wl.to_causal(to_np(bb.dxBC)), dconv_w=to_np(bb.dconv_w),
                ddt_raw=wl.to_causal(to_np(bb.ddt_raw)), ddt_bias=to_np(bb.ddt_bias),
                dA_log=to_np(bb.dA_log), dD=to_np(bb.dD))


@pytest.fixture(scope="module", params=SMALL)
def bwd_run(request):
    wl = _bwd_small(request.param)
    log(f"[backward] case {wl.name}: b={wl.batch} L={wl.seqlen} H={wl.nheads} P={wl.headdim} "
        f"N={wl.dstate} G={wl.ngroups} Q={wl.chunk} act={wl.act} segs={len(wl.segments)} "
        f"layout={wl.layout} packed={wl.seq_idx is not None}")
    p, x, fb, bb = run_fwd_bwd(wl)
    return wl, p, x, fb, bb


def test_backward_summary(bwd_run):
    """Per segment: dL/dS_in from its own outputs (oracle initial-state gradient) and a_block."""
    wl, p, x, fb, bb = bwd_run
    v = oracle_v(wl)
    S, b, H, P, N = len(wl.segments), wl.batch, wl.nheads, wl.headdim, wl.dstate
    summ = to_np(bb.summary)
    Lk = summ[:S * b * H * P * N].reshape(S, b, H, P, N)
    ak = summ[S * b * H * P * N:].reshape(S, b, H)
    fwd_a = to_np(fb.summary)[S * b * H * P * N:].reshape(S, b, H)
    np.testing.assert_allclose(ak, fwd_a, rtol=1e-6, atol=0)  # product taken in reverse order
    seq = wl.causal_seq_idx()
    dt_raw = wl.to_causal(wl.dt_raw)
    dy = wl.to_causal(wl.dy)
    for k, (a, e) in enumerate(causal_ranges(wl)):
        s = None if seq is None else seq[:, a:e]
        g = oracle.ssd_bwd(v[:, a:e], dt_raw[:, a:e], wl.dt_bias, wl.A_log, wl.D, dy[:, a:e],
                           nheads=H, headdim=P, dstate=N, ngroups=wl.ngroups, dt_min=wl.dt_min,
                           dt_max=wl.dt_max, seq_idx=s, init=np.zeros((b, H, P, N)),
                           want_dinit=True)["dinit"]
        if seq is not None and a > 0:
            for r in range(b):
                if seq[r, a] != seq[r, a - 1]:
                    g[r] = 0.0  # the segment starts a new sequence: no state reaches it
        assert_close(Lk[k], g, wl.act, f"dL/dS_in local[{k}]")


def test_backward_gradients(bwd_run):
    wl, p, x, fb, bb = bwd_run
    ref = oracle.backward(wl)
    got = gpu_grads(wl, bb)
    for name in GRADS:
        assert_close(got[name], ref[name], wl.act, name)


def test_backward_phases_equal_composite(bwd_run):
    """summary -> reverse scan -> pass -> chunks -> conv backward, called one by one
    through the C ABI, gives the composite ssd_segment_bwd's gradients bit for bit."""
    import mamba2_ssd_chunked_amd as ssd
    wl, p, x, fb, bb = bwd_run
    s = ssd.Segments(wl.segments)
    b2 = ssd.BackwardBuffers.allocate(p, s, x["xBC"].device)
    ssd.ssd_segment_bwd_summary(p, s, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"],
                                x["A_log"], x["seq_idx"], x["dy"], b2.summary, b2.ws)
    ssd.ssd_boundary_scan(p, s.n, b2.summary, None, True, b2.dS_out)
    ssd.ssd_segment_bwd_pass(p, s, x["seq_idx"], x["dy"], fb.S_in, b2.dS_out, b2.ws)
    ssd.ssd_segment_bwd_chunks(p, s, x["D"], x["seq_idx"], x["dy"], b2.ws)
    ssd.ssd_conv1d_bwd(p, s, x["xBC"], x["conv_w"], x["dt_raw"], x["dt_bias"], x["A_log"],
                       x["seq_idx"], b2.ws, b2.dxBC, b2.ddt_raw, b2.dconv_w, b2.ddt_bias,
                       b2.dA_log, b2.dD)
    torch.cuda.synchronize()
    for name in ("dxBC", "ddt_raw", "dconv_w", "ddt_bias", "dA_log", "dD"):
        assert torch.equal(getattr(b2, name), getattr(bb, name)), name


def test_backward_mixer_shard_full():
    wl = W.config("mixer_shard_bwd_bf16")
    log(f"[backward] {wl.name}")
    _, _, _, bb = run_fwd_bwd(wl)
    ref = oracle.backward(wl)
    got = gpu_grads(wl, bb)
    for name in GRADS:
        assert_close(got[name], ref[name], wl.act, f"mixer shard {name}")


def test_backward_packed_thd_full():
    """32768 packed tokens, lengths U[512, 8192], 4 segments: every gradient."""
    wl = W.make_workload("packed_thd_bwd_bf16", **W.WORKLOADS["packed_thd_bf16"], with_dy=True)
    log(f"[backward] {wl.name}")
    _, _, _, bb = run_fwd_bwd(wl)
    ref = oracle.backward(wl)
    got = gpu_grads(wl, bb)
    for name in GRADS:
        assert_close(got[name], ref[name], wl.act, f"packed thd {name}")


def test_maximum_segment_count():
    """SSD_MAX_SEGMENTS (64) segments of one 64-token chunk each, with packed
    sequences crossing them: y and every gradient against the oracle.  Each walk
    then covers a single slice."""
    wl = W.make_workload("max_segments", batch=1, seqlen=4096, nheads=2, headdim=64,
                         dstate=64, ngroups=1, chunk=64, act="bf16", seed=309, nseg=64,
                         packed=(30, 400), with_dy=True)
    log(f"[backward] {wl.name}: {len(wl.segments)} segments")
    _, _, fb, bb = run_fwd_bwd(wl)
    ref = oracle.backward(wl)
    assert_close(wl.to_causal(to_np(fb.y)), ref["y"], wl.act, "y, 64 segments")
    got = gpu_grads(wl, bb)
    for name in GRADS:
        assert_close(got[name], ref[name], wl.act, f"{name}, 64 segments")


@pytest.mark.parametrize("cfg", ["long_context_bf16", "long_context_virtual_bf16"])
def test_backward_long_context_whole_groups(cfg):
    """131072 tokens, 64 heads in 8 groups: the full backward on the GPU; every gradient
    of the first and the last group (heads 0-7 and 56-63: their x channels and the
    groups' B and C channels in dxBC and dconv_w, ddt_raw, ddt_bias, dA_log, dD)
    against the oracle restricted to that group."""
    wl = W.make_workload(cfg.replace("_bf16", "_bwd_bf16"), **W.WORKLOADS[cfg], with_dy=True)
    log(f"[backward] {wl.name} whole groups")
    _, _, _, bb = run_fwd_bwd(wl)
    hpg = wl.nheads // wl.ngroups
    for g in (0, wl.ngroups - 1):
        heads = list(range(g * hpg, (g + 1) * hpg))
        ref = oracle.backward(wl, heads=heads)
        ch = torch.from_numpy(ref["channels"]).to(bb.dxBC.device)
        hs = torch.tensor(heads, device=bb.dxBC.device)
        got = dict(dxBC=wl.to_causal(to_np(bb.dxBC.index_select(2, ch))),
                   dconv_w=to_np(bb.dconv_w.index_select(0, ch)),
                   ddt_raw=wl.to_causal(to_np(bb.ddt_raw.index_select(2, hs))),
                   ddt_bias=to_np(bb.ddt_bias)[heads], dA_log=to_np(bb.dA_log)[heads],
                   dD=to_np(bb.dD)[heads])
        assert ref["dxBC"].shape[2] == hpg * wl.headdim + 2 * wl.dstate
        for name in GRADS:
            assert_close(got[name], ref[name], wl.act, f"{cfg} {name} group {g}")
        del ref


def test_tiny_gradients_against_finite_differences():
    """Central differences of L = <dy, y> with the float64 oracle forward, sampled entries."""
    import copy
    wl = _bwd_small("tiny_f32")
    log("[backward] tiny_f32 finite differences")
    _, _, _, bb = run_fwd_bwd(wl)
    got = gpu_grads(wl, bb)

    def loss(field, arr):
        w2 = copy.copy(wl)
        setattr(w2, field, arr)
        return float((oracle.forward(w2) * wl.to_causal(wl.dy)).sum())

    rng = np.random.default_rng(9)
    eps = 1e-3
    for name, field in [("dxBC", "xBC"), ("dconv_w", "conv_w"), ("ddt_raw", "dt_raw"),
                        ("ddt_bias", "dt_bias"), ("dA_log", "A_log"), ("dD", "D")]:
        base = getattr(wl, field)
        idx = rng.choice(base.size, size=min(8, base.size), replace=False)
        scale = np.sqrt(np.mean(got[name] ** 2)) + 1e-12
        for fi in idx:
            plus = base.copy().reshape(-1)
            minus = base.copy().reshape(-1)
            plus[fi] = np.float32(plus[fi] + eps)
            minus[fi] = np.float32(minus[fi] - eps)
            h = float(plus[fi]) - float(minus[fi])
            fd = (loss(field, plus.reshape(base.shape)) - loss(field, minus.reshape(base.shape))) / h
            # the memory-order index of a token array equals the causal one here (contiguous)
            an = got[name].reshape(-1)[fi]
            assert abs(fd - an) <= 1e-3 * max(abs(fd), scale), (name, int(fi), fd, an)


def test_backward_determinism():
    wl = _bwd_small("bf16_thd")
    log("[backward] determinism")
    _, x, _, b1 = run_fwd_bwd(wl)
    r1 = [t.clone() for t in (b1.dxBC, b1.ddt_raw, b1.dconv_w, b1.ddt_bias, b1.dA_log, b1.dD)]
    _, _, _, b2 = run_fwd_bwd(wl, inputs=x)
    r2 = (b2.dxBC, b2.ddt_raw, b2.dconv_w, b2.ddt_bias, b2.dA_log, b2.dD)
    for a, c in zip(r1, r2):
        assert torch.equal(a, c)


def test_backward_reset_isolation_is_bitwise():
    """Changing dy inside one packed sequence leaves every other sequence's dxBC and ddt bit-identical."""
    wl = W.make_workload("iso_bwd", batch=1, seqlen=4096, nheads=4, headdim=64, dstate=128,
                         ngroups=1, chunk=256, act="bf16", seed=308, nseg=4, packed=(300, 1400),
                         with_dy=True)
    log("[backward] reset isolation")
    x = device_inputs(wl)
    _, _, _, b1 = run_fwd_bwd(wl, inputs=x)
    d1, t1 = b1.dxBC.clone(), b1.ddt_raw.clone()
    seq = wl.seq_idx[0]
    target = int(seq[len(seq) // 2])
    mask = torch.from_numpy(seq == target).cuda()
    x2 = dict(x)
    x2["dy"] = x["dy"].clone()
    x2["dy"][0, mask] = (x["dy"][0, mask].float() * 1.7 - 0.3).to(x["dy"].dtype)
    _, _, _, b2 = run_fwd_bwd(wl, inputs=x2)
    keep = ~mask
    assert torch.equal(d1[0, keep], b2.dxBC[0, keep])
    assert torch.equal(t1[0, keep], b2.ddt_raw[0, keep])
    assert not torch.equal(d1[0, mask], b2.dxBC[0, mask])
