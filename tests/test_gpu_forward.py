"""GPU parity of the forward path against the CPU oracle (through the C ABI).

Component checks (conv, boundary scan, segment summaries, zero-state output,
correction) and end-to-end checks on small workloads that span several tiles,
unequal segments, packed sequences that start inside chunks and the virtual
front/back layout, plus the full-size workloads (the 131072-token ones on sampled
heads).  Tolerances: float32 inputs, max relative error 1e-4 (floored at the
output RMS); bf16 inputs, relative RMS error 2e-2.
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_workloads as W
from ssd_testlib import (assert_close, causal_ranges, device_inputs, err_fp32, log, oracle_segment,
                         oracle_v, problem_of, rms, run_forward, to_np)

pytestmark = pytest.mark.gpu


def _small(name):
    mk = W.make_workload
    if name in ("tiny_f32", "slow_tiny_f32"):
        return W.config(name)
    if name == "f32_head_thd":
        return mk(name, batch=2, seqlen=512, nheads=4, headdim=64, dstate=128, ngroups=2,
                  chunk=64, act="f32", seed=101, seg_lens=[128, 256, 128],
                  lengths=[37, 150, 1, 200, 124])
    if name == "f32_virtual":
        return mk(name, batch=1, seqlen=512, nheads=2, headdim=32, dstate=32, ngroups=1,
                  chunk=64, act="f32", seed=102, nseg=4, layout="virtual", slow_decay=True)
    if name == "bf16_small":
        return mk(name, batch=2, seqlen=2048, nheads=4, headdim=64, dstate=128, ngroups=1,
                  chunk=256, act="bf16", seed=103, nseg=4)
    if name == "bf16_virtual":
        return mk(name, batch=1, seqlen=2048, nheads=4, headdim=64, dstate=128, ngroups=2,
                  chunk=256, act="bf16", seed=104, nseg=4, layout="virtual", slow_decay=True)
    if name == "bf16_thd":
        return mk(name, batch=1, seqlen=4096, nheads=4, headdim=64, dstate=128, ngroups=1,
                  chunk=256, act="bf16", seed=105, nseg=4, packed=(100, 1500))
    if name == "bf16_q64":
        return mk(name, batch=1, seqlen=1024, nheads=4, headdim=64, dstate=64, ngroups=2,
                  chunk=64, act="bf16", seed=106, seg_lens=[64, 320, 640], slow_decay=True)
    if name == "bf16_spans":
        # long segments on few heads: the state walk splits them into spans of
        # four chunks (8 spans), composed afterwards
        return mk(name, batch=1, seqlen=8192, nheads=2, headdim=64, dstate=128, ngroups=1,
                  chunk=256, act="bf16", seed=108, seg_lens=[2048, 6144], packed=(700, 3000),
                  slow_decay=True)
    if name == "f32_spans":
        # float32, chunk 64: spans of sixteen chunks, two per segment
        return mk(name, batch=2, seqlen=2048, nheads=2, headdim=32, dstate=32, ngroups=1,
                  chunk=64, act="f32", seed=109, nseg=1, packed=(300, 900), slow_decay=True)
    if name == "bf16_q128":
        return mk(name, batch=2, seqlen=1024, nheads=2, headdim=32, dstate=64, ngroups=1,
                  chunk=128, act="bf16", seed=107, nseg=2, packed=(60, 300))
    raise KeyError(name)


SMALL = ["tiny_f32", "slow_tiny_f32", "f32_head_thd", "f32_virtual", "bf16_small", "bf16_virtual", "bf16_thd",
         "bf16_q64", "bf16_q128", "bf16_spans", "f32_spans"]


@pytest.fixture(scope="module", params=SMALL)
def small_run(request):
    wl = _small(request.param)
    log(f"[forward] case {wl.name}: b={wl.batch} L={wl.seqlen} H={wl.nheads} P={wl.headdim} "
        f"N={wl.dstate} G={wl.ngroups} Q={wl.chunk} act={wl.act} segs={len(wl.segments)} "
        f"layout={wl.layout} packed={wl.seq_idx is not None}")
    p, x, bufs = run_forward(wl, fused=False)
    return wl, p, x, bufs


def test_conv(small_run):
    wl, p, x, bufs = small_run
    g = wl.to_causal(to_np(bufs.xBC_conv))
    o = oracle_v(wl)
    # float32: fp32 accumulation error only; bf16: plus one rounding to bf16 (2^-9 relative)
    tol = 1e-5 if wl.act == "f32" else 2.0 ** -8
    err = err_fp32(g, o)
    log(f"  conv max rel err (floored at RMS) {err:.3e}")
    assert err <= tol


def test_summaries_and_zero_state_output(small_run):
    """S_ext, a_block and y_zero of every segment vs the oracle run of that segment alone."""
    wl, p, x, bufs = small_run
    v = oracle_v(wl)
    S, b, H, P, N = len(wl.segments), wl.batch, wl.nheads, wl.headdim, wl.dstate
    summ = to_np(bufs.summary)
    S_ext = summ[:S * b * H * P * N].reshape(S, b, H, P, N)
    a_blk = summ[S * b * H * P * N:].reshape(S, b, H)
    yz = wl.to_causal(to_np(bufs.y_zero))
    seq = wl.causal_seq_idx()
    v_no_x = v.copy()
    v_no_x[..., :H * P] = 0.0  # with x = 0 the final state is exactly a_block * init
    for k, (a, e) in enumerate(causal_ranges(wl)):
        y0, f0 = oracle_segment(wl, v, k)
        _, f1 = oracle_segment(wl, v_no_x, k, init=np.ones((b, H, P, N)))
        a_ref = f1[:, :, 0, 0]
        assert_close(S_ext[k], f0, wl.act, f"S_ext[{k}]")
        assert_close(yz[:, a:e], y0, wl.act, f"y_zero[{k}]")
        np.testing.assert_allclose(a_blk[k], a_ref, rtol=1e-4, atol=1e-30)
        if seq is not None:
            for r in range(b):
                lo = seq[r, a - 1] if a > 0 else seq[r, a]
                if seq[r, e - 1] != lo:
                    assert np.all(a_blk[k, r] == 0.0), "a_block must be exactly 0 across a reset"


def test_apply_init_state_random_states(small_run):
    """Correction pass with random S_in equals the oracle run of each segment from S_in."""
    import mamba2_ssd_chunked_amd as ssd
    wl, p, x, bufs = small_run
    S, b, H, P, N = len(wl.segments), wl.batch, wl.nheads, wl.headdim, wl.dstate
    rng = np.random.default_rng(77)
    S_in = rng.standard_normal((S, b, H, P, N)).astype(np.float32)
    S_dev = torch.from_numpy(S_in).cuda()
    y = torch.empty_like(bufs.y)
    ssd.ssd_apply_init_state(p, wl.segments, bufs.y_zero, bufs.xBC_conv, x["D"], x["seq_idx"],
                             S_dev, bufs.ws, y)
    torch.cuda.synchronize()
    g = wl.to_causal(to_np(y))
    v = oracle_v(wl)
    for k, (a, e) in enumerate(causal_ranges(wl)):
        yk, _ = oracle_segment(wl, v, k, init=S_in[k].astype(np.float64), D_zero=False)
        assert_close(g[:, a:e], yk, wl.act, f"y(S_in random)[{k}]")


def test_end_to_end(small_run):
    wl, p, x, bufs = small_run
    g = wl.to_causal(to_np(bufs.y))
    o = oracle.forward(wl)
    assert_close(g, o, wl.act, "y")


def test_fused_output_end_to_end(small_run):
    """States first, boundary scan, then the fused output pass (true entering
    states and D x in one pass) against the oracle, from the workspace the
    unfused run filled."""
    import mamba2_ssd_chunked_amd as ssd
    wl, p, x, bufs = small_run
    y = torch.empty_like(bufs.y)
    ssd.ssd_segment_output_fused(p, wl.segments, bufs.xBC_conv, x["D"], x["seq_idx"], bufs.S_in,
                                 bufs.ws, y)
    torch.cuda.synchronize()
    g = wl.to_causal(to_np(y))
    o = oracle.forward(wl)
    assert_close(g, o, wl.act, "y (fused output)")


def test_fused_output_random_states(small_run):
    """The fused output pass from random S_in equals the oracle run of each
    segment from that S_in (every chunk's entering state carries it)."""
    import mamba2_ssd_chunked_amd as ssd
    wl, p, x, bufs = small_run
    S, b, H, P, N = len(wl.segments), wl.batch, wl.nheads, wl.headdim, wl.dstate
    rng = np.random.default_rng(78)
    S_in = rng.standard_normal((S, b, H, P, N)).astype(np.float32)
    y = torch.empty_like(bufs.y)
    ssd.ssd_segment_output_fused(p, wl.segments, bufs.xBC_conv, x["D"], x["seq_idx"],
                                 torch.from_numpy(S_in).cuda(), bufs.ws, y)
    torch.cuda.synchronize()
    g = wl.to_causal(to_np(y))
    v = oracle_v(wl)
    for k, (a, e) in enumerate(causal_ranges(wl)):
        yk, _ = oracle_segment(wl, v, k, init=S_in[k].astype(np.float64), D_zero=False)
        assert_close(g[:, a:e], yk, wl.act, f"y fused (S_in random)[{k}]")


# --------------------------------------------------------------------------- boundary scan


@pytest.mark.parametrize("nseg", [1, 2, 5, 16, 64])
def test_boundary_scan_against_float64_loop(nseg):
    """Random block decays a ~ U(0, 1) so every term of the composition matters."""
    import mamba2_ssd_chunked_amd as ssd
    log(f"[scan] nseg={nseg}")
    p = ssd.make_problem(batch=2, seqlen=64 * nseg, nheads=3, headdim=16, dstate=16, ngroups=1,
                         chunk=64, conv_width=4, act="f32")
    rng = np.random.default_rng(nseg)
    bh, pn = 2 * 3, 16 * 16
    M = rng.standard_normal((nseg, bh, pn)).astype(np.float32)
    a = rng.uniform(0, 1, (nseg, bh)).astype(np.float32)
    init = rng.standard_normal((bh, pn)).astype(np.float32)
    summ = torch.from_numpy(np.concatenate([M.reshape(-1), a.reshape(-1)])).cuda()
    for reverse in (0, 1):
        for use_init in (False, True):
            out = torch.empty(nseg * bh * pn, device="cuda")
            fin = torch.empty(bh * pn, device="cuda")
            ssd.ssd_boundary_scan(p, nseg, summ, torch.from_numpy(init).cuda() if use_init else None,
                                  bool(reverse), out, fin)
            torch.cuda.synchronize()
            cur = init.astype(np.float64) if use_init else np.zeros((bh, pn))
            ref = np.zeros((nseg, bh, pn))
            order = range(nseg - 1, -1, -1) if reverse else range(nseg)
            for k in order:
                ref[k] = cur
                cur = a[k].astype(np.float64)[:, None] * cur + M[k]
            np.testing.assert_allclose(to_np(out).reshape(nseg, bh, pn), ref, rtol=1e-5, atol=1e-5)
            np.testing.assert_allclose(to_np(fin).reshape(bh, pn), cur, rtol=1e-5, atol=1e-5)


# --------------------------------------------------------------------------- invariants


def test_segment_count_does_not_change_result():
    """One segment vs sixteen: the same answer within the bf16 tolerance."""
    kw = dict(batch=1, seqlen=4096, nheads=4, headdim=64, dstate=128, ngroups=1, chunk=256,
              act="bf16", seed=201, slow_decay=True)
    one = W.make_workload("one", nseg=1, **kw)
    many = W.make_workload("many", nseg=16, **kw)
    log("[invariant] 1 vs 16 segments")
    _, _, b1 = run_forward(one)
    _, _, b2 = run_forward(many)
    assert_close(to_np(b2.y), to_np(b1.y), "bf16", "y(16 segs) vs y(1 seg)")


def test_virtual_equals_contiguous():
    kw = dict(batch=1, seqlen=4096, nheads=4, headdim=64, dstate=128, ngroups=2, chunk=256,
              act="bf16", seed=202, nseg=4, slow_decay=True)
    c = W.make_workload("contig", layout="contiguous", **kw)
    v = W.make_workload("virt", layout="virtual", **kw)
    log("[invariant] virtual vs contiguous")
    _, _, bc = run_forward(c)
    _, _, bv = run_forward(v)
    assert_close(v.to_causal(to_np(bv.y)), to_np(bc.y), "bf16", "virtual vs contiguous")


def test_reset_isolation_is_bitwise():
    """Changing one packed sequence leaves every other sequence's output bit-identical."""
    wl = W.make_workload("iso", batch=1, seqlen=4096, nheads=4, headdim=64, dstate=128, ngroups=1,
                         chunk=256, act="bf16", seed=203, nseg=4, packed=(300, 1400))
    log("[invariant] reset isolation")
    x = device_inputs(wl)
    _, _, b1 = run_forward(wl, inputs=x)
    y1 = b1.y.clone()
    seq = wl.seq_idx[0]
    target = int(seq[len(seq) // 2])
    mask = torch.from_numpy(seq == target).cuda()
    x2 = dict(x)
    x2["xBC"] = x["xBC"].clone()
    x2["xBC"][0, mask] = (x["xBC"][0, mask].float() * -1.5 + 0.25).to(x["xBC"].dtype)
    x2["dt_raw"] = x["dt_raw"].clone()
    x2["dt_raw"][0, mask] = (x["dt_raw"][0, mask].float() + 0.7).to(x["dt_raw"].dtype)
    _, _, b2 = run_forward(wl, inputs=x2)
    y2 = b2.y
    keep = ~mask
    assert torch.equal(y1[0, keep], y2[0, keep])
    assert not torch.equal(y1[0, mask], y2[0, mask])


def test_determinism():
    wl = _small("bf16_thd")
    log("[invariant] determinism")
    _, x, b1 = run_forward(wl)
    y1 = b1.y.clone()
    s1 = b1.summary.clone()
    _, _, b2 = run_forward(wl, inputs=x)
    assert torch.equal(y1, b2.y) and torch.equal(s1, b2.summary)


# --------------------------------------------------------------------------- full sizes


@pytest.mark.parametrize("cfg,fused", [("mixer_shard_bf16", True), ("mixer_shard_bf16", False),
                                       ("packed_thd_bf16", True), ("slow_mixer_shard_bf16", True)])
def test_full_config(cfg, fused):
    wl = W.config(cfg)
    log(f"[full] {cfg} fused={fused}")
    _, _, bufs = run_forward(wl, fused=fused)
    g = wl.to_causal(to_np(bufs.y))
    o = oracle.forward(wl)
    assert_close(g, o, wl.act, f"y {cfg}")


@pytest.mark.parametrize("cfg", ["long_context_bf16", "long_context_virtual_bf16"])
def test_long_context_all_heads(cfg):
    """131072 tokens, 64 heads in 8 groups: y of every head against the oracle, one
    group at a time (the oracle restricted to a group's heads and channels gives
    exactly the full problem's values for them)."""
    wl = W.config(cfg)
    log(f"[full] {cfg} all heads")
    _, _, bufs = run_forward(wl)
    hpg = wl.nheads // wl.ngroups
    for g in range(wl.ngroups):
        heads = list(range(g * hpg, (g + 1) * hpg))
        got = wl.to_causal(to_np(bufs.y[:, :, g * hpg:(g + 1) * hpg]))
        o = oracle.forward(wl, heads=heads)
        assert_close(got, o, wl.act, f"y {cfg} group {g}")
