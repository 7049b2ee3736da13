"""Pins for the CPU oracle: it must agree with things other than itself.

Each test ties one part of the oracle to an independent statement of the
mathematics: hand-derived fixtures (tests/golden), a brute-force quadratic
(SSD-matrix) form, torch's conv1d, closed forms, library filters, invariants
of state passing, finite differences and torch autograd of the quadratic form.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle
import ssd_workloads as W

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_fixture(name):
    rows = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _v_from_parts(x, B, C):
    """Pack per-token x [L,H,P], B [L,G,N], C [L,G,N] into v [1, L, C]."""
    L = x.shape[0]
    return np.concatenate([x.reshape(L, -1), B.reshape(L, -1), C.reshape(L, -1)], axis=1)[None]


# ---------------------------------------------------------------- golden fixtures


@pytest.mark.parametrize("case", ["plain", "reset"])
def test_golden_three_token(case):
    rows = [r for r in _read_fixture("ssd_three_token.txt") if r[0] == case]
    x = np.array([float(r[2]) for r in rows]).reshape(3, 1, 1)
    B = np.array([float(r[3]) for r in rows]).reshape(3, 1, 1)
    C = np.array([float(r[4]) for r in rows]).reshape(3, 1, 1)
    want = np.array([float(r[5]) for r in rows])
    seq = np.array([[0, 0, 1]], np.int32) if case == "reset" else None
    y = oracle.ssd_fwd(_v_from_parts(x, B, C), np.full((1, 3, 1), 20.0), np.zeros(1),
                       np.zeros(1), np.full(1, 0.5), nheads=1, headdim=1, dstate=1, ngroups=1,
                       dt_min=1e-3, dt_max=0.125, seq_idx=seq)
    np.testing.assert_allclose(y.reshape(3), want, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("case", ["plain", "reset"])
def test_golden_conv_impulse(case):
    rows = [r for r in _read_fixture("conv_impulse.txt") if r[0] == case]
    want_u = np.array([float(r[2]) for r in rows])
    L = len(rows)
    xBC = np.zeros((1, L, 1), np.float32)
    xBC[0, 0, 0] = 1.0
    w = np.array([[0.5, -1.0, 2.0, 3.0]], np.float32)
    seq = np.array([[0, 0, 1, 1, 1, 1]], np.int32) if case == "reset" else None
    u, v = oracle.conv_silu(xBC, w, seq)
    np.testing.assert_array_equal(u.reshape(L), want_u)
    sig = 1.0 / (1.0 + np.exp(-want_u))
    np.testing.assert_allclose(v.reshape(L), want_u * sig, rtol=1e-15)


# ---------------------------------------------------------------- brute-force quadratic form


def _brute_quadratic(v, dt_raw, dt_bias, A_log, D, H, P, N, G, dt_min, dt_max, seq_idx=None):
    """y = (Lambda o C B^T)(dt o x) + D x, built as an explicit L x L matrix per head.

    Lambda[i, j] = exp(sum_{r=j+1..i} dt_r A) for j <= i within one sequence,
    0 otherwise.  Written independently of the oracle's recurrence.
    """
    b, L, Cc = v.shape
    hpg = H // G
    y = np.zeros((b, L, H, P))
    for bi in range(b):
        for h in range(H):
            g = h // hpg
            x = v[bi, :, h * P:(h + 1) * P]
            Bm = v[bi, :, H * P + g * N:H * P + (g + 1) * N]
            Cm = v[bi, :, H * P + G * N + g * N:H * P + G * N + (g + 1) * N]
            z = dt_raw[bi, :, h].astype(np.float64) + float(dt_bias[h])
            dt = np.clip(np.logaddexp(0.0, z), float(np.float32(dt_min)), float(np.float32(dt_max)))
            A = -math.exp(float(A_log[h]))
            lam = np.zeros((L, L))
            for i in range(L):
                for j in range(i + 1):
                    if seq_idx is not None and seq_idx[bi, i] != seq_idx[bi, j]:
                        continue
                    lam[i, j] = math.exp(A * dt[j + 1:i + 1].sum())
            M = lam * (Cm @ Bm.T)
            y[bi, :, h, :] = M @ (dt[:, None] * x) + float(D[h]) * x
    return y


@pytest.mark.parametrize("packed", [False, True])
def test_recurrence_matches_quadratic_form(packed):
    wl = W.make_workload("pin", batch=2, seqlen=48, nheads=4, headdim=3, dstate=5, ngroups=2,
                         chunk=16, act="f32", seed=7,
                         lengths=[5, 1, 20, 22] if packed else None)
    seq = wl.seq_idx
    _, v = oracle.conv_silu(wl.xBC, wl.conv_w, seq)
    y = oracle.ssd_fwd(v, wl.dt_raw, wl.dt_bias, wl.A_log, wl.D, nheads=4, headdim=3, dstate=5,
                       ngroups=2, seq_idx=seq)
    yb = _brute_quadratic(v, wl.dt_raw, wl.dt_bias, wl.A_log, wl.D, 4, 3, 5, 2,
                          wl.dt_min, wl.dt_max, seq)
    np.testing.assert_allclose(y, yb, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- conv against torch


@pytest.mark.parametrize("width", [2, 4])
def test_conv_matches_torch_conv1d(width):
    rng = np.random.default_rng(3)
    b, L, C = 2, 37, 11
    x = rng.standard_normal((b, L, C)).astype(np.float32)
    w = rng.standard_normal((C, width)).astype(np.float32)
    u, v = oracle.conv_silu(x, w)
    xt = torch.from_numpy(x.astype(np.float64)).transpose(1, 2)
    wt = torch.from_numpy(w.astype(np.float64)).unsqueeze(1)
    ref = torch.nn.functional.conv1d(xt, wt, groups=C, padding=width - 1)[..., :L]
    ref = ref.transpose(1, 2).numpy()
    np.testing.assert_allclose(u, ref, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(v, torch.nn.functional.silu(torch.from_numpy(ref)).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_conv_resets_equal_separate_sequences():
    rng = np.random.default_rng(4)
    lens = [3, 9, 1, 12]
    L, C = sum(lens), 6
    x = rng.standard_normal((1, L, C)).astype(np.float32)
    w = rng.standard_normal((C, 4)).astype(np.float32)
    _, seq = W.seq_idx_from_lengths(np.array(lens))
    _, v = oracle.conv_silu(x, w, seq[None])
    o = 0
    for n in lens:
        _, vs = oracle.conv_silu(x[:, o:o + n], w)
        np.testing.assert_array_equal(v[:, o:o + n], vs)
        o += n


# ---------------------------------------------------------------- closed forms


def test_no_decay_is_causal_linear_attention():
    """A -> 0 and D = 0: y_t = sum_{j<=t} dt_j (C_t . B_j) x_j, a running sum."""
    rng = np.random.default_rng(5)
    L, P, N = 30, 4, 3
    x = rng.standard_normal((L, 1, P))
    B = rng.standard_normal((L, 1, N))
    C = rng.standard_normal((L, 1, N))
    dt_raw = rng.standard_normal((1, L, 1)).astype(np.float32)
    y = oracle.ssd_fwd(_v_from_parts(x, B, C), dt_raw, np.zeros(1), np.full(1, -60.0),
                       np.zeros(1), nheads=1, headdim=P, dstate=N, ngroups=1)
    dt = np.clip(np.log1p(np.exp(dt_raw[0, :, 0].astype(np.float64))),
                 float(np.float32(1e-3)), float(np.float32(0.1)))
    S = np.cumsum(dt[:, None, None] * x[:, 0, :, None] * B[:, 0, None, :], axis=0)
    want = np.einsum("tpn,tn->tp", S, C[:, 0])
    np.testing.assert_allclose(y[0, :, 0], want, rtol=1e-12, atol=1e-13)


def test_scalar_state_is_geometric_filter():
    """P = N = 1, B = C = 1, dt clamped: y = lfilter([dt], [1, -exp(dt A)], x) + D x."""
    from scipy.signal import lfilter
    rng = np.random.default_rng(6)
    L = 200
    x = rng.standard_normal((L, 1, 1))
    ones = np.ones((L, 1, 1))
    A_log = np.float32(0.7)
    A = -math.exp(float(A_log))
    dt = float(np.float32(0.1))
    y = oracle.ssd_fwd(_v_from_parts(x, ones, ones), np.full((1, L, 1), 30.0), np.zeros(1),
                       np.full(1, A_log), np.full(1, 0.25), nheads=1, headdim=1, dstate=1,
                       ngroups=1)
    want = lfilter([dt], [1.0, -math.exp(dt * A)], x[:, 0, 0]) + 0.25 * x[:, 0, 0]
    np.testing.assert_allclose(y[0, :, 0, 0], want, rtol=1e-12, atol=1e-13)


def test_single_token_and_dt_path():
    """One token: y0 = dt0 (C0 . B0) x0 + D x0.  dt0 = softplus(raw + bias) = 0.05 exactly."""
    rng = np.random.default_rng(8)
    P, N = 5, 7
    x = rng.standard_normal((1, 1, P))
    B = rng.standard_normal((1, 1, N))
    C = rng.standard_normal((1, 1, N))
    bias = np.float32(math.log(math.expm1(0.05)))  # inverse softplus of 0.05
    y = oracle.ssd_fwd(_v_from_parts(x, B, C), np.zeros((1, 1, 1)), np.full(1, bias),
                       np.zeros(1), np.full(1, -1.5), nheads=1, headdim=P, dstate=N, ngroups=1)
    dt = math.log1p(math.exp(float(bias)))
    assert abs(dt - 0.05) < 1e-8
    want = dt * float(C[0, 0] @ B[0, 0]) * x[0, 0] - 1.5 * x[0, 0]
    np.testing.assert_allclose(y[0, 0, 0], want, rtol=1e-13)
    # clamp: a very large or very negative raw value pins dt to the bounds
    for raw, dt_want in [(40.0, np.float32(0.1)), (-40.0, np.float32(1e-3))]:
        y = oracle.ssd_fwd(_v_from_parts(x, B, C), np.full((1, 1, 1), raw), np.zeros(1),
                           np.zeros(1), np.zeros(1), nheads=1, headdim=P, dstate=N, ngroups=1)
        np.testing.assert_allclose(y[0, 0, 0], float(dt_want) * float(C[0, 0] @ B[0, 0]) * x[0, 0],
                                   rtol=1e-13)


# ---------------------------------------------------------------- state-passing invariants


def _small(seed=11, **kw):
    base = dict(batch=1, seqlen=96, nheads=2, headdim=4, dstate=3, ngroups=1, chunk=16,
                act="f32", seed=seed, slow_decay=True)
    base.update(kw)
    return W.make_workload("inv", **base)


def _kw(wl):
    return dict(nheads=wl.nheads, headdim=wl.headdim, dstate=wl.dstate, ngroups=wl.ngroups,
                dt_min=wl.dt_min, dt_max=wl.dt_max)


@pytest.mark.parametrize("lengths", [None, [10, 50, 36]])
def test_segmented_equals_unsegmented(lengths):
    """Running segment k from the final state of segment k-1 reproduces the full run."""
    wl = _small(lengths=lengths)
    seq = wl.seq_idx
    _, v = oracle.conv_silu(wl.xBC, wl.conv_w, seq)
    y_full = oracle.ssd_fwd(v, wl.dt_raw, wl.dt_bias, wl.A_log, wl.D, seq_idx=seq, **_kw(wl))
    cuts = [0, 17, 40, 41, 96]
    state = None
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        s = None if seq is None else seq[:, a:b]
        if s is not None and a > 0 and state is not None and seq[0, a] != seq[0, a - 1]:
            state = np.zeros_like(state)  # the segment's first token starts a new sequence
        y, state = oracle.ssd_fwd(v[:, a:b], wl.dt_raw[:, a:b], wl.dt_bias, wl.A_log, wl.D,
                                  seq_idx=s, init=state, want_final=True, **_kw(wl))
        parts.append(y)
    np.testing.assert_allclose(np.concatenate(parts, axis=1), y_full, rtol=1e-12, atol=1e-13)


def test_segment_map_is_affine_in_initial_state():
    """S_out = a_block * S_in + S_ext with a scalar a_block = exp(A sum dt); y affine in S_in."""
    wl = _small(seqlen=64)
    _, v = oracle.conv_silu(wl.xBC, wl.conv_w)
    rng = np.random.default_rng(12)
    S1 = rng.standard_normal((1, 2, 4, 3))
    S2 = rng.standard_normal((1, 2, 4, 3))
    run = lambda S: oracle.ssd_fwd(v, wl.dt_raw, wl.dt_bias, wl.A_log, wl.D, init=S,
                                   want_final=True, **_kw(wl))
    y0, f0 = run(np.zeros_like(S1))
    y1, f1 = run(S1)
    y2, f2 = run(S2)
    y12, f12 = run(S1 + 2.5 * S2)
    np.testing.assert_allclose(y12 - y0, (y1 - y0) + 2.5 * (y2 - y0), rtol=1e-10, atol=1e-12)
    for h in range(2):
        ratio = (f1 - f0)[0, h] / S1[0, h]
        assert np.allclose(ratio, ratio.flat[0], rtol=1e-9)
        z = wl.dt_raw[0, :, h].astype(np.float64) + float(wl.dt_bias[h])
        dt = np.clip(np.logaddexp(0, z), float(np.float32(1e-3)), float(np.float32(0.1)))
        a_block = math.exp(-math.exp(float(wl.A_log[h])) * dt.sum())
        np.testing.assert_allclose(ratio.flat[0], a_block, rtol=1e-10)
        assert 0.05 < a_block < 0.99  # slow-decay workload: the scan really composes


def test_reset_kills_initial_state_and_isolates_sequences():
    wl = _small(seqlen=64, lengths=[20, 44])
    _, v = oracle.conv_silu(wl.xBC, wl.conv_w, wl.seq_idx)
    S = np.random.default_rng(13).standard_normal((1, 2, 4, 3))
    y0, f0 = oracle.ssd_fwd(v, wl.dt_raw, wl.dt_bias, wl.A_log, wl.D, seq_idx=wl.seq_idx,
                            init=np.zeros_like(S), want_final=True, **_kw(wl))
    y1, f1 = oracle.ssd_fwd(v, wl.dt_raw, wl.dt_bias, wl.A_log, wl.D, seq_idx=wl.seq_idx,
                            init=S, want_final=True, **_kw(wl))
    np.testing.assert_array_equal(f0, f1)           # a_block is exactly 0 across a reset
    np.testing.assert_array_equal(y0[:, 20:], y1[:, 20:])
    assert np.abs(y0[:, :20] - y1[:, :20]).max() > 1e-6


def test_packed_equals_each_sequence_alone():
    lens = [7, 30, 1, 26]
    wl = _small(seqlen=64, lengths=lens, slow_decay=False)
    y = oracle.forward(wl)
    o = 0
    for n in lens:
        _, v = oracle.conv_silu(wl.xBC[:, o:o + n], wl.conv_w)
        ys = oracle.ssd_fwd(v, wl.dt_raw[:, o:o + n], wl.dt_bias, wl.A_log, wl.D, **_kw(wl))
        np.testing.assert_array_equal(y[:, o:o + n], ys)
        o += n


def test_head_subset_matches_full_run():
    wl = W.make_workload("sub", batch=1, seqlen=64, nheads=8, headdim=4, dstate=4, ngroups=4,
                         chunk=16, act="bf16", seed=21)
    y = oracle.forward(wl)
    ys = oracle.forward(wl, heads=[2, 3, 6, 7])
    np.testing.assert_array_equal(ys, y[:, :, [2, 3, 6, 7]])


@pytest.mark.parametrize("heads", [[2, 3, 6, 7], [2, 6]])
def test_head_subset_backward_matches_full_run(heads):
    """Gradients that belong to one head alone are unchanged when the problem is
    restricted to a subset of heads (with their groups' B and C channels); with
    every head of each touched group ([2, 3, 6, 7]: groups 1 and 3) the groups'
    B and C channel gradients are whole and come back too."""
    wl = W.make_workload("sub_bwd", batch=2, seqlen=64, nheads=8, headdim=4, dstate=4,
                         ngroups=4, chunk=16, act="bf16", seed=22, lengths=[20, 1, 43],
                         with_dy=True)
    full = oracle.backward(wl)
    sub = oracle.backward(wl, heads=heads)
    P, N, H, G = wl.headdim, wl.dstate, wl.nheads, wl.ngroups
    ch = np.concatenate([np.arange(h * P, (h + 1) * P) for h in heads])
    if len(heads) == 4:
        for g in (1, 3):
            ch = np.concatenate([ch, H * P + g * N + np.arange(N)])
        for g in (1, 3):
            ch = np.concatenate([ch, H * P + G * N + g * N + np.arange(N)])
    np.testing.assert_array_equal(sub["channels"], ch)
    np.testing.assert_allclose(sub["dxBC"], full["dxBC"][:, :, ch], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub["dconv_w"], full["dconv_w"][ch], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(sub["ddt_raw"], full["ddt_raw"][:, :, heads], rtol=1e-12,
                               atol=1e-14)
    for k in ("ddt_bias", "dA_log", "dD"):
        np.testing.assert_allclose(sub[k], full[k][heads], rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------- gradients


def _torch_quadratic_loss(xBC, w, dt_raw, dt_bias, A_log, D, dy, H, P, N, G, seq):
    """Full path in torch float64 via the quadratic form; differentiated by autograd."""
    b, L, C = xBC.shape
    Wd = w.shape[1]
    xt = torch.nn.functional.pad(xBC.transpose(1, 2), (Wd - 1, 0))
    if seq is None:
        u = torch.nn.functional.conv1d(xt, w.unsqueeze(1), groups=C)
    else:
        cols = []
        for t in range(L):
            acc = 0
            for k in range(Wd):
                s = t - (Wd - 1) + k
                if s < 0 or seq[0, s] != seq[0, t]:
                    continue
                acc = acc + w[:, k] * xBC[:, s, :]
            cols.append(acc if torch.is_tensor(acc) else torch.zeros(b, C, dtype=xBC.dtype))
        u = torch.stack(cols, dim=2)
    vv = torch.nn.functional.silu(u).transpose(1, 2)
    hpg = H // G
    loss = 0
    idx = torch.arange(L)
    causal = (idx[:, None] >= idx[None, :])
    if seq is not None:
        s = torch.from_numpy(np.asarray(seq[0]))
        causal = causal & (s[:, None] == s[None, :])
    for h in range(H):
        g = h // hpg
        x = vv[:, :, h * P:(h + 1) * P]
        Bm = vv[:, :, H * P + g * N:H * P + (g + 1) * N]
        Cm = vv[:, :, H * P + G * N + g * N:H * P + G * N + (g + 1) * N]
        dt = torch.clamp(torch.nn.functional.softplus(dt_raw[:, :, h] + dt_bias[h]),
                         float(np.float32(1e-3)), float(np.float32(0.1)))
        A = -torch.exp(A_log[h])
        cs = torch.cumsum(dt * A, dim=1)
        seg = cs[:, :, None] - cs[:, None, :]
        lam = torch.where(causal, torch.exp(torch.where(causal, seg, torch.zeros_like(seg))),
                          torch.zeros_like(seg))
        M = lam * (Cm @ Bm.transpose(1, 2))
        y = M @ (dt[:, :, None] * x) + D[h] * x
        loss = loss + (y * dy[:, :, h, :]).sum()
    return loss


@pytest.mark.parametrize("packed", [False, True])
def test_adjoint_matches_autograd_of_quadratic_form(packed):
    wl = W.make_workload("grad", batch=2, seqlen=40, nheads=4, headdim=3, dstate=4, ngroups=2,
                         chunk=8, act="f32", seed=31, with_dy=True,
                         lengths=[9, 1, 30] if packed else None)
    g = oracle.backward(wl)
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    xBC, w, dtr, dtb, al, D = (t(wl.xBC), t(wl.conv_w), t(wl.dt_raw), t(wl.dt_bias),
                               t(wl.A_log), t(wl.D))
    loss = _torch_quadratic_loss(xBC, w, dtr, dtb, al, D, torch.from_numpy(wl.dy.astype(np.float64)),
                                 4, 3, 4, 2, wl.seq_idx)
    loss.backward()
    for name, ref in [("dxBC", xBC), ("dconv_w", w), ("ddt_raw", dtr), ("ddt_bias", dtb),
                      ("dA_log", al), ("dD", D)]:
        np.testing.assert_allclose(g[name], ref.grad.numpy(), rtol=1e-9, atol=1e-10,
                                   err_msg=name)


def _near_clamp(wl, field, fi, margin):
    z = wl.dt_raw.astype(np.float64) + wl.dt_bias.astype(np.float64)[None, None, :]
    sp = np.logaddexp(0.0, z)
    dist = np.minimum(np.abs(sp - float(np.float32(wl.dt_min))),
                      np.abs(sp - float(np.float32(wl.dt_max))))
    if field == "dt_raw":
        return dist.reshape(-1)[fi] < margin
    return (dist[..., fi] < margin).any()


def test_adjoint_matches_finite_differences():
    """Central differences of L = <dy, y> in float64 on a config-0-like problem."""
    wl = W.make_workload("fd", batch=1, seqlen=64, nheads=2, headdim=4, dstate=4, ngroups=1,
                         chunk=16, act="f32", seed=41, with_dy=True, lengths=[25, 39])
    g = oracle.backward(wl)

    def loss(**over):
        import copy
        w2 = copy.copy(wl)
        for k, val in over.items():
            setattr(w2, k, val)
        return float((oracle.forward(w2) * wl.dy).sum())

    rng = np.random.default_rng(42)
    eps = 1e-4
    for name, field in [("dxBC", "xBC"), ("dconv_w", "conv_w"), ("ddt_raw", "dt_raw"),
                        ("ddt_bias", "dt_bias"), ("dA_log", "A_log"), ("dD", "D")]:
        base = getattr(wl, field).astype(np.float64)
        flat_idx = rng.choice(base.size, size=min(6, base.size), replace=False)
        for fi in flat_idx:
            # The oracle reads float32 inputs: perturb by a float32-representable step.
            plus = base.copy().reshape(-1)
            minus = base.copy().reshape(-1)
            plus[fi] += eps
            minus[fi] -= eps
            hp = np.float32(plus[fi]) - np.float32(base.reshape(-1)[fi])
            hm = np.float32(base.reshape(-1)[fi]) - np.float32(minus[fi])
            lp = loss(**{field: plus.reshape(base.shape).astype(np.float32)})
            lm = loss(**{field: minus.reshape(base.shape).astype(np.float32)})
            fd = (lp - lm) / (float(hp) + float(hm))
            an = g[name].reshape(-1)[fi]
            if field in ("dt_raw", "dt_bias") and _near_clamp(wl, field, fi, 2 * eps):
                continue  # the clamp has a kink there; a central difference straddles it
            assert abs(fd - an) <= 2e-3 * max(1.0, abs(an)), (name, fi, fd, an)


def test_adjoint_dot_product_identity():
    """The dot-product test of an adjoint: along one random direction v over every input
    at once, <dy, y(x + d+)> - <dy, y(x - d-)> = <J^T dy, d+ + d-> up to third order in
    the step, with J^T dy the oracle's gradients and d+-, the float32-representable steps
    of size 1e-4 v.  Entries of dt_raw near a clamp bound (a kink of the dt path) get no
    step, and neither does dt_bias (it moves every token of its head)."""
    import copy
    wl = W.make_workload("dot", batch=1, seqlen=64, nheads=2, headdim=4, dstate=4, ngroups=1,
                         chunk=16, act="f32", seed=43, with_dy=True, lengths=[30, 34])
    g = oracle.backward(wl)
    rng = np.random.default_rng(44)
    eps = 1e-4
    fields = [("dxBC", "xBC"), ("dconv_w", "conv_w"), ("ddt_raw", "dt_raw"),
              ("dA_log", "A_log"), ("dD", "D")]
    plus, minus = copy.copy(wl), copy.copy(wl)
    predicted = 0.0
    for gname, field in fields:
        base = getattr(wl, field).astype(np.float64)
        v = rng.standard_normal(base.shape)
        if field == "dt_raw":
            keep = np.array([not _near_clamp(wl, "dt_raw", i, 4 * eps) for i in range(base.size)])
            v = v * keep.reshape(base.shape)
        p32 = (base + eps * v).astype(np.float32)
        m32 = (base - eps * v).astype(np.float32)
        setattr(plus, field, p32)
        setattr(minus, field, m32)
        step = p32.astype(np.float64) - m32.astype(np.float64)
        predicted += float((g[gname].astype(np.float64) * step).sum())
    measured = float((oracle.forward(plus) * wl.dy).sum() - (oracle.forward(minus) * wl.dy).sum())
    assert abs(predicted) > 1e-6
    assert abs(measured - predicted) <= 1e-5 * abs(predicted), (measured, predicted)


# ---------------------------------------------------------------- initial state in the adjoint
#
# The boundary scan hands every segment an initial state S_in and the reverse scan
# hands back dL/dS_in (Megatron-LM #6808, first commit: S_out = a_block S_in + S_ext,
# and the backward mirrors it with a reverse scan).  The oracle's adjoint with a
# non-zero initial state (its t = 0 terms and the gradient of the initial state
# itself) is pinned here at the level of the post-conv recurrence.


def _init_problem(seed, lengths=None):
    """A small post-conv problem with a random initial state and upstream gradient."""
    rng = np.random.default_rng(seed)
    b, L, H, P, N, G = 2, 40, 4, 3, 4, 2
    C = H * P + 2 * G * N
    v = rng.standard_normal((b, L, C))
    dt_raw = rng.standard_normal((b, L, H)).astype(np.float32)
    dt_bias = (rng.standard_normal(H) * 0.5 - 2.5).astype(np.float32)
    A_log = rng.uniform(0.0, math.log(4.0), H).astype(np.float32)
    D = rng.standard_normal(H).astype(np.float32)
    init = rng.standard_normal((b, H, P, N))
    dy = rng.standard_normal((b, L, H, P)).astype(np.float32)
    seq = None
    if lengths is not None:
        seq = np.ascontiguousarray(np.broadcast_to(
            np.repeat(np.arange(len(lengths)), lengths).astype(np.int32), (b, L)))
    kw = dict(nheads=H, headdim=P, dstate=N, ngroups=G, dt_min=1e-3, dt_max=0.1, seq_idx=seq)
    return dict(v=v, dt_raw=dt_raw, dt_bias=dt_bias, A_log=A_log, D=D, init=init, dy=dy), kw


def _torch_loss_with_init(v, dt_raw, dt_bias, A_log, D, init, dy, H, P, N, G, seq):
    """<dy, y> with y from the quadratic (SSD-matrix) form plus the initial-state term
    exp(cs_i) C_i . init[p, :] for tokens i of the row's first sequence, where cs is the
    inclusive cumulative sum of dt A from the row start (the state before the first
    token decays by that token's factor).  Written independently of the oracle."""
    b, L, _ = v.shape
    hpg = H // G
    idx = torch.arange(L)
    causal = idx[:, None] >= idx[None, :]
    first = torch.ones(b, L, dtype=torch.bool)
    if seq is not None:
        s = torch.from_numpy(np.asarray(seq))
        causal = causal[None] & (s[:, :, None] == s[:, None, :])
        first = s == s[:, :1]
    else:
        causal = causal[None].expand(b, L, L)
    lo, hi = float(np.float32(1e-3)), float(np.float32(0.1))
    loss = 0
    for h in range(H):
        g = h // hpg
        x = v[:, :, h * P:(h + 1) * P]
        Bm = v[:, :, H * P + g * N:H * P + (g + 1) * N]
        Cm = v[:, :, H * P + G * N + g * N:H * P + G * N + (g + 1) * N]
        dt = torch.clamp(torch.nn.functional.softplus(dt_raw[:, :, h] + dt_bias[h]), lo, hi)
        cs = torch.cumsum(dt * (-torch.exp(A_log[h])), dim=1)
        seg = cs[:, :, None] - cs[:, None, :]
        lam = torch.where(causal, torch.exp(torch.where(causal, seg, torch.zeros_like(seg))),
                          torch.zeros_like(seg))
        y = (lam * (Cm @ Bm.transpose(1, 2))) @ (dt[:, :, None] * x) + D[h] * x
        dec = torch.where(first, torch.exp(cs), torch.zeros_like(cs))
        y = y + dec[:, :, None] * (Cm @ init[:, h].transpose(1, 2))
        loss = loss + (y * dy[:, :, h, :]).sum()
    return loss


@pytest.mark.parametrize("lengths", [None, [13, 27]])
def test_adjoint_with_initial_state_matches_autograd(lengths):
    """Every gradient of the oracle's adjoint under a non-zero initial state, dinit
    included, against torch autograd of the quadratic form with the initial-state term."""
    a, kw = _init_problem(51, lengths)
    g = oracle.ssd_bwd(a["v"], a["dt_raw"], a["dt_bias"], a["A_log"], a["D"], a["dy"],
                       init=a["init"], want_dinit=True, **kw)
    t = lambda z: torch.tensor(np.asarray(z, np.float64), requires_grad=True)
    v, dtr, dtb, al, D, ini = (t(a["v"]), t(a["dt_raw"]), t(a["dt_bias"]), t(a["A_log"]),
                               t(a["D"]), t(a["init"]))
    loss = _torch_loss_with_init(v, dtr, dtb, al, D, ini, torch.from_numpy(a["dy"].astype(np.float64)),
                                 kw["nheads"], kw["headdim"], kw["dstate"], kw["ngroups"],
                                 kw["seq_idx"])
    loss.backward()
    # the forward itself under the initial state
    y = oracle.ssd_fwd(a["v"], a["dt_raw"], a["dt_bias"], a["A_log"], a["D"], init=a["init"], **kw)
    np.testing.assert_allclose(float((y * a["dy"]).sum()), loss.item(), rtol=1e-11)
    for name, ref in [("dv", v), ("ddt_raw", dtr), ("ddt_bias", dtb), ("dA_log", al),
                      ("dD", D), ("dinit", ini)]:
        np.testing.assert_allclose(g[name], ref.grad.numpy(), rtol=1e-9, atol=1e-10, err_msg=name)
    if lengths is not None:
        # tokens after the first reset cannot see the initial state
        assert np.any(g["dinit"] != 0.0)


def test_initial_state_gradient_matches_finite_differences():
    """dL/dinit and, under a non-zero initial state, dL/d(dt_raw) and dL/dA_log by
    central differences of the oracle forward (the loss is linear in init, so those
    differences are exact up to rounding)."""
    a, kw = _init_problem(52, [22, 18])
    g = oracle.ssd_bwd(a["v"], a["dt_raw"], a["dt_bias"], a["A_log"], a["D"], a["dy"],
                       init=a["init"], want_dinit=True, **kw)

    def loss(**over):
        z = dict(a, **over)
        y = oracle.ssd_fwd(z["v"], z["dt_raw"], z["dt_bias"], z["A_log"], z["D"],
                           init=z["init"], **kw)
        return float((y * a["dy"]).sum())

    eps = 1e-5
    base = a["init"]
    for fi in range(base.size):
        p, m = base.copy().reshape(-1), base.copy().reshape(-1)
        p[fi] += eps
        m[fi] -= eps
        fd = (loss(init=p.reshape(base.shape)) - loss(init=m.reshape(base.shape))) / (2 * eps)
        an = g["dinit"].reshape(-1)[fi]
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), ("dinit", fi, fd, an)
    # t = 0 of every row: the only token whose dt term sees the initial state directly
    rng = np.random.default_rng(53)
    checks = [("ddt_raw", "dt_raw", (r, 0, h)) for r in range(2) for h in range(4)]
    checks += [("ddt_raw", "dt_raw", tuple(rng.integers(0, s) for s in a["dt_raw"].shape))
               for _ in range(6)]
    checks += [("dA_log", "A_log", (h,)) for h in range(4)]
    sp = np.logaddexp(0.0, a["dt_raw"].astype(np.float64) + a["dt_bias"][None, None, :])
    for gname, field, ix in checks:
        if field == "dt_raw" and min(abs(sp[ix] - float(np.float32(1e-3))),
                                     abs(sp[ix] - float(np.float32(0.1)))) < 1e-3:
            continue  # at a clamp kink a central difference straddles it
        base32 = a[field]
        h = 1e-3
        p, m = base32.copy(), base32.copy()
        p[ix] = np.float32(p[ix] + h)
        m[ix] = np.float32(m[ix] - h)
        step = float(p[ix]) - float(m[ix])
        fd = (loss(**{field: p}) - loss(**{field: m})) / step
        an = g[gname][ix]
        assert abs(fd - an) <= 2e-4 * max(1.0, abs(an)), (gname, ix, fd, an)


def test_adjoint_dot_product_identity_with_initial_state():
    """The dot-product test of the adjoint along one random direction over every input
    of the recurrence and the initial state at once."""
    a, kw = _init_problem(54, [19, 21])
    g = oracle.ssd_bwd(a["v"], a["dt_raw"], a["dt_bias"], a["A_log"], a["D"], a["dy"],
                       init=a["init"], want_dinit=True, **kw)
    rng = np.random.default_rng(55)
    eps = 1e-4
    sp = np.logaddexp(0.0, a["dt_raw"].astype(np.float64) + a["dt_bias"][None, None, :])
    far = (np.minimum(np.abs(sp - float(np.float32(1e-3))), np.abs(sp - float(np.float32(0.1))))
           > 4 * eps)
    plus, minus = dict(a), dict(a)
    predicted = 0.0
    for gname, field in [("dv", "v"), ("ddt_raw", "dt_raw"), ("dA_log", "A_log"), ("dD", "D"),
                         ("dinit", "init")]:
        base = a[field].astype(np.float64)
        d = rng.standard_normal(base.shape)
        if field == "dt_raw":
            d = d * far
        dt = a[field].dtype
        pz = (base + eps * d).astype(dt)
        mz = (base - eps * d).astype(dt)
        plus[field], minus[field] = pz, mz
        predicted += float((g[gname] * (pz.astype(np.float64) - mz.astype(np.float64))).sum())

    def lval(z):
        y = oracle.ssd_fwd(z["v"], z["dt_raw"], z["dt_bias"], z["A_log"], z["D"],
                           init=z["init"], **kw)
        return float((y * a["dy"]).sum())

    measured = lval(plus) - lval(minus)
    assert abs(predicted) > 1e-6
    assert abs(measured - predicted) <= 1e-6 * abs(predicted), (measured, predicted)
