"""Seeded synthetic workloads for the Mamba2 conv1d + SSD state-passing path.

This module only draws random numbers and lays out workload structure
(shapes, segment tables, packed-sequence lengths, memory permutations).
It holds none of the method's arithmetic, so both the CPU oracle and the
HIP path can take their inputs from it without sharing any computation.

Value distributions (all seeded through ``numpy.random.default_rng``):
  xBC    ~ N(0, 1)                       pre-conv activations, [b, L, H*P + 2*G*N]
  conv_w ~ 0.5 * N(0, 1)                 depthwise conv taps, [C, W]
  dt_raw ~ N(0, 1)                       [b, L, H]
  dt_bias: per head, softplus^-1(exp(U(ln 1e-3, ln 1e-1)))   (Mamba2-style init)
  A_log  ~ U(0, ln 16)                   so A = -exp(A_log) lies in [-16, -1]
  D      ~ N(0, 1)                       [H]
  dy     ~ N(0, 1)                       [b, L, H, P] (backward workloads)
Slow-decay variants replace dt_bias by softplus^-1(1e-3) on every head and
draw A_log ~ U(ln 0.1, 0), so a segment's block decay stays far from zero.

bf16 workloads are drawn in float32 and rounded to bf16 (round to nearest
even); the stored float32 arrays hold exactly the bf16 values, so the oracle
and the device see identical inputs.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

DT_MIN = 1e-3
DT_MAX = 0.1


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), kept as float32."""
    # Finite float32 bit patterns stay below 2**32 after adding at most 0x8000.
    u = np.array(a, dtype=np.float32, copy=True).view(np.uint32)
    bias = (u >> np.uint32(16)) & np.uint32(1)
    bias += np.uint32(0x7FFF)
    u += bias
    u &= np.uint32(0xFFFF0000)
    return u.view(np.float32)


def _inv_softplus(y: np.ndarray) -> np.ndarray:
    # y = log(1 + e^x)  <=>  x = y + log(1 - e^-y)
    y = np.asarray(y, dtype=np.float64)
    return (y + np.log(-np.expm1(-y))).astype(np.float32)


@dataclass
class Workload:
    """One problem instance: shapes, segment table, packed layout and tensors.

    Token arrays are stored in *memory order*.  ``perm[m]`` is the causal
    (original) position of the token held at memory position ``m``; for
    contiguous layouts it is the identity.  ``segments`` lists ``(start, len)``
    in causal order, ``start`` being a memory offset.
    """
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    conv_width: int
    act: str                      # "f32" or "bf16"
    segments: List[Tuple[int, int]]
    perm: np.ndarray              # [L] int64, memory position -> causal position
    seq_idx: Optional[np.ndarray]  # [b, L] int32 in memory order, or None
    cu_seqlens: Optional[np.ndarray]
    xBC: np.ndarray               # [b, L, C] float32 (bf16-exact when act == "bf16")
    conv_w: np.ndarray            # [C, W] float32
    dt_raw: np.ndarray            # [b, L, H] float32 (bf16-exact when act == "bf16")
    dt_bias: np.ndarray           # [H] float32
    A_log: np.ndarray             # [H] float32
    D: np.ndarray                 # [H] float32
    dy: Optional[np.ndarray] = None  # [b, L, H, P] (bf16-exact when act == "bf16")
    dt_min: float = DT_MIN
    dt_max: float = DT_MAX
    layout: str = "contiguous"
    notes: dict = field(default_factory=dict)

    @property
    def conv_dim(self) -> int:
        return self.nheads * self.headdim + 2 * self.ngroups * self.dstate

    @property
    def tokens(self) -> int:
        return self.batch * self.seqlen

    def to_causal(self, a: np.ndarray, axis: int = 1) -> np.ndarray:
        """Reorder a memory-order token axis into causal order."""
        if self.layout == "contiguous":
            return a
        inv = np.empty_like(self.perm)
        inv[self.perm] = np.arange(self.perm.size)
        return np.take(a, inv, axis=axis)

    def causal_seq_idx(self) -> Optional[np.ndarray]:
        return None if self.seq_idx is None else self.to_causal(self.seq_idx, axis=1)


def contiguous_segments(L: int, nseg: int) -> List[Tuple[int, int]]:
    assert L % nseg == 0
    s = L // nseg
    return [(k * s, s) for k in range(nseg)]


def virtual_layout(L: int, cp: int) -> Tuple[List[Tuple[int, int]], np.ndarray]:
    """Front/back balanced layout with 2*cp half-shards (DualChunkSwap order).

    Causal half-shard ``h_k`` (k = 0..2cp-1) covers causal tokens
    [k*s, (k+1)*s).  Rank r holds (h_r, h_{2cp-1-r}), so memory holds
    h_0, h_{2cp-1}, h_1, h_{2cp-2}, ..., h_{cp-1}, h_cp.  Returns the segment
    table (causal order, memory offsets) and the memory->causal permutation.
    """
    n = 2 * cp
    assert L % n == 0
    s = L // n
    slot_of = {}
    for r in range(cp):
        slot_of[r] = 2 * r
        slot_of[n - 1 - r] = 2 * r + 1
    segs = [(slot_of[k] * s, s) for k in range(n)]
    perm = np.empty(L, dtype=np.int64)
    for k in range(n):
        m0 = slot_of[k] * s
        perm[m0:m0 + s] = np.arange(k * s, (k + 1) * s)
    return segs, perm


def packed_lengths(rng: np.random.Generator, total: int, lo: int, hi: int) -> np.ndarray:
    """Draw sequence lengths in [lo, hi] until they reach ``total``; the last is cut."""
    lens = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return np.asarray(lens, dtype=np.int64)


def seq_idx_from_lengths(lens: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    seq_idx = np.repeat(np.arange(len(lens), dtype=np.int32), lens)
    return cu, seq_idx


def make_workload(name: str, *, batch: int, seqlen: int, nheads: int, headdim: int,
                  dstate: int, ngroups: int, chunk: int, conv_width: int = 4,
                  act: str = "bf16", nseg: int = 1, layout: str = "contiguous",
                  seed: int = 0, packed: Optional[Tuple[int, int]] = None,
                  lengths: Optional[List[int]] = None, slow_decay: bool = False,
                  with_dy: bool = False, seg_lens: Optional[List[int]] = None) -> Workload:
    """Build a seeded workload.

    ``packed=(lo, hi)`` draws packed sequence lengths U[lo, hi] over each row
    (the same lengths for every row); ``lengths`` gives them explicitly.
    ``nseg`` is the number of causal segments.  With ``layout="virtual"`` it
    must be even and memory holds the balanced front/back order with
    cp = nseg // 2 (see ``virtual_layout``).  ``seg_lens`` gives contiguous
    segments of unequal lengths instead.
    """
    rng = np.random.default_rng(seed)
    H, P, N, G, W = nheads, headdim, dstate, ngroups, conv_width
    C = H * P + 2 * G * N
    L = seqlen

    if seg_lens is not None:
        assert layout == "contiguous" and sum(seg_lens) == L
        starts = np.concatenate([[0], np.cumsum(seg_lens)[:-1]])
        segs = [(int(a), int(n)) for a, n in zip(starts, seg_lens)]
        perm = np.arange(L, dtype=np.int64)
    elif layout == "contiguous":
        segs = contiguous_segments(L, nseg)
        perm = np.arange(L, dtype=np.int64)
    elif layout == "virtual":
        assert nseg % 2 == 0
        segs, perm = virtual_layout(L, nseg // 2)
    else:
        raise ValueError(layout)

    seq_idx_c = None
    cu = None
    if lengths is not None:
        lens = np.asarray(lengths, dtype=np.int64)
        assert int(lens.sum()) == L
        cu, seq_idx_c = seq_idx_from_lengths(lens)
    elif packed is not None:
        lens = packed_lengths(rng, L, packed[0], packed[1])
        cu, seq_idx_c = seq_idx_from_lengths(lens)

    xBC = rng.standard_normal((batch, L, C), dtype=np.float32)
    conv_w = (0.5 * rng.standard_normal((C, W), dtype=np.float32)).astype(np.float32)
    dt_raw = rng.standard_normal((batch, L, H), dtype=np.float32)
    if slow_decay:
        dt_bias = np.full(H, _inv_softplus(np.float64(1e-3)), dtype=np.float32)
        A_log = rng.uniform(math.log(0.1), 0.0, size=H).astype(np.float32)
    else:
        dt0 = np.exp(rng.uniform(math.log(1e-3), math.log(1e-1), size=H))
        dt_bias = _inv_softplus(dt0)
        A_log = rng.uniform(0.0, math.log(16.0), size=H).astype(np.float32)
    D = rng.standard_normal(H, dtype=np.float32)
    dy = rng.standard_normal((batch, L, H, P), dtype=np.float32) if with_dy else None

    if act == "bf16":
        xBC = round_to_bf16(xBC)
        dt_raw = round_to_bf16(dt_raw)
        if dy is not None:
            dy = round_to_bf16(dy)
    elif act != "f32":
        raise ValueError(act)

    # Causal-order draws are placed into memory order.
    if layout != "contiguous":
        xBC = xBC[:, perm]
        dt_raw = dt_raw[:, perm]
        if dy is not None:
            dy = dy[:, perm]
    seq_idx = None
    if seq_idx_c is not None:
        seq_idx = np.ascontiguousarray(np.broadcast_to(seq_idx_c[perm], (batch, L))).astype(np.int32)

    return Workload(name=name, batch=batch, seqlen=L, nheads=H, headdim=P, dstate=N,
                    ngroups=G, chunk=chunk, conv_width=W, act=act, segments=segs,
                    perm=perm, seq_idx=seq_idx, cu_seqlens=cu,
                    xBC=np.ascontiguousarray(xBC), conv_w=conv_w,
                    dt_raw=np.ascontiguousarray(dt_raw), dt_bias=dt_bias,
                    A_log=A_log, D=D,
                    dy=None if dy is None else np.ascontiguousarray(dy),
                    layout=layout)


# Named workloads (seeds fixed per workload).
WORKLOADS = {
    # 1 x 256 tokens, 2 heads, P = N = 16, chunk 64, float32, 2 segments
    "tiny_f32": dict(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, ngroups=1, chunk=64,
                     act="f32", nseg=2, seed=1000),
    # Mamba2 mixer shard: 2 x 8192 tokens, 32 heads, P 64, N 128, 8 segments of 1024
    "mixer_shard_bf16": dict(batch=2, seqlen=8192, nheads=32, headdim=64, dstate=128, ngroups=1,
                             chunk=256, act="bf16", nseg=8, seed=1001),
    # long context: 131072 tokens, 64 heads in 8 groups, 8 contiguous segments
    "long_context_bf16": dict(batch=1, seqlen=131072, nheads=64, headdim=64, dstate=128,
                              ngroups=8, chunk=256, act="bf16", nseg=8, seed=1002),
    # the same, as 16 half-shards in the virtual front/back layout
    "long_context_virtual_bf16": dict(batch=1, seqlen=131072, nheads=64, headdim=64, dstate=128,
                                      ngroups=8, chunk=256, act="bf16", nseg=16,
                                      layout="virtual", seed=1002),
    # packed variable-length batch: 32768 tokens, lengths U[512, 8192], 4 segments
    "packed_thd_bf16": dict(batch=1, seqlen=32768, nheads=32, headdim=64, dstate=128, ngroups=1,
                            chunk=256, act="bf16", nseg=4, packed=(512, 8192), seed=1003),
    # the mixer shard with an upstream gradient dy (forward + backward)
    "mixer_shard_bwd_bf16": dict(batch=2, seqlen=8192, nheads=32, headdim=64, dstate=128,
                                 ngroups=1, chunk=256, act="bf16", nseg=8, seed=1001,
                                 with_dy=True),
    # slow-decay variants: block decays far from 0 so the scan composes segments
    "slow_tiny_f32": dict(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, ngroups=1,
                          chunk=64, act="f32", nseg=2, seed=2000, slow_decay=True),
    "slow_mixer_shard_bf16": dict(batch=2, seqlen=8192, nheads=32, headdim=64, dstate=128,
                                  ngroups=1, chunk=256, act="bf16", nseg=8, seed=2001,
                                  slow_decay=True),
}


def config(name: str) -> Workload:
    """Build one of the named workloads."""
    return make_workload(name, **WORKLOADS[name])
