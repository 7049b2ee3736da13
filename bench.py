"""Benchmark of the conv1d + SSD state-passing path on one MI355X.

One step = one pass of the whole hot path (forward and backward) over one
batch of synthetic input, every call going through the C ABI on torch's
current stream:
  forward : ssd_conv1d_fwd -> ssd_segment_states -> ssd_boundary_scan
            -> ssd_segment_output_fused (output pass with the correction folded in)
  backward: ssd_segment_bwd_summary -> ssd_boundary_scan (reverse)
            -> ssd_segment_bwd_pass -> ssd_segment_bwd_chunks -> ssd_conv1d_bwd
Workload: 2 rows x 8192 tokens, 32 heads, headdim 64, d_state 128, 1 group,
chunk 256, conv width 4, bf16 activations with FP32 state, cut into 8
contiguous causal segments of 1024 tokens (one device's context-parallel
shard each).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line (rank 0).  Per-call durations ("calls") come from a
breakdown pass of K steps with HIP events around every call.  The timed region
(K further steps, the headline value) records events around one call only:
the call whose single kernel takes the most time, whose duration there gives
the roofline entry.  After the timed region, two probe kernels (a 1 GiB copy and
a bf16 MFMA loop, libssd_probe.so) measure the achievable HBM and MFMA rates;
the roofline and MFMA entries give fractions of those beside the fractions of
the published peaks.
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, published
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, published
F32_PEAK_TFLOPS = 157.3      # MI355X dense fp32 MFMA, published

METRIC = "SSD fwd(+bwd) tokens/s on 1 MI355X; % of MFMA peak and HBM GB/s"
DEFAULT_WORKLOAD = "mixer_shard_bwd_bf16"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="a name from ssd_workloads.WORKLOADS (default: the mixer shard with dy, "
                         "forward+backward)")
    ap.add_argument("--pass", dest="which", default=None, choices=["fwd", "fwd+bwd"],
                    help="default: fwd+bwd when the workload has dy, else fwd")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra-configs", action="store_true",
                    help="time only the chosen workload (by default the headline run also times "
                         "the forward of every other configuration)")
    ap.add_argument("--conv-fused", action="store_true",
                    help="run the headline's forward conv-fused (ssd_conv_segment_states and "
                         "ssd_conv_segment_output instead of ssd_conv1d_fwd and the two phases)")
    ap.add_argument("--cpu-runs", type=int, default=8)
    ap.add_argument("--copy-probe-mb", type=int, default=0,
                    help="run one device-to-device copy of this many MB before timing, so that "
                         "hardware byte counters can be calibrated against a known size")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the achievable-peak probes (copy kernel, MFMA loop) run after timing")
    ap.add_argument("--summarize-mfma", metavar="PMC_DB",
                    help="no GPU work: read a rocprofv3 --pmc database with SQ_VALU_MFMA_BUSY_CYCLES, "
                         "GRBM_GUI_ACTIVE and SQ_INSTS_VALU_MFMA_MOPS_BF16 of a run with the peak "
                         "probes, and print every kernel's MFMA-busy fraction as JSON")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DB", "WRITE_DB"),
                    help="no GPU work: read two rocprofv3 --pmc databases (FETCH_SIZE, then "
                         "WRITE_SIZE) of a run made with --copy-probe-mb, and print the per-launch "
                         "HBM traffic of every kernel as JSON, calibrated against the copy")
    return ap.parse_args()


# The kernel each single-kernel call launches: a regex over kernel_short() names.
CALL_KERNEL = {
    "ssd_conv1d_fwd": r"k_conv1d_silu<",
    "ssd_segment_output_fused": r"k_chunk_y<",
    "ssd_conv_segment_output": r"k_chunk_y<",
    "ssd_boundary_scan": r"k_boundary_scan<",
    "ssd_boundary_scan(reverse)": r"k_boundary_scan<",
    "ssd_segment_bwd_chunks": r"k_chunk_bwd(_hb)?<",
}
CSRC = os.path.join(ROOT, "mamba2_ssd_chunked_amd", "csrc")


def source_digest():
    """sha256 over the HIP/C++ sources: counter figures are only valid for these exact kernels."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        # the peak probes are measurement kernels, not kernels of the path
        if name.endswith((".hip", ".h", ".cpp")) and not name.startswith("peak_probes"):
            h.update(name.encode())
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(f.read())
    return h.hexdigest()


def kernel_short(sym):
    """Kernel name with its mangled template arguments, e.g. k_state_walk_pair<DF16bLi64ELi128ELb0ELi2E>."""
    import re
    m = re.match(r"_ZN3ssd\d+(k_\w+?)I(.*?)EEv", sym)
    if m:
        return f"{m.group(1)}<{m.group(2)}>"
    m = re.match(r"_ZN3ssd\d+(k_\w+?)E", sym)
    if m:
        return m.group(1) + "<>"
    m = re.match(r"ssd::(k_\w+)", sym)
    return m.group(1) + "<>" if m else sym


def summarize_traffic(fetch_db, write_db, probe_mb):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB, summed over the counter's instances),
    averaged per kernel, each scaled by known bytes / counted bytes of the largest
    __amd_rocclr_copyBuffer dispatch (the copy probe: reads and writes probe_mb MiB)."""
    import collections
    import sqlite3

    def per_dispatch(db, counter):
        vals = collections.defaultdict(float)
        names = {}
        cur = sqlite3.connect(db).cursor()
        for disp, kname, cname, val in cur.execute(
                "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
            if cname == counter:
                vals[disp] += val
                names[disp] = kname
        return vals, names

    probe_kib = probe_mb * 1024.0
    out = {"probe_bytes": probe_mb * (1 << 20), "kernels": {}}
    for counter, db in (("FETCH_SIZE", fetch_db), ("WRITE_SIZE", write_db)):
        vals, names = per_dispatch(db, counter)
        copies = [vals[k] for k in vals if "copyBuffer" in names[k]]
        if not copies:
            raise SystemExit(f"no copy-probe dispatch in {db}")
        counted = max(copies)
        factor = probe_kib / counted
        if not 0.25 <= factor <= 4.0:
            raise SystemExit(f"{counter}: copy probe counted {counted} KiB for {probe_kib} KiB")
        out[counter] = {"probe_counted_KiB": counted, "factor": round(factor, 4)}
        per_k = collections.defaultdict(list)
        for k, v in vals.items():
            if "copyBuffer" not in names[k]:
                per_k[kernel_short(names[k])].append(v)
        for kn, vs in per_k.items():
            e = out["kernels"].setdefault(kn, {})
            e[counter + "_KiB"] = round(statistics.mean(vs), 1)
            e[counter + "_bytes"] = round(statistics.mean(vs) * 1024 * factor)
            e["dispatches"] = len(vs)
    for e in out["kernels"].values():
        e["hbm_bytes"] = e.get("FETCH_SIZE_bytes", 0) + e.get("WRITE_SIZE_bytes", 0)
    out["source_sha256"] = source_digest()
    return out


SIMDS = 256 * 4  # MI355X: 256 CUs of 4 SIMDs


def summarize_mfma(db):
    """Per kernel, the mean over its dispatches of
      busy = sum of SQ_VALU_MFMA_BUSY_CYCLES / (max GRBM_GUI_ACTIVE * SIMDS)
    (the counters' own MfmaUtil formula) and of the executed MFMA flops
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 counts 512 flops).  The absolute busy figure depends on
    how the counter's instances map to SIMDs, so every kernel's figure is also given as a
    fraction of that of the busier MFMA-loop probe (k_probe_mfma16 / k_probe_mfma32, waves
    of independent products only): the matrix-core time a plain kernel reaches."""
    import collections
    import re
    import sqlite3
    cur = sqlite3.connect(db).cursor()
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    names = {}
    for disp, kname, cname, val in cur.execute(
            "select dispatch_id, kernel_name, counter_name, value from counters_collection"):
        acc[disp][cname].append(val)
        names[disp] = kname
    per_k = collections.defaultdict(lambda: {"busy": [], "gflop": []})
    for disp, cs in acc.items():
        gui = max(cs.get("GRBM_GUI_ACTIVE", [0]))
        if gui <= 0 or "SQ_VALU_MFMA_BUSY_CYCLES" not in cs:
            continue
        m = re.search(r"k_probe_\w+", names[disp])
        e = per_k[m.group(0) if m else kernel_short(names[disp])]
        e["busy"].append(sum(cs["SQ_VALU_MFMA_BUSY_CYCLES"]) / (gui * SIMDS))
        e["gflop"].append(sum(cs.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", [0])) * 512 / 1e9)
    out = {"simds": SIMDS, "kernels": {}}
    for kn, e in per_k.items():
        out["kernels"][kn] = {"mfma_busy": round(statistics.mean(e["busy"]), 4),
                              "executed_bf16_GFLOP": round(statistics.mean(e["gflop"]), 3),
                              "dispatches": len(e["busy"])}
    probes = [k for k in out["kernels"] if k.startswith("k_probe_mfma")]
    if probes:
        ref = max(probes, key=lambda k: out["kernels"][k]["mfma_busy"])
        out["probe"] = ref
        for e in out["kernels"].values():
            e["busy_vs_probe"] = round(e["mfma_busy"] / out["kernels"][ref]["mfma_busy"], 4)
    out["source_sha256"] = source_digest()
    return out


def measure_peaks(torch, dev, stream):
    """Achievable peaks of plain kernels on this GPU (libssd_probe.so): HBM GB/s of a
    1 GiB device copy (read + write bytes / time, median of 10), and bf16 MFMA TFLOP/s
    of the MFMA loop (2048 workgroups of 4 waves, median of 5), checked against its
    closed-form output."""
    from mamba2_ssd_chunked_amd import probes
    nb = 1 << 30
    src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    ts = []
    for rep in range(12):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        probes.probe_copy(src, dst)
        b.record(stream)
        if rep >= 2:
            ts.append((a, b))
    torch.cuda.synchronize()
    copy_ms = statistics.median(a.elapsed_time(b) for a, b in ts)
    if not bool(torch.equal(src, dst)):
        raise RuntimeError("copy probe produced wrong bytes")
    del src, dst
    blocks, iters = 2048, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    rate = {}
    for shape in (16, 32):
        ts = []
        for rep in range(7):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            flops = probes.probe_mfma(out, blocks, iters, shape)
            b.record(stream)
            if rep >= 2:
                ts.append((a, b))
        torch.cuda.synchronize()
        mfma_ms = statistics.median(a.elapsed_time(b) for a, b in ts)
        if not bool(torch.all(out == probes.mfma_expected(iters, shape))):
            raise RuntimeError(f"MFMA probe ({shape}) output differs from its closed form")
        rate[shape] = round(flops / (mfma_ms * 1e-3) / 1e12, 1)
    return {"hbm_GBps": round(2 * nb / (copy_ms * 1e-3) / 1e9, 1),
            "bf16_mfma_TFLOPs": max(rate.values()),
            "bf16_mfma_TFLOPs_by_shape": {f"{s}x{s}": v for s, v in rate.items()},
            "probes": "1 GiB device copy, 64-thread workgroups of 4 KiB (read + write bytes); "
                      "bf16 MFMA loops of 16x16x32 (8 independent chains per wave) and "
                      f"32x32x16 (4 chains), 2048 x 256 threads, {iters} rounds; the faster"}


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter summary of this
    workload, or None when it is missing or the sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_sha256") != source_digest():
        return None
    import re
    hits = [e for k, e in t["kernels"].items() if re.match(kernel, k)]
    return hits[0]["hbm_bytes"] if len(hits) == 1 else None


def head_block(wl):
    """Heads per workgroup of the head-blocked chunk backward (largest divisor of the
    heads per group up to 8); 1 when the per-head kernel runs (headdim above 64)."""
    if wl.headdim > 64:
        return 1
    hpg = wl.nheads // wl.ngroups
    return max(c for c in range(1, 9) if hpg % c == 0)


def algorithmic_bytes(wl):
    """Bytes each call must move at minimum: its own inputs and outputs, with every
    workspace intermediate counted once where one pass writes it and another reads
    it, and no per-head copies of per-group quantities."""
    e = 2 if wl.act == "bf16" else 4
    b, L, H, P, N, G, Q = (wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups,
                           wl.chunk)
    S = len(wl.segments)
    BL = b * L
    C = H * P + 2 * G * N
    seq = 4 * BL if wl.seq_idx is not None else 0
    nchunk = L // Q
    qt = Q // 16
    hst_chunks = b * (nchunk - S)  # entering states of every non-first chunk of a segment
    hst = hst_chunks * H * P * N * e
    st_all = b * nchunk * H * P * N  # one P x N matrix per chunk and head
    gram = b * nchunk * G * (qt * (qt + 1) // 2) * 256 * e
    summary = S * b * H * (P * N + 1) * 4
    states = S * b * H * P * N * 4
    dtcs = 2 * BL * H * 4
    dy = BL * H * P * e
    x, bc = BL * H * P * e, BL * 2 * G * N * e
    nhb = H // head_block(wl)
    dbc_part = BL * nhb * 2 * N * e  # dB, dC per head block
    tokp = 5 * BL * H * 4            # per-token ddt partial sums
    return {
        "ssd_conv1d_fwd": 2 * BL * C * e + C * wl.conv_width * 4 + seq,
        # dt prep (dt_raw in, dt and cumsum out), the walk (x, B in; entering states and
        # summary out) and the Gram tiles (B, C in; tiles out)
        "ssd_segment_states": BL * H * e + dtcs + x + bc // 2 + dtcs + hst + summary + bc + gram + seq,
        "ssd_boundary_scan": summary + states,
        # x, C, Gram tiles, entering states, S_in, decays in; y out
        "ssd_segment_output_fused": x + bc // 2 + gram + hst + states + dtcs + x + seq,
        # conv-fused forward: the B/C conv (raw B, C in, convolved out), then the states
        # phase reading the raw x (same bytes as the convolved x; the halo rows are
        # L1/L2 hits); the output pass reading the raw x; each with its conv taps
        "ssd_conv_segment_states": 2 * bc + 2 * G * N * wl.conv_width * 4
                                   + BL * H * e + dtcs + x + bc // 2 + dtcs + hst + summary
                                   + bc + gram + seq + H * P * wl.conv_width * 4,
        "ssd_conv_segment_output": x + bc // 2 + gram + hst + states + dtcs + x + seq
                                   + H * P * wl.conv_width * 4,
        "ssd_segment_output": x + bc // 2 + gram + hst + dtcs + BL * H * P * 4 + seq,
        "ssd_apply_init_state": BL * H * P * 4 + x + bc // 2 + BL * H * 4 + states + x + seq,
        # conv recompute (xBC in, conv output out), dt prep, the transposed Gram tiles
        # (B, C in), the reverse walk of every segment from zero (dy, C, cumsum in;
        # summary out)
        "ssd_segment_bwd_summary": BL * C * e + BL * C * e + BL * H * e + dtcs + bc + gram
                                   + dy + bc // 2 + dtcs // 2 + summary + seq,
        "ssd_boundary_scan(reverse)": summary + states,
        # the reverse walk from dS_out (dy, C, cumsum in; exit gradient of every chunk
        # out) and the forward walk from S_in (x, B, dt, cumsum in; entering state of
        # every chunk out)
        "ssd_segment_bwd_pass": dy + x + bc + dtcs + 2 * states + 2 * st_all * e + seq,
        # x, B, C, dy, decays, exit gradient and entering state per chunk, Gram tiles
        # in; d(conv output) of x, dB and dC per head block, ddt partial sums out
        "ssd_segment_bwd_chunks": BL * C * e + dy + dtcs + 2 * st_all * e + gram + x
                                  + dbc_part + tokp + seq,
        # ddt partials and dt_raw in, ddt_raw out; dB / dC partials summed per group;
        # xBC and d(conv output) in, dxBC out
        "ssd_conv1d_bwd": tokp + 2 * BL * H * e + dbc_part + bc + BL * C * e + x + bc
                          + BL * C * e + seq,
    }


def output_flops(wl):
    """MFMA flops of the output pass: the decay-weighted Gram tiles times X over causal
    pairs, and C H^T.  The Gram tiles C B^T themselves are formed once per group by the
    Gram pass of ssd_segment_states, not here."""
    b, L, H, P, N, Q = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.chunk
    per_chunk_head = Q * (Q + 1) // 2 * 2 * P + 2 * Q * P * N
    return b * (L // Q) * H * per_chunk_head


def chunk_bwd_flops(wl):
    """MFMA flops of ssd_segment_bwd_chunks over causal pairs only: per head dy x^T and
    its weighted product with dy (dx), the four state products (G B, H C, G^T x,
    H^T dy); per head block the products of the head-summed weights with C (dB) and
    B (dC)."""
    b, L, H, P, N, Q = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.chunk
    pairs = Q * (Q + 1) // 2
    per_head = 2 * pairs * 2 * P + 4 * 2 * Q * P * N
    per_block = 2 * pairs * 2 * N
    return b * (L // Q) * (H * per_head + H // head_block(wl) * per_block)


def path_floor_bytes(wl):
    """Method floors of the whole path (bytes), each pass counting its own inputs and
    outputs once:
      survey_fwd: conv, segment-local SSD with an FP32 y_zero and the summary, boundary
                  scan, correction pass (the passes of the unfused order);
      f1_fwd    : the states-first order (conv, states and summary, scan, one output pass
                  writing y): no y_zero;
      bwd       : the backward's summary phase and segment phase each reading xBC, dt_raw
                  and dy once, the summaries and scanned states of both scans, dxBC and
                  ddt written once (chunk states kept on chip)."""
    e = 2 if wl.act == "bf16" else 4
    b, L, H, P, N, G = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups
    S = len(wl.segments)
    BL, C = b * L, H * P + 2 * G * N
    summ = S * b * H * (P * N + 1) * 4
    st = S * b * H * P * N * 4
    conv = 2 * BL * C * e
    scan = summ + st
    survey = (conv + (BL * C * e + BL * H * e + BL * H * P * 4 + summ) + scan
              + (BL * H * P * 4 + BL * (H * P + G * N) * e + st + BL * H * P * e + BL * H * 4))
    f1 = (conv + (BL * (H * P + G * N) * e + BL * H * e + summ) + scan
          + (BL * (H * P + G * N) * e + st + BL * H * e + BL * H * P * e))
    bwd = (2 * BL * C * e + 2 * BL * H * e + 2 * BL * H * P * e + 2 * summ + 2 * st
           + BL * C * e + BL * H * e)
    return {"survey_fwd": survey, "f1_fwd": f1, "bwd": bwd}


def cpu_baseline(wl, runs, backward, heads=None):
    """The oracle timed on this host.  `heads` restricts it to a sample of heads (the
    value is then scaled to all heads: the oracle's work is per head)."""
    import oracle
    threads = oracle.num_threads()
    times = []
    for _ in range(runs):
        t = time.perf_counter()
        if backward:
            oracle.backward(wl, heads=heads)  # runs the forward too
        else:
            oracle.forward(wl, heads=heads)
        times.append(time.perf_counter() - t)
    med = statistics.median(times)
    what = "forward + backward (adjoint)" if backward else "forward"
    frac = 1.0 if heads is None else len(heads) / wl.nheads
    sample = (f"the whole workload ({wl.tokens} tokens, all heads)" if heads is None else
              f"heads {heads[0]}-{heads[-1]} of {wl.nheads} over all {wl.tokens} tokens, "
              f"scaled to all heads")
    return {"value": round(wl.tokens * frac / med, 1), "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{sample}, float64 token-by-token recurrence, {what}, median of {runs} "
                      f"runs ({med:.2f} s each)"}


def run_workload(wl, which, steps, warmup, dev, copy_probe_mb=0, conv_fused=False):
    """Times one workload: a breakdown pass with events around every call, then
    `steps` whole steps with events around the dominant single-kernel call only.
    conv_fused: the forward runs the conv inside the two forward phases.
    Returns the measurements (no JSON formatting)."""
    import numpy as np
    import torch

    import mamba2_ssd_chunked_amd as ssd

    do_bwd = which == "fwd+bwd"
    act = torch.bfloat16 if wl.act == "bf16" else torch.float32
    f32 = torch.float32
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    xBC, conv_w, dt_raw = t(wl.xBC, act), t(wl.conv_w, f32), t(wl.dt_raw, act)
    dt_bias, A_log, D = t(wl.dt_bias, f32), t(wl.A_log, f32), t(wl.D, f32)
    seq = None if wl.seq_idx is None else t(wl.seq_idx, torch.int32)
    dy = t(wl.dy, act) if do_bwd else None
    p = ssd.make_problem(batch=wl.batch, seqlen=wl.seqlen, nheads=wl.nheads, headdim=wl.headdim,
                         dstate=wl.dstate, ngroups=wl.ngroups, chunk=wl.chunk,
                         conv_width=wl.conv_width, act=wl.act, dt_min=wl.dt_min,
                         dt_max=wl.dt_max)
    segs = ssd.Segments(wl.segments)
    bufs = ssd.ForwardBuffers.allocate(p, segs, dev)
    bb = ssd.BackwardBuffers.allocate(p, segs, dev) if do_bwd else None
    stream = torch.cuda.current_stream()

    calls = [
        ("ssd_conv1d_fwd", lambda: ssd.ssd_conv1d_fwd(p, segs, xBC, conv_w, seq, bufs.xBC_conv)),
        ("ssd_segment_states", lambda: ssd.ssd_segment_states(
            p, segs, bufs.xBC_conv, dt_raw, dt_bias, A_log, seq, bufs.summary, bufs.ws)),
        ("ssd_boundary_scan", lambda: ssd.ssd_boundary_scan(
            p, segs.n, bufs.summary, None, False, bufs.S_in)),
        ("ssd_segment_output_fused", lambda: ssd.ssd_segment_output_fused(
            p, segs, bufs.xBC_conv, D, seq, bufs.S_in, bufs.ws, bufs.y)),
    ]
    if conv_fused:
        calls = [
            ("ssd_conv_segment_states", lambda: ssd.ssd_conv_segment_states(
                p, segs, xBC, conv_w, dt_raw, dt_bias, A_log, seq, bufs.summary, bufs.ws)),
            ("ssd_boundary_scan", lambda: ssd.ssd_boundary_scan(
                p, segs.n, bufs.summary, None, False, bufs.S_in)),
            ("ssd_conv_segment_output", lambda: ssd.ssd_conv_segment_output(
                p, segs, xBC, conv_w, D, seq, bufs.S_in, bufs.ws, bufs.y)),
        ]
    if do_bwd:
        calls += [
            ("ssd_segment_bwd_summary", lambda: ssd.ssd_segment_bwd_summary(
                p, segs, xBC, conv_w, dt_raw, dt_bias, A_log, seq, dy, bb.summary, bb.ws)),
            ("ssd_boundary_scan(reverse)", lambda: ssd.ssd_boundary_scan(
                p, segs.n, bb.summary, None, True, bb.dS_out)),
            ("ssd_segment_bwd_pass", lambda: ssd.ssd_segment_bwd_pass(
                p, segs, seq, dy, bufs.S_in, bb.dS_out, bb.ws)),
            ("ssd_segment_bwd_chunks", lambda: ssd.ssd_segment_bwd_chunks(
                p, segs, D, seq, dy, bb.ws)),
            ("ssd_conv1d_bwd", lambda: ssd.ssd_conv1d_bwd(
                p, segs, xBC, conv_w, dt_raw, dt_bias, A_log, seq, bb.ws, bb.dxBC, bb.ddt_raw,
                bb.dconv_w, bb.ddt_bias, bb.dA_log, bb.dD)),
        ]
    single_kernel = set(CALL_KERNEL)

    def step(events=None, only=None):
        """One pass of every call; with `events`, record [start, end] around each call
        (or, with `only`, around that call alone)."""
        for i, (_, fn) in enumerate(calls):
            rec = events is not None and (only is None or i == only)
            if rec:
                events[i if only is None else 0][0].record(stream)
            fn()
            if rec:
                events[i if only is None else 0][1].record(stream)

    def new_events(n):
        return [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n)]
                for _ in range(steps)]

    if copy_probe_mb:
        nb = copy_probe_mb * (1 << 20)
        src = torch.ones(nb // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    # A garbage-collection pass inside the timed region stalls the host long
    # enough to drain the launch queue and idle the GPU: collect now, then keep
    # the collector off until the timing is done.
    gc.collect()
    gc.disable()
    try:
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()

        # Breakdown pass (not the timed region): events around every call give the
        # per-call times.  Each event record adds a few microseconds between calls,
        # so the step is timed separately below with events around one call only.
        ev = new_events(len(calls))
        for k in range(steps):
            step(ev[k])
        torch.cuda.synchronize()
        abytes = algorithmic_bytes(wl)
        per_call = {}
        for i, (name, _) in enumerate(calls):
            each = [ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(steps)]
            ms = statistics.mean(each)
            per_call[name] = {"ms": round(ms, 5), "max_ms": round(max(each), 5),
                              "algorithmic_MB": round(abytes[name] / 1e6, 2),
                              "GB_per_s": round(abytes[name] / (ms * 1e-3) / 1e9, 1)}
        dom = max((n for n in single_kernel if n in per_call), key=lambda n: per_call[n]["ms"])
        dom_i = [name for name, _ in calls].index(dom)

        # Timed region: K whole steps, with HIP events on the launch stream around the
        # dominant kernel's call only (its duration for the roofline line).
        evd = new_events(1)
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        t0.record(stream)
        for k in range(steps):
            step(evd[k], only=dom_i)
        t1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
    finally:
        gc.enable()
    ms_step = t0.elapsed_time(t1) / steps
    dom_ms = statistics.mean(evd[k][0][0].elapsed_time(evd[k][0][1]) for k in range(steps))
    return {"ms_step": ms_step, "dom": dom, "dom_ms": dom_ms, "abytes": abytes,
            "per_call": per_call, "wall": wall}


def flops_entries(wl, m, do_bwd, peaks=None):
    mfma_peak = BF16_PEAK_TFLOPS if wl.act == "bf16" else F32_PEAK_TFLOPS
    mfma = {}
    out_call = ("ssd_conv_segment_output" if "ssd_conv_segment_output" in m["per_call"]
                else "ssd_segment_output_fused")
    for name, fl in [(out_call, output_flops(wl))] + \
            ([("ssd_segment_bwd_chunks", chunk_bwd_flops(wl))] if do_bwd else []):
        ms = m["dom_ms"] if name == m["dom"] else m["per_call"][name]["ms"]
        tf = fl / (ms * 1e-3) / 1e12
        mfma[name] = {"achieved": round(tf, 2), "peak": mfma_peak, "unit": "TFLOP/s",
                      "frac": round(tf / mfma_peak, 4), "algorithmic_GFLOP": round(fl / 1e9, 2)}
        if peaks and wl.act == "bf16":
            mfma[name]["achievable_peak"] = peaks["bf16_mfma_TFLOPs"]
            mfma[name]["achievable_frac"] = round(tf / peaks["bf16_mfma_TFLOPs"], 4)
    return mfma


def path_entry(wl, ms_step, do_bwd):
    """t_floor / t_measured of the whole path at the published HBM peak."""
    fl = path_floor_bytes(wl)
    out = {}
    for key, fwd in (("survey", fl["survey_fwd"]), ("states_first", fl["f1_fwd"])):
        total = fwd + (fl["bwd"] if do_bwd else 0)
        t_floor = total / (HBM_PEAK_GBS * 1e9)
        out[key] = {"floor_MB": round(total / 1e6, 1), "t_floor_ms": round(t_floor * 1e3, 5),
                    "frac": round(t_floor / (ms_step * 1e-3), 4)}
    return out


# One rank's shard at cp8, at its real shape: the contiguous shard (b rows of L/8
# tokens) and the virtual layout's two half-shards run as 2b rows of L/16 tokens
# (Megatron-LM #6808, "Why virtual is the mode to prefer": 2 x batch program
# instances); one causal segment per row, no predecessor on this GPU.
SHARDS = [("mixer_shard_bf16", "fwd+bwd"), ("mixer_shard_bf16", "fwd"), ("long_context_bf16", "fwd")]


def shard_latency(steps, warmup, dev):
    import torch

    import ssd_workloads as W
    out = {}
    for name, which in SHARDS:
        base = dict(W.WORKLOADS[name])
        L, b = base["seqlen"], base["batch"]
        entry = {}
        for layout, bb, ll in (("contiguous", b, L // 8), ("virtual", 2 * b, L // 16)):
            kw = dict(base, batch=bb, seqlen=ll, nseg=1, layout="contiguous",
                      with_dy=which == "fwd+bwd")
            wl = W.make_workload(f"{name}_shard_{layout}", **kw)
            m = run_workload(wl, which, steps, warmup, dev)
            torch.cuda.empty_cache()
            entry[layout] = {"batch": bb, "seq_len": ll, "us_per_call_sequence": round(m["ms_step"] * 1e3, 2),
                             "tokens_per_s": round(wl.tokens / (m["ms_step"] * 1e-3), 1)}
        out[f"{name}:{which}"] = entry
    return out


# Configurations measured beside the headline (forward of each; the headline is the
# forward + backward of the mixer shard), and the head sample their oracle baseline uses.
EXTRA_CONFIGS = [("tiny_f32", None), ("mixer_shard_bf16", None), ("packed_thd_bf16", None),
                 ("long_context_bf16", list(range(8))),
                 ("long_context_virtual_bf16", list(range(8)))]


def main():
    args = parse()
    if args.summarize_mfma:
        print(json.dumps(summarize_mfma(args.summarize_mfma), indent=1))
        return
    if args.summarize_traffic:
        if not args.copy_probe_mb:
            raise SystemExit("--summarize-traffic needs the --copy-probe-mb of the profiled run")
        print(json.dumps(summarize_traffic(*args.summarize_traffic, args.copy_probe_mb), indent=1))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import ssd_workloads as W

    wl = W.config(args.workload)
    which = args.which or ("fwd+bwd" if wl.dy is not None else "fwd")
    if which == "fwd+bwd" and wl.dy is None:
        raise SystemExit("this workload has no dy; use --pass fwd")
    do_bwd = which == "fwd+bwd"
    dev = torch.device("cuda:0")
    m = run_workload(wl, which, args.steps, args.warmup, dev, args.copy_probe_mb,
                     conv_fused=args.conv_fused)
    torch.cuda.empty_cache()
    peaks = None if args.no_peaks else measure_peaks(torch, dev, torch.cuda.current_stream())
    ms_step, dom, dom_ms, abytes = m["ms_step"], m["dom"], m["dom_ms"], m["abytes"]
    achieved = round(abytes[dom] / (dom_ms * 1e-3) / 1e9, 1)

    result = {
        "metric": METRIC,
        "value": round(wl.tokens / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.act,
        "data": "synthetic (seeded N(0,1) activations, Mamba2-style dt_bias and A_log)",
        "config": {"workload": wl.name, "pass": which, "batch": wl.batch,
                   "seq_len": wl.seqlen, "nheads": wl.nheads, "headdim": wl.headdim,
                   "dstate": wl.dstate, "ngroups": wl.ngroups, "chunk": wl.chunk,
                   "conv_width": wl.conv_width, "segments": len(wl.segments),
                   "layout": wl.layout, "packed": wl.seq_idx is not None,
                   "conv_fused": args.conv_fused},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic(wl.name, CALL_KERNEL[dom]),
                     "kernel_ms": round(dom_ms, 5),
                     "algorithmic_MB": round(abytes[dom] / 1e6, 2)},
        "path_roofline": path_entry(wl, ms_step, do_bwd),
        "achievable_peaks": peaks,
        "mfma": flops_entries(wl, m, do_bwd, peaks),
        "calls": m["per_call"],  # from the breakdown pass, events around every call
        "wall_s_timed_region": round(m["wall"], 4),
    }
    if peaks:
        result["roofline"]["achievable_peak"] = peaks["hbm_GBps"]
        result["roofline"]["achievable_frac"] = round(achieved / peaks["hbm_GBps"], 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_runs, do_bwd)

    # the other configurations, forward, one line each inside the same JSON object
    if not args.no_extra_configs and args.workload == DEFAULT_WORKLOAD:
        extra = {}
        for name, heads in EXTRA_CONFIGS:
            xw = W.config(name)
            xm = run_workload(xw, "fwd", args.steps, args.warmup, dev)
            torch.cuda.empty_cache()
            xd = xm["dom"]
            xa = xm["abytes"][xd] / (xm["dom_ms"] * 1e-3) / 1e9
            e = {"value": round(xw.tokens / (xm["ms_step"] * 1e-3), 1), "unit": "tokens/s",
                 "ms_per_step": round(xm["ms_step"], 5), "pass": "fwd", "dtype": xw.act,
                 "config": {"batch": xw.batch, "seq_len": xw.seqlen, "nheads": xw.nheads,
                            "headdim": xw.headdim, "dstate": xw.dstate, "ngroups": xw.ngroups,
                            "chunk": xw.chunk, "segments": len(xw.segments),
                            "layout": xw.layout, "packed": xw.seq_idx is not None},
                 "roofline": {"bound": "hbm", "kernel": xd, "achieved": round(xa, 1),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s",
                              "frac": round(xa / HBM_PEAK_GBS, 4),
                              "kernel_ms": round(xm["dom_ms"], 5),
                              "algorithmic_MB": round(xm["abytes"][xd] / 1e6, 2)},
                 "path_roofline": path_entry(xw, xm["ms_step"], False),
                 "mfma": flops_entries(xw, xm, False),
                 "calls": {k: v["ms"] for k, v in xm["per_call"].items()}}
            # the same forward with the conv inside the two forward phases
            xf = run_workload(xw, "fwd", args.steps, args.warmup, dev, conv_fused=True)
            torch.cuda.empty_cache()
            fo = xf["per_call"]["ssd_conv_segment_output"]
            e["conv_fused"] = {"value": round(xw.tokens / (xf["ms_step"] * 1e-3), 1),
                               "ms_per_step": round(xf["ms_step"], 5),
                               "output_pass_frac": round(fo["GB_per_s"] / HBM_PEAK_GBS, 4),
                               "calls": {k: v["ms"] for k, v in xf["per_call"].items()}}
            if not args.no_cpu_baseline:
                e["cpu_baseline"] = cpu_baseline(xw, 1, False, heads=heads)
            extra[name] = e
            del xw, xm
            gc.collect()
        result["configs"] = extra
        result["per_shard"] = shard_latency(args.steps, args.warmup, dev)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
