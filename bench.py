"""Benchmark of the conv1d + SSD state-passing path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input,
every call going through the C ABI on torch's current stream:
  ssd_conv1d_fwd -> ssd_segment_states -> ssd_segment_output
  -> ssd_boundary_scan -> ssd_apply_init_state.
Workload: 2 rows x 8192 tokens, 32 heads, headdim 64, d_state 128, 1 group,
chunk 256, conv width 4, bf16 activations with FP32 state, cut into 8
contiguous causal segments of 1024 tokens (one device's context-parallel
shard each).  Inputs are resident in HBM before timing starts.

Prints ONE JSON line (rank 0).  Per-call durations come from HIP events
recorded around every call inside the timed region; the roofline entry uses
the call whose single kernel takes the most time.
"""
from __future__ import annotations

import argparse
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="1", help="workload: 1, 2c, 2v or 3")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-runs", type=int, default=3)
    return ap.parse_args()


def algorithmic_bytes(wl):
    """Bytes each call must move at minimum (its own inputs and outputs)."""
    e = 2 if wl.act == "bf16" else 4
    b, L, H, P, N, G, Q = (wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.ngroups,
                           wl.chunk)
    S = len(wl.segments)
    BL = b * L
    C = H * P + 2 * G * N
    seq = 4 * BL if wl.seq_idx is not None else 0
    nchunk = L // Q
    hst_chunks = b * (nchunk - S)  # entering states of every non-first chunk of a segment
    hst = hst_chunks * H * P * N * e
    summary = S * b * H * (P * N + 1) * 4
    states = S * b * H * P * N * 4
    dtcs = 2 * BL * H * 4
    return {
        "ssd_conv1d_fwd": 2 * BL * C * e + C * wl.conv_width * 4 + seq,
        "ssd_segment_states": BL * (H * P + G * N) * e + BL * H * e + 2 * dtcs + hst + summary + seq,
        "ssd_segment_output": BL * C * e + hst + dtcs + BL * H * P * 4 + seq,
        "ssd_boundary_scan": summary + states,
        "ssd_apply_init_state": BL * H * P * 4 + BL * (H * P + G * N) * e + BL * H * 4 + states
                                + BL * H * P * e + seq,
    }


def output_flops(wl):
    """MFMA flops of ssd_segment_output: causal C B^T, its product with X, and C H^T."""
    b, L, H, P, N, Q = wl.batch, wl.seqlen, wl.nheads, wl.headdim, wl.dstate, wl.chunk
    per_chunk_head = Q * (Q + 1) // 2 * 2 * (N + P) + 2 * Q * P * N
    return b * (L // Q) * H * per_chunk_head


def cpu_baseline(wl, runs):
    import oracle
    threads = oracle.num_threads()
    times = []
    for _ in range(runs):
        t = time.perf_counter()
        oracle.forward(wl)
        times.append(time.perf_counter() - t)
    med = statistics.median(times)
    return {"value": wl.tokens / med, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"the whole workload ({wl.tokens} tokens, all heads), float64 token-by-token "
                      f"recurrence, median of {runs} runs ({med:.2f} s each)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import mamba2_ssd_chunked_amd as ssd
    import ssd_workloads as W

    wl = W.config(args.config)
    dev = torch.device("cuda:0")
    act = torch.bfloat16 if wl.act == "bf16" else torch.float32
    f32 = torch.float32
    t = lambda a, dt: torch.from_numpy(np.ascontiguousarray(a)).to(dev, dt)
    xBC, conv_w, dt_raw = t(wl.xBC, act), t(wl.conv_w, f32), t(wl.dt_raw, act)
    dt_bias, A_log, D = t(wl.dt_bias, f32), t(wl.A_log, f32), t(wl.D, f32)
    seq = None if wl.seq_idx is None else t(wl.seq_idx, torch.int32)
    p = ssd.make_problem(batch=wl.batch, seqlen=wl.seqlen, nheads=wl.nheads, headdim=wl.headdim,
                         dstate=wl.dstate, ngroups=wl.ngroups, chunk=wl.chunk,
                         conv_width=wl.conv_width, act=wl.act, dt_min=wl.dt_min,
                         dt_max=wl.dt_max)
    segs = ssd.Segments(wl.segments)
    bufs = ssd.ForwardBuffers.allocate(p, segs, dev)
    stream = torch.cuda.current_stream()

    calls = [
        ("ssd_conv1d_fwd", lambda: ssd.ssd_conv1d_fwd(p, segs, xBC, conv_w, seq, bufs.xBC_conv)),
        ("ssd_segment_states", lambda: ssd.ssd_segment_states(
            p, segs, bufs.xBC_conv, dt_raw, dt_bias, A_log, seq, bufs.summary, bufs.ws)),
        ("ssd_segment_output", lambda: ssd.ssd_segment_output(
            p, segs, bufs.xBC_conv, seq, bufs.ws, bufs.y_zero)),
        ("ssd_boundary_scan", lambda: ssd.ssd_boundary_scan(
            p, segs.n, bufs.summary, None, False, bufs.S_in)),
        ("ssd_apply_init_state", lambda: ssd.ssd_apply_init_state(
            p, segs, bufs.y_zero, bufs.xBC_conv, D, seq, bufs.S_in, bufs.ws, bufs.y)),
    ]
    single_kernel = {"ssd_conv1d_fwd", "ssd_segment_output", "ssd_boundary_scan",
                     "ssd_apply_init_state"}

    def step(events=None):
        for i, (_, fn) in enumerate(calls):
            if events is not None:
                events[i][0].record(stream)
            fn()
            if events is not None:
                events[i][1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in calls]
          for _ in range(args.steps)]
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    for k in range(args.steps):
        step(ev[k])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / args.steps

    abytes = algorithmic_bytes(wl)
    per_call = {}
    for i, (name, _) in enumerate(calls):
        ms = statistics.mean(ev[k][i][0].elapsed_time(ev[k][i][1]) for k in range(args.steps))
        per_call[name] = {"ms": round(ms, 5), "algorithmic_MB": round(abytes[name] / 1e6, 2),
                          "GB_per_s": round(abytes[name] / (ms * 1e-3) / 1e9, 1)}
    dom = max(single_kernel, key=lambda n: per_call[n]["ms"])
    achieved = per_call[dom]["GB_per_s"]
    fl = output_flops(wl)
    out_ms = per_call["ssd_segment_output"]["ms"]
    mfma_peak = BF16_PEAK_TFLOPS if wl.act == "bf16" else F32_PEAK_TFLOPS
    out_tflops = fl / (out_ms * 1e-3) / 1e12

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
        "config": {"workload": wl.name, "pass": "forward", "batch": wl.batch,
                   "seq_len": wl.seqlen, "nheads": wl.nheads, "headdim": wl.headdim,
                   "dstate": wl.dstate, "ngroups": wl.ngroups, "chunk": wl.chunk,
                   "conv_width": wl.conv_width, "segments": len(wl.segments),
                   "layout": wl.layout, "packed": wl.seq_idx is not None},
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None},
        "mfma": {"kernel": "ssd_segment_output", "achieved": round(out_tflops, 2),
                 "peak": mfma_peak, "unit": "TFLOP/s", "frac": round(out_tflops / mfma_peak, 4)},
        "calls": per_call,
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wl, args.cpu_runs)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
