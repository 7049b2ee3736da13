"""Build libssd.so (gfx950) in-tree with hipcc, and beside it libssd_probe.so,
the achievable-peak probes that the roofline figures are also quoted against.

All HIP sources are compiled for gfx950 only, with packed-FP32 instructions
disabled (-Xclang -target-feature -Xclang -packed-fp32-ops).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libssd.so")
PROBE_LIB = os.path.join(HERE, "libssd_probe.so")
BUILD_DIR = os.path.join(ROOT, "_build")
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["ssd_api.cpp", "conv1d.hip", "ssd_fwd.hip", "scan.hip", "ssd_bwd.hip", "noalloc.hip"]
PROBE_SOURCES = ["peak_probes.hip"]
# The probes' MFMA loops keep their accumulators in ordinary VGPRs, updated in
# place: with accumulation registers the allocator copies every chain's
# accumulator between registers each round, and the copies wait for the
# products.  (The SSD kernels get the in-place VGPR form without the flag.)
EXTRA_FLAGS = {"peak_probes.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include"), "-Wno-unused-command-line-argument"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC] + FLAGS + EXTRA_FLAGS.get(src, []) + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs: list, lib: str) -> None:
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed for {os.path.basename(lib)}:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Compile every source, link libssd.so and libssd_probe.so; returns the
    path of libssd.so."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    _link(objs[:len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {os.path.basename(PROBE_LIB)}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
