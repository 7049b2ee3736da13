"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers in tests/sanitize/: the C ABI's host validation (every entry point
given arguments it must refuse, workspace queries over a grid of shapes,
extreme sizes that must be refused without overflow) linked against the
library's sources built with sanitized host code, and the CPU oracle's entry
points on a small packed problem with an initial state.  No GPU is used: the
validation refuses every call before a launch.  Any sanitizer report aborts the
driver (errors are not recoverable) and fails the test.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mamba2_ssd_chunked_amd", "csrc")
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# sanitizers on the host compilation only: the device code is built as usual
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]
SOURCES = ["ssd_api.cpp", "conv1d.hip", "ssd_fwd.hip", "scan.hip", "ssd_bwd.hip", "noalloc.hip"]

pytestmark = pytest.mark.slow


def _run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return r


def _env():
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1:exitcode=87"
    return env


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = str(tmp_path / "oracle_driver")
    _run(["gcc", "-g", "-O1", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
          "-fopenmp", "-o", exe, os.path.join(SAN, "oracle_driver.c"),
          os.path.join(ROOT, "oracle", "ssd_oracle.c"), "-lm"])
    r = _run([exe], env=_env())
    assert "oracle outputs finite: 1" in r.stdout


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_validation_under_sanitizers(tmp_path):
    import concurrent.futures as cf
    common = ["--offload-arch=gfx950", "-O1", "-g", "-fPIC", "-std=c++17",
              "-I", os.path.join(ROOT, "include"), "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-Wno-unused-command-line-argument"] + HOST_SAN

    def compile_one(src):
        obj = str(tmp_path / (src + ".o"))
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        _run([HIPCC] + common + lang + ["-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with cf.ThreadPoolExecutor(max_workers=6) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    drv = str(tmp_path / "abi_driver.o")
    _run([HIPCC, "-g", "-O1", "-x", "c", "-I", os.path.join(ROOT, "include")] + HOST_SAN
         + ["-c", os.path.join(SAN, "abi_driver.c"), "-o", drv])
    exe = str(tmp_path / "abi_driver")
    _run([HIPCC, "--offload-arch=gfx950", "-o", exe, drv] + objs + HOST_SAN)
    r = _run([exe], env=_env())
    assert "0 failed checks" in r.stdout
