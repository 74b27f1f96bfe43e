"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU
only, no GPU call): the library's host pass (argument checks, path choice,
the launch planner and its event model, tuning overrides) built with hipcc
with the sanitizers on the host side only, and the CPU oracle built with gcc,
each driven by a program under tests/sanitize/ that reports any memory or
undefined-behaviour error and exits non-zero."""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# leak reports would come from the HIP runtime's process-lifetime state; the
# checks here are for invalid accesses and undefined behaviour
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="4")


def run(cmd, **kw):
    return subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, **kw)


def check_clean(r):
    out = r.stdout
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_host_pass_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "host_api_check")
    srcs = sorted(glob.glob(os.path.join(ROOT, "linear_layer_backward_amd", "csrc", "*.hip")))
    # the checks below never launch a kernel: device code unoptimised (fast to build)
    cmd = [HIPCC, "-O1", "-g", "-std=c++17", "--offload-arch=gfx950",
           "-Xarch_device", "-O0", "-Xarch_device", "-g0",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
           *srcs, os.path.join(HERE, "host_api_check.cpp"),
           "-L/opt/rocm/lib", "-lrocprofiler-sdk-roctx", "-Wl,-rpath,/opt/rocm/lib", "-o", exe]
    b = run(cmd)
    assert b.returncode == 0, b.stdout[-4000:]
    check_clean(run([exe], env=ENV, timeout=600))


def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_check")
    b = run(["gcc", "-O1", "-g", "-std=c99", "-fopenmp", "-fsanitize=address,undefined",
             "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
             os.path.join(ROOT, "oracle", "mmb_oracle.c"), os.path.join(HERE, "oracle_check.c"),
             "-lm", "-o", exe])
    assert b.returncode == 0, b.stdout[-4000:]
    check_clean(run([exe], env=ENV, timeout=300))
