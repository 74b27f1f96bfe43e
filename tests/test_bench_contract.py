"""The benchmark's output contract: one JSON line with the metric, the
roofline and the CPU baseline.  The CPU test checks the one-GPU refusal; the
GPU test runs every operation briefly in this process."""
import contextlib
import io
import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def run_bench(argv):
    import bench
    out, err = io.StringIO(), io.StringIO()
    with contextlib.redirect_stdout(out), contextlib.redirect_stderr(err):
        rc = bench.main(argv)
    return rc, out.getvalue(), err.getvalue()


def test_more_than_one_gpu_is_refused():
    rc, out, err = run_bench(["--gpus", "2"])
    assert rc == 2 and out == "" and "one GPU" in err


@pytest.mark.gpu
@pytest.mark.parametrize("argv", [
    [], ["--config", "2"], ["--op", "forward"], ["--op", "backward_sr"], ["--op", "layernorm"]],
    ids=["default", "fp32_qkv", "forward", "backward_sr", "layernorm"])
def test_json_line(argv):
    rc, out, _ = run_bench(argv + ["--steps", "3", "--warmup", "3", "--no-cpu-baseline"])
    assert rc == 0
    lines = [ln for ln in out.splitlines() if ln.strip()]
    assert len(lines) == 1
    d = json.loads(lines[0])
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
              "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config", "roofline"):
        assert k in d, k
    assert d["n_gpus"] == 1 and d["steps"] == 3 and d["warmup"] == 3
    # the warm-up runs on past --warmup until 300 ms of GPU time have gone by
    assert d["warmup_steps_run"] >= 3 and d["warmup_ms"] >= 300
    assert d["value"] > 0 and d["ms_per_step"] > 0 and d["higher_is_better"] is True
    assert d["data"] == "synthetic" and "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] in ("mfma", "hbm") and r["achieved"] > 0 and r["peak"] > 0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-3
    assert r["traffic"] is None or r["traffic"] > 0
    if r["bound"] == "mfma":
        assert r["hbm_gbs_algorithmic"] > 0 and r["hbm_peak_gbs"] == 8000.0
        assert (r["hbm_gbs_measured"] is None) == (r["traffic"] is None)
        assert r["mfma_busy"] is None or 0 < r["mfma_busy"] <= 100
    # the cold-cache figure: each launch after a 512 MiB stream through the caches
    assert r["launch_ms_flushed"] > 0 and r["achieved_flushed"] > 0
