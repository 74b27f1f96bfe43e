"""Benchmark of the linear-layer backward pass (dinp + dweight + dbias) on one
MI355X, and (--op forward) of the forward product out = inp.W^T + bias at the
same layer shapes.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 4] [--op backward]

A step is one whole backward pass over the workload (one mmb_backward call;
two for the MLP pair).  Prints one JSON line: TFLOP/s over the timed steps,
which run back to back (4*B*T*C*OC flops plus B*T*OC adds for the bias), the
dominant kernel's MFMA roofline fraction from HIP events recorded around each
launch of a second run of as many steps on the stream it runs on, and the CPU
oracle timed on a bounded sample of the same workload on the host's cores.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "matmul-backward TFLOP/s (dinp+dweight+dbias) at GPT-2 fc shape; % MFMA peak"
METRIC_FORWARD = "matmul-forward TFLOP/s (inp.W^T + bias) at GPT-2 layer shape; % MFMA peak"
METRIC_SR = ("matmul-backward TFLOP/s (dinp+dweight+dbias, bf16 dweight/dbias stochastically "
             "rounded) at GPT-2 layer shape; % MFMA peak")
# MI355X dense peaks (AMD published): bf16 MFMA 2.5 PFLOP/s (256 CUs x 2.4 GHz
# x 4096 flop/clk/CU = 2516.6 TFLOP/s), fp32 MFMA 157.3 TFLOP/s
PEAK_TFLOPS = {"bf16": 2516.6, "f32": 157.3}
# the one kernel a step launches, per operation and compute type
KERNEL_NAME = {"bf16": "mmb_tiles_bf16_kernel", "f32": "mmb_tiles_kernel"}
KERNEL_NAME_FORWARD = {"bf16": "mmb_fwd_bf16_kernel", "f32": "mmb_fwd_kernel"}
KERNEL_NAME_SR = {"bf16": "mmb_tiles_bf16_sr_kernel"}
METRIC_LN = "layernorm-backward GB/s (dinp+dweight+dbias) at the page's B=8 T=1024 C=1600; % HBM peak"
HBM_PEAK_GBS = 8000.0


def flushed_launch_ms(step, stream, K: int, flush_mib: int) -> float:
    """Average duration of K launches, each after streaming a flush_mib MiB
    device copy (larger than the 256 MB last-level cache and the L2s), timed
    with HIP events on the launch stream: the cold-cache counterpart of the
    warm, back-to-back figures."""
    import torch
    n = flush_mib * (1 << 20) // 4
    a = torch.empty(n, dtype=torch.float32, device=stream.device).fill_(1.0)
    b = torch.empty_like(a)
    ms = []
    for _ in range(K):
        b.copy_(a)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    del a, b
    return float(np.mean(ms))


def warm_up(step, stream, W: int, min_ms: float):
    """W steps, then more, back to back, until at least min_ms of GPU time has
    gone by: the GPU raises its clocks over the first tens of milliseconds of
    continuous work, and a few warm-up steps would time that ramp instead of
    the steady state a training loop runs in.  Returns (steps run, GPU ms)."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    n = 0
    for _ in range(W):
        step()
        n += 1
    e1.record(stream)
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    while ms < min_ms:
        # estimate the per-step time from what ran so far, then enqueue the rest
        # in one batch (a probe of 4 steps when none ran yet)
        per = ms / n if n else 0.0
        batch = 4 if per <= 0 else max(1, min(100000, int((min_ms - ms) / per) + 1))
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(batch):
            step()
        b1.record(stream)
        b1.synchronize()
        ms += b0.elapsed_time(b1)
        n += batch
    return n, ms


def backward_bytes(c) -> int:
    """Algorithmic HBM bytes of one backward call: read dout, inp and weight
    once, read and write dinp and dweight once, write dbias."""
    es = 2 if c.dtype == "bf16" else 4
    return es * (c.BT * c.OC + c.BT * c.C + c.OC * c.C + 2 * c.BT * c.C + 2 * c.OC * c.C
                 + (c.OC if c.with_bias else 0))


def forward_bytes(c) -> int:
    """Algorithmic HBM bytes of one forward call: read inp, weight and the
    bias once, write out."""
    es = 2 if c.dtype == "bf16" else 4
    return es * (c.BT * c.C + c.OC * c.C + (c.OC if c.with_bias else 0) + c.BT * c.OC)


def layernorm_bytes(c) -> int:
    """Algorithmic HBM bytes of one LayerNorm backward: read dout, inp and
    the old dinp and write dinp (BT*C each), read weight, mean and rstd, read
    and write dweight and dbias."""
    es = 2 if c.dtype == "bf16" else 4
    return es * (4 * c.BT * c.C + c.C + 2 * c.BT + 4 * c.C)


def bench_layernorm(args):
    """--op layernorm: the LayerNorm backward at the page's benchmark shape
    (B=8, T=1024, C=1600, bf16 as the page's build), HBM-bound."""
    import torch
    from linear_layer_backward_amd import mmb
    from linear_layer_backward_amd import workloads as wl
    dev = torch.device("cuda:0")
    dt = args.ln_dtype
    c = wl.layernorm_case(8, 1024, 1600, dt, seed=1)
    print(f"[bench] workload: {c.name}", file=sys.stderr, flush=True)

    def up(a):
        raw = wl.storage(np.asarray(a, np.float32).ravel(), c.dtype)
        if dt == "bf16":
            return torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(raw.copy()).to(dev)

    b = [up(a) for a in (c.dinp0, c.dweight0, c.dbias0, c.dout, c.inp, c.weight, c.mean, c.rstd)]
    stream = torch.cuda.current_stream(dev)
    code = mmb.MMB_BF16 if dt == "bf16" else mmb.MMB_FP32

    def step():
        mmb.mmb_layernorm_backward(*b, c.B, c.T, c.C, code, stream)

    warm_steps, warm_ms = warm_up(step, stream, args.warmup, args.min_warmup_ms)
    torch.cuda.synchronize(dev)
    K = args.steps
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(K):
        step()
    t1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / K
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, z in ev:
        a.record(stream)
        step()
        z.record(stream)
    torch.cuda.synchronize(dev)
    launch_ms = float(np.mean([a.elapsed_time(z) for a, z in ev]))
    nbytes = layernorm_bytes(c)
    cold_ms = flushed_launch_ms(step, stream, K, args.flush_mib) if args.flush_mib > 0 else None
    out = {
        "metric": METRIC_LN, "value": round(nbytes / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "warmup_steps_run": warm_steps,
        "warmup_ms": round(warm_ms, 1), "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dt,
        "data": "synthetic",
        "config": {"workload": c.name, "B": c.B, "T": c.T, "C": c.C, "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / (launch_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(nbytes / (launch_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("ln_bwd_rows", 0, ln_slug(dt)),
                     "lds_busy": measured_util("ln_bwd_rows", 0, "lds_util_pct", ln_slug(dt)),
                     "kernel": "ln_bwd_rows + ln_bwd_reduce (one call)",
                     "launch_ms": round(launch_ms, 5),
                     "launch_ms_flushed": None if cold_ms is None else round(cold_ms, 5),
                     "achieved_flushed": None if cold_ms is None
                     else round(nbytes / (cold_ms * 1e-3) / 1e9, 1)},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        import oracle
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        # the whole workload, repeated for at least 2 s (one pass is short)
        reps, t = 0, time.perf_counter()
        while True:
            oracle.layernorm_backward(c.dout, c.inp, c.weight, c.mean, c.rstd, B=c.B, T=c.T,
                                      C=c.C)
            reps += 1
            dt_s = time.perf_counter() - t
            if dt_s >= 2.0:
                break
        sb = reps * nbytes
        out["cpu_baseline"] = {"value": sb / dt_s / 1e9, "unit": "GB/s", "cores": oracle.threads(),
                               "kind": "oracle",
                               "sample": f"{c.name}: the whole call {reps} times; fp64 OpenMP, "
                                         f"{dt_s:.2f} s for {sb:.3e} bytes"}
    print(json.dumps(out), flush=True)
    return 0


def kernel_name(op: str, dtype: str) -> str:
    table = {"forward": KERNEL_NAME_FORWARD, "backward_sr": KERNEL_NAME_SR}.get(op, KERNEL_NAME)
    return table[dtype]


def forward_bias(case):
    """The forward's bias for a workload case: N(0, 0.02) in the case's dtype
    (seeded), or None where the layer has no bias (the LM head)."""
    from linear_layer_backward_amd import workloads as wl
    return wl.normal(7000 + case.OC, (case.OC,), 0.02, case.dtype) if case.with_bias else None


def forward_flops(case) -> int:
    """2*B*T*C*OC for the product, plus one add per output for the bias."""
    return 2 * case.BT * case.C * case.OC + (case.BT * case.OC if case.with_bias else 0)


# the sources each kernel's code and launch plan come from (the shared headers
# and the planner included); counters taken on other sources are stale
_COMMON = ["mmb_internal.h", "mmb_numeric.h", "mmb_tile_common.h", "mmb_plan.h", "mmb_plan.hip"]
KERNEL_SOURCES = {
    "mmb_tiles_bf16_kernel": ["mmb_tiles_bf16.hip"] + _COMMON,
    "mmb_tiles_bf16_sr_kernel": ["mmb_tiles_bf16.hip"] + _COMMON,
    "mmb_fwd_bf16_kernel": ["mmb_tiles_bf16.hip"] + _COMMON,
    "mmb_tiles_kernel": ["mmb_tiles.hip"] + _COMMON,
    "mmb_fwd_kernel": ["mmb_tiles.hip"] + _COMMON,
    "ln_bwd_rows": ["mmb_layernorm.hip", "mmb_internal.h", "mmb_numeric.h"],
}


def source_digest(kernel: str = None) -> str:
    """sha256 over the HIP sources of `kernel` (all of them when None)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "linear_layer_backward_amd", "csrc")
    names = KERNEL_SOURCES.get(kernel)
    files = ([os.path.join(csrc, n) for n in sorted(names)] if names
             else sorted(glob.glob(os.path.join(csrc, "*"))))
    for f in files:
        h.update(os.path.basename(f).encode())
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def ln_slug(dtype: str = "bf16") -> str:
    return f"layernorm_{dtype}_B8_T1024_C1600"


LN_SLUG = ln_slug("bf16")


def measured_traffic(kernel: str, cfg: int, slug: str = None):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    this workload, if it was taken on the current kernel sources."""
    from linear_layer_backward_amd import workloads as wl
    slug = slug or wl.CONFIG_SLUGS[cfg]
    path = os.path.join(ROOT, "profiles", f"{kernel}_{slug}_counters.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_digest:\s*(\w+)", text, re.M)
    b = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not b or m.group(1) != source_digest(kernel):
        return None
    return float(b.group(1))


def measured_util(kernel: str, cfg: int, field: str, slug: str = None):
    """A utilisation figure (percent) from the committed rocprofv3 counter
    summary of this workload (<kernel>_<workload>_util.txt), if it was taken
    on the current kernel sources."""
    from linear_layer_backward_amd import workloads as wl
    slug = slug or wl.CONFIG_SLUGS[cfg]
    path = os.path.join(ROOT, "profiles", f"{kernel}_{slug}_util.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_digest:\s*(\w+)", text, re.M)
    b = re.search(rf"^{field}:\s*([0-9.eE+-]+)", text, re.M)
    if not m or not b or m.group(1) != source_digest(kernel):
        return None
    return float(b.group(1))


# one rocprofv3 --pmc pass of utilisation counters (8 SQ counters and
# GRBM_GUI_ACTIVE, within one pass's hardware limits)
UTIL_COUNTERS = ["MfmaUtil", "LdsUtil", "VALUBusy", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES",
                 "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_MFMA", "SQ_INSTS_LDS"]


def summarize_util(kernel: str, workload: str, run_dir: str, digest_kernel: str = None) -> str:
    """Text summary of one rocprofv3 --pmc pass of UTIL_COUNTERS over a
    workload: the matrix-core busy share (MfmaUtil: MFMA busy cycles over the
    SIMDs' active cycles), the LDS busy share (LdsUtil), VALU busy, the share
    of wave cycles spent waiting on LDS instructions, and LDS bank conflicts
    per LDS-active cycle."""
    mean = {c: _counter_mean(run_dir, c, kernel)[0] for c in UTIL_COUNTERS}
    n = _counter_mean(run_dir, "MfmaUtil", kernel)[1]
    lds_wait = mean["SQ_WAIT_INST_LDS"] / mean["SQ_WAVE_CYCLES"] if mean["SQ_WAVE_CYCLES"] else 0
    lines = [
        f"kernel: {kernel}",
        f"workload: {workload}",
        f"source_digest: {source_digest(digest_kernel or kernel)}",
        f"dispatches: {n}",
        f"mfma_util_pct: {mean['MfmaUtil']:.2f}",
        f"lds_util_pct: {mean['LdsUtil']:.2f}",
        f"valu_busy_pct: {mean['VALUBusy']:.2f}",
        f"lds_wait_share_of_wave_cycles_pct: {100 * lds_wait:.2f}",
        f"lds_bank_conflict_cycles: {mean['SQ_LDS_BANK_CONFLICT']:.4e}",
        f"mfma_instructions: {mean['SQ_INSTS_MFMA']:.4e}",
        f"lds_instructions: {mean['SQ_INSTS_LDS']:.4e}",
    ]
    return "\n".join(lines) + "\n"


def _counter_mean(run_dir: str, counter: str, kernel: str):
    """Mean per-dispatch value of one rocprofv3 counter for kernels whose
    name contains `kernel`, from the counter_collection CSVs under run_dir."""
    import csv
    vals = []
    for f in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                if row["Counter_Name"] == counter and kernel in row["Kernel_Name"]:
                    vals.append(float(row["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {kernel} under {run_dir}")
    return float(np.mean(vals)), len(vals)


def summarize_counters(cfg: int, dirs, copy_mib: int, op: str = "backward",
                       ln_dtype: str = "bf16") -> str:
    """Text summary of two FETCH_SIZE / WRITE_SIZE passes over the workload and
    the same two passes over a plain copy of copy_mib MiB: the copy kernel's
    readings fix the KiB-per-counter-unit scale of each counter.  The figure
    is per step: the MLP pair launches its kernel twice, and a LayerNorm call
    is a row kernel and a reduce kernel."""
    from linear_layer_backward_amd import workloads as wl
    fetch_dir, write_dir, cal_fetch_dir, cal_write_dir = dirs
    if op == "layernorm":
        kernels, per_step = ["ln_bwd_rows", "ln_bwd_reduce"], 1
        digest_kernel = "ln_bwd_rows"
        name = f"LayerNorm backward {ln_dtype} B=8 T=1024 C=1600"
    else:
        kernels = [kernel_name(op, "bf16" if cfg >= 4 else "f32")]
        digest_kernel = kernels[0]
        per_step = len(wl.config_cases(cfg)) if cfg == 3 else 1
        name = wl.CONFIG_NAMES[cfg] + (" (forward product)" if op == "forward" else "")
    copy_kib = copy_mib * 1024.0
    cf, ncf = _counter_mean(cal_fetch_dir, "FETCH_SIZE", "__amd_rocclr_copyBuffer")
    cw, ncw = _counter_mean(cal_write_dir, "WRITE_SIZE", "__amd_rocclr_copyBuffer")
    sf, sw = copy_kib / cf, copy_kib / cw
    lines = [
        f"kernel: {' + '.join(kernels)}",
        f"workload: {name}",
        f"source_digest: {source_digest(digest_kernel)}",
        f"copy calibration: {copy_mib} MiB each way; FETCH_SIZE {cf:.1f} ({ncf} dispatches), "
        f"WRITE_SIZE {cw:.1f} ({ncw}); scale fetch {sf:.4f}, write {sw:.4f}",
    ]
    total = 0.0
    for k in kernels:
        kf, nkf = _counter_mean(fetch_dir, "FETCH_SIZE", k)
        kw, nkw = _counter_mean(write_dir, "WRITE_SIZE", k)
        fetch_b, write_b = kf * sf * 1024 * per_step, kw * sw * 1024 * per_step
        total += fetch_b + write_b
        lines += [f"{k} FETCH_SIZE mean {kf:.1f} over {nkf} dispatches, {per_step} per step -> "
                  f"{fetch_b:.4e} bytes per step",
                  f"{k} WRITE_SIZE mean {kw:.1f} over {nkw} dispatches, {per_step} per step -> "
                  f"{write_b:.4e} bytes per step"]
    lines.append(f"hbm_bytes_per_launch: {total:.6e}")
    return "\n".join(lines) + "\n"


def summarize_trace(run_dir: str, log: str, title: str, digest_kernel: str) -> str:
    """Text summary of one rocprofv3 --kernel-trace --stats run of bench.py:
    the per-kernel statistics table and the bench line of the same run."""
    stats = glob.glob(os.path.join(run_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not stats:
        raise SystemExit(f"no kernel_stats.csv under {run_dir}")
    line = [ln for ln in open(log).read().splitlines() if ln.startswith("{")][-1]
    return (f"# {title}: kernel trace\n"
            f"source_digest: {source_digest(digest_kernel)}\n\n"
            f"run_kernel_stats.csv:\n{open(stats[0]).read().strip()}\n\n"
            f"bench.py line of the same run (launch_ms from HIP events on the launch stream):\n"
            f"{line}\n")


def upload(case, dev):
    import torch
    from linear_layer_backward_amd import workloads as wl

    def up(a):
        raw = wl.storage(np.asarray(a, np.float32).ravel(), case.dtype)
        if case.dtype == "bf16":
            return torch.from_numpy(raw.view(np.int16).copy()).view(torch.bfloat16).to(dev)
        return torch.from_numpy(raw.copy()).to(dev)

    return dict(dinp=up(case.dinp0), dweight=up(case.dweight0),
                dbias=up(case.dbias0) if case.with_bias else None,
                dout=up(case.dout), inp=up(case.inp), weight=up(case.weight))


def cpu_baseline_forward(case, bias, target_s: float = 12.0):
    """The oracle's forward (unchanged) on the first `rows` rows of out,
    sized from a probe to about target_s seconds."""
    import oracle
    x64 = case.inp.astype(np.float64)
    w64 = case.weight.astype(np.float64)
    b64 = None if bias is None else bias.astype(np.float64)

    def run(rows):
        xr = np.ascontiguousarray(x64[:rows])
        t0 = time.perf_counter()
        oracle.forward(xr, w64, b64, B=1, T=rows, C=case.C, OC=case.OC)
        dt = time.perf_counter() - t0
        return dt, 2 * rows * case.C * case.OC + (rows * case.OC if bias is not None else 0)

    threads = oracle.threads()
    r0 = max(threads, 16)
    t, _ = run(r0)
    rows = int(min(case.BT, r0 * max(1.0, target_s / max(t, 1e-3))))
    dt, flops = run(rows)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{case.name}, forward: out rows 0..{rows - 1} of {case.BT}; "
                      f"fp64 OpenMP, {dt:.1f} s for {flops:.3e} flops"}


def cpu_baseline(case, target_s: float = 12.0):
    """The oracle (unchanged) on a bounded sample of the workload: the first
    `rows` rows of dinp and the first `chans` rows of dweight (plus their
    dbias entries), sized from a probe to about target_s seconds."""
    import oracle
    d64 = case.dout.astype(np.float64)
    x64 = case.inp.astype(np.float64)
    w64 = case.weight.astype(np.float64)

    def run(rows, chans):
        dr = np.ascontiguousarray(d64[:rows])
        dc = np.ascontiguousarray(d64[:, :chans])
        t0 = time.perf_counter()
        oracle.dinp(dr, w64, None, B=1, T=rows, C=case.C, OC=case.OC)
        oracle.dweight(dc, x64, None, B=case.B, T=case.T, C=case.C, OC=chans)
        if case.with_bias:
            oracle.dbias(dc, B=case.B, T=case.T, OC=chans)
        dt = time.perf_counter() - t0
        flops = 2 * rows * case.C * case.OC + 2 * chans * case.BT * case.C
        if case.with_bias:
            flops += chans * case.BT
        return dt, flops

    threads = oracle.threads()
    r0, c0 = max(threads, 16), max(threads, 4)
    t, _ = run(r0, c0)
    scale = max(1.0, target_s / max(t, 1e-3))
    rows = int(min(case.BT, r0 * scale))
    chans = int(min(case.OC, c0 * scale))
    dt, flops = run(rows, chans)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"{case.name}: dinp rows 0..{rows - 1} of {case.BT}, dweight"
                      f"{'+dbias' if case.with_bias else ''} channels 0..{chans - 1} of "
                      f"{case.OC}; fp64 OpenMP, {dt:.1f} s for {flops:.3e} flops"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    # the GPU needs a few tens of milliseconds of back-to-back work to reach its
    # steady clocks: fewer warm-up steps measure the ramp, not the kernel
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--min-warmup-ms", type=float, default=300.0, metavar="MS",
                    help="keep warming up, whatever --warmup says, until this much GPU time of "
                         "back-to-back steps has run (the clocks ramp over the first tens of ms)")
    ap.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--unpadded-vocab", action="store_true",
                    help="with --config 5: the LM head at the real vocabulary (OC = 50257, "
                         "ragged rows, packed copies on the MFMA tiles) instead of 50304")
    ap.add_argument("--op", default="backward",
                    choices=["backward", "forward", "backward_sr", "layernorm"],
                    help="backward (the metric), the forward product at the same shapes, or the "
                         "bf16 backward with stochastically rounded dweight/dbias")
    ap.add_argument("--ln-dtype", default="bf16", choices=["bf16", "f32"],
                    help="storage type of --op layernorm (the page's build is bf16)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush-mib", type=int, default=512, metavar="MIB",
                    help="also time each launch after streaming MIB MiB through the caches "
                         "(cold-cache figure; 0 = skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("DIR", "LOG"),
                    help="print the kernel-trace summary of a rocprofv3 --kernel-trace --stats "
                         "run (output DIR) of this bench, whose stdout is in LOG")
    ap.add_argument("--summarize-util", metavar="DIR",
                    help="print the utilisation summary (MFMA, LDS, VALU busy) of the dominant "
                         "kernel from a rocprofv3 --pmc run of bench.UTIL_COUNTERS in DIR")
    ap.add_argument("--summarize-counters", nargs=4, metavar="DIR",
                    help="print the HBM-traffic summary from rocprofv3 --pmc output dirs: "
                         "workload FETCH_SIZE, workload WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE "
                         "(the copy run made with --copy-calibration MIB)")
    args = ap.parse_args(argv)

    if args.summarize_trace:
        from linear_layer_backward_amd import workloads as wl
        if args.op == "layernorm":
            k = "ln_bwd_rows"
            title = f"ln_bwd_rows + ln_bwd_reduce, LayerNorm backward {args.ln_dtype} B=8 T=1024 C=1600"
        else:
            k = kernel_name(args.op, "bf16" if args.config >= 4 else "f32")
            title = f"{k}, workload {wl.CONFIG_NAMES[args.config]}" + (
                " (forward product)" if args.op == "forward" else "")
        print(summarize_trace(args.summarize_trace[0], args.summarize_trace[1], title, k), end="")
        return 0

    if args.summarize_util:
        from linear_layer_backward_amd import workloads as wl
        if args.op == "layernorm":
            k, name = "ln_bwd_rows", f"LayerNorm backward {args.ln_dtype} B=8 T=1024 C=1600"
        else:
            k = kernel_name(args.op, "bf16" if args.config >= 4 else "f32")
            name = wl.CONFIG_NAMES[args.config] + (" (forward product)" if args.op == "forward"
                                                    else "")
        print(summarize_util(k, name, args.summarize_util), end="")
        return 0

    if args.summarize_counters:
        print(summarize_counters(args.config, args.summarize_counters,
                                 args.copy_calibration or 256, args.op, args.ln_dtype), end="")
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported: the "
              "multi-GPU (data-parallel) sharding is a design note only.", file=sys.stderr)
        return 2

    import torch
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        a = torch.ones(n, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": n * 4, "launches": 5}))
        return 0

    if args.op == "layernorm":
        return bench_layernorm(args)

    from linear_layer_backward_amd import mmb
    from linear_layer_backward_amd import workloads as wl

    fwd = args.op == "forward"
    sr = args.op == "backward_sr"
    cases = wl.config_cases(args.config)
    if args.unpadded_vocab:
        if args.config != 5:
            print("--unpadded-vocab goes with --config 5", file=sys.stderr)
            return 2
        cases = [wl.lm_head_unpadded_case()]
    if sr and cases[0].dtype != "bf16":
        print("--op backward_sr needs a bf16 workload (--config 4 or 5)", file=sys.stderr)
        return 2
    print(f"[bench] workload: {wl.CONFIG_NAMES[args.config]}"
          + (" (forward product)" if fwd else ""), file=sys.stderr, flush=True)
    bufs = [upload(c, dev) for c in cases]
    stream = torch.cuda.current_stream(dev)
    codes = [mmb.MMB_BF16 if c.dtype == "bf16" else mmb.MMB_FP32 for c in cases]
    biases = [forward_bias(c) for c in cases]
    if fwd:
        tdt = {"bf16": torch.bfloat16, "f32": torch.float32}
        for c, b, bias in zip(cases, bufs, biases):
            b["out"] = torch.empty(c.BT * c.OC, dtype=tdt[c.dtype], device=dev)
            b["bias"] = (None if bias is None else
                         torch.from_numpy(np.asarray(bias, np.float32)).to(dev).to(tdt[c.dtype]))

    def step():
        for c, b, code in zip(cases, bufs, codes):
            if fwd:
                mmb.mmb_forward_stream(b["out"], b["inp"], b["weight"], b["bias"], c.B, c.T,
                                       c.C, c.OC, code, stream)
            elif sr:
                mmb.mmb_backward_sr(b["dinp"], b["dweight"], b["dbias"], b["dout"], b["inp"],
                                    b["weight"], c.B, c.T, c.C, c.OC, 1234, stream)
            else:
                mmb.mmb_backward_stream(b["dinp"], b["dweight"], b["dbias"], b["dout"], b["inp"],
                                        b["weight"], c.B, c.T, c.C, c.OC, code, stream)

    warm_steps, warm_ms = warm_up(step, stream, args.warmup, args.min_warmup_ms)
    torch.cuda.synchronize(dev)

    # The K timed steps run back to back with nothing between them: an event
    # recorded between two launches holds the second one back by several
    # microseconds.  The kernel's own duration is then taken over K more
    # steps, each bracketed by events on the launch stream.
    K = args.steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(K):
        step()
    t_end.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        step()
        ev[i][1].record(stream)
    torch.cuda.synchronize(dev)
    launch_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    cold_ms = flushed_launch_ms(step, stream, K, args.flush_mib) if args.flush_mib > 0 else None

    flops = sum(forward_flops(c) if fwd else c.flops() for c in cases)
    dtype = cases[0].dtype
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (launch_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype]
    kernel = kernel_name(args.op, dtype)
    # counter summaries exist for the five workloads, not the unpadded LM head
    traffic = None if args.unpadded_vocab else measured_traffic(kernel, args.config)
    nbytes = sum(forward_bytes(c) if fwd else backward_bytes(c) for c in cases)
    gbs = lambda b: round(b / (launch_ms * 1e-3) / 1e9, 1)

    out = {
        "metric": METRIC_FORWARD if fwd else (METRIC_SR if sr else METRIC),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "warmup_steps_run": warm_steps,
        "warmup_ms": round(warm_ms, 1),
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": (wl.CONFIG_NAMES[args.config].replace("OC=50304", "OC=50257")
                                if args.unpadded_vocab else wl.CONFIG_NAMES[args.config])
                   + (" (forward product)" if fwd else "")
                   + (" (stochastic rounding)" if sr else ""),
                   "calls": [{"B": c.B, "T": c.T, "C": c.C, "OC": c.OC, "bias": c.with_bias}
                             for c in cases],
                   "flops_per_step": flops, "bytes_per_step": nbytes},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic, "kernel": kernel,
                     "launch_ms": round(launch_ms, 5),
                     # HBM rates against the 8 TB/s peak: algorithmic bytes, and the
                     # copy-calibrated counter bytes, each over the launch duration
                     "hbm_gbs_algorithmic": gbs(nbytes),
                     "hbm_gbs_measured": None if traffic is None else gbs(traffic),
                     "hbm_peak_gbs": HBM_PEAK_GBS,
                     # matrix-core busy share of the kernel's cycles (rocprofv3 MfmaUtil)
                     "mfma_busy": None if args.unpadded_vocab
                     else measured_util(kernel, args.config, "mfma_util_pct"),
                     "launch_ms_flushed": None if cold_ms is None else round(cold_ms, 5),
                     "achieved_flushed": None if cold_ms is None
                     else round(flops / (cold_ms * 1e-3) / 1e12, 2)},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        out["cpu_baseline"] = (cpu_baseline_forward(cases[0], biases[0]) if fwd
                               else cpu_baseline(cases[0]))
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
