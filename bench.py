#!/usr/bin/env python3
"""Throughput of the batch-invariant selected-token logp path on one MI355X.

Default workload (one "step" = the whole hot path over one batch):
  logits bf16 [8192, 151936] ~ N(0, 3) (Qwen3-8B vocabulary), 10% of rows
  ignored, upstream gradient g ~ N(0, 1) fp32, tile width 4096;
  step = logp_fwd (logp + lse) followed by logp_bwd (dlogits bf16 [N, V]).

Inputs are generated on the device before timing (synthetic, seeded).  Prints
one JSON line.  `value` is rows/s over the timed steps; the roofline object
prices the dominant kernel's algorithmic bytes against the MI355X HBM peak;
cpu_baseline times the float64 CPU oracle on a bounded row sample of the same
workload.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
                    [--workload fwd_bwd|fwd|linear|linear_bwd]
"""

import argparse
import hashlib
import json
import os
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = {
    "logp_fwd_fused_kernel": ["invariant_token_log_amd/csrc/logp_kernels.hip",
                              "invariant_token_log_amd/csrc/logp_device.h"],
    "logp_bwd_kernel": ["invariant_token_log_amd/csrc/logp_kernels.hip",
                        "invariant_token_log_amd/csrc/logp_device.h"],
    "linear_stats_dma": ["invariant_token_log_amd/csrc/linear_logp.hip",
                         "invariant_token_log_amd/csrc/mfma_gemm.h",
                         "invariant_token_log_amd/csrc/logp_device.h"],
}


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary
    (profiles/traffic_<kernel>_<workload>.txt), or None when absent or when
    the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.strip().split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def ramp(torch, fn, seconds):
    """Run fn() untimed until `seconds` of wall time have passed, so that the
    GPU clocks have left their idle state before any warmup or timed step."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_events(torch, fn, steps):
    """Mean device time of fn() over `steps` calls, with events on the
    current stream (the stream every library call launches on)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return sum(a.elapsed_time(b) for a, b in ev) / steps


def bench_fwd_bwd(args, torch, itl, synth):
    n, v, w = 8192, synth.QWEN3_VOCAB, 4096
    dev = torch.device("cuda", 0)
    c = synth.qwen3_fwd_bwd(n=n, v=v, device=dev)
    x, t, g = c["logits"], c["targets"], c["grad"]
    n_active = int((t != -100).sum().item())
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    dl = torch.empty_like(x)

    def fwd():
        itl.logp_fwd(x, t, -100, w, logp_out=logp, lse_out=lse)

    def bwd():
        itl.logp_bwd(x, t, lse, g, -100, w, dlogits_out=dl)

    def step():
        fwd()
        bwd()

    ramp(torch, step, args.ramp_s)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    # per-kernel averages over a second timed pass of the same steps
    fwd_ms = time_events(torch, fwd, args.steps)
    bwd_ms = time_events(torch, bwd, args.steps)

    fwd_bytes = n_active * v * 2 + n * (8 + 4 + 4)
    bwd_bytes = n_active * v * 2 + n * v * 2 + n * (8 + 4 + 4)
    step_bytes = fwd_bytes + bwd_bytes
    kernels = {
        "logp_fwd_fused_kernel": dict(ms=fwd_ms, bytes=fwd_bytes),
        "logp_bwd_kernel": dict(ms=bwd_ms, bytes=bwd_bytes),
    }
    for k in kernels.values():
        k["gbps"] = k["bytes"] / (k["ms"] * 1e-3) / 1e9
        k["hbm_frac"] = k["gbps"] / HBM_PEAK_GBS
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    traffic = measured_traffic(dom, "qwen3_8192x151936")
    roofline = {"bound": "hbm", "achieved": round(kernels[dom]["gbps"], 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kernels[dom]["gbps"] / HBM_PEAK_GBS, 4),
                "traffic": traffic, "kernel": dom,
                "algorithmic_bytes_per_launch": kernels[dom]["bytes"]}
    gbps = step_bytes / (ms_step * 1e-3) / 1e9
    out = {
        "metric": "rows/s and achieved HBM GB/s (% of peak), N=8192 V=151936 bf16 fwd+bwd",
        "value": round(n / (ms_step * 1e-3), 1), "unit": "rows/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_8b_vocab_logp_fwd_bwd", "n": n, "v": v,
                   "tile_width": w, "ignored_rows": n - n_active, "num_shards": 1},
        "gb_per_s": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "algorithmic_bytes_per_step": step_bytes,
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv)
                        for kk, vv in d.items()} for k, d in kernels.items()},
        "roofline": roofline,
        "wall_s_timed": round(wall, 4),
    }
    sample = None
    if not args.no_cpu_baseline:
        sample = dict(x=x, t=t, g=g, n=n, v=v)
    return out, sample


def cpu_baseline_fwd_bwd(sample, max_rows, budget_s):
    """The float64 oracle (forward then backward) on the leading rows of the
    same workload, single process, in 64-row blocks until `budget_s` seconds
    of oracle time are spent or `max_rows` rows are done.  Device-to-host
    copies happen between blocks and are not timed."""
    import oracle

    block = 64
    done, spent = 0, 0.0
    while done < max_rows and spent < budget_s:
        r1 = min(max_rows, done + block)
        xs = sample["x"][done:r1].float().cpu().numpy()
        ts = sample["t"][done:r1].cpu().numpy()
        gs = sample["g"][done:r1].cpu().numpy()
        t0 = time.perf_counter()
        _, lse = oracle.logp_fwd(xs, ts)
        d = oracle.logp_bwd(xs, ts, gs, lse=lse)
        spent += time.perf_counter() - t0
        del d
        done = r1
    return {"value": round(done / spent, 2), "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"first {done} rows of the same [8192, 151936] bf16 batch, float64 "
                      f"numpy forward+backward in {block}-row blocks, {spent:.1f} s of "
                      "oracle time (one thread)",
            "cpu": cpu_model()}


def bench_fwd(args, torch, itl, synth):
    n, v, w = 4096, synth.QWEN3_VOCAB, 4096
    dev = torch.device("cuda", 0)
    c = synth.qwen3_fwd(n=n, v=v, device=dev)
    x, t = c["logits"], c["targets"]
    n_active = int((t != -100).sum().item())
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)

    def fwd():
        itl.logp_fwd(x, t, -100, w, logp_out=logp, lse_out=lse)

    ramp(torch, fwd, args.ramp_s)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()
    ms = time_events(torch, fwd, args.steps)
    byts = n_active * v * 2 + n * 16
    gbps = byts / (ms * 1e-3) / 1e9
    return {
        "metric": "rows/s and achieved HBM GB/s (% of peak), N=4096 V=151936 bf16 fwd",
        "value": round(n / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_vocab_logp_fwd", "n": n, "v": v, "tile_width": w,
                   "ignored_rows": n - n_active},
        "gb_per_s": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("logp_fwd_fused_kernel",
                                                 "qwen3_4096x151936"),
                     "kernel": "logp_fwd_fused_kernel"},
    }, None


def bench_linear(args, torch, itl, synth, prepared=False):
    n, h, v = 4096, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB
    dev = torch.device("cuda", 0)
    c = synth.qwen3_linear(n=n, h=h, v=v, device=dev)
    hid, wt, t = c["hidden"], c["weight"], c["targets"]
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)
    ws = torch.empty(itl.lib().linear_logp_fwd_workspace_bytes(n, h, v, 256),
                     dtype=torch.uint8, device=dev)
    # prepared: the weight re-laid once per weight version, outside the timed
    # calls
    pw = itl.prepare_weight(wt) if prepared else None

    def run():
        itl.linear_logp_fwd(hid, wt, t, -100, 256, logp_out=logp, lse_out=lse, workspace=ws,
                            prepared_weight=pw)

    ramp(torch, run, args.ramp_s)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ms = time_events(torch, run, args.steps)
    flops = 2.0 * n * h * v
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "rows/s and MFMA TFLOP/s (% of peak), fused LM-head+logp N=4096 H=4096 "
                  "V=151936 bf16" + (", prepared weight" if prepared else ""),
        "value": round(n / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_lm_head_linear_logp" + ("_prepared" if prepared else ""),
                   "n": n, "h": h, "v": v, "tile_width": 256},
        "tflops": round(tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4),
                     "traffic": None if prepared else measured_traffic(
                         "linear_stats_dma", "qwen3_4096x4096x151936"),
                     "kernel": "linear_logp_fwd (all launches: blocking the hidden rows, "
                               "linear_stats_dma, the merge; linear_stats_dma is 98% of it)"},
    }
    sample = None
    if not args.no_cpu_baseline:
        sample = dict(h=hid, w=wt, t=t)
    return out, sample


def bench_linear_bwd(args, torch, itl, synth, saved=False, prepared=False):
    n, h, v = 4096, synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB
    dev = torch.device("cuda", 0)
    c = synth.qwen3_linear(n=n, h=h, v=v, device=dev, ignore_frac=0.05)
    hid, wt, t = c["hidden"], c["weight"], c["targets"]
    g = synth.normal_matrix(1, n, 1.0, torch.float32, 1055, dev)[0]
    # saved: the forward keeps its fp32 logits (2.5 GB here) and the backward
    # reads them instead of recomputing h W^T
    _, lse, *rest = itl.linear_logp_fwd(hid, wt, t, return_logits=saved,
                                        logits_dtype=torch.float32)
    z = rest[0] if saved else None
    # prepared: the weight re-laid once per weight version, outside the timed
    # step
    wtp = itl.prepare_weight(wt) if prepared else None
    dh = torch.empty(n, h, dtype=torch.float32, device=dev)
    dw = torch.empty(v, h, dtype=torch.float32, device=dev)
    ws = torch.empty(itl.lib().linear_logp_bwd_workspace_bytes(n, h, v, 256), dtype=torch.uint8,
                     device=dev)

    def run():
        itl.linear_logp_bwd(hid, wt, t, lse, g, dhidden_out=dh, dweight_out=dw, workspace=ws,
                            saved_logits=z, prepared_weight=wtp)

    ramp(torch, run, args.ramp_s)
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    ms = time_events(torch, run, args.steps)
    # z recomputed (not when saved), dh = dz W, dW = dz^T h
    flops = (2 if saved else 3) * 2.0 * n * h * v
    tflops = flops / (ms * 1e-3) / 1e12
    return {
        "metric": "rows/s and MFMA TFLOP/s (% of peak), fused LM-head+logp backward N=4096 "
                  "H=4096 V=151936 bf16" + (", logits saved by the forward (fp32)" if saved
                                            else ", logits recomputed")
                  + (", prepared weight" if prepared else ""),
        "value": round(n / (ms * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_lm_head_linear_logp_bwd" + ("_saved" if saved else "")
                   + ("_prepared" if prepared else ""),
                   "n": n, "h": h, "v": v, "tile_width": 256, "outputs": "dh, dW fp32"},
        "tflops": round(tflops, 2),
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / BF16_MFMA_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "linear_logp_bwd (all launches: dz, the transposes, "
                               "two products)"},
        "extra_memory_bytes": n * v * 4 if saved else 0,
    }, None


def cpu_baseline_linear(sample, rows):
    import oracle

    h = sample["h"][:rows].float().cpu().numpy()
    w = sample["w"].float().cpu().numpy()
    t = sample["t"][:rows].cpu().numpy()
    t0 = time.perf_counter()
    oracle.linear_logp_fwd(h, w, t)
    dt = time.perf_counter() - t0
    threads = os.environ.get("OMP_NUM_THREADS") or str(len(os.sched_getaffinity(0)))
    return {"value": round(rows / dt, 2), "unit": "rows/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {rows} rows, float64 numpy h @ W^T then logp, {dt:.1f} s "
                      "(BLAS threads = cores)",
            "cpu": cpu_model()}


# ---------------------------------------------------------------------------
# HBM traffic summaries from two rocprofv3 --pmc runs (FETCH_SIZE, then
# WRITE_SIZE) of `bench.py --calibrate-copy`: counters are KiB per dispatch and
# are scaled by what the same counter reads on the plain 1 GiB device copies
# that --calibrate-copy runs first (1 GiB read + 1 GiB written each).
# ---------------------------------------------------------------------------

def _short_kernel(name):
    base = name.replace("(anonymous namespace)", "").split("(")[0].split("<")[0]
    return base.split("::")[-1].strip()


def _counter_rows(run_dir, counter):
    """(dispatch id, short kernel name, value) of every dispatch in the
    counter_collection CSV files under run_dir."""
    import csv
    import glob

    per = {}
    for path in glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"),
                          recursive=True):
        with open(path) as f:
            for row in csv.DictReader(f):
                if row.get("Counter_Name") != counter:
                    continue
                key = (path, row["Dispatch_Id"])
                name = _short_kernel(row["Kernel_Name"])
                val = float(row["Counter_Value"])
                if key in per:
                    per[key] = (name, per[key][1] + val)
                else:
                    per[key] = (name, val)
    return [(k[1], nm, v) for k, (nm, v) in sorted(per.items(), key=lambda kv: int(kv[0][1]))]


def _algorithmic_bytes(workload, kernel):
    """Algorithmic bytes per launch of a kernel on a workload: the logits of
    active rows read once (forward and backward), the gradient written once
    for every row, plus 16 B of per-row scalars; for the fused LM head the
    weight and hidden states read once and the per-row outputs."""
    if workload == "qwen3_8192x151936":
        n, v = 8192, 151936
        act = n - int(0.10 * n)
        if kernel == "logp_bwd_kernel":
            return act * v * 2 + n * v * 2 + n * 16
        return act * v * 2 + n * 16
    if workload == "qwen3_4096x151936":
        n, v = 4096, 151936
        return (n - int(0.05 * n)) * v * 2 + n * 16
    if workload == "qwen3_4096x4096x151936":
        n, h, v = 4096, 4096, 151936
        return v * h * 2 + n * h * 2 + n * 16
    raise ValueError(workload)


def summarize_traffic(fetch_dir, write_dir, workload, kernels, fetch_cmd, write_cmd):
    fetch = _counter_rows(fetch_dir, "FETCH_SIZE")
    write = _counter_rows(write_dir, "WRITE_SIZE")

    def calib(rows):
        vals = sorted(v for _, nm, v in rows if nm == "__amd_rocclr_copyBuffer")[-3:]
        if len(vals) < 3:
            raise SystemExit("no 1 GiB calibration copies found (run with --calibrate-copy)")
        return sum(vals) / len(vals)

    cf, cw = calib(fetch), calib(write)
    written = []
    for k in kernels:
        fv = [v for _, nm, v in fetch if nm == k]
        wv = [v for _, nm, v in write if nm == k]
        if not fv or not wv:
            raise SystemExit(f"kernel {k} not found in the counter runs")
        f_kib, w_kib = sum(fv) / len(fv), sum(wv) / len(wv)
        fs, ws = 1048576.0 / cf, 1048576.0 / cw
        hbm = (f_kib * fs + w_kib * ws) * 1024.0
        alg = _algorithmic_bytes(workload, k)
        path = os.path.join(PROFILES, f"traffic_{k}_{workload}.txt")
        with open(path, "w") as f:
            f.write(f"# HBM traffic of {k} on workload {workload}, from two rocprofv3 --pmc runs\n")
            f.write(f"# fetch command: {fetch_cmd}\n# write command: {write_cmd}\n")
            f.write("# counters are KiB per dispatch; scale factors come from the same counters "
                    "read on\n# plain 1 GiB device copies (__amd_rocclr_copyBuffer, 1 GiB read + "
                    "1 GiB written) in the same run\n")
            f.write(f"kernel={k}\nworkload={workload}\n")
            f.write(f"source_sha256_16={kernel_source_hash(k)}\n")
            f.write(f"dispatches_fetch={len(fv)}\ndispatches_write={len(wv)}\n")
            f.write(f"fetch_kib_per_dispatch={f_kib:.1f}\nwrite_kib_per_dispatch={w_kib:.1f}\n")
            f.write(f"copy_fetch_kib_per_gib={cf:.1f}\ncopy_write_kib_per_gib={cw:.1f}\n")
            f.write(f"fetch_scale={fs:.5f}\nwrite_scale={ws:.5f}\n")
            f.write(f"hbm_bytes_per_launch={hbm:.0f}\nalgorithmic_bytes_per_launch={alg}\n")
            f.write(f"traffic_over_algorithmic={hbm / alg:.4f}\n")
        written.append(path)
    return written


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ramp-s", type=float, default=0.5,
                    help="untimed seconds of steps before the warmup steps (GPU clock ramp)")
    ap.add_argument("--workload", default="fwd_bwd",
                    choices=["fwd_bwd", "fwd", "linear", "linear_bwd", "linear_bwd_saved",
                             "linear_bwd_prepared", "linear_prepared"])
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows for the CPU oracle baseline (0 = workload default)")
    ap.add_argument("--cpu-budget-s", type=float, default=15.0,
                    help="oracle time budget of the CPU baseline (fwd_bwd workload)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="first run three plain 1 GiB device copies (a known byte count "
                         "for scaling HBM counters)")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn two rocprofv3 --pmc output folders (FETCH_SIZE, "
                         "WRITE_SIZE) of this workload into profiles/traffic_*.txt")
    ap.add_argument("--pmc-commands", nargs=2, metavar=("FETCH_CMD", "WRITE_CMD"),
                    default=("?", "?"), help="the two commands, recorded in the summaries")
    args = ap.parse_args()
    if args.summarize_traffic:
        wl, ks = {"fwd_bwd": ("qwen3_8192x151936", ["logp_fwd_fused_kernel", "logp_bwd_kernel"]),
                  "fwd": ("qwen3_4096x151936", ["logp_fwd_fused_kernel"]),
                  "linear": ("qwen3_4096x4096x151936", ["linear_stats_dma"])}[args.workload]
        for p in summarize_traffic(*args.summarize_traffic, wl, ks, *args.pmc_commands):
            print(p)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(rows are independent, so data-parallel scaling needs no exchange); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")

    import torch

    sys.path.insert(0, ROOT)
    import invariant_token_log_amd as itl
    import synth

    if not torch.cuda.is_available():
        sys.exit("no ROCm GPU visible")
    itl.lib()  # fail loudly if the HIP library is missing
    if args.calibrate_copy:
        src = torch.ones(1 << 29, dtype=torch.bfloat16, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    runner = {"fwd_bwd": bench_fwd_bwd, "fwd": bench_fwd, "linear": bench_linear,
              "linear_bwd": bench_linear_bwd,
              "linear_bwd_saved": lambda *a: bench_linear_bwd(*a, saved=True),
              "linear_bwd_prepared": lambda *a: bench_linear_bwd(*a, prepared=True),
              "linear_prepared": lambda *a: bench_linear(*a, prepared=True)}[args.workload]
    out, sample = runner(args, torch, itl, synth)
    if sample is not None:
        if args.workload == "fwd_bwd":
            out["cpu_baseline"] = cpu_baseline_fwd_bwd(sample, args.cpu_rows or 8192,
                                                       args.cpu_budget_s)
        elif args.workload == "linear":
            out["cpu_baseline"] = cpu_baseline_linear(sample, args.cpu_rows or 512)
    if "cpu_baseline" in out and out["cpu_baseline"]["value"]:
        out["gpu_over_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    out["contract_id"] = itl.contract_id()
    out["device"] = torch.cuda.get_device_name(0)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
