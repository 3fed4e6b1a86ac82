#!/usr/bin/env python3
"""Throughput of the batch-invariant selected-token logp path on one MI355X.

Default workload (one "step" = the whole hot path over one batch):
  logits bf16 [8192, 151936] ~ N(0, 3) (Qwen3-8B vocabulary), 10% of rows
  ignored, upstream gradient g ~ N(0, 1) fp32, tile width 4096;
  step = logp_fwd (logp + lse) followed by logp_bwd (dlogits bf16 [N, V]).

Inputs are generated on the device before timing (synthetic, seeded).  Prints
one JSON line.  `value` is rows/s over the timed steps; the roofline object
prices the dominant kernel's algorithmic bytes against the MI355X HBM peak and
against the read and copy rates measured in the same run.  After the headline
timing the default run also times, on their own inputs: the N = 4096 forward
workload, the fused LM head (forward with and without a prepared weight,
backward) at N = H = 4096, V = 151936 and its decode-sized forward (N = 1 and
64) ("secondary"); and the float64 CPU
oracle on the host's cores over the whole headline batch, a forward-only pass
over the N = 4096 forward batch, and one core on 256 rows ("cpu_baseline").
Every input buffer is fingerprinted with SHA-256 ("inputs_sha256").

    python bench.py [--gpus 1] [--steps 20] [--warmup 5]
                    [--workload fwd_bwd|fwd|linear|linear_prepared|linear_bwd|...]
"""

import argparse
import hashlib
import re
import json
import os
import statistics
import sys
import time

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor figure
ROOT = os.path.dirname(os.path.abspath(__file__))
PROFILES = os.path.join(ROOT, "profiles")
MAX_CPU_WORKERS = 16  # the host-core share of one GPU on the benchmark boxes
ORACLE_CHUNK_ROWS = 16
KERNEL_SOURCES = {
    "logp_fwd_fused_kernel": ["invariant_token_log_amd/csrc/logp_kernels.hip",
                              "invariant_token_log_amd/csrc/logp_device.h"],
    "logp_bwd_kernel": ["invariant_token_log_amd/csrc/logp_kernels.hip",
                        "invariant_token_log_amd/csrc/logp_device.h"],
    "linear_stats_dma": ["invariant_token_log_amd/csrc/linear_logp.hip",
                         "invariant_token_log_amd/csrc/mfma_gemm.h",
                         "invariant_token_log_amd/csrc/logp_device.h"],
    "linear_dz_saved_kernel": ["invariant_token_log_amd/csrc/linear_bwd.hip",
                               "invariant_token_log_amd/csrc/mfma_gemm.h",
                               "invariant_token_log_amd/csrc/logp_device.h"],
}
# The fused backward at N = H = 4096, V = 151936 with 204 rows ignored and the
# default vocabulary chunk (32768 columns: 5 chunks over Vp = 152064).
LINEAR_BWD_CHUNKS = 5


def _code_only(text):
    """Source text without comments, trailing blanks and empty lines, so that
    a comment edit does not retire counters taken on the same code."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", line).rstrip() for line in text.splitlines())
    return "\n".join(line for line in lines if line)


def kernel_source_hash(kernel):
    """SHA-256 (first 16 hex digits) of the code of a kernel's sources."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
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


def measured_valu(kernel, workload):
    """VALU-busy percent of a streaming kernel from the committed rocprofv3
    counter summary (profiles/valu_logp_fwd_bwd_<workload>.txt), or None when
    absent or when the kernel source changed since the counters were taken."""
    path = os.path.join(PROFILES, f"valu_logp_fwd_bwd_{workload}.txt")
    if not os.path.exists(path):
        return None
    src, busy = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("source_sha256_16="):
                src = line.strip().split("=", 1)[1]
            elif line.startswith(kernel + ":"):
                for item in line.split():
                    if item.startswith("VALUBusy_pct="):
                        busy = float(item.split("=", 1)[1])
    if src != kernel_source_hash(kernel):
        return None
    return busy


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ---------------------------------------------------------------------------
# CPU oracle baseline.  The worker pool is forked at start-up, before torch
# is imported, so the workers never hold any GPU state; they import numpy and
# the oracle only.  Inputs reach them as raw bf16 bits in a file under
# /dev/shm (a host copy of the device buffer), which they widen to float32
# exactly, as the oracle's callers do.
# ---------------------------------------------------------------------------

def _worker_init():
    # one thread per worker process: the pool supplies the parallelism
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[k] = "1"
    # keep freed blocks of the oracle's per-chunk arrays (about 20 MB each) in
    # the heap instead of returning them to the kernel, so that chunk after
    # chunk reuses memory rather than faulting fresh pages in
    try:
        import ctypes

        libc = ctypes.CDLL("libc.so.6")
        libc.mallopt(-3, 32 << 20)  # M_MMAP_THRESHOLD: heap up to 32 MiB blocks
        libc.mallopt(-1, 1 << 30)   # M_TRIM_THRESHOLD
    except (OSError, AttributeError):
        pass


def _oracle_chunk(task):
    """Worker: the float64 oracle on rows [r0, r1) of a [n, v] bf16 file.
    Returns (rows, seconds) with the widening and the oracle timed."""
    kind, path, n, v, r0, r1, t, g = task
    import numpy as np

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle

    raw = np.memmap(path, dtype=np.uint16, mode="r", shape=(n, v))
    t0 = time.perf_counter()
    x = (raw[r0:r1].astype(np.uint32) << 16).view(np.float32)
    _, lse = oracle.logp_fwd(x, t)
    if kind == "fwd_bwd":
        d = oracle.logp_bwd(x, t, g, lse=lse)
        del d
    dt = time.perf_counter() - t0
    del raw, x
    return r1 - r0, dt


def _warm(_):
    """Worker: import numpy and the oracle and touch a chunk's worth of
    memory, so that timed chunks find a warm process."""
    import numpy as np

    if ROOT not in sys.path:
        sys.path.insert(0, ROOT)
    import oracle

    x = np.zeros((ORACLE_CHUNK_ROWS, 151936), dtype=np.float32)
    t = np.zeros(ORACLE_CHUNK_ROWS, dtype=np.int64)
    _, lse = oracle.logp_fwd(x, t)
    oracle.logp_bwd(x, t, np.ones(ORACLE_CHUNK_ROWS, dtype=np.float32), lse=lse)
    return os.getpid()


def make_pool():
    import multiprocessing as mp

    cores = min(MAX_CPU_WORKERS, len(os.sched_getaffinity(0)))
    return mp.get_context("fork").Pool(cores, initializer=_worker_init), cores


def host_bits(torch, x, path):
    """Host copy of a 2-D bf16 device tensor as raw 16-bit words in a file
    under /dev/shm (returned as a writable memmap)."""
    import numpy as np

    mm = np.memmap(path, dtype=np.uint16, mode="w+", shape=tuple(x.shape))
    torch.from_numpy(mm.view(np.int16)).copy_(x.view(torch.int16))
    mm.flush()
    return mm


def sha256_of(buf):
    """SHA-256 of a host buffer (numpy array or memmap) as stored."""
    import numpy as np

    h = hashlib.sha256()
    a = np.ascontiguousarray(buf)
    mv = memoryview(a).cast("B")
    step = 1 << 28
    for i in range(0, len(mv), step):
        h.update(mv[i:i + step])
    return h.hexdigest()


def oracle_rate(pool, cores, kind, path, n, v, t, g, rows=None, single=False):
    """rows/s of the oracle over the first `rows` rows (all by default), on
    the pool's cores (contiguous row chunks) or on one worker."""
    import numpy as np

    rows = n if rows is None else rows
    tasks = []
    for r0 in range(0, rows, ORACLE_CHUNK_ROWS):
        r1 = min(rows, r0 + ORACLE_CHUNK_ROWS)
        tasks.append((kind, path, n, v, r0, r1, np.ascontiguousarray(t[r0:r1]),
                      None if g is None else np.ascontiguousarray(g[r0:r1])))
    t0 = time.perf_counter()
    if single:
        done = [pool.apply(_oracle_chunk, (task,)) for task in tasks]
    else:
        done = list(pool.imap_unordered(_oracle_chunk, tasks))
    wall = time.perf_counter() - t0
    cpu_s = sum(d[1] for d in done)
    return rows / wall, wall, cpu_s


# ---------------------------------------------------------------------------
# GPU timing helpers
# ---------------------------------------------------------------------------

def ramp(torch, fn, seconds):
    """Run fn() untimed until `seconds` of wall time have passed, so that the
    GPU clocks have left their idle state before any warmup or timed step."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_launches(torch, fn, steps):
    """Device time of each of `steps` calls of fn(), from events on the
    current stream (the stream every library call launches on)."""
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    for a, b in ev:
        a.record()
        fn()
        b.record()
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def stats_ms(ms):
    return {"ms": round(sum(ms) / len(ms), 4), "median_ms": round(statistics.median(ms), 4),
            "min_ms": round(min(ms), 4)}


def timed(torch, fn, args):
    """Ramp, warmup, then per-launch timing: the mean / median / min dict."""
    ramp(torch, fn, args.ramp_s)
    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
    return stats_ms(time_launches(torch, fn, args.steps))


def probe_lib():
    """The bandwidth probes built next to the library (libitl_ceiling.so)."""
    import ctypes

    from invariant_token_log_amd.build import PROBE_PATH

    if not os.path.exists(PROBE_PATH):
        raise RuntimeError(f"{PROBE_PATH} is missing: build with "
                           "`python -m invariant_token_log_amd.build`")
    lib = ctypes.CDLL(PROBE_PATH)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.itl_probe_read.argtypes = [vp, sz, vp, vp]
    lib.itl_probe_read.restype = ctypes.c_int
    lib.itl_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.itl_probe_copy.restype = ctypes.c_int
    return lib


def measured_ceilings(torch, src, dst, args):
    """Read and copy rates (GB/s) of the probe kernels over the benchmark's
    own buffers: a read of src, a copy src -> dst (same size)."""
    lib = probe_lib()
    nbytes = src.numel() * src.element_size()
    sink = torch.zeros(1, dtype=torch.int32, device=src.device)
    stream = torch.cuda.current_stream().cuda_stream

    def rd():
        if lib.itl_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), stream):
            raise RuntimeError("itl_probe_read failed")

    def cp():
        if lib.itl_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream):
            raise RuntimeError("itl_probe_copy failed")

    r = timed(torch, rd, args)
    c = timed(torch, cp, args)
    return {"read_gbps": round(nbytes / (r["median_ms"] * 1e-3) / 1e9, 1),
            "copy_gbps": round(2 * nbytes / (c["median_ms"] * 1e-3) / 1e9, 1),
            "bytes_read": nbytes, "bytes_copied": nbytes,
            "pattern": "one 16-byte chunk per thread in address order, non-temporal loads "
                       "(and stores), medians over the timed launches"}


# ---------------------------------------------------------------------------
# Workloads
# ---------------------------------------------------------------------------

QWEN_N_FB, QWEN_N_F = 8192, 4096


def _kernel_entry(st, nbytes):
    d = dict(st)
    d["bytes"] = nbytes
    d["gbps"] = round(nbytes / (st["ms"] * 1e-3) / 1e9, 1)
    d["hbm_frac"] = round(d["gbps"] / HBM_PEAK_GBS, 4)
    d["gbps_median"] = round(nbytes / (st["median_ms"] * 1e-3) / 1e9, 1)
    return d


def bench_fwd_bwd(args, torch, itl, synth, ctx):
    n, v, w = QWEN_N_FB, synth.QWEN3_VOCAB, 4096
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
    # per-kernel figures over a second timed pass of the same launches
    fwd_st = stats_ms(time_launches(torch, fwd, args.steps))
    bwd_st = stats_ms(time_launches(torch, bwd, args.steps))

    fwd_bytes = n_active * v * 2 + n * (8 + 4 + 4)
    bwd_bytes = n_active * v * 2 + n * v * 2 + n * (8 + 4 + 4)
    step_bytes = fwd_bytes + bwd_bytes
    kernels = {"logp_fwd_fused_kernel": _kernel_entry(fwd_st, fwd_bytes),
               "logp_bwd_kernel": _kernel_entry(bwd_st, bwd_bytes)}
    ceil = measured_ceilings(torch, x, dl, args)
    dom = max(kernels, key=lambda k: kernels[k]["ms"])
    kd = kernels[dom]
    traffic = measured_traffic(dom, "qwen3_8192x151936")
    roofline = {"bound": "hbm", "achieved": kd["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(kd["gbps"] / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": dom,
                "valu_busy_pct": {k: measured_valu(k, "qwen3_8192x151936") for k in kernels},
                "algorithmic_bytes_per_launch": kd["bytes"],
                "measured_ceiling": dict(ceil, **{
                    "bwd_frac_of_copy": round(kernels["logp_bwd_kernel"]["gbps_median"]
                                              / ceil["copy_gbps"], 4),
                    "fwd_frac_of_read": round(kernels["logp_fwd_fused_kernel"]["gbps_median"]
                                              / ceil["read_gbps"], 4)})}
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
        "kernels": kernels,
        "roofline": roofline,
        "wall_s_timed": round(wall, 4),
    }
    del logp, lse, dl
    tn, gn = t.cpu().numpy(), g.cpu().numpy()
    path = ctx.shm_path("fwd_bwd_logits")
    xb = host_bits(torch, x, path)
    ctx.inputs["fwd_bwd"] = {"logits_bf16": sha256_of(xb), "targets_i64": sha256_of(tn),
                             "grad_f32": sha256_of(gn)}
    del x, c
    torch.cuda.empty_cache()
    ctx.cpu_jobs.append(("fwd_bwd", path, n, v, tn, gn))
    return out


def secondary_fwd(args, torch, itl, synth, ctx):
    """The N = 4096 forward workload (1% spike rows, 5% ignored)."""
    n, v, w = QWEN_N_F, synth.QWEN3_VOCAB, 4096
    dev = torch.device("cuda", 0)
    c = synth.qwen3_fwd(n=n, v=v, device=dev)
    x, t = c["logits"], c["targets"]
    n_active = int((t != -100).sum().item())
    logp = torch.empty(n, dtype=torch.float32, device=dev)
    lse = torch.empty(n, dtype=torch.float32, device=dev)

    def fwd():
        itl.logp_fwd(x, t, -100, w, logp_out=logp, lse_out=lse)

    st = timed(torch, fwd, args)
    byts = n_active * v * 2 + n * 16
    res = dict(_kernel_entry(st, byts), workload="qwen3_8b_vocab_logp_fwd", n=n, v=v,
               tile_width=w, ignored_rows=n - n_active,
               rows_per_s=round(n / (st["ms"] * 1e-3), 1),
               traffic=measured_traffic("logp_fwd_fused_kernel", "qwen3_4096x151936"))
    tn = t.cpu().numpy()
    path = ctx.shm_path("fwd_logits")
    xb = host_bits(torch, x, path)
    ctx.inputs["fwd"] = {"logits_bf16": sha256_of(xb), "targets_i64": sha256_of(tn)}
    del x, c, logp, lse
    torch.cuda.empty_cache()
    ctx.cpu_jobs.append(("fwd", path, n, v, tn, None))
    return res


def _linear_case(torch, synth, ignore_frac=0.0, n=4096):
    h, v = synth.QWEN3_HIDDEN, synth.QWEN3_VOCAB
    dev = torch.device("cuda", 0)
    c = synth.qwen3_linear(n=n, h=h, v=v, device=dev, ignore_frac=ignore_frac)
    return n, h, v, c["hidden"], c["weight"], c["targets"]


def _mfma_entry(st, flops):
    d = dict(st)
    d["tflops"] = round(flops / (st["ms"] * 1e-3) / 1e12, 2)
    d["mfma_frac"] = round(d["tflops"] / BF16_MFMA_PEAK_TFLOPS, 4)
    d["tflops_median"] = round(flops / (st["median_ms"] * 1e-3) / 1e12, 2)
    return d


def linear_fwd_stats(args, torch, itl, synth, prepared, ctx=None):
    n, h, v, hid, wt, t = _linear_case(torch, synth)
    dev = hid.device
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

    st = timed(torch, run, args)
    res = _mfma_entry(st, 2.0 * n * h * v)
    if ctx is not None and "linear" not in ctx.inputs:
        ctx.inputs["linear"] = {"hidden_bf16": sha256_of(hid.view(torch.int16).cpu().numpy()),
                                "weight_bf16": sha256_of(wt.view(torch.int16).cpu().numpy()),
                                "targets_i64": sha256_of(t.cpu().numpy())}
    return res, (hid, wt, t)


def linear_bwd_stats(args, torch, itl, synth, saved=False, prepared=False, vocab_chunk=0):
    n, h, v, hid, wt, t = _linear_case(torch, synth, ignore_frac=0.05)
    dev = hid.device
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
    ws = torch.empty(itl.linear_logp_bwd_workspace_bytes(n, h, v, prepared=prepared,
                                                         saved_logits=saved,
                                                         vocab_chunk=vocab_chunk),
                     dtype=torch.uint8, device=dev)

    def run():
        itl.linear_logp_bwd(hid, wt, t, lse, g, dhidden_out=dh, dweight_out=dw, workspace=ws,
                            saved_logits=z, prepared_weight=wtp, vocab_chunk=vocab_chunk)

    st = timed(torch, run, args)
    # z recomputed (not when saved), dh = dz W, dW = dz^T h
    flops = (2 if saved else 3) * 2.0 * n * h * v
    res = _mfma_entry(st, flops)
    res["workspace_bytes"] = ws.numel()
    res["vocab_chunk"] = vocab_chunk or "default"
    return res, n * v * 4 if saved else 0


def standalone_fwd(args, torch, itl, synth, ctx):
    r = secondary_fwd(args, torch, itl, synth, ctx)
    gbps = r["gbps"]
    return {
        "metric": "rows/s and achieved HBM GB/s (% of peak), N=4096 V=151936 bf16 fwd",
        "value": r["rows_per_s"], "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": r["workload"], "n": r["n"], "v": r["v"],
                   "tile_width": r["tile_width"], "ignored_rows": r["ignored_rows"]},
        "gb_per_s": gbps, "hbm_frac": round(gbps / HBM_PEAK_GBS, 4),
        "kernels": {"logp_fwd_fused_kernel": {k: r[k] for k in
                                              ("ms", "median_ms", "min_ms", "bytes", "gbps")}},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbps / HBM_PEAK_GBS, 4), "traffic": r["traffic"],
                     "kernel": "logp_fwd_fused_kernel"},
    }


def linear_decode(args, torch, itl, synth, prepared):
    """Decode-sized fused LM head (N = 1 and 64 rows, the narrow tile): the
    weight streams from HBM once per call, so the rate is weight bytes / time
    against the HBM peak."""
    out = {}
    for n in (1, 64):
        _, h, v, hid, wt, t = _linear_case(torch, synth, n=n)
        logp = torch.empty(n, dtype=torch.float32, device=hid.device)
        lse = torch.empty(n, dtype=torch.float32, device=hid.device)
        ws = torch.empty(max(itl.lib().linear_logp_fwd_workspace_bytes(n, h, v, 256), 1),
                         dtype=torch.uint8, device=hid.device)
        pw = itl.prepare_weight(wt) if prepared else None

        def run():
            itl.linear_logp_fwd(hid, wt, t, -100, 256, logp_out=logp, lse_out=lse, workspace=ws,
                                prepared_weight=pw)

        st = timed(torch, run, args)
        d = _kernel_entry(st, v * h * 2 + n * h * 2 + n * 16)
        d["rows"] = n
        out[f"n{n}"] = d
        del hid, wt, t, pw, ws
        torch.cuda.empty_cache()
    return out


def standalone_linear_decode(args, torch, itl, synth, prepared):
    r = linear_decode(args, torch, itl, synth, prepared)
    d = r["n64"]
    return {
        "metric": "weight-stream GB/s (% of HBM peak), fused LM-head+logp decode N=64 H=4096 "
                  "V=151936 bf16" + (", prepared weight" if prepared else ""),
        "value": d["gbps"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": d["ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "qwen3_8b_lm_head_linear_logp_decode"
                               + ("_prepared" if prepared else ""),
                   "n": 64, "h": 4096, "v": synth.QWEN3_VOCAB, "tile_width": 256},
        "sizes": r,
        "roofline": {"bound": "hbm", "achieved": d["gbps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": d["hbm_frac"], "traffic": None,
                     "kernel": "linear_logp_fwd (the 64-row tile and the merge)"},
    }


def standalone_linear(args, torch, itl, synth, ctx, prepared):
    r, _ = linear_fwd_stats(args, torch, itl, synth, prepared, ctx)
    n = 4096
    out = {
        "metric": "rows/s and MFMA TFLOP/s (% of peak), fused LM-head+logp N=4096 H=4096 "
                  "V=151936 bf16" + (", prepared weight" if prepared else ""),
        "value": round(n / (r["ms"] * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_lm_head_linear_logp" + ("_prepared" if prepared else ""),
                   "n": n, "h": 4096, "v": synth.QWEN3_VOCAB, "tile_width": 256},
        "tflops": r["tflops"], "median_ms": r["median_ms"], "min_ms": r["min_ms"],
        "roofline": {"bound": "mfma", "achieved": r["tflops"],
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": r["mfma_frac"],
                     "traffic": None if prepared else measured_traffic(
                         "linear_stats_dma", "qwen3_4096x4096x151936"),
                     "kernel": "linear_logp_fwd (all launches: blocking the hidden rows, "
                               "linear_stats_dma, the merge; linear_stats_dma is 98% of it)"},
    }
    return out


def standalone_linear_bwd(args, torch, itl, synth, ctx, saved=False, prepared=False):
    r, extra = linear_bwd_stats(args, torch, itl, synth, saved, prepared, args.vocab_chunk)
    n = 4096
    return {
        "metric": "rows/s and MFMA TFLOP/s (% of peak), fused LM-head+logp backward N=4096 "
                  "H=4096 V=151936 bf16" + (", logits saved by the forward (fp32)" if saved
                                            else ", logits recomputed")
                  + (", prepared weight" if prepared else ""),
        "value": round(n / (r["ms"] * 1e-3), 1), "unit": "rows/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": r["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "qwen3_8b_lm_head_linear_logp_bwd" + ("_saved" if saved else "")
                   + ("_prepared" if prepared else ""),
                   "n": n, "h": 4096, "v": synth.QWEN3_VOCAB, "tile_width": 256,
                   "outputs": "dh, dW fp32"},
        "tflops": r["tflops"], "median_ms": r["median_ms"], "min_ms": r["min_ms"],
        "roofline": {"bound": "mfma", "achieved": r["tflops"],
                     "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": r["mfma_frac"], "traffic": None,
                     "kernel": "linear_logp_bwd (all launches: the hidden rows' re-layout and "
                               "transpose, dz, the two products)"},
        "extra_memory_bytes": extra, "workspace_bytes": r["workspace_bytes"],
        "vocab_chunk": r["vocab_chunk"],
    }


def default_secondary(args, torch, itl, synth, ctx):
    """Measurements after the headline's timed region: the N = 4096 forward
    workload, the fused LM head at N = H = 4096, V = 151936 (forward, with a
    prepared weight, backward with the default and a whole-vocabulary chunk)
    and at decode sizes (N = 1 and 64)."""
    sec = {"fwd_qwen3_4096x151936": secondary_fwd(args, torch, itl, synth, ctx)}
    r, _ = linear_fwd_stats(args, torch, itl, synth, False, ctx)
    sec["linear_fwd_qwen3_4096x4096x151936"] = r
    torch.cuda.empty_cache()
    r, _ = linear_fwd_stats(args, torch, itl, synth, True, None)
    sec["linear_fwd_prepared_qwen3_4096x4096x151936"] = r
    torch.cuda.empty_cache()
    r, _ = linear_bwd_stats(args, torch, itl, synth)
    sec["linear_bwd_qwen3_4096x4096x151936"] = r
    torch.cuda.empty_cache()
    # the memory trade-off: the whole vocabulary in one chunk (largest
    # workspace, fewest launches), the same bits
    r, _ = linear_bwd_stats(args, torch, itl, synth, vocab_chunk=synth.QWEN3_VOCAB)
    sec["linear_bwd_one_chunk_qwen3_4096x4096x151936"] = r
    torch.cuda.empty_cache()
    # decode-sized fused forward (the narrow tile): weight-stream GB/s
    sec["linear_decode_qwen3_4096x151936"] = linear_decode(args, torch, itl, synth, False)
    sec["linear_decode_prepared_qwen3_4096x151936"] = linear_decode(args, torch, itl, synth, True)
    return sec


class Ctx:
    """Per-run state: input fingerprints, pending CPU jobs, /dev/shm files."""

    def __init__(self):
        self.inputs = {}
        self.cpu_jobs = []
        self.files = []

    def shm_path(self, name):
        base = "/dev/shm" if os.path.isdir("/dev/shm") else "/tmp"
        p = os.path.join(base, f"itl_bench_{os.getpid()}_{name}.u16")
        self.files.append(p)
        return p

    def cleanup(self):
        for p in self.files:
            try:
                os.remove(p)
            except OSError:
                pass


def cpu_baselines(pool, cores, ctx):
    """The float64 oracle over the recorded host copies: the first job on
    the pool's cores (the whole batch), the others forward-only on the pool,
    and one core on 256 rows of the first job."""
    if not ctx.cpu_jobs:
        return None
    pool.map(_warm, range(4 * cores), chunksize=1)
    kind, path, n, v, t, g = ctx.cpu_jobs[0]
    rate, wall, cpu_s = oracle_rate(pool, cores, kind, path, n, v, t, g)
    one, one_wall, _ = oracle_rate(pool, cores, kind, path, n, v, t, g, rows=256, single=True)
    what = "forward+backward" if kind == "fwd_bwd" else "forward"
    out = {"value": round(rate, 1), "unit": "rows/s", "cores": cores, "kind": "oracle",
           "sample": f"all {n} rows of the same [{n}, {v}] bf16 batch, float64 numpy {what} "
                     f"(bf16 widened to float32 in the workers) in {ORACLE_CHUNK_ROWS}-row "
                     f"chunks over a pool of {cores} processes, {wall:.2f} s wall, "
                     f"{cpu_s:.1f} s of worker time; device-to-host copy not timed",
           "cpu": cpu_model(),
           "single_core": {"value": round(one, 1), "unit": "rows/s", "cores": 1,
                           "sample": f"first 256 rows of the same batch on one worker, "
                                     f"{one_wall:.2f} s"}}
    for kind2, path2, n2, v2, t2, _ in ctx.cpu_jobs[1:]:
        r2, w2, c2 = oracle_rate(pool, cores, "fwd", path2, n2, v2, t2, None)
        out["fwd_only_qwen3_4096x151936" if n2 == QWEN_N_F else f"fwd_only_{n2}x{v2}"] = {
            "value": round(r2, 1), "unit": "rows/s", "cores": cores,
            "sample": f"all {n2} rows of the [{n2}, {v2}] bf16 forward batch, float64 numpy "
                      f"forward, {w2:.2f} s wall, {c2:.1f} s of worker time"}
    return out


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
    if workload == "qwen3_4096x4096x151936_bwd_saved":
        # per launch, averaged over one backward's launches: the saved-logits
        # dz kernel reads the active rows' fp32 logits and writes dz_c (bf16,
        # padded to Vp columns) once per chunk
        n, v, vp = 4096, 151936, 152064
        act = n - int(0.05 * n)
        if kernel == "linear_dz_saved_kernel":
            return (act * v * 4 + n * vp * 2) // LINEAR_BWD_CHUNKS
    raise ValueError((workload, kernel))


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


def cpu_baseline_linear(hid, wt, t, rows):
    import oracle

    h = hid[:rows].float().cpu().numpy()
    w = wt.float().cpu().numpy()
    tt = t[:rows].cpu().numpy()
    t0 = time.perf_counter()
    oracle.linear_logp_fwd(h, w, tt)
    dt = time.perf_counter() - t0
    threads = os.environ.get("OMP_NUM_THREADS") or str(len(os.sched_getaffinity(0)))
    return {"value": round(rows / dt, 2), "unit": "rows/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"first {rows} rows, float64 numpy h @ W^T then logp, {dt:.1f} s "
                      "(BLAS threads = cores)",
            "cpu": cpu_model()}


def run(args, ctx, pool, cores):
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
    wl = args.workload
    if wl == "fwd_bwd":
        out = bench_fwd_bwd(args, torch, itl, synth, ctx)
        if not args.no_secondary:
            out["secondary"] = default_secondary(args, torch, itl, synth, ctx)
    elif wl == "fwd":
        out = standalone_fwd(args, torch, itl, synth, ctx)
    elif wl in ("linear", "linear_prepared"):
        out = standalone_linear(args, torch, itl, synth, ctx, wl == "linear_prepared")
    elif wl in ("linear_decode", "linear_decode_prepared"):
        out = standalone_linear_decode(args, torch, itl, synth, wl == "linear_decode_prepared")
    else:
        out = standalone_linear_bwd(args, torch, itl, synth, ctx,
                                    saved=wl == "linear_bwd_saved",
                                    prepared=wl == "linear_bwd_prepared")
    if pool is not None:
        out["cpu_baseline"] = cpu_baselines(pool, cores, ctx)
        if wl == "fwd_bwd" and not args.no_secondary and out["cpu_baseline"]:
            # the fused LM head's oracle (h W^T in float64, then logp) on a
            # 64-row sample of the N = H = 4096 workload
            _, h, v, hid, wt, t = _linear_case(torch, synth)
            out["cpu_baseline"]["linear_fwd_qwen3_4096x4096x151936"] = cpu_baseline_linear(
                hid, wt, t, 64)
            del hid, wt, t
            torch.cuda.empty_cache()
    elif wl == "linear" and not args.no_cpu_baseline:
        _, h, v, hid, wt, t = _linear_case(torch, synth)
        out["cpu_baseline"] = cpu_baseline_linear(hid, wt, t, args.cpu_rows or 512)
    if out.get("cpu_baseline") and out["cpu_baseline"]["value"]:
        out["gpu_over_cpu"] = round(out["value"] / out["cpu_baseline"]["value"], 1)
    if ctx.inputs:
        out["inputs_sha256"] = ctx.inputs
    out["contract_id"] = itl.contract_id()
    out["device"] = torch.cuda.get_device_name(0)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--ramp-s", type=float, default=0.5,
                    help="untimed seconds of launches before the warmup (GPU clock ramp)")
    ap.add_argument("--workload", default="fwd_bwd",
                    choices=["fwd_bwd", "fwd", "linear", "linear_bwd", "linear_bwd_saved",
                             "linear_bwd_prepared", "linear_prepared", "linear_decode",
                             "linear_decode_prepared"])
    ap.add_argument("--cpu-rows", type=int, default=0,
                    help="rows for the fused LM head's CPU oracle baseline (0 = 512)")
    ap.add_argument("--vocab-chunk", type=int, default=0,
                    help="fused backward workloads: vocabulary columns per pass (0 = default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true",
                    help="default workload: skip the measurements after the headline")
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
                  "linear": ("qwen3_4096x4096x151936", ["linear_stats_dma"]),
                  "linear_bwd_saved": ("qwen3_4096x4096x151936_bwd_saved",
                                       ["linear_dz_saved_kernel"]),
                  }[args.workload]
        for p in summarize_traffic(*args.summarize_traffic, wl, ks, *args.pmc_commands):
            print(p)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(rows are independent, so data-parallel scaling needs no exchange); "
              f"--gpus {args.gpus} is not supported.", file=sys.stderr)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        sys.exit("--steps must be >= 1 and --warmup >= 0")
    pool, cores = None, 0
    if not args.no_cpu_baseline and args.workload in ("fwd_bwd", "fwd"):
        pool, cores = make_pool()  # before torch is imported: no GPU state in the workers
    ctx = Ctx()
    try:
        out = run(args, ctx, pool, cores)
    finally:
        ctx.cleanup()
        if pool is not None:
            pool.terminate()
            pool.join()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
