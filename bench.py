"""Benchmark: Swin3D shifted-window attention on one MI355X.

One step = one call of the library over the whole stage-1 latent grid of a
0.25-degree encoder (B=1, D=4, H=180, W=360: 259,200 tokens, 8 heads,
head_dim 64, window (2, 6, 12), shift (1, 3, 6), bf16 I/O, -100 bias): every
step of the path (index map, gather, masked softmax attention, scatter)
runs inside that call. Inputs are seeded synthetic tensors already resident
in device memory when the timed region starts.

Prints one JSON line with the throughput (tokens/s), the roofline position
of the kernel and the fp64 CPU oracle timed on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "window-attention tokens/s at 0.25° stage-1 shape; % of HBM/MFMA roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_MFMA_PEAK_TFLOPS = 2516.6  # MI355X dense bf16
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 (matrix)
KERNEL_SRC = os.path.join(ROOT, "swin3d_window_attention_amd", "csrc", "wattn_bf16.hip")
# every input of the headline launch: the kernel, the host code that builds its
# plan and arguments, the public header, and the build script (compiler flags)
LAUNCH_INPUTS = [KERNEL_SRC] + [os.path.join(ROOT, *f) for f in (
    ("swin3d_window_attention_amd", "csrc", "fastdiv.h"),
    ("swin3d_window_attention_amd", "csrc", "plan.h"),
    ("swin3d_window_attention_amd", "csrc", "api.cpp"),
    ("include", "swin3d_wattn.h"),
    ("swin3d_window_attention_amd", "build.py"))]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_wattn_bf16_stage1.json")
# the shapes the pages measure, besides the headline: a tiny FP32 check, the
# stage-2 shape without and with shift, the padded stage-3 shape and the
# high-resolution large-logit stress grid
CONFIG_WORKLOADS = ("tiny_f32", "stage2_s0", "stage2", "stage3_pad", "stress_hres")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_work(wl):
    """Bytes: read Q, K, V and write O once per real token. FLOPs: 4 n^2 dh per window-head, n the
    real (not padding) slots of the window: the dense products among its real tokens, masked or
    not (N^2 where the grid needs no padding). The real slots of a window are the product over the
    axes of its real positions along each, so the sum of n^2 over windows is the product over the
    axes of the sums of squares."""
    elt = 2 if wl.dtype == "bf16" else 4
    nbytes = 4 * wl.tokens * wl.heads * wl.head_dim * elt
    n = 1
    sq = 1
    for x, w, s in zip((wl.D, wl.H, wl.W), wl.window, wl.shift):
        nw = -(-x // w)
        P = nw * w
        n *= nw
        sq *= sum(sum(1 for o in range(w) if (k * w + o + s) % P < x) ** 2 for k in range(nw))
    n *= wl.B
    flops = 4 * sq * wl.B * wl.head_dim * wl.heads
    return nbytes, flops, n


def kernel_digest() -> str:
    """SHA-256 over every input of the headline launch (file names and contents, in order)."""
    h = hashlib.sha256()
    for path in LAUNCH_INPUTS:
        h.update(os.path.relpath(path, ROOT).encode() + b"\0")
        with open(path, "rb") as f:
            h.update(f.read())
        h.update(b"\0")
    return h.hexdigest()


def measured_traffic():
    """HBM bytes per launch from the committed PMC summary, if the kernel is unchanged since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("launch_sha256") != kernel_digest():
        return None
    return t.get("traffic_bytes_per_launch")


def _cpu_time():
    r = resource.getrusage(resource.RUSAGE_SELF)
    return r.ru_utime + r.ru_stime


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _pool_run(task, budget_s: float):
    """Run task(worker, i) on a pool of threads, one per core this process may use, each
    worker repeating its tasks until budget_s of wall time has passed since the start (a
    task in flight at the deadline is finished and counted). BLAS runs one thread per
    worker. Returns (tasks done per worker, wall seconds, CPU seconds, workers)."""
    from concurrent.futures import ThreadPoolExecutor

    n = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(limits=1)
    except ImportError:  # pragma: no cover - BLAS then keeps its own threading
        limit = None
    try:
        c0, t0 = _cpu_time(), time.perf_counter()

        def worker(w):
            done = 0
            while True:
                task(w, done)
                done += 1
                if time.perf_counter() - t0 >= budget_s:
                    return done

        with ThreadPoolExecutor(max_workers=n) as ex:
            counts = list(ex.map(worker, range(n)))
        wall, cpu = time.perf_counter() - t0, _cpu_time() - c0
    finally:
        if limit is not None:
            limit.restore_original_limits()
    return counts, wall, cpu, n


def _baseline_record(value, sample, wall, cpu, workers):
    return {
        "value": value,
        "unit": "tokens/s",
        "cores": max(1, int(round(cpu / wall))),
        "kind": "oracle",
        "sample": sample,
        "cpu_seconds": round(cpu, 2),
        "workers": workers,
        "cores_available": len(os.sched_getaffinity(0)),
        "cpu_model": cpu_model(),
    }


def cpu_baseline(wl, budget_s: float, bias: float = -100.0):
    """The fp64 oracle, as it stands, timed on a bounded sample of the same workload for about
    budget_s of wall time, on a thread pool with one worker per available core (BLAS at one
    thread per worker). Where the grid is no larger than the stage-1 one, each task is one call
    of the whole-grid oracle on one head (worker w's task i takes head (w + i * workers) mod
    heads); otherwise each task is a seeded batch of 16 random windows with every head, read
    from the same inputs."""
    import numpy as np

    import datagen
    import oracle

    grid = (wl.D, wl.H, wl.W)
    nwin = oracle.window_count(wl.B, grid, wl.window)
    if wl.tokens * wl.heads * wl.head_dim <= 259200 * 8 * 64:
        q, k, v = (datagen.full_f64(wl, t) for t in ("q", "k", "v"))
        workers = len(os.sched_getaffinity(0))

        def task(w, i):
            h = (w + i * workers) % wl.heads
            sl = (Ellipsis, slice(h, h + 1), slice(None))
            oracle.swin3d_window_attention(q[sl], k[sl], v[sl], wl.window, wl.shift, wl.scale, bias)

        counts, wall, cpu, n = _pool_run(task, budget_s)
        del q, k, v
        done = sum(counts)
        frac = done / wl.heads
        sample = (f"fp64 numpy oracle on the whole {wl.name} grid, one head per call, {done} head "
                  f"pass{'es' if done > 1 else ''} ({done * nwin} window-heads = {frac:.2f} x the workload) "
                  f"on {n} threads in {wall:.1f} s")
    else:
        host = {t: datagen.full_io(wl, t) for t in ("q", "k", "v")}

        def fetch(t, b, c):
            a = host[t][b, c[:, 0], c[:, 1], c[:, 2]]
            return (datagen.bf16_bits_to_f32(a) if wl.dtype == "bf16" else a).astype(np.float64)

        nw = [oracle.padded_extent(x, w) // w for x, w in zip(grid, wl.window)]

        def task(w, i):
            rng = np.random.default_rng([12345, w, i])
            wins = [(int(rng.integers(wl.B)),) + tuple(int(rng.integers(m)) for m in nw) for _ in range(16)]
            oracle.windows_attention(fetch, wl.B, grid, wl.heads, wl.head_dim, wl.window, wl.shift, wl.scale,
                                     bias, wins)

        counts, wall, cpu, n = _pool_run(task, budget_s)
        del host
        done = 16 * sum(counts)
        frac = done / nwin
        sample = (f"fp64 numpy oracle on {done} seeded random windows of the {wl.name} grid, all {wl.heads} "
                  f"heads ({frac:.4f} x the workload) on {n} threads in {wall:.1f} s")
    return _baseline_record(wl.tokens * frac / wall, sample, wall, cpu, n)


def cpu_baseline_adaln(wl, a, budget_s: float):
    """The fp64 AdaLN + residual oracle on blocks of 4,096 rows of the same inputs (worker w's
    task i takes block (w + i * workers), cycling over the rows; the block at the end of the rows
    is shorter) on a thread pool with one worker per available core, for about budget_s of wall
    time. Counts the rows actually processed."""
    import numpy as np

    import datagen
    import oracle.adaln as oadaln

    def f64(x, dt):
        return (datagen.bf16_bits_to_f32(x) if dt == "bf16" else x).astype(np.float64)

    step = 4096
    nblocks = -(-wl.rows // step)
    workers = len(os.sched_getaffinity(0))
    rows_done = [0] * workers

    def task(w, i):
        r = ((w + i * workers) % nblocks) * step
        sl = slice(r, min(wl.rows, r + step))
        oadaln.adaln_residual(f64(a["x"][:, sl], wl.x_dtype), f64(a["res"][:, sl], wl.res_dtype),
                              a["gamma"].astype(np.float64), a["beta"].astype(np.float64), wl.eps)
        rows_done[w] += (sl.stop - sl.start) * wl.B

    counts, wall, cpu, n = _pool_run(task, budget_s)
    n_rows = sum(rows_done)
    sample = (f"fp64 numpy oracle on {sum(counts)} blocks of up to {step} rows x {wl.B} batch ({n_rows} rows) "
              f"of the {wl.name} inputs on {n} threads in {wall:.1f} s")
    return _baseline_record(n_rows / wall, sample, wall, cpu, n)


def copy_calibration(nbytes: int, steps: int):
    """A plain device copy of known size, for scaling the HBM byte counters of a profiler."""
    import torch

    n = nbytes // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    print(json.dumps({"copy_bytes_read": n * 2, "copy_bytes_written": n * 2, "steps": steps,
                      "gbs_read_plus_write": 2 * n * 2 / dt / 1e9}), flush=True)


def device_copy_gbs(torch, nbytes: int) -> float:
    """Read + write GB/s of a plain device-to-device copy of nbytes (torch's copy kernel), best of 3
    rounds of 10, with HIP events on the current stream."""
    src = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    best = float("inf")
    for _ in range(3):
        st, en = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st.record()
        for _ in range(10):
            dst.copy_(src)
        en.record()
        torch.cuda.synchronize()
        best = min(best, st.elapsed_time(en) / 10)
    del src, dst
    return 2 * nbytes / (best / 1e3) / 1e9


def write_traffic(prof_dir: str, copy_bytes: int = 536870912):
    """Turn four rocprofv3 --pmc runs into the traffic summary that bench.py reports: FETCH_SIZE
    and WRITE_SIZE (KiB per dispatch) of the stage-1 kernel, each scaled by what the same counter
    reads for a plain device copy of copy_bytes (subfolders fetch, write, copyfetch, copywrite
    of prof_dir, as written by the commands in profiles/wattn_bf16_item_stage1_hbm_traffic.md).
    Host only; records the SHA-256 of the launch inputs (kernel source, plan and argument code,
    header, build flags) the counters were taken on."""
    import csv
    import glob

    def mean_counter(sub, counter, name_part):
        vals = []
        for f in glob.glob(os.path.join(prof_dir, sub, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] == counter and name_part in r["Kernel_Name"]:
                    vals.append(float(r["Counter_Value"]))
        if not vals:
            sys.exit(f"bench.py: no {counter} rows for {name_part!r} under {prof_dir}/{sub}")
        return sum(vals) / len(vals)

    fetch = mean_counter("fetch", "FETCH_SIZE", "wattn_bf16_item")
    write = mean_counter("write", "WRITE_SIZE", "wattn_bf16_item")
    cfetch = mean_counter("copyfetch", "FETCH_SIZE", "copyBuffer")
    cwrite = mean_counter("copywrite", "WRITE_SIZE", "copyBuffer")
    fscale = copy_bytes / 1024 / cfetch
    wscale = copy_bytes / 1024 / cwrite
    import datagen
    nbytes = algorithmic_work(datagen.WORKLOADS["stage1"])[0]
    out = {
        "kernel": "wattn_bf16_item",
        "workload": "stage-1 latent grid B=1 D=4 H=180 W=360, 8 heads, head_dim 64, window (2,6,12), "
                    "shift (1,3,6), bf16",
        "launch_inputs": [os.path.relpath(f, ROOT) for f in LAUNCH_INPUTS],
        "launch_sha256": kernel_digest(),
        "fetch_size_kib_per_dispatch": fetch,
        "write_size_kib_per_dispatch": write,
        "copy_calibration": {"bytes_read": copy_bytes, "bytes_written": copy_bytes, "fetch_size_kib": cfetch,
                             "write_size_kib": cwrite, "fetch_scale": fscale, "write_scale": wscale},
        "read_bytes_per_launch": fetch * 1024 * fscale,
        "write_bytes_per_launch": write * 1024 * wscale,
        "traffic_bytes_per_launch": (fetch * fscale + write * wscale) * 1024,
        "algorithmic_bytes_per_launch": nbytes,
    }
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out), flush=True)


def bench_adaln(args):
    """The fused AdaLN + residual step at the stage-1 token count (one JSON line)."""
    import torch

    import datagen
    import swin3d_window_attention_amd as sw

    wl = datagen.ADALN_WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    a = datagen.adaln_inputs(wl)
    x = datagen.to_torch(a["x"], wl.x_dtype).to(dev)
    res = datagen.to_torch(a["res"], wl.res_dtype).to(dev)
    g, b = (torch.from_numpy(a[k]).to(dev) for k in ("gamma", "beta"))
    out_dtype = torch.float32 if wl.out_dtype == "f32" else torch.bfloat16
    out = torch.empty(wl.shape, dtype=out_dtype, device=dev)
    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        sw.adaln_residual(x, res, g, b, wl.eps, out=out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while (time.perf_counter() - t0) * 1e3 < args.warmup_ms:
        for _ in range(20):
            sw.adaln_residual(x, res, g, b, wl.eps, out=out)
        torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(args.steps):
        sw.adaln_residual(x, res, g, b, wl.eps, out=out)
    end.record(stream)
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    log(f"[bench] adaln {ms * 1000:.1f} us per step")
    elt = {"bf16": 2, "f32": 4}
    n = wl.B * wl.rows * wl.C
    nbytes = n * (elt[wl.x_dtype] + elt[wl.res_dtype] + elt[wl.out_dtype]) + 2 * wl.B * wl.C * 4
    gbs = nbytes / (ms / 1e3) / 1e9
    # context: the same launches writing ROTATE_OUTPUTS output buffers in turn (see output_rotation)
    rotation = None
    out_bytes = out.numel() * out.element_size()
    if not args.no_output_rotation and out_bytes <= ROTATE_MAX_BYTES:
        outs = [torch.empty_like(out) for _ in range(ROTATE_OUTPUTS)]
        i = [0]

        def run_rot():
            sw.adaln_residual(x, res, g, b, wl.eps, out=outs[i[0] % ROTATE_OUTPUTS])
            i[0] += 1

        rms, _ = warm_then_time(torch, run_rot, stream, args.steps, max(args.warmup, ROTATE_OUTPUTS), 100.0)
        del outs
        rg = nbytes / (rms / 1e3) / 1e9
        rotation = {"buffers": ROTATE_OUTPUTS, "bytes_per_buffer": out_bytes, "us_per_step": rms * 1e3,
                    "tokens_per_s": wl.B * wl.rows / (rms / 1e3),
                    "roofline": {"bound": "hbm", "achieved": rg, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": rg / HBM_PEAK_GBS}}
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        cpu = cpu_baseline_adaln(wl, a, args.cpu_budget)
    print(json.dumps({
        "metric": "fused AdaLN + residual tokens/s at the 0.25-degree stage-1 token count",
        "value": wl.B * wl.rows / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": f"x {wl.x_dtype}, residual {wl.res_dtype}, out {wl.out_dtype}, f32 math",
        "data": "synthetic (seeded)",
        "config": {"workload": wl.name, "B": wl.B, "rows": wl.rows, "C": wl.C, "eps": wl.eps},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": None},
        "output_rotation": rotation, "algorithmic_bytes_per_launch": nbytes, "cpu_baseline": cpu,
    }), flush=True)


def warm_then_time(torch, run, stream, steps: int, warmup: int, warmup_ms: float):
    """warmup calls, then more until the GPU has run for warmup_ms (engine clocks ramp up under
    sustained load; a cold first pass reads about 10% slow), then `steps` back-to-back calls
    between two HIP events on the launch stream. Returns (ms per call, extra warm-up calls)."""
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    extra = 0
    while (time.perf_counter() - t0) * 1e3 < warmup_ms:
        for _ in range(20):
            run()
        torch.cuda.synchronize()
        extra += 20
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    for _ in range(steps):
        run()
    end.record(stream)
    torch.cuda.synchronize()
    return start.elapsed_time(end) / steps, extra


ROTATE_OUTPUTS = 8           # output buffers cycled by output_rotation()
ROTATE_MAX_BYTES = 1 << 30   # larger outputs exceed the 256 MB Infinity Cache at least four times over


def output_rotation(torch, wl, run_into, like, stream, steps: int, warmup: int):
    """Context for a timed workload: the same launches, but each writes the next of ROTATE_OUTPUTS
    output buffers (8 x the output, well beyond the 256 MB Infinity Cache). Back-to-back launches
    into one output buffer find much of the previous launch's output still in that cache, and
    rewrite those lines there before they are ever written back to HBM; here every launch's output
    reaches HBM, as it does for an output that goes to fresh memory. None for outputs above
    ROTATE_MAX_BYTES (whose launches already write back all but a cache's worth)."""
    out_bytes = like.numel() * like.element_size()
    if out_bytes > ROTATE_MAX_BYTES:
        return None
    outs = [torch.empty_like(like) for _ in range(ROTATE_OUTPUTS)]
    i = [0]

    def run():
        run_into(outs[i[0] % ROTATE_OUTPUTS])
        i[0] += 1

    ms, _ = warm_then_time(torch, run, stream, steps, max(warmup, ROTATE_OUTPUTS), 100.0)
    del outs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    r = roofline_of(wl, ms)
    return {"buffers": ROTATE_OUTPUTS, "bytes_per_buffer": out_bytes, "us_per_step": ms * 1e3,
            "tokens_per_s": wl.tokens / (ms / 1e3), "roofline": r}


def roofline_of(wl, ms: float) -> dict:
    """Position of one launch of workload wl taking ms against the bound of its kernel: HBM bytes
    at 8 TB/s or products at the matrix-core peak of their own type, whichever takes longer."""
    nbytes, flops, _ = algorithmic_work(wl)
    sec = ms / 1e3
    mfma_peak = F32_MFMA_PEAK_TFLOPS if wl.plan_dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
    if flops / (mfma_peak * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9):
        a = flops / sec / 1e12
        return {"bound": "mfma", "achieved": a, "peak": mfma_peak, "unit": "TFLOP/s", "frac": a / mfma_peak}
    a = nbytes / sec / 1e9
    return {"bound": "hbm", "achieved": a, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": a / HBM_PEAK_GBS}


def bench_configs(torch, dev, stream, args, names=CONFIG_WORKLOADS) -> dict:
    """The other measured shapes, each timed like the headline (same warm-up and event protocol,
    inputs resident on the device, the same bias). Inputs of one shape are freed before the next
    is generated."""
    import datagen
    import swin3d_window_attention_amd as sw

    out = {}
    for name in names:
        wl = datagen.WORKLOADS[name]
        log(f"[bench] config {name}: inputs {wl.shape} {wl.dtype}")
        x = {t: datagen.to_torch(datagen.full_io(wl, t), wl.dtype).to(dev) for t in ("q", "k", "v")}
        o = torch.empty_like(x["q"])
        plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.plan_dtype, scale=wl.scale,
                       cross_region_bias=args.bias)
        info = plan.info()
        ms, _ = warm_then_time(torch, lambda: plan.run(x["q"], x["k"], x["v"], o), stream, args.steps,
                               args.warmup, min(args.warmup_ms, 200.0))
        rot = None if args.no_output_rotation else output_rotation(
            torch, wl, lambda oo: plan.run(x["q"], x["k"], x["v"], oo), o, stream, args.steps, args.warmup)
        nbytes, flops, nwin = algorithmic_work(wl)
        out[name] = {
            "shape": {"B": wl.B, "grid": [wl.D, wl.H, wl.W], "heads": wl.heads, "head_dim": wl.head_dim,
                      "window": list(wl.window), "shift": list(wl.shift), "dtype": wl.dtype,
                      "windows": nwin, "masked_windows": info.n_masked_windows, "kernel": info.kernel},
            "us_per_step": ms * 1e3,
            "tokens_per_s": wl.tokens / (ms / 1e3),
            "steps": args.steps,
            "algorithmic_bytes_per_launch": nbytes,
            "algorithmic_flops_per_launch": flops,
            "roofline": roofline_of(wl, ms),
            "output_rotation": rot,
        }
        log(f"[bench] config {name}: {ms * 1e3:.1f} us per step, "
            f"{out[name]['roofline']['frac']:.3f} of the {out[name]['roofline']['bound']} roofline")
        del x, o, plan
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--warmup-ms", type=float, default=300.0, help="minimum warm-up time on the GPU")
    ap.add_argument("--bias", type=float, default=-100.0)
    ap.add_argument("--workload", default="stage1",
                    help="stage1 (default, the headline line) or another workload: stage2, stage2_s0, "
                         "stage3_pad, stress_hres (bf16), stage1_f32_split, stage3_pad_f32_split, "
                         "stress_f32_split (FP32 I/O on the split-bf16 matrix-core kernel), "
                         "stage1_f32, stage3_pad_f32, stress_f32 (exact FP32 on the matrix cores), "
                         "stage1_h4d128, stage1_w2x12x12 (whole window in LDS), "
                         "stage1_w4x12x24, stage1_w3x12x12_h4d128 (K/V streamed through LDS), "
                         "adaln_stage1 (the fused AdaLN + residual step)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true",
                    help="with the headline workload: skip timing the other shapes (" +
                         ", ".join(CONFIG_WORKLOADS) + ") that the line reports under 'configs'")
    ap.add_argument("--no-output-rotation", action="store_true",
                    help="skip the output_rotation context (the same launches writing eight output buffers "
                         "in turn), e.g. so that a profiler's kernel statistics hold the timed protocol only")
    ap.add_argument("--cold", action="store_true",
                    help="flush the 256 MB Infinity Cache (read a 1 GiB buffer) before every timed "
                         "launch and time each launch with its own events")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device copy of BYTES bytes (profiler counter calibration)")
    ap.add_argument("--write-traffic", metavar="DIR",
                    help="host only: write the stage-1 traffic summary from rocprofv3 FETCH_SIZE / "
                         "WRITE_SIZE runs under DIR (fetch, write, copyfetch, copywrite)")
    args = ap.parse_args()

    if args.write_traffic:
        write_traffic(args.write_traffic)
        return

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the attention shards by head or batch with no communication, but no multi-GPU "
              "path is built", file=sys.stderr)
        sys.exit(2)

    if args.copy_calibration:
        copy_calibration(args.copy_calibration, args.steps)
        return
    if args.workload.startswith("adaln"):
        bench_adaln(args)
        return

    import torch

    import datagen
    import swin3d_window_attention_amd as sw

    wl = datagen.WORKLOADS[args.workload]
    if wl.plan_dtype not in ("bf16", "f32_split", "f32"):
        sys.exit(f"bench.py: workload {wl.name} is a {wl.dtype} parity case, not a benchmark")
    headline = wl.name == "stage1"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log(f"[bench] inputs {wl.shape} {wl.dtype}")
    x = {t: datagen.to_torch(datagen.full_io(wl, t), wl.dtype).to(dev) for t in ("q", "k", "v")}
    o = torch.empty_like(x["q"])
    plan = sw.Plan(*wl.shape, window=wl.window, shift=wl.shift, dtype=wl.plan_dtype, scale=wl.scale,
                   cross_region_bias=args.bias)
    info = plan.info()
    stream = torch.cuda.current_stream(dev)

    def run():
        plan.run(x["q"], x["k"], x["v"], o)

    if args.cold:
        # a read-only pass over 1 GiB replaces the cache contents with clean, unrelated lines
        # (a write pass would leave dirty lines that the timed kernel then has to write back)
        warm_then_time(torch, run, stream, 1, args.warmup, args.warmup_ms)
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(args.steps)]
        torch.cuda.synchronize()
        for s, e in evs:
            torch.amax(flush, dim=0, out=sink)
            s.record(stream)
            run()
            e.record(stream)
        torch.cuda.synchronize()
        ms = sum(s.elapsed_time(e) for s, e in evs) / args.steps
        del flush
    else:
        ms, extra = warm_then_time(torch, run, stream, args.steps, args.warmup, args.warmup_ms)
        log(f"[bench] warmup {args.warmup} + {extra} steps done; timed {args.steps} steps")
    log(f"[bench] {ms * 1000:.1f} us per step{' (cold cache)' if args.cold else ''}")

    # context, after the timed region: single launches each between their own
    # events (median and min of 20; the pages' method, the mean of 5 after 2
    # warm-ups), and a plain device copy for the fraction of what this device
    # moves in practice
    def single_launches(n):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for st, en in evs:
            st.record(stream)
            plan.run(x["q"], x["k"], x["v"], o)
            en.record(stream)
        torch.cuda.synchronize()
        return [st.elapsed_time(en) * 1000 for st, en in evs]

    singles = sorted(single_launches(20))
    for _ in range(2):
        plan.run(x["q"], x["k"], x["v"], o)
    pages_mean5 = sum(single_launches(5)) / 5
    rotation = None if args.cold or args.no_output_rotation else output_rotation(
        torch, wl, lambda oo: plan.run(x["q"], x["k"], x["v"], oo), o, stream, args.steps, args.warmup)
    copy_gbs = device_copy_gbs(torch, 1 << 29)

    configs = None
    if headline and not args.no_configs:
        configs = bench_configs(torch, dev, stream, args)

    nbytes, flops, nwin = algorithmic_work(wl)
    sec = ms / 1e3
    tokens_per_s = wl.tokens / sec
    gbs = nbytes / sec / 1e9
    tflops = flops / sec / 1e12
    frac_hbm = gbs / HBM_PEAK_GBS
    # the matrix-core peak of the products' own type (exact FP32 runs FP32 MFMAs)
    mfma_peak = F32_MFMA_PEAK_TFLOPS if wl.plan_dtype == "f32" else BF16_MFMA_PEAK_TFLOPS
    frac_mfma = tflops / mfma_peak
    mfma_bound = flops / (mfma_peak * 1e12) > nbytes / (HBM_PEAK_GBS * 1e9)

    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] timing the fp64 oracle on the host")
        cpu = cpu_baseline(wl, args.cpu_budget, args.bias)

    line = {
        "metric": METRIC,
        "value": tokens_per_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16" if wl.dtype == "bf16"
                  else "f32 I/O, bf16x3 split products, f32 softmax" if wl.plan_dtype == "f32_split"
                  else "f32"),
        "data": ("synthetic (seeded iid N(0,1) rounded to bf16)" if wl.dtype == "bf16"
                 else "synthetic (seeded iid float32 draws)"),
        "config": {
            "workload": ("0.25-degree stage-1-like window attention" if headline
                         else f"{wl.name} window attention"),
            "B": wl.B, "grid": [wl.D, wl.H, wl.W], "heads": wl.heads, "head_dim": wl.head_dim,
            "window": list(wl.window), "shift": list(wl.shift), "cross_region_bias": args.bias,
            "tokens": wl.tokens, "windows": nwin, "masked_windows": info.n_masked_windows,
            "cache": ("flushed (1 GiB read) before each launch" if args.cold
                      else "warm (back-to-back launches)"),
        },
        "roofline": ({
            "bound": "mfma",
            "achieved": tflops,
            "peak": mfma_peak,
            "unit": "TFLOP/s",
            "frac": frac_mfma,
            "traffic": None,
        } if mfma_bound else {
            "bound": "hbm",
            "achieved": gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": frac_hbm,
            "traffic": measured_traffic() if headline else None,
        }),
        "mfma": {"achieved_tflops": tflops, "peak_tflops": mfma_peak, "frac": frac_mfma},
        "single_launch_us": {"median": singles[len(singles) // 2], "min": singles[0], "count": len(singles),
                             "mean_of_5_after_2_warmups": pages_mean5},
        "device_copy": {"gbs_read_plus_write": copy_gbs, "bytes": 1 << 29,
                        "algorithmic_frac_of_copy": gbs / copy_gbs},
        "output_rotation": rotation,
        "algorithmic_bytes_per_launch": nbytes,
        "algorithmic_flops_per_launch": flops,
        "cpu_baseline": cpu,
    }
    if configs is not None:
        line["configs"] = configs
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
