"""Host-side pieces of bench.py (CPU only): the algorithmic work it divides by, the traffic summary
it reports, the oracle baselines it times, and the one-GPU guard."""
import json
import os
import subprocess
import sys

import pytest

import bench
import datagen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_algorithmic_work_stage1():
    """Stage 1: 259,200 tokens x 8 heads x 64 dims x 2 bytes x 4 tensors, and 4 N^2 dh FLOPs for
    each of 1,800 windows x 8 heads."""
    nbytes, flops, nwin = bench.algorithmic_work(datagen.WORKLOADS["stage1"])
    assert nbytes == 1_061_683_200
    assert nwin == 1800
    assert flops == 4 * 144 * 144 * 64 * 8 * 1800 == 76_441_190_400


def test_algorithmic_work_counts_real_tokens_only():
    """Stage 3 pads 45 x 90 to 48 x 96: bytes count the real tokens, FLOPs every padded window."""
    nbytes, flops, nwin = bench.algorithmic_work(datagen.WORKLOADS["stage3_pad"])
    assert nbytes == 4 * (4 * 45 * 90) * 32 * 64 * 2
    assert nwin == 2 * 8 * 8
    assert flops == 4 * 144 * 144 * 64 * 32 * 128


def test_traffic_summary_matches_the_kernel_source():
    """The committed HBM traffic summary was taken on the current single-tile kernel source, and
    its bytes equal the algorithmic bytes within 0.1%."""
    t = bench.measured_traffic()
    assert t is not None, "traffic summary missing or taken on another kernel source"
    with open(bench.TRAFFIC_FILE) as f:
        summary = json.load(f)
    assert summary["algorithmic_bytes_per_launch"] == bench.algorithmic_work(datagen.WORKLOADS["stage1"])[0]
    assert abs(t / summary["algorithmic_bytes_per_launch"] - 1.0) < 1e-3


@pytest.mark.parametrize("name", ["tiny_f32", "stage3_pad"])
def test_cpu_baseline_whole_heads(name):
    r = bench.cpu_baseline(datagen.WORKLOADS[name], 0.05)
    assert r["kind"] == "oracle" and r["unit"] == "tokens/s" and r["value"] > 0 and r["cores"] >= 1
    assert "one head per call" in r["sample"]


def test_cpu_baseline_adaln():
    wl = datagen.AdalnWorkload("adaln_small", 2, 5000, 256, "bf16", "f32", "f32", 3)
    r = bench.cpu_baseline_adaln(wl, datagen.adaln_inputs(wl), 0.05)
    assert r["kind"] == "oracle" and r["value"] > 0 and "blocks of 4096 rows" in r["sample"]


def test_more_than_one_gpu_is_refused():
    """bench.py runs on one GPU: --gpus 2 exits with status 2 and says so, before touching a GPU."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_help_lists_every_bench_workload():
    """Every stage, stress and shape workload can be named on the command line and is listed in
    --help (the tiny case is a smoke and test input only)."""
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0
    text = " ".join(r.stdout.split())
    for name in datagen.WORKLOADS:
        if name != "tiny_f32":
            assert name in text, name
    assert "adaln_stage1" in text
