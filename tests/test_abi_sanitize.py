"""The C ABI's host logic (descriptor validation, plan arithmetic, span / overlap / alignment
checks of run and run_strided, the AdaLN descriptor checks) built with AddressSanitizer and
UndefinedBehaviorSanitizer and driven over a grid of valid and invalid descriptors
(`tests/native/abi_sanitize.cpp`, stub kernel launchers, no GPU)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_abi_under_sanitizers(tmp_path):
    exe = tmp_path / "abi_sanitize"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROOT, "swin3d_window_attention_amd", "csrc"),
           os.path.join(ROOT, "swin3d_window_attention_amd", "csrc", "api.cpp"),
           os.path.join(ROOT, "tests", "native", "abi_sanitize.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True, timeout=300)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1:abort_on_error=1"})
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.startswith("ok:"), r.stdout
