"""Host-side logic of the HIP path that runs without a GPU: the launch-time
fast division behind the kernels' index math, the argument checks under
sanitizers, and the bench's buffer rotation and traffic bookkeeping."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_positional_encoding_amd", "csrc")


def test_fast_division_exact(tmp_path):
    exe = tmp_path / "fastdiv_check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC,
                    os.path.join(ROOT, "tests", "host_checks", "fastdiv_check.cpp"), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "bad 0" in out.stdout


def test_argument_checks_under_sanitizers(tmp_path):
    """The C ABI's argument validation, built with g++ under AddressSanitizer
    and UndefinedBehaviorSanitizer (host code only), on three million random
    and extreme argument sets: no sanitizer report, and every accepted call
    describes a launch whose offsets fit in 64 bits."""
    exe = tmp_path / "plan_fuzz"
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-I", CSRC, "-I", os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "host_checks", "plan_fuzz.cpp"), os.path.join(CSRC, "rope_plan.cpp"),
                    "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stdout + out.stderr
    assert "bad 0" in out.stdout


def test_bench_rotation_and_line_bytes():
    sys.path.insert(0, ROOT)
    import bench
    import workloads as W
    # c3: one 128-byte line of a 384-byte row per row; c4 bf16: two lines (straddle)
    assert bench.slice_line_bytes(W.WORKLOADS["c3"]) == 4 * 4096 * 128 * 128
    assert bench.slice_line_bytes(W.WORKLOADS["c4"]) == 16 * 8192 * 32 * 256
    assert bench.rotating_copies(W.WORKLOADS["c3"]) == 3
    assert bench.rotating_copies(W.WORKLOADS["c4"]) == 1


def test_bench_refuses_more_than_one_gpu():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True)
    assert res.returncode == 2 and "one GPU" in res.stderr


def test_traffic_is_dropped_when_the_kernel_changes(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    md = tmp_path / "t.md"
    md.write_text('```json\n{"kernel_source_sha256_16": "%s", "launches": {"c4:bwd": {"hbm_bytes_per_launch": 5}}}\n```\n'
                  % bench.kernel_source_hash())
    monkeypatch.setattr(bench, "TRAFFIC_MD", str(md))
    assert bench.committed_traffic("c4", "bwd")["hbm_bytes_per_launch"] == 5
    md.write_text('```json\n{"kernel_source_sha256_16": "0000", "launches": {"c4:bwd": {"hbm_bytes_per_launch": 5}}}\n```\n')
    assert bench.committed_traffic("c4", "bwd") is None


def test_rope_inv_freq_follows_the_recipe():
    """rope_inv_freq(L, base) gives the frequencies of "ANE实战RoPE位置编码在MIL中的
    纯ANE实现", section 第一步 (θ = p / base^(2i/h), i < h/2), as doubles: each is
    base^(-2i/L) evaluated with 50 significant digits (the decimal module)
    and compared with the returned double: the two differ by less than one
    unit in the last place (the double power is faithfully rounded; it need
    not be the nearest double, 2^-0.5 is not), and the first is 1."""
    import decimal
    import math

    import numpy as np

    sys.path.insert(0, ROOT)
    import transformer_positional_encoding_amd as rp
    ctx = decimal.Context(prec=50)
    for L in (2, 32, 64, 128, 1024):
        for base in (10000.0, 500000.0, 2.0):
            f = rp.rope_inv_freq(L, base).numpy()
            assert f.dtype == np.float64 and f.shape == (L // 2,)
            assert f[0] == 1.0
            b = decimal.Decimal(base)
            for i in range(L // 2):
                exact = ctx.power(b, ctx.divide(decimal.Decimal(-2 * i), decimal.Decimal(L)))
                ref = float(exact)
                err = abs(decimal.Decimal(float(f[i])) - exact)
                assert err < decimal.Decimal(math.ulp(ref)), (L, base, i, f[i], exact)
            assert np.all(np.diff(f) < 0)
