"""A plain C program (tests/c_abi/rope_c_consumer.c, built by
__graft_entry__.build()) that uses the library through the C ABI alone: HIP
runtime memory and streams, no PyTorch and no Python in the process. It
compares the in-place, out-of-place, multi-tensor and position entry points
with the C oracle element by element and checks the documented status codes."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi", "rope_c_consumer")


def _run(*args, timeout):
    if not os.path.exists(EXE):
        pytest.fail(f"{EXE} is missing: run __graft_entry__.build()")
    res = subprocess.run([EXE, *args], capture_output=True, text=True, timeout=timeout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.strip().endswith("all ok"), res.stdout
    return res.stdout


def test_c_client_argument_checks_without_a_gpu():
    """Errors, no-ops and the launch plan return before any HIP call."""
    out = _run("--no-gpu", timeout=60)
    assert "ROPE_ERR_NULLPTR" in out and "ROPE_ERR_INVALID" in out
    assert sum(line.startswith("ok   ") for line in out.splitlines()) == 15


@pytest.mark.gpu
def test_c_client_on_the_gpu():
    out = _run(timeout=120)
    for case in ("per-batch tables", "MLA-like", "rotate_half, bwd out of place", "fp32 tables", "Q and K",
                 "odd start", "per-head tables", "bf16 positions", "fp32 positions"):
        assert case in out, case
