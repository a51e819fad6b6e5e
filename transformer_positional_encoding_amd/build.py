"""Build librope_partial.so (HIP, gfx950) in-tree with hipcc.

    python -m transformer_positional_encoding_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "librope_partial.so")
SOURCES = [os.path.join(CSRC, "rope_kernels.hip"), os.path.join(CSRC, "rope_plan.cpp")]
# The bare access-pattern probe the benchmark times beside the kernels (its
# own library; the rotation library does not use it).
PROBE_LIB_PATH = os.path.join(LIB_DIR, "libhbm_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "probe", "hbm_probe.hip")]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared", "-fvisibility=hidden",
        # no packed fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wno-unused-command-line-argument",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(sources: list[str], out: str, verbose: bool) -> str:
    os.makedirs(LIB_DIR, exist_ok=True)
    tmp = out + ".tmp"
    cmd = [hipcc()] + compile_flags() + sources + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed to build {os.path.basename(out)}")
    os.replace(tmp, out)
    return out


def build(verbose: bool = False) -> str:
    """Build the rotation library and the benchmark's access-pattern probe;
    returns the rotation library's path."""
    _compile(SOURCES, LIB_PATH, verbose)
    _compile(PROBE_SOURCES, PROBE_LIB_PATH, verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
