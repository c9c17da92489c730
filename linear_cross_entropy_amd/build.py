"""Compile the gfx950 HIP libraries in-tree with hipcc: libcce.so (the loss and its
gradients) and libcce_probe.so (measured MFMA, LDS and load ceilings of the device)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "cce.hip")
LIB = os.path.join(HERE, "libcce.so")
PROBE_SRC = os.path.join(HERE, "csrc", "probe.hip")
PROBE_LIB = os.path.join(HERE, "libcce_probe.so")
INCLUDE = os.path.join(ROOT, "include")

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed-fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _compile(src: str, lib: str, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = lib + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-I", INCLUDE, src, "-o", tmp]
    r = subprocess.run(cmd, capture_output=not verbose, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + (r.stderr or "") + (r.stdout or ""))
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    """Always recompiles both libraries; returns the path of libcce.so."""
    _compile(SRC, LIB, verbose)
    _compile(PROBE_SRC, PROBE_LIB, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
