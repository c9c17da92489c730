"""Time the fp64 oracle at full size on this host: forward and backward
separately for every synthetic workload, as a CPU baseline for the GPU path.

    python oracle/time_full.py [--workloads tiny,qwen2.5-0.5b-head,...] [--plain-rows 256]

The blocked form (fp64 matrix products per block of rows) runs every row of
every workload; the plain loops (C, OpenMP) run the first --plain-rows rows of
each, their rate scaled to tokens/s.  The backward uses the filter threshold
2^-12 and the workload's reduction.  Prints a markdown table with the host's
CPU model, logical CPUs, RAM and the threads each form used.

Test infrastructure: it loads the oracle and nothing of the HIP path.
"""
from __future__ import annotations

import argparse
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import oracle  # noqa: E402
import synthetic_inputs as si  # noqa: E402

EPS = 2.0 ** -12


def host():
    model = "unknown"
    for line in open("/proc/cpuinfo"):
        if line.startswith("model name"):
            model = line.split(":", 1)[1].strip()
            break
    ram = 0
    for line in open("/proc/meminfo"):
        if line.startswith("MemTotal"):
            ram = int(line.split()[1]) // (1024 * 1024)
    return model, os.cpu_count(), ram


class Progress:
    """Prints the blocked form's progress at most every 30 s."""

    def __init__(self, what):
        self.what, self.t0, self.last = what, time.perf_counter(), time.perf_counter()

    def __call__(self, done, total):
        now = time.perf_counter()
        if now - self.last >= 30.0:
            self.last = now
            print(f"  {self.what}: {done} / {total} rows, {now - self.t0:.0f} s", flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workloads", default=",".join(w.name for w in si.FULL))
    ap.add_argument("--plain-rows", type=int, default=256)
    args = ap.parse_args()
    names = args.workloads.split(",")
    model, ncpu, ram = host()
    print(f"host: {model}, {ncpu} logical CPUs, {ram} GiB RAM; blocked form on "
          f"{torch.get_num_threads()} torch threads, plain loops on {oracle.threads()} OpenMP "
          f"threads", flush=True)
    rows = []
    for w in si.FULL:
        if w.name not in names:
            continue
        E, C, x = si.generate(w)
        E64, C64, xs = E.double().numpy(), C.double().numpy(), x.numpy()
        g = si.upstream_grad(w).double().numpy()
        del E, C
        t0 = time.perf_counter()
        _, lse, _ = oracle.forward_blocked(E64, C64, xs, -100, w.reduction,
                                           progress=Progress(f"{w.name} forward"))
        tf = time.perf_counter() - t0
        print(f"{w.name}: blocked forward {tf:.1f} s", flush=True)
        t0 = time.perf_counter()
        oracle.backward_blocked(E64, C64, xs, g, -100, w.reduction, eps=EPS, lse=lse,
                                progress=Progress(f"{w.name} backward"))
        tb = time.perf_counter() - t0
        print(f"{w.name}: blocked backward {tb:.1f} s", flush=True)
        r = min(args.plain_rows, w.N)
        gs = np.where(xs[:r] != -100, 1.0 / max(int((xs != -100).sum()), 1), 0.0)
        if w.reduction == "none":
            gs = np.where(xs[:r] != -100, g[:r], 0.0)
        t0 = time.perf_counter()
        oracle.forward(E64[:r], C64, xs[:r], -100, "none")
        pf = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.backward(E64[:r], C64, xs[:r], gs, -100, "none", eps=EPS)
        pb = time.perf_counter() - t0
        print(f"{w.name}: plain loops on {r} rows: forward {pf:.1f} s, backward {pb:.1f} s",
              flush=True)
        rows.append((w, tf, tb, r, pf, pb))
        del E64, C64
    print()
    print("| workload | N | V | D | blocked fwd s | blocked bwd s | blocked tokens/s (fwd+bwd) |"
          " plain rows | plain fwd s | plain bwd s | plain tokens/s (fwd+bwd) |")
    print("|---|---:|---:|---:|---:|---:|---:|---:|---:|---:|---:|")
    for w, tf, tb, r, pf, pb in rows:
        print(f"| {w.name} | {w.N} | {w.V} | {w.D} | {tf:.1f} | {tb:.1f} | {w.N / (tf + tb):.1f} |"
              f" {r} | {pf:.1f} | {pb:.1f} | {r / (pf + pb):.2f} |")


if __name__ == "__main__":
    main()
