"""Benchmark: one fwd+bwd step of Cut Cross-Entropy on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload gemma2-2b-head]

A step is the whole hot path on one batch: cce_forward (logit tiles, online
log-sum-exp, merge) and cce_backward (recompute, G, filter, dC, dE) at the
Gemma-2-2B head shape N=8192, V=256000, D=2304 in bf16 with filter_eps=2^-12
and mean reduction.  Inputs are seeded synthetic data of that shape (the
recipe is in synthetic_inputs.py), resident in HBM before timing starts.

Prints one JSON line with tokens/s, the roofline of the dominant kernel
(per-kernel HIP events recorded by the library on the launch stream), the
forward / backward split of each step (median, min, max), the rate against
this device's measured MFMA peak, and the CPU oracle timed on a bounded
sample of the same workload.  --hw-probe measures the device's ceilings
instead (MFMA rate, LDS read and load bandwidth in and past L2).
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fwd+bwd tokens/sec and % bf16 MFMA peak at N=8192,V=256000,D=2304"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
FAMILIES = ("fwd_lse", "target", "fwd_merge", "bwd_step", "transpose", "gather", "vocab_order",
            "small", "bwd_de", "bwd_dc", "bwd_g", "bwd_t")


def kernel_flops(name, N, V, D, kC=1.0, kE=1.0):
    """The method's MFMA flops of one step for a kernel family: 2*N*V*D for the
    forward's logits; for the backward step kernel the recompute (2*N*V*D) plus
    dC and dE at the fraction of 32x32 units each keeps (2*N*V*D*k each): work
    on filtered units is skipped and not counted.  With --role-split the
    backward's roles are families of their own (bwd_g, bwd_dc, bwd_de)."""
    per = 2.0 * N * V * D
    return {"fwd_lse": per, "bwd_step": (1.0 + kC + kE) * per, "bwd_g": per, "bwd_dc": kC * per,
            "bwd_de": kE * per}.get(name, 0.0)


def dense_flops(name, N, V, D):
    """The same kernels' flops with no unit filtered (3 contractions in the backward)."""
    per = 2.0 * N * V * D
    return {"fwd_lse": per, "bwd_step": 3.0 * per, "bwd_g": per, "bwd_dc": per,
            "bwd_de": per}.get(name, 0.0)


def host_description():
    """CPU model, logical CPUs and RAM of this host (for the CPU baseline)."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    ram = 0
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                ram = int(line.split()[1]) // (1024 * 1024)
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(), "ram_gib": ram}


def kernel_source_sha256():
    """sha256 of the kernel source with comments and blank lines removed, so
    that only a change to the code itself retires a counter summary."""
    import hashlib
    import re
    src = os.path.join(ROOT, "linear_cross_entropy_amd", "csrc", "cce.hip")
    text = re.sub(r"//[^\n]*", "", open(src).read())
    lines = [ln.rstrip() for ln in text.splitlines() if ln.strip()]
    return hashlib.sha256("\n".join(lines).encode()).hexdigest()


def traffic_record(kernel, workload):
    """HBM traffic of `kernel` per launch from the committed counter summary
    (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by the same counters read on a
    plain copy of known size), or None when there is no summary or the kernel
    source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None, "no counter summary"
    rec = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            rec[k.strip()] = v.strip()
    sha = kernel_source_sha256()
    if rec.get("source_sha256") != sha:
        return None, "kernel source changed since the counters were taken"
    b = (float(rec["fetch_kib_per_launch"]) * float(rec["fetch_scale"]) +
         float(rec["write_kib_per_launch"]) * float(rec["write_scale"])) * 1024.0
    return b, os.path.relpath(path, ROOT)


def copy_calibration(mib):
    """A plain device copy of known size, for scaling the traffic counters."""
    import torch
    n = int(mib) << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "copies": 5}), flush=True)


def _probe_lib():
    """ctypes view of libcce_probe.so (measured device ceilings), or None if not built."""
    import ctypes
    from linear_cross_entropy_amd.build import PROBE_LIB
    if not os.path.exists(PROBE_LIB):
        return None
    lib = ctypes.CDLL(PROBE_LIB)
    f, d = ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_double)
    lib.cce_probe_mfma.argtypes = [ctypes.c_int, f, d]
    lib.cce_probe_lds.argtypes = [f, d]
    lib.cce_probe_stream.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, f, d]
    return lib


def _probe_call(fn, *args):
    """Runs one probe; returns (ms, amount) or raises on a HIP error."""
    import ctypes
    ms, amount = ctypes.c_float(), ctypes.c_double()
    rc = fn(*args, ctypes.byref(ms), ctypes.byref(amount))
    if rc != 0:
        raise RuntimeError(f"probe failed with HIP error {rc}")
    return ms.value, amount.value


def mfma_probe_tflops():
    """Measured bf16 MFMA rate (v_mfma_f32_16x16x32_bf16 on register operands,
    pseudo-random values) of this device, TFLOP/s, or None without the probe."""
    lib = _probe_lib()
    if lib is None:
        return None
    rates = sorted(f / (m * 1e-3) / 1e12 for m, f in (_probe_call(lib.cce_probe_mfma, 0)
                                                      for _ in range(3)))
    return rates[1]  # median of three


def hw_probe():
    """The device ceilings the kernels are read against: MFMA rate, LDS read
    bandwidth, and 16-byte-per-lane loads from every compute unit at once
    (direct to LDS and into registers) from L2-resident windows and from
    footprints past L2."""
    import torch
    torch.cuda.init()
    lib = _probe_lib()
    if lib is None:
        raise SystemExit("libcce_probe.so is not built (linear_cross_entropy_amd.build.build())")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = {"probe": "device ceilings", "cus": cus}
    for zeros in (0, 1):
        rates = [f / (m * 1e-3) / 1e12 for m, f in (_probe_call(lib.cce_probe_mfma, zeros)
                                                    for _ in range(3))]
        out["mfma_bf16_tflops" + ("_zero_operands" if zeros else "")] = [round(r, 1)
                                                                         for r in rates]
    ms, b = _probe_call(lib.cce_probe_lds)
    out["lds_read_GBps_per_cu"] = round(b / (ms * 1e-3) / 1e9 / cus, 1)
    out["lds_read_bytes_per_clk_per_cu_at_2p4GHz"] = round(b / (ms * 1e-3) / cus / 2.4e9, 1)
    loads = []
    # (window KiB, shared): 1 MiB shared by all (L2); own windows of 64 KiB (2 MiB per XCD,
    # L2), 256 KiB (8 MiB per XCD, 64 MiB in all), 4 MiB (1 GiB in all)
    for win_kib, shared in ((1024, 1), (64, 0), (256, 0), (4096, 0)):
        for to_lds in (1, 0):
            ms, b = _probe_call(lib.cce_probe_stream, win_kib * 1024, shared, to_lds)
            loads.append({"window_KiB": win_kib, "windows": "shared" if shared else "own",
                          "footprint_MiB": win_kib * (1 if shared else cus) / 1024,
                          "path": "direct-to-LDS" if to_lds else "registers",
                          "TBps": round(b / (ms * 1e-3) / 1e12, 2),
                          "GBps_per_cu": round(b / (ms * 1e-3) / 1e9 / cus, 1)})
    out["loads"] = loads
    print(json.dumps(out), flush=True)


def cpu_baseline(w, E, C, x, eps, rows=256, filter_mode="both", vocab_sort=False):
    """The oracle, as it stands, on the first `rows` tokens (one filter-unit block)
    with the full vocabulary and hidden size: fwd + bwd, timed on the host."""
    import numpy as np
    import oracle
    oracle._load()
    Es = E[:rows].double().numpy()
    xs = x[:rows].numpy()
    C64 = C.double().numpy()
    nv = max(int((x != -100).sum()), 1)
    g = np.where(xs != -100, 1.0 / nv, 0.0)
    t0 = time.perf_counter()
    oracle.forward(Es, C64, xs, -100, "none")
    order = oracle.vocab_order(Es, C64, xs, -100)[0] if vocab_sort else None
    oracle.backward(Es, C64, xs, g, -100, "none", eps=eps, filter_mode=filter_mode,
                    vocab_order=order)
    dt = time.perf_counter() - t0
    return {"value": rows / dt, "unit": "tokens/s", "cores": oracle.threads(), "kind": "oracle",
            "sample": f"first {rows} tokens of {w.name} (full V={w.V}, D={w.D}), fp64 fwd+bwd "
                      f"with filter eps={eps:g} ({filter_mode}"
                      f"{', vocabulary sorted on the sample' if vocab_sort else ''}), {dt:.1f} s",
            "host": host_description()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gemma2-2b-head")
    ap.add_argument("--eps", type=float, default=2.0 ** -12)
    ap.add_argument("--filter-mode", default="both", choices=["both", "full_c", "full_e"],
                    help="contractions that take the filtered gradient (both; full_c: dC "
                         "unfiltered; full_e: dE unfiltered)")
    ap.add_argument("--vocab-sort", action="store_true",
                    help="take the backward's vocabulary by descending average logit "
                         "(cce_vocab_order + cce_backward_sorted, both inside every step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--tokens", type=int, default=None,
                    help="override the workload's token count N (same V, D and generator)")
    ap.add_argument("--ignored-rows", type=int, default=None,
                    help="override the workload's count of ignore_index rows (seeded positions)")
    ap.add_argument("--literal-beta", action="store_true",
                    help="the generator's literal target margin 0.5*sqrt(D) logit standard "
                         "deviations (a degenerate softmax: nearly every unit filtered)")
    ap.add_argument("--role-split", action="store_true",
                    help="diagnostic: run each role of the backward step in a launch of its own "
                         "and report the roles' times (a slower step than the fused launch)")
    ap.add_argument("--copy-calibration", type=int, metavar="MIB", default=0,
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    ap.add_argument("--hw-probe", action="store_true",
                    help="only measure the device ceilings (MFMA rate, LDS and load bandwidth)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.hw_probe:
        hw_probe()
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (the hot path is a single-GPU kernel); "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic_inputs as si
    import linear_cross_entropy_amd as lce

    w = {x.name: x for x in si.FULL + si.VARIANTS}[args.workload]
    if args.tokens is not None:
        w = dataclasses.replace(w, N=args.tokens)
    if args.ignored_rows is not None:
        w = dataclasses.replace(w, ignore_rows=args.ignored_rows)
    if args.literal_beta:
        w = dataclasses.replace(w, beta=None)
    t0 = time.perf_counter()
    E, C, x = si.generate(w)
    gen_s = time.perf_counter() - t0
    dev = torch.device("cuda:0")
    Ed, Cd, xd = E.to(dev), C.to(dev), x.to(dev)
    N, D = E.shape
    V = C.shape[0]
    grad = si.upstream_grad(w).to(dev)
    torch.cuda.synchronize()
    # device memory in use before the library runs anything (hipMemGetInfo):
    # the delta at the peak below also holds what torch's allocator does not
    # see, such as the library's static per-device arrays
    free0, total_mem = torch.cuda.mem_get_info(dev)
    # memory beyond the resident inputs: the workspace and every output of a step
    base_mem = torch.cuda.memory_allocated(dev)
    torch.cuda.reset_peak_memory_stats(dev)
    fb, bb = lce.cce_workspace_bytes(N, V, D)
    # the forward's workspace is dead once its outputs are written, so one
    # buffer serves both calls (stream order keeps them apart)
    ws = torch.empty(max(fb, bb), dtype=torch.uint8, device=dev)

    def step(stats=False):
        loss, lse = lce.cce_forward(Ed, Cd, xd, -100, w.reduction, workspace=ws)
        order = lce.cce_vocab_order(Ed, Cd, xd, -100, workspace=ws) if args.vocab_sort else None
        out = lce.cce_backward(Ed, Cd, xd, lse, grad, -100, w.reduction, args.eps,
                               with_stats=stats, workspace=ws, filter_mode=args.filter_mode,
                               vocab_order=order)
        return (loss, lse, order) + tuple(out)

    print(f"[bench] {w.name} N={N} V={V} D={D} generated in {gen_s:.1f}s; warmup {args.warmup}",
          file=sys.stderr, flush=True)
    held = step(stats=True)  # every output of one step held while the peak is read
    torch.cuda.synchronize()
    stats = held[-1]
    peak_extra = torch.cuda.max_memory_allocated(dev) - base_mem
    free1, _ = torch.cuda.mem_get_info(dev)
    del held
    for _ in range(args.warmup):
        step()

    lce.profile_enable(True, roles=args.role_split)
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms = t_start.elapsed_time(t_end) / args.steps

    kernels = {}
    for fam in FAMILIES:
        n, tot = lce.profile_query(fam)
        if n:
            kernels[fam] = {"launches_per_step": n / args.steps, "ms_per_step": tot / args.steps}
    lce.profile_enable(False)
    # Timing protocol: a second pass of the same steps with events around the
    # forward and the backward of each step (median, min, max); the headline
    # above comes from the untouched loop.
    fwd_ms, bwd_ms, step_ms = [], [], []
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        loss, lse = lce.cce_forward(Ed, Cd, xd, -100, w.reduction, workspace=ws)
        ev[i][1].record()
        order = lce.cce_vocab_order(Ed, Cd, xd, -100, workspace=ws) if args.vocab_sort else None
        lce.cce_backward(Ed, Cd, xd, lse, grad, -100, w.reduction, args.eps, workspace=ws,
                         filter_mode=args.filter_mode, vocab_order=order)
        ev[i][2].record()
    torch.cuda.synchronize()
    for e0, e1, e2 in ev:
        fwd_ms.append(e0.elapsed_time(e1))
        bwd_ms.append(e1.elapsed_time(e2))
        step_ms.append(e0.elapsed_time(e2))

    def dist(v):
        v = sorted(v)
        m = len(v) // 2
        med = v[m] if len(v) % 2 else 0.5 * (v[m - 1] + v[m])
        return {"median": round(med, 4), "min": round(v[0], 4), "max": round(v[-1], 4)}

    try:
        mfma_peak = mfma_probe_tflops()
    except RuntimeError:
        mfma_peak = None
    kept = 1.0 - stats["units_skipped"] / max(stats["units_total"], 1)
    # dC and dE at their kept fractions (1 for the contraction a variant leaves unfiltered)
    kC = 1.0 if args.filter_mode == "full_c" else kept
    kE = 1.0 if args.filter_mode == "full_e" else kept
    dom = max((k for k in kernels if kernel_flops(k, N, V, D) > 0),
              key=lambda k: kernels[k]["ms_per_step"])
    dom_ms = kernels[dom]["ms_per_step"]
    dom_launches = kernels[dom]["launches_per_step"]
    ach = kernel_flops(dom, N, V, D, kC, kE) / (dom_ms * 1e-3) / 1e12
    for k, v in kernels.items():
        f = kernel_flops(k, N, V, D, kC, kE)
        if f:
            v["tflops"] = round(f / (v["ms_per_step"] * 1e-3) / 1e12, 1)
            v["tflops_dense_equivalent"] = round(dense_flops(k, N, V, D) /
                                                 (v["ms_per_step"] * 1e-3) / 1e12, 1)

    traffic, traffic_src = traffic_record(dom, w.name)
    if args.filter_mode != "both":
        traffic, traffic_src = None, "the committed counters were taken with filter_mode both"
    if args.vocab_sort:
        traffic, traffic_src = None, "the committed counters were taken without vocabulary sorting"
    nominal = 8.0 * N * V * D
    # forward and recompute, then dC and dE at their kept fractions
    effective = (4.0 + 2.0 * kC + 2.0 * kE) * N * V * D
    tflops = nominal / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC,
        "value": N / (ms * 1e-3),
        "unit": "tokens/s",
        # the same rate over the rows that are not ignore_index
        "valid_tokens_per_s": int((x != -100).sum()) / (ms * 1e-3),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes of the Gemma 2 2B head, no real weights)",
        "config": {"workload": w.name + ("-as-written" if args.literal_beta else ""),
                   "N": N, "V": V, "D": D, "reduction": w.reduction,
                   "filter_eps": args.eps, "filter_mode": args.filter_mode,
                   "ignored_rows": w.ignore_rows, "vocab_sort": bool(args.vocab_sort),
                   "role_split": bool(args.role_split)},
        "pct_bf16_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
        "tflops_nominal": round(tflops, 1),
        "tflops_effective": round(effective / (ms * 1e-3) / 1e12, 1),
        # the same nominal rate against this device's measured MFMA rate (bf16
        # 16x16x32 on register operands, random values: the chip's power limit)
        "mfma_probe_tflops": round(mfma_peak, 1) if mfma_peak else None,
        "pct_measured_mfma_peak": round(100.0 * tflops / mfma_peak, 2) if mfma_peak else None,
        "timing": {"steps": args.steps, "step_ms": dist(step_ms), "fwd_ms": dist(fwd_ms),
                   "bwd_ms": dist(bwd_ms),
                   "note": "a second pass with events around each step's forward and backward"},
        "filter": {"units_total": stats["units_total"], "units_skipped": stats["units_skipped"],
                   "unit": "32x32", "kept_fraction": round(kept, 4)},
        "peak_extra_mem_MiB": round(peak_extra / 2 ** 20, 1),
        # hipMemGetInfo: device memory in use with every output of a step held, less
        # before the first library call (torch's cached blocks and the library's
        # static arrays included)
        "device_used_extra_MiB": round((free0 - free1) / 2 ** 20, 1),
        # dE + dC in bf16: the least any method can hold
        "mem_lower_bound_MiB": round((N * D + V * D) * 2 / 2 ** 20, 1),
        "roofline": {
            "kernel": dom,
            "bound": "mfma",
            "achieved": round(ach, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(ach / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_source": traffic_src,
            "dense_equivalent_frac": round(dense_flops(dom, N, V, D) / (dom_ms * 1e-3) / 1e12 /
                                           PEAK_BF16_TFLOPS, 4),
            "per_launch": f"{kernel_flops(dom, N, V, D, kC, kE) / dom_launches:.4g} flops "
                          f"(method's work: recompute + dC, dE at kept fraction {kept:.4f}) avg "
                          f"over {dom_launches:g} launches per step, "
                          f"{dom_ms / dom_launches:.3f} ms avg",
        },
        "kernels": kernels,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, E, C, x, args.eps, filter_mode=args.filter_mode,
                                           vocab_sort=args.vocab_sort)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
