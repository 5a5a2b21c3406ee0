"""Benchmark: NVFP4 Four Over Six quantization on one MI355X.

One step is one pass of the whole hot path over one synthetic tensor: the amax
pass (clear + streaming max), then the block pass (alpha, both candidate scales,
FP4 rounding, error, selection, packed codes + E4M3 scales).  The step calls the
two C-ABI entry points nvfp4_amax and nvfp4_quantize_from_amax back to back --
the same kernels, in the same order, as nvfp4_quantize -- so that HIP events on
the launch stream can time each pass inside the timed region.

Default workload: the 4096 x 14336 bf16 weight (N(0, 0.02^2), 0.1 % of entries
x20), Four Over Six with the MSE rule, packed output.  Inputs are generated once
on the host, copied to HBM and rotated over enough copies that every step reads
data that the 256 MB Infinity Cache no longer holds.

Printed: one JSON line (see the keys below).  value = algorithmic bytes of a step
(2 B/elem amax read + 2.5625 B/elem block pass) / step time, in GB/s.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 4/6 quantize GB/s (bf16 in) and % of HBM peak; 4/6-vs-rtn6 overhead"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MALL_BYTES = 256 << 20          # Infinity Cache
AMAX_BPE = 2.0                  # bytes per element: bf16 read
PACKED_BPE = 2.0 + 0.5 + 1.0 / 16   # bf16 read + 4-bit code + 1 scale byte per 16
FQ_BPE = 4.0                    # bf16 read + bf16 write
KERNEL_SRC = os.path.join(ROOT, "nvfp4_block_scaled_amax_amd", "csrc", "nvfp4_amax.hip")
COUNTERS = os.path.join(ROOT, "profiles", "quantize_kernel_counters.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_digest() -> str:
    with open(KERNEL_SRC, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()[:16]


def read_counters(workload, mode, rule):
    """HBM traffic per dispatch of the block-pass kernel from the committed rocprofv3
    counter summary, or None when absent or taken on a different kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    want = "%s %s %s" % (workload, mode, rule)
    for line in open(COUNTERS):
        if line.startswith("TRAFFIC "):
            f = dict(kv.split("=", 1) for kv in line.split()[1:])
            if f.get("source") == source_digest() and f.get("case", "").replace(",", " ") == want:
                return float(f["bytes_per_dispatch"])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="weight")
    ap.add_argument("--mode", default="four_over_six")
    ap.add_argument("--rule", default="mse")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="timed steps only (for rocprofv3 runs): no extra legs")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import nvfp4_block_scaled_amax_amd as nv
    from nvfp4_block_scaled_amax_amd import workloads as W

    nv.lib()                                   # raises if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    wl = W.WORKLOADS[args.workload]
    fq = any(o == "fakequant" for (m, r, o) in wl.runs if (m, r) == (args.mode, args.rule))
    log("[bench] generating %s %s" % (wl.name, wl.shape))
    x_cpu = W.generate(wl.name)
    N = x_cpu.numel()
    E = wl.shape[0] if len(wl.shape) == 3 else 1
    step_bpe = AMAX_BPE + (FQ_BPE if fq else PACKED_BPE)
    pass_bpe = FQ_BPE if fq else PACKED_BPE
    one_set = N * 2 + (N * 2 if fq else N // 2 + N // 16)
    R = max(2, math.ceil(3 * MALL_BYTES / one_set) + 1)
    log("[bench] %d rotating buffer sets of %.1f MB" % (R, one_set / 1e6))
    xs = [x_cpu.to(dev) for _ in range(R)]
    lead = (E,) if len(wl.shape) == 3 else ()
    rows, cols = wl.shape[-2], wl.shape[-1]
    if fq:
        outs = [torch.empty_like(xs[0]) for _ in range(R)]
    else:
        outs = [(torch.empty(lead + (rows, cols // 2), dtype=torch.uint8, device=dev),
                 torch.empty(lead + (rows, cols // 16), dtype=torch.uint8, device=dev))
                for _ in range(R)]
    amaxs = [torch.empty(E, dtype=torch.float32, device=dev) for _ in range(R)]
    alphas = [torch.empty(E, dtype=torch.float32, device=dev) for _ in range(R)]

    def block_pass(i, mode, rule):
        if fq:
            nv.fakequant_from_amax(xs[i], amaxs[i], mode, rule, out=outs[i], alpha=alphas[i])
        else:
            nv.quantize_from_amax(xs[i], amaxs[i], mode, rule, codes=outs[i][0],
                                  scales=outs[i][1], alpha=alphas[i])

    def step(i):
        nv.amax(xs[i], out=amaxs[i])
        block_pass(i, args.mode, args.rule)

    for s in range(args.warmup):
        step(s % R)
    torch.cuda.synchronize()

    # ---- timed region: K steps, HIP events between the two passes on the launch stream
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        i = s % R
        ev[s][0].record()
        nv.amax(xs[i], out=amaxs[i])
        ev[s][1].record()
        block_pass(i, args.mode, args.rule)
        ev[s][2].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    amax_us = np.array([e[0].elapsed_time(e[1]) * 1e3 for e in ev])
    pass_us = np.array([e[1].elapsed_time(e[2]) * 1e3 for e in ev])
    value = step_bpe * N / (ms_step * 1e-3) / 1e9

    pass_gbps = pass_bpe * N / (pass_us.mean() * 1e-6) / 1e9
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (wl.name, wl.description), "shape": list(wl.shape),
                   "elements": N, "mode": args.mode, "rule": args.rule,
                   "output": "fakequant" if fq else "packed", "block": 16,
                   "rotating_buffer_sets": R},
    }
    traffic = read_counters(wl.name, args.mode, args.rule)
    result["roofline"] = {
        "bound": "hbm", "achieved": round(pass_gbps, 1), "peak": HBM_PEAK_GBPS,
        "unit": "GB/s", "frac": round(pass_gbps / HBM_PEAK_GBPS, 4),
        "traffic": traffic,
        "kernel": "quantize_kernel<%s,%s,%s>" % (args.mode, args.rule, "fq" if fq else "packed"),
        "bytes_per_launch": int(pass_bpe * N), "avg_launch_us": round(float(pass_us.mean()), 2),
    }
    result["passes"] = {
        "amax": {"avg_us": round(float(amax_us.mean()), 2), "p50_us": round(float(np.median(amax_us)), 2),
                 "GBps": round(AMAX_BPE * N / (amax_us.mean() * 1e-6) / 1e9, 1)},
        "block": {"avg_us": round(float(pass_us.mean()), 2), "p50_us": round(float(np.median(pass_us)), 2),
                  "p10_us": round(float(np.percentile(pass_us, 10)), 2),
                  "p90_us": round(float(np.percentile(pass_us, 90)), 2),
                  "GBps": round(pass_gbps, 1), "frac_hbm": round(pass_gbps / HBM_PEAK_GBPS, 4)},
    }

    if args.profile:
        # a plain device copy of known size (256 MiB read + 256 MiB written), so that a
        # counter run of this command can calibrate FETCH_SIZE / WRITE_SIZE against it
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    else:
        # ---- block pass alone on cold buffers (no amax pass before it), and rtn6 on the same
        def time_pass(mode, rule, reps):
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
            for r in range(reps):
                i = r % R
                evs[r][0].record()
                block_pass(i, mode, rule)
                evs[r][1].record()
            torch.cuda.synchronize()
            return np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        for i in range(R):
            nv.amax(xs[i], out=amaxs[i])
        torch.cuda.synchronize()
        reps = max(K, 2 * R)
        cold46 = time_pass(args.mode, args.rule, reps)
        cold6 = time_pass("rtn6", "mse", reps)
        cold46b = time_pass(args.mode, args.rule, reps)
        t46 = float(np.median(np.concatenate([cold46, cold46b])))
        t6 = float(np.median(cold6))
        result["passes"]["block_cold"] = {"p50_us": round(t46, 2),
                                          "GBps": round(pass_bpe * N / (t46 * 1e-6) / 1e9, 1)}
        result["passes"]["rtn6_block_cold"] = {"p50_us": round(t6, 2),
                                               "GBps": round(pass_bpe * N / (t6 * 1e-6) / 1e9, 1)}
        result["overhead_4over6_vs_rtn6"] = round(t46 / t6 - 1.0, 4)

        # ---- the single-call dynamic entry point end to end (4 launches)
        evs = []
        for r in range(reps):
            i = r % R
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            if fq:
                nv.fakequant(xs[i], args.mode, args.rule, out=outs[i], alpha=alphas[i])
            else:
                nv.quantize(xs[i], args.mode, args.rule, codes=outs[i][0], scales=outs[i][1],
                            alpha=alphas[i])
            b.record()
            evs.append((a, b))
        torch.cuda.synchronize()
        e2e = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
        result["passes"]["dynamic_entry_point"] = {"p50_us": round(float(np.median(e2e)), 2)}

        # ---- device copy bandwidth (read + write), a second denominator
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(10):
            dst.copy_(src)
        b.record()
        torch.cuda.synchronize()
        copy_gbps = 10 * 2 * src.numel() / (a.elapsed_time(b) * 1e-3) / 1e9
        result["copy_GBps"] = round(copy_gbps, 1)
        result["passes"]["block"]["frac_copy"] = round(pass_gbps / copy_gbps, 4)
        del src, dst

    if not args.no_cpu_baseline and not args.profile:
        result["cpu_baseline"] = cpu_baseline(x_cpu, wl, args, step_bpe)

    print(json.dumps(result), flush=True)


def cpu_baseline(x_cpu, wl, args, step_bpe):
    """The CPU oracle (untuned, test infrastructure) on a bounded sample of the workload:
    the leading rows of the tensor (of the first experts for batched workloads), the whole
    hot path (amax + block pass), on the host's cores."""
    import numpy as np

    import oracle
    from nvfp4_block_scaled_amax_amd import workloads as W
    cores = max(1, min(16, os.cpu_count() or 1))
    x = W.bits(x_cpu)
    if x.ndim == 3:
        sample = x[:2]
        desc = "first 2 of %d experts (%d elements)" % (x.shape[0], sample.size)
    else:
        rows = min(x.shape[0], max(1, (64 * 1024 * 1024) // x.shape[1]))
        sample = x[:rows]
        desc = "first %d of %d rows (%d elements)" % (rows, x.shape[0], sample.size)
    oracle.build()
    reps, times = 0, []
    while reps < 20 and (reps < 3 or sum(times) < 10.0):     # about 10 s of wall clock
        t0 = time.perf_counter()
        oracle.quantize(sample, args.mode, args.rule, nthreads=cores, want_y=False)
        times.append(time.perf_counter() - t0)
        reps += 1
    dt = float(np.median(times))
    return {"value": round(step_bpe * sample.size / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "sample": desc + ", median of %d runs" % reps,
            "seconds_per_run": round(dt, 3)}


if __name__ == "__main__":
    main()
