"""Benchmark: NVFP4 Four Over Six quantization on one MI355X.

One step is one pass of the whole hot path over one synthetic input: the amax
pass (clear + streaming max), then the block pass (alpha, both candidate scales,
FP4 rounding, error, selection, packed codes + E4M3 scales).  The step calls the
C-ABI entry points nvfp4_amax and nvfp4_quantize_from_amax back to back -- the
kernels of nvfp4_quantize_batched, in the same order.

Default workload: the largest configuration, a mixture-of-experts weight batch of
64 experts of 2048 x 5120 bf16 (expert e: sigma_e * N(0, 1), sigma_e
log-uniform in [0.005, 0.05]), Four Over Six with the MSE rule, packed output,
one alpha per expert, one launch per pass.  `--workload weight|act|large|tiny`
selects the other configurations.  Inputs are generated once on the host,
copied to HBM and rotated over enough copies that each step starts on data the
256 MB Infinity Cache no longer holds.

Timing:
  * timed region: K steps captured as one HIP graph, uploaded to the device
    (hipGraphUpload) and replayed once, bracketed by torch.cuda.synchronize() (so
    host launch overhead is not timed); gives
    ms_per_step and value = the operation's own bytes / step time: the bf16
    input once plus the codes and scales out (2.5625 B/elem), or the bf16 input
    and output (4 B/elem fake-quant).  The HBM bytes the two-pass step moves
    (the amax pass reads the input a second time: 4.5625 or 6 B/elem) are
    reported separately as hbm_bytes_per_step.
  * per-kernel legs: graphs of back-to-back launches of one pass over rotating
    cold buffers, one untimed replay, then HIP events recorded on the launch stream
    before and after each of 5 replays; the average launch of the block pass is the
    roofline figure.  Also
    timed this way: the rtn6 block pass, the amax pass, the two-pass and the
    single-read dynamic calls, the diagnostics call (with and without error
    statistics) and dequantize (packed -> bf16).
Printed: one JSON line.
"""
from __future__ import annotations

import argparse
import ctypes
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
DEQUANT_BPE = 0.5 + 1.0 / 16 + 2.0   # 4-bit code + scale byte read, bf16 written
KERNEL_SRC = os.path.join(ROOT, "nvfp4_block_scaled_amax_amd", "csrc", "nvfp4_amax.hip")
COUNTERS = os.path.join(ROOT, "profiles", "quantize_kernel_counters.txt")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


_HIP = None


def graph_upload(g, stream):
    """hipGraphUpload of an instantiated graph before its first replay.  Otherwise the first
    replay pays for the upload: on the 20-step MoE graph, 583 against 520 us per step."""
    global _HIP
    if _HIP is None:
        _HIP = ctypes.CDLL("libamdhip64.so")
    rc = _HIP.hipGraphUpload(ctypes.c_void_p(g.raw_cuda_graph_exec()),
                             ctypes.c_void_p(stream.cuda_stream))
    if rc != 0:
        raise RuntimeError("hipGraphUpload failed (%d)" % rc)


def source_digest(path: str = KERNEL_SRC) -> str:
    """First 16 hex digits of the SHA-256 of the kernel source's code: comments and white space
    removed (string and character literals kept as written), so that an edit to comments or
    layout alone keeps the committed counters, and any change to device or host code drops
    them."""
    text = open(path, encoding="utf-8").read()
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                                    # string or character literal
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    code = "".join("".join(out).split())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def read_counters(workload, mode, rule):
    """HBM bytes per dispatch of the block-pass kernel from the committed rocprofv3 counter
    summary (FETCH_SIZE and WRITE_SIZE, each scaled by a plain copy's reading), or None when
    absent or taken on a different kernel source."""
    if not os.path.exists(COUNTERS):
        return None
    want = "%s,%s,%s" % (workload, mode, rule)
    for line in open(COUNTERS):
        if line.startswith("TRAFFIC "):
            f = dict(kv.split("=", 1) for kv in line.split()[1:])
            if f.get("source") == source_digest() and f.get("case") == want:
                return int(float(f["bytes_per_dispatch"]))
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--workload", default="moe")
    ap.add_argument("--mode", default="four_over_six")
    ap.add_argument("--rule", default="mse")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="counter runs: add a plain 256 MiB device copy (calibration), "
                         "skip the CPU baseline")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path; a tensor "
              "would be sharded by rows with one all-reduce(MAX) of its amax "
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
    pass_bpe = FQ_BPE if fq else PACKED_BPE
    step_bpe = AMAX_BPE + pass_bpe
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

    def block_pass(i, mode=args.mode, rule=args.rule):
        if fq:
            nv.fakequant_from_amax(xs[i], amaxs[i], mode, rule, out=outs[i], alpha=alphas[i])
        else:
            nv.quantize_from_amax(xs[i], amaxs[i], mode, rule, codes=outs[i][0],
                                  scales=outs[i][1], alpha=alphas[i])

    def amax_pass(i):
        nv.amax(xs[i], out=amaxs[i])

    def step(i):
        amax_pass(i)
        block_pass(i)

    def dynamic_call(i):
        if fq:
            nv.fakequant(xs[i], args.mode, args.rule, out=outs[i], alpha=alphas[i])
        else:
            nv.quantize(xs[i], args.mode, args.rule, codes=outs[i][0], scales=outs[i][1],
                        alpha=alphas[i])

    ws = torch.empty(nv.FUSED_WS_WORDS * E, dtype=torch.int32, device=dev)
    # packed inputs for the dequantize leg, and outputs for it and for the diagnostics leg
    if fq:
        pk = [(torch.empty(lead + (rows, cols // 2), dtype=torch.uint8, device=dev),
               torch.empty(lead + (rows, cols // 16), dtype=torch.uint8, device=dev))
              for _ in range(R)]
        ys = outs
    else:
        pk = outs
        ys = [torch.empty_like(xs[0]) for _ in range(R)]
    qstar = [torch.empty_like(pk[0][1]) for _ in range(R)]
    count4 = torch.empty(E, dtype=torch.int32, device=dev)
    stats = torch.empty((E, len(nv.STATS)), dtype=torch.float64, device=dev)
    stats_ws = torch.empty(nv.diag_ws_words(E), dtype=torch.int32, device=dev)

    def dequant_call(i):
        nv.dequantize(pk[i][0], pk[i][1], alphas[i], out=ys[i])

    def diag_call(i, with_stats):
        st = nv.lib().nvfp4_quantize_diag(
            xs[i].data_ptr(), E, rows, cols, 16, nv.MODES[args.mode], nv.RULES[args.rule],
            pk[i][0].data_ptr(), pk[i][1].data_ptr(), alphas[i].data_ptr(),
            qstar[i].data_ptr(), count4.data_ptr(), stats.data_ptr() if with_stats else None,
            stats_ws.data_ptr() if with_stats else None, torch.cuda.current_stream().cuda_stream)
        assert st == 0, st

    def fused_call(i):
        if fq:
            nv.fakequant_fused(xs[i], args.mode, args.rule, out=outs[i], alpha=alphas[i],
                               workspace=ws)
        else:
            nv.quantize_fused(xs[i], args.mode, args.rule, codes=outs[i][0], scales=outs[i][1],
                              alpha=alphas[i], workspace=ws)

    def capture(fn, count):
        """One HIP graph of `count` back-to-back calls fn(0), fn(1), ... (buffers mod R)."""
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(min(count, R)):
                fn(i % R)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(count):
                fn(i % R)
        graph_upload(g, torch.cuda.current_stream())
        torch.cuda.synchronize()
        return g

    def replay_us(g, count, reps=5):
        """(events around one replay) / count in microseconds, over reps replays after one
        untimed replay: (median, min, max)."""
        g.replay()
        torch.cuda.synchronize()
        out = []
        for _ in range(reps):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            g.replay()
            b.record()
            torch.cuda.synchronize()
            out.append(a.elapsed_time(b) * 1e3 / count)
        return float(np.median(out)), float(np.min(out)), float(np.max(out))

    # ---- per-kernel legs: back-to-back launches of one pass over cold rotating buffers
    B = max(4 * R, 32)
    for i in range(R):
        amax_pass(i)
        if fq:      # packed codes of the same tensor for the dequantize leg
            nv.quantize_from_amax(xs[i], amaxs[i], args.mode, args.rule, codes=pk[i][0],
                                  scales=pk[i][1], alpha=alphas[i])
    torch.cuda.synchronize()
    legs, spread = {}, {}
    for name, fn in (("block", block_pass),
                     ("rtn6_block", lambda i: block_pass(i, "rtn6", "mse")),
                     ("block_again", block_pass),          # 4/6 once more: drift check
                     ("amax", amax_pass),
                     ("dynamic_entry_point", dynamic_call),
                     ("fused_entry_point", fused_call),
                     ("diagnostics", lambda i: diag_call(i, False)),
                     ("diagnostics_with_stats", lambda i: diag_call(i, True)),
                     ("dequantize", dequant_call),
                     ("block_warm", lambda i: block_pass(0))):   # one buffer set: input in cache
        g = capture(fn, B)
        legs[name], lo, hi = replay_us(g, B)
        spread[name] = [round(lo, 2), round(hi, 2)]
        del g
        log("[bench] leg %s: %.2f us per launch (min %.2f, max %.2f over replays)"
            % (name, legs[name], lo, hi))
    # ---- timed region: K steps in one graph, replayed once.  It runs after the per-kernel
    # legs, so that the GPU has been busy for a while when it starts (right after the inputs are
    # generated, the first steps ran up to 6 % slower than in steady state).
    K = args.steps
    log("[bench] capturing %d warmup + %d timed steps" % (args.warmup, K))
    g_warm = capture(step, max(1, args.warmup))
    g_steps = capture(step, K)
    g_warm.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g_steps.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    value = pass_bpe * N / (ms_step * 1e-3) / 1e9          # the operation's own bytes
    # a second replay, outside the timed region, with events: the steady-state step time
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    g_steps.replay()
    b.record()
    torch.cuda.synchronize()
    again_us = a.elapsed_time(b) * 1e3 / K
    del g_warm, g_steps
    log("[bench] timed region: %.1f us/step (a second replay: %.1f us/step)"
        % (ms_step * 1e3, again_us))

    block_leg = "block" if legs["block"] <= legs["block_again"] else "block_again"
    t_block = legs[block_leg]
    t_rtn6 = legs["rtn6_block"]
    block_gbps = pass_bpe * N / (t_block * 1e-6) / 1e9

    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "%s: %s" % (wl.name, wl.description), "shape": list(wl.shape),
                   "elements": N, "mode": args.mode, "rule": args.rule,
                   "output": "fakequant" if fq else "packed", "block": 16,
                   "rotating_buffer_sets": R, "timed_as": "one HIP graph of K steps",
                   "input_sha256": W.sha256(x_cpu)[:16]},
        "roofline": {
            "bound": "hbm", "achieved": round(block_gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(block_gbps / HBM_PEAK_GBPS, 4),
            "traffic": read_counters(wl.name, args.mode, args.rule),
            "kernel": "quantize_kernel<%s,%s,%s>" % (args.mode, args.rule,
                                                     "fakequant" if fq else "packed"),
            "bytes_per_launch": int(pass_bpe * N), "avg_launch_us": round(t_block, 2),
            "launches_timed": B, "buffers": "cold (rotating)",
        },
        "passes": {
            "block": {"avg_us": round(t_block, 2), "GBps": round(block_gbps, 1),
                      "frac_hbm": round(block_gbps / HBM_PEAK_GBPS, 4),
                      "Gelem_per_s": round(N / (t_block * 1e-6) / 1e9, 2),
                      "replay_min_max_us": spread[block_leg],
                      "warm_avg_us": round(legs["block_warm"], 2)},
            "rtn6_block": {"avg_us": round(t_rtn6, 2),
                           "GBps": round(pass_bpe * N / (t_rtn6 * 1e-6) / 1e9, 1),
                           "replay_min_max_us": spread["rtn6_block"]},
            "amax": {"avg_us": round(legs["amax"], 2),
                     "GBps": round(AMAX_BPE * N / (legs["amax"] * 1e-6) / 1e9, 1),
                     "replay_min_max_us": spread["amax"]},
            "step": {"Gelem_per_s": round(N / (ms_step * 1e-3) / 1e9, 2),
                     "op_bytes_per_step": int(pass_bpe * N),
                     "hbm_bytes_per_step": int(step_bpe * N),
                     "hbm_GBps": round(step_bpe * N / (ms_step * 1e-3) / 1e9, 1),
                     "second_replay_us_per_step": round(again_us, 2)},
            "dynamic_entry_point": {"avg_us": round(legs["dynamic_entry_point"], 2)},
            "fused_entry_point": {
                "avg_us": round(legs["fused_entry_point"], 2),
                "blocks_per_lane": nv.fused_blocks_per_lane(wl.shape, args.mode, args.rule, fq),
                "GBps": round(pass_bpe * N / (legs["fused_entry_point"] * 1e-6) / 1e9, 1),
                "speedup_vs_dynamic": round(legs["dynamic_entry_point"] /
                                            legs["fused_entry_point"], 3)},
            "diagnostics": {"avg_us": round(legs["diagnostics"], 2),
                            "with_stats_avg_us": round(legs["diagnostics_with_stats"], 2)},
            "dequantize": {"avg_us": round(legs["dequantize"], 2),
                           "GBps": round(DEQUANT_BPE * N / (legs["dequantize"] * 1e-6) / 1e9, 1)},
        },
        "overhead_4over6_vs_rtn6": round(t_block / t_rtn6 - 1.0, 4),
    }

    # ---- device copy bandwidth (read + write of 1 GiB), a second denominator
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
    result["passes"]["block"]["frac_copy"] = round(block_gbps / copy_gbps, 4)
    del src, dst
    if args.profile:
        # a plain device copy of known size (256 MiB read + 256 MiB written), so that a
        # counter run of this command can calibrate FETCH_SIZE / WRITE_SIZE against it
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_cpu_baseline and not args.profile:
        result["cpu_baseline"] = cpu_baseline(x_cpu, wl, args, pass_bpe)

    print(json.dumps(result), flush=True)


def cpu_threads():
    """(threads used, CPUs this process may run on, CPUs the host reports).  The oracle runs
    on every CPU it may use, up to 16: a one-GPU machine allots 16 host CPUs to its GPU, whatever
    the host reports."""
    host = os.cpu_count() or 1
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = host
    return max(1, min(16, usable)), usable, host


def cpu_baseline(x_cpu, wl, args, bpe):
    """The CPU oracle (untuned, test infrastructure) on a bounded sample of the workload:
    the whole hot path (amax + block pass) on the leading rows of the tensor (the first
    experts for batched workloads), on the host's cores; median of repeated runs.  GB/s on
    the same bytes as the GPU value (the operation's own bytes)."""
    import numpy as np

    import oracle
    from nvfp4_block_scaled_amax_amd import workloads as W
    cores, usable, host = cpu_threads()
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
    while reps < 60 and (reps < 3 or sum(times) < 12.0):     # about 12 s of wall clock
        t0 = time.perf_counter()
        oracle.quantize(sample, args.mode, args.rule, nthreads=cores, want_y=False)
        times.append(time.perf_counter() - t0)
        reps += 1
    dt = float(np.median(times))
    # one thread, on the first eighth of the sample (about 1 s per run), median of 3
    small = sample[: max(1, sample.shape[0] // 8)]
    t1 = []
    for _ in range(3):
        t0 = time.perf_counter()
        oracle.quantize(small, args.mode, args.rule, nthreads=1, want_y=False)
        t1.append(time.perf_counter() - t0)
    dt1 = float(np.median(t1))
    return {"value": round(bpe * sample.size / dt / 1e9, 4), "unit": "GB/s", "cores": cores,
            "kind": "oracle", "sample": desc + ", median of %d runs" % reps,
            "seconds_per_run": round(dt, 3), "cpu_model": cpu_model(),
            "host_cpus": host, "usable_cpus": usable,
            "threads_note": "the oracle's threads: every usable CPU up to 16, the host CPUs "
                            "a one-GPU box allots to its GPU",
            "single_thread": {"value": round(bpe * small.size / dt1 / 1e9, 4),
                              "unit": "GB/s", "cores": 1,
                              "sample": "first %d elements of that sample, median of 3 runs"
                                        % small.size,
                              "seconds_per_run": round(dt1, 3)}}


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
