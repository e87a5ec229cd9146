"""Benchmark: tiled GEMM TFLOP/s on one MI355X, with roofline and CPU baseline.

A step is one call of the library's GEMM on the bf16 4096 x 4096 x 4096 workload
with the fused ReLU epilogue (row-major A and B, N(0,1) entries cast to bf16,
fp32 accumulation, bf16 output), inputs already resident in HBM.  W untimed
warm-up steps, then K timed steps between a synchronize on each side.

Warm-up: at least W steps and at least WARM_MS of back-to-back launches.  After
the seconds of host-side input generation the card sits at idle clocks, and
this kernel only settles at its sustained speed after about 30 ms of launches
(measured: 126 us for the first 50 launches, 107 us from launch 300 on).  The
launches actually run are reported as ``warmup_launches``.

Printed: ONE JSON line (rank 0) with
  value         whole-job TFLOP/s = 2 M N K * K_steps / elapsed (host clock),
  roofline      the kernel's average duration (HIP events recorded on the
                stream it runs on, around the K timed launches), against the
                bf16 dense MFMA peak; the per-launch median / p10 / p90 of a
                separate pass; the shader clock the kernel ran at (the
                library's clock record: shader-clock counter against the
                100 MHz reference counter inside the kernel, one workgroup per
                XCD) and the fraction of the peak at that clock,
  cpu_baseline  the C oracle timed on host cores on a bounded row sample,
  workloads     the other workload shapes, each timed the same way with warm
                caches (same buffers) and cold caches (operands rotated over
                copies larger than the 256 MB MALL), with the oracle timed on
                a row sample of each.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "GEMM TFLOP/s and % of MI355X dense MFMA peak (4096³ bf16/fp32, 1 GPU)"
# MI355X dense matrix peaks (256 CUs at 2.4 GHz): bf16/fp16 4096 FLOP/clk/CU,
# fp32 256 FLOP/clk/CU; HBM3E 8 TB/s.
PEAK_CLOCK_GHZ = 2.4
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3,
               # scaled MFMA: E2M1 x E2M1 at the fp4 rate, E4M3 x E2M1 at the fp8 rate
               "mx_e2m1": 10066.3, "mx_e4m3": 5033.2,
               # 2:4 sparse MFMA, dense-equivalent rate (twice the dense bf16/fp16 rate)
               "sp24_bf16": 5033.2, "sp24_f16": 5033.2}
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_4096_relu"
OTHER = ["f32_4096", "bf16_4000x4032x4096_relu", "f16_1024", "f32_512", "w4_256x8192x8192",
         "w4_16x8192x8192", "w4_1x8192x8192", "mx_e2m1_8192", "mx_e4m3_8192",
         "sp24_bf16_4096_relu", "bf16_6144x4096x4096_relu", "bf16_3072_relu"]
# Workloads whose run time is the operand stream from HBM: their headline
# bandwidth is the cold-cache one.
MEMORY_BOUND = ("w4_1x8192x8192", "w4_16x8192x8192")
WARM_MS = 40.0      # GPU work before a workload's timed launches (clock ramp-up)
COLD_BYTES = 1 << 30  # operand copies rotated by the cold timing (> 256 MB MALL)
CLOCK_MS = 400.0    # back-to-back launches while the shader clock is recorded


def load_traffic(workload: str):
    """Fabric bytes per launch from the committed rocprofv3 counter summary, if
    it was taken with the configuration and swizzle group the library launches
    now and on that kernel's current sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from tiled_dense_gemm_07_amd.traffic import source_hash, workload_launch

    config, group = workload_launch(workload)
    if (rec.get("config") != config or rec.get("group_m") != group or
            rec.get("source_hash") != source_hash(config)):
        return None
    return rec


def make_device_inputs(w, dev):
    import numpy as np
    import torch

    from tiled_dense_gemm_07_amd import synth

    inp = synth.make_inputs(w, integer=False)
    tdt = {synth.F32: torch.float32, synth.F16: torch.float16, synth.BF16: torch.bfloat16}
    if w.op == "gemm":
        view = np.int32 if w.dtype == synth.F32 else np.int16
        A = torch.from_numpy(inp["A"].view(view)).view(tdt[w.dtype]).to(dev)
        B = torch.from_numpy(inp["B"].view(view)).view(tdt[w.dtype]).to(dev)
        C = torch.empty((w.M, w.N), dtype=tdt[w.dtype], device=dev)
        return inp, (A, B, C)
    if w.op == "mx":
        t = tuple(torch.from_numpy(inp[k]).to(dev) for k in ("Aq", "As", "Wq", "Ws"))
        return inp, t + (torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev),)
    if w.op == "sp24":
        Ac = torch.from_numpy(inp["Ac"].view(np.int16)).view(tdt[w.dtype]).to(dev)
        B = torch.from_numpy(inp["B"].view(np.int16)).view(tdt[w.dtype]).to(dev)
        Ai = torch.from_numpy(inp["Ai"]).to(dev)
        return inp, (Ac, Ai, B, torch.empty((w.M, w.N), dtype=tdt[w.dtype], device=dev))
    A = torch.from_numpy(inp["A"].view(np.int16)).view(torch.bfloat16).to(dev)
    Wq = torch.from_numpy(inp["Wq"]).to(dev)
    Ws = torch.from_numpy(inp["Ws"]).to(dev)
    C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
    return inp, (A, Wq, Ws, C)


def launcher(w, tensors, stream):
    from tiled_dense_gemm_07_amd import binding

    epi = "relu" if w.relu else None
    if w.op == "gemm":
        A, B, C = tensors
        return lambda: binding.gemm(A, B, C=C, epilogue=epi, stream=stream)
    if w.op == "sp24":
        Ac, Ai, B, C = tensors
        return lambda: binding.gemm_sp24(Ac, Ai, B, C=C, epilogue=epi, stream=stream)
    if w.op == "mx":
        Aq, As, Wq, Ws, C = tensors
        return lambda: binding.gemm_mx(w.dtype, Aq, As, Wq, Ws, C=C, epilogue=epi, stream=stream)
    A, Wq, Ws, C = tensors
    return lambda: binding.dequant_gemm_w4(A, Wq, Ws, C=C, epilogue=epi, stream=stream)


def launch_ms(fn, stream) -> float:
    """One launch's duration (ms) from an event pair around five launches."""
    import torch

    fn()
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        fn()
    b.record(stream)
    stream.synchronize()
    return max(a.elapsed_time(b) / 5, 1e-3)


def warm_up(fn, stream, warmup: int) -> int:
    """At least `warmup` launches and at least WARM_MS of back-to-back work;
    returns the launches run."""
    n = max(warmup, min(int(WARM_MS / launch_ms(fn, stream)) + 1, 5000))
    for _ in range(n):
        fn()
    stream.synchronize()
    return n + 6


def time_mean(fn, stream, launches: int) -> float:
    """Average kernel duration (ms): one HIP event pair on the kernel's stream
    around `launches` back-to-back launches."""
    import torch

    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(launches):
        fn()
    b.record(stream)
    stream.synchronize()
    return a.elapsed_time(b) / launches


def time_each(fns, stream, launches: int) -> dict:
    """Per-launch durations (ms) from one event pair around each launch
    (launch i runs fns[i % len(fns)]): median, p10, p90, mean.  Each event
    pair adds a few microseconds, so for short kernels these read high: the
    spread, not the level, is what they show (levels come from back-to-back
    timing and from the kernel trace)."""
    import numpy as np
    import torch

    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fns[i % len(fns)]()
        b.record(stream)
    stream.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in evs])
    return {"median_ms": round(float(np.median(t)), 5), "p10_ms": round(float(np.percentile(t, 10)), 5),
            "p90_ms": round(float(np.percentile(t, 90)), 5), "mean_ms": round(float(t.mean()), 5),
            "launches": launches}


def measure_clock(fn, stream, once_ms: float) -> dict:
    """The shader clock the kernel runs at, from the library's clock record:
    CLOCK_MS of back-to-back launches in 20 batches; after each batch, the
    record of its last launch (one workgroup per XCD: shader-clock counter
    against the 100 MHz reference counter at its start and end)."""
    import numpy as np
    import torch

    from tiled_dense_gemm_07_amd import binding

    stamps = torch.zeros(32, dtype=torch.int64, device=torch.device("cuda:0"))
    per = max(5, int(CLOCK_MS / once_ms / 20))
    clocks = []
    binding.set_clock_stamps(stamps)
    try:
        for _ in range(20):
            stamps.zero_()
            for _ in range(per):
                fn()
            stream.synchronize()
            clocks.extend(binding.stamp_clock_ghz(stamps.cpu().tolist()))
    finally:
        binding.set_clock_stamps(None)
    c = np.array(clocks)
    if c.size == 0:
        raise RuntimeError("no clock records")
    return {"sustained_clock_ghz": round(float(np.median(c)), 4),
            "clock_p10_ghz": round(float(np.percentile(c, 10)), 4),
            "clock_p90_ghz": round(float(np.percentile(c, 90)), 4),
            "clock_records": int(c.size),
            "clock_source": "s_memtime / s_memrealtime in workgroups 0-7 of the kernel"}


def time_cold(w, tensors, stream, launches: int = 40) -> dict:
    """Average kernel duration with each launch on a different copy of the
    inputs (together COLD_BYTES or more), so nothing is cache-resident: one
    event pair around back-to-back launches that cycle through the copies
    (an event pair per launch adds several microseconds to each launch)."""
    import torch

    per = sum(x.numel() * x.element_size() for x in tensors)
    copies = max(4, -(-COLD_BYTES // per))
    sets = [tuple(x.clone() for x in tensors) for _ in range(copies)]
    fns = [launcher(w, s_, stream) for s_ in sets]
    n = max(launches, 2 * copies)
    for i in range(n):  # warm-up pass (clocks), itself cold
        fns[i % copies]()
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(n):
        fns[i % copies]()
    b.record(stream)
    stream.synchronize()
    ms = a.elapsed_time(b) / n
    gbs = w.algorithmic_bytes() / (ms * 1e-3) / 1e9
    tf = w.flops / (ms * 1e-3) / 1e12
    del sets, fns
    return {"kernel_ms": round(ms, 5), "launches": n, "copies": copies, "tflops": round(tf, 2),
            "gbs_algorithmic": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def dtype_name(w):
    from tiled_dense_gemm_07_amd import synth

    if w.op == "mx":
        return "mx_" + synth.MX_NAMES[w.dtype]
    if w.op == "sp24":
        return "sp24_" + {synth.F16: "f16", synth.BF16: "bf16"}[w.dtype]
    return {synth.F32: "f32", synth.F16: "f16", synth.BF16: "bf16"}[w.dtype]


def oracle_rows(w, inp, rows: int):
    """The oracle on rows 0 .. rows-1 of C (every row is an independent sum)."""
    import numpy as np

    import oracle

    if w.op == "gemm":
        return oracle.gemm_f64(np.ascontiguousarray(inp["A"][:rows]), inp["B"], w.dtype, w.relu)
    if w.op == "dequant_w4":
        return oracle.dequant_w4_f64(np.ascontiguousarray(inp["A"][:rows]), inp["Wq"], inp["Ws"],
                                     w.relu)
    if w.op == "mx":
        return oracle.mx_gemm_f64(w.dtype, np.ascontiguousarray(inp["Aq"][:rows]),
                                  np.ascontiguousarray(inp["As"][:rows]), inp["Wq"], inp["Ws"],
                                  w.relu)
    return oracle.gemm_sp24_f64(np.ascontiguousarray(inp["Ac"][:rows]),
                                np.ascontiguousarray(inp["Ai"][:rows]), inp["B"], w.dtype, w.relu)


def cpu_baseline(w, inp, budget_s: float) -> dict:
    """The oracle, as it stands, on the first R rows of C; R grows until one
    call takes about a quarter of the budget (or covers all of C)."""
    import oracle

    rows = 1
    while True:
        t0 = time.perf_counter()
        oracle_rows(w, inp, rows)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s / 4 or rows >= w.M:
            break
        rows = min(w.M, max(rows * 2, int(rows * (budget_s / 4) / max(elapsed, 1e-3))))
    flops = 2.0 * rows * w.N * w.K
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s",
            "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "rows 0..%d of C for the %s workload (%d x %d x %d fp64 sums, %.2f s)"
                      % (rows - 1, w.name, rows, w.N, w.K, elapsed),
            "seconds": round(elapsed, 3)}


def bench_workload(name, dev, stream, cpu_budget_s):
    import torch

    from tiled_dense_gemm_07_amd import binding, synth

    ow = synth.WORKLOADS[name]
    inp, t = make_device_inputs(ow, dev)
    fn = launcher(ow, t, stream)
    warm_up(fn, stream, 5)
    mean_ms = time_mean(fn, stream, 30)
    dist = time_each([fn], stream, 50)
    tf = ow.flops / (mean_ms * 1e-3) / 1e12
    gbs = ow.algorithmic_bytes() / (mean_ms * 1e-3) / 1e9
    dn = dtype_name(ow)
    rec = {
        "kernel_ms": round(mean_ms, 5), "tflops": round(tf, 2),
        "frac_mfma_peak": round(tf / PEAK_TFLOPS[dn], 4),
        "gbs_algorithmic": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
        "per_launch": dist,
        "config": binding.query_config({"gemm": 0, "dequant_w4": 1, "mx": 2, "sp24": 3}[ow.op],
                                       ow.M, ow.N, ow.K, ow.dtype)}
    try:
        ck = measure_clock(fn, stream, mean_ms)
        rec["sustained_clock_ghz"] = ck["sustained_clock_ghz"]
        rec["frac_mfma_peak_at_clock"] = round(
            tf / (PEAK_TFLOPS[dn] * ck["sustained_clock_ghz"] / PEAK_CLOCK_GHZ), 4)
    except Exception as e:
        rec["sustained_clock_ghz"] = "unavailable: %s" % e
    rec["cold"] = time_cold(ow, t, stream)
    tr = load_traffic(name)
    if tr is not None:
        # L2 <-> fabric bytes per launch from the committed counter record
        rec["fabric_bytes_per_launch"] = int(tr["fabric_bytes_per_launch"])
        rec["fabric_over_algorithmic"] = round(tr["fabric_bytes_per_launch"] /
                                               ow.algorithmic_bytes(), 3)
        if tr.get("cold"):
            # counters taken on the cold rotation: every fabric byte came from HBM
            rec["hbm_gbs_counters_cold"] = round(
                tr["fabric_bytes_per_launch"] / (rec["cold"]["kernel_ms"] * 1e-3) / 1e9, 1)
    del t
    torch.cuda.empty_cache()
    if cpu_budget_s > 0:
        rec["cpu_baseline"] = cpu_baseline(ow, inp, cpu_budget_s)
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
    ap.add_argument("--workloads", default=None,
                    help="comma-separated subset of the other workloads")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch

    from tiled_dense_gemm_07_amd import binding, synth

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    binding.load_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    w = synth.WORKLOADS[HEADLINE]
    inp, tensors = make_device_inputs(w, dev)
    fn = launcher(w, tensors, stream)

    warm = warm_up(fn, stream, args.warmup)
    # timed region: exactly K steps; one event pair on the kernel's stream
    # around them gives the average launch duration (launches run back to
    # back, so this is the kernel's own time plus the gaps between launches)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        fn()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps
    value = w.flops * args.steps / wall / 1e12
    kernel_ms = ev0.elapsed_time(ev1) / args.steps

    achieved = w.flops / (kernel_ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS[dtype_name(w)]
    traffic = load_traffic(HEADLINE)
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic["fabric_bytes_per_launch"] if traffic else None,
                "kernel_ms": round(kernel_ms, 5),
                "algorithmic_flops_per_launch": w.flops,
                "algorithmic_bytes_per_launch": w.algorithmic_bytes()}
    # after the timed region: per-launch distribution and the sustained clock
    roofline["per_launch"] = time_each([fn], stream, 200)
    try:
        ck = measure_clock(fn, stream, kernel_ms)
        roofline.update(ck)
        ghz = ck["sustained_clock_ghz"]
        roofline["peak_at_clock"] = round(peak * ghz / PEAK_CLOCK_GHZ, 1)
        roofline["frac_at_clock"] = round(achieved / roofline["peak_at_clock"], 4)
    except Exception as e:
        roofline["sustained_clock_ghz"] = "unavailable: %s" % e
    roofline["cold"] = time_cold(w, tensors, stream)

    workloads = {}
    if not args.no_workloads:
        names = OTHER if not args.workloads else args.workloads.split(",")
        for name in names:
            workloads[name] = bench_workload(name, dev, stream,
                                             0.0 if args.no_cpu_baseline else 1.5)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp, 12.0)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "warmup_launches": warm,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": HEADLINE, "M": w.M, "N": w.N, "K": w.K, "epilogue": "relu",
                   "layout": "row-major A[M,K], B[K,N]",
                   "kernel": binding.query_config(0, w.M, w.N, w.K, w.dtype)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
