"""Benchmark: tiled GEMM TFLOP/s on one MI355X, with roofline and CPU baseline.

A step is one call of the library's GEMM on the bf16 4096 x 4096 x 4096 workload
with the fused ReLU epilogue (row-major A and B, N(0,1) entries cast to bf16,
fp32 accumulation, bf16 output), inputs already resident in HBM.  W untimed
warm-up steps, then K timed steps between a synchronize on each side.

The default warm-up is long (300 steps, about 35 ms of GEMM work): after the
seconds of host-side input generation the card sits at idle clocks, and back-
to-back launches of this kernel only settle at their sustained speed after
about 30 ms (measured: 126 us for the first 50 launches, 107 us from launch
300 on).

Printed: ONE JSON line (rank 0) with
  value       whole-job TFLOP/s = 2 M N K * K_steps / elapsed,
  roofline    the kernel's average duration (HIP events recorded on the
              stream it runs on, around the K timed launches), against the
              bf16 dense MFMA peak,
  cpu_baseline the C oracle timed on host cores on a bounded row sample,
  workloads   the other workload shapes (fp32 / fp16 GEMMs, the non-divisible
              bf16 GEMM, the 4-bit dequant GEMM and its decode-like probes,
              the MX-format GEMMs, the 2:4 sparse GEMM), each timed the same
              way.
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
PEAK_TFLOPS = {"bf16": 2516.6, "f16": 2516.6, "f32": 157.3,
               # scaled MFMA: E2M1 x E2M1 at the fp4 rate, E4M3 x E2M1 at the fp8 rate
               "mx_e2m1": 10066.3, "mx_e4m3": 5033.2,
               # 2:4 sparse MFMA, dense-equivalent rate (twice the dense bf16/fp16 rate)
               "sp24_bf16": 5033.2, "sp24_f16": 5033.2}
PEAK_HBM_GBS = 8000.0
HEADLINE = "bf16_4096_relu"
OTHER = ["f32_4096", "bf16_4000x4032x4096_relu", "f16_1024", "f32_512", "w4_256x8192x8192",
         "w4_16x8192x8192", "w4_1x8192x8192", "mx_e2m1_8192", "mx_e4m3_8192",
         "sp24_bf16_4096_relu"]


def load_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken with the configuration the library launches now and on that
    kernel's current sources; else None."""
    path = os.path.join(ROOT, "profiles", "traffic_%s.json" % workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    from tiled_dense_gemm_07_amd.traffic import source_hash, workload_config

    config = workload_config(workload)
    if rec.get("config") != config or rec.get("source_hash") != source_hash(config):
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


WARM_MS = 40.0  # GPU work before a workload's timed launches (clock ramp-up)


def time_kernel(fn, stream, launches: int, warmup: int):
    """Average kernel duration (ms): one HIP event pair on the stream the
    kernel runs on, around `launches` back-to-back launches.  The warm-up is at least
    `warmup` launches and at least WARM_MS of back-to-back work, so the card
    has left its idle clocks (the inputs are generated on the host first)."""
    import torch

    # one launch's duration from an event pair around a few launches (a host
    # clock around one launch would mostly time the launch and the sync)
    fn()
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        fn()
    b.record(stream)
    stream.synchronize()
    once_ms = max(a.elapsed_time(b) / 5, 1e-3)
    for _ in range(max(warmup, min(int(WARM_MS / once_ms) + 1, 5000))):
        fn()
    stream.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(launches):
        fn()
    b.record(stream)
    stream.synchronize()
    return {"mean_ms": a.elapsed_time(b) / launches}


# Workloads whose run time is the operand stream from HBM: also timed with
# the operands rotated over copies larger than the caches (256 MB MALL,
# 8 x 4 MB L2), so every launch reads its bytes from HBM.
MEMORY_BOUND = ("w4_1x8192x8192", "w4_16x8192x8192")
COLD_BYTES = 1 << 30


def time_cold(w, tensors, stream, launches: int = 40):
    """Kernel duration with each launch on a different copy of the inputs
    (together COLD_BYTES or more), so nothing is cache-resident."""
    import torch

    from tiled_dense_gemm_07_amd import binding

    per = sum(x.numel() * x.element_size() for x in tensors)
    copies = max(4, -(-COLD_BYTES // per))
    sets = [tuple(x.clone() for x in tensors) for _ in range(copies)]
    fns = [launcher(w, s_, stream) for s_ in sets]
    for f in fns[:4]:
        f()
    stream.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fns[i % copies]()
        b.record(stream)
    stream.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    mean = sum(ts) / len(ts)
    gbs = w.algorithmic_bytes() / (mean * 1e-3) / 1e9
    del sets, fns
    return {"copies": copies, "kernel_ms": round(mean, 5), "kernel_ms_min": round(ts[0], 5),
            "gbs_algorithmic": round(gbs, 1), "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4)}


def dtype_name(w):
    from tiled_dense_gemm_07_amd import synth

    if w.op == "mx":
        return "mx_" + synth.MX_NAMES[w.dtype]
    if w.op == "sp24":
        return "sp24_" + {synth.F16: "f16", synth.BF16: "bf16"}[w.dtype]
    return {synth.F32: "f32", synth.F16: "f16", synth.BF16: "bf16"}[w.dtype]


def cpu_baseline(w, inp, budget_s: float = 12.0):
    """The oracle, as it stands, on the first R rows of C; R grows until one
    call takes a good part of the budget."""
    import numpy as np

    import oracle

    A, B = inp["A"], inp["B"]
    rows = 4
    elapsed = 0.0
    while True:
        t0 = time.perf_counter()
        oracle.gemm_f64(np.ascontiguousarray(A[:rows]), B, w.dtype, w.relu)
        elapsed = time.perf_counter() - t0
        if elapsed >= budget_s / 4 or rows >= w.M:
            break
        rows = min(w.M, max(rows * 2, int(rows * (budget_s / 4) / max(elapsed, 1e-3))))
    flops = 2.0 * rows * w.N * w.K
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "rows 0..%d of C = A @ B for the %s workload (%d x %d x %d fp64 sums, "
                      "%.1f s)" % (rows - 1, w.name, rows, w.N, w.K, elapsed),
            "seconds": elapsed}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true")
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

    for _ in range(args.warmup):
        fn()
    torch.cuda.synchronize()
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
                "traffic": traffic["hbm_bytes_per_launch"] if traffic else None,
                "kernel_ms": round(kernel_ms, 5),
                "algorithmic_flops_per_launch": w.flops,
                "algorithmic_bytes_per_launch": w.algorithmic_bytes()}
    # the matrix cores' own ceiling on this card: the same MFMA work on
    # register operands, no memory traffic (power-limited clock)
    try:
        from tiled_dense_gemm_07_amd import clockprobe

        roofline["mfma_ceiling"] = [clockprobe.measure("random"), clockprobe.measure("zeros")]
    except Exception as e:  # the probe is context only
        roofline["mfma_ceiling"] = "unavailable: %s" % e

    workloads = {}
    if not args.no_workloads:
        for name in OTHER:
            ow = synth.WORKLOADS[name]
            _, t = make_device_inputs(ow, dev)
            r = time_kernel(launcher(ow, t, stream), stream, launches=30, warmup=5)
            tf = ow.flops / (r["mean_ms"] * 1e-3) / 1e12
            gbs = ow.algorithmic_bytes() / (r["mean_ms"] * 1e-3) / 1e9
            dn = dtype_name(ow)
            workloads[name] = {
                "kernel_ms": round(r["mean_ms"], 5), "tflops": round(tf, 2),
                "frac_mfma_peak": round(tf / PEAK_TFLOPS[dn], 4),
                "gbs_algorithmic": round(gbs, 1),
                "frac_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                "config": binding.query_config({"gemm": 0, "dequant_w4": 1, "mx": 2, "sp24": 3}[ow.op],
                                               ow.M, ow.N, ow.K, ow.dtype)}
            if name in MEMORY_BOUND:
                workloads[name]["cold"] = time_cold(ow, t, stream)
            tr = load_traffic(name)
            if tr is not None:
                # L2 <-> fabric bytes per launch from the committed counter record
                workloads[name]["traffic_bytes"] = int(tr["hbm_bytes_per_launch"])
                workloads[name]["gbs_counters"] = round(
                    tr["hbm_bytes_per_launch"] / (r["mean_ms"] * 1e-3) / 1e9, 1)
            del t
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, inp)

    line = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
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
