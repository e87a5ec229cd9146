"""Measured fabric traffic of one kernel launch, from rocprofv3 counters.

FETCH_SIZE and WRITE_SIZE (KiB per dispatch) count traffic between the L2s
and the memory fabric: the 256 MB MALL serves part of it, so these are
*fabric* bytes, an upper bound on HBM bytes.  With ``--cold`` the profiled
program rotates the operands over copies larger than the MALL, so every
launch's first touch of each operand byte comes from HBM.  The counters' scale
is calibrated with one plain elementwise kernel that reads and writes a known
number of bytes (1 GiB each way, larger than the MALL) in the same process:
factor = true bytes / counter bytes.  gfx950 issues 128-byte requests that
FETCH_SIZE counts as 64 bytes, hence a fetch factor near 2; a cold record whose
fabric bytes come out near the algorithmic bytes of a kernel that reads every
byte once (the weight-streaming dequant kernel) checks that factor for its
family.  Two separate counter passes are needed (FETCH_SIZE, then WRITE_SIZE):

    rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/f -o f -- \\
        python -m tiled_dense_gemm_07_amd.traffic run --workload bf16_4096_relu
    rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/w -o w -- \\
        python -m tiled_dense_gemm_07_amd.traffic run --workload bf16_4096_relu
    python -m tiled_dense_gemm_07_amd.traffic summarize --workload bf16_4096_relu \\
        --fetch OUT/f/f_counter_collection.csv --write OUT/w/w_counter_collection.csv \\
        --out profiles/traffic_bf16_4096_relu.json

(add ``--cold`` to both ``run`` commands and to ``summarize`` for a cold record).

The summary records which compiled configuration ran and a hash of the
sources that kernel is built from; the benchmark reports the traffic only
while both still match.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
COPY_BYTES = 1 << 30  # 1 GiB read + 1 GiB written by the calibration copy


# Sources each kernel family is built from (its header, the shared helpers and
# the scheduler); a change to any of them invalidates a stored traffic record.
_FAMILY_SOURCES = {
    "dma": ["tg_kernel_dma.h", "tg_kernel.h", "tg_sched.h"],
    "dma_w4": ["tg_kernel_dma_w4.h", "tg_kernel_dma.h", "tg_kernel.h", "tg_sched.h"],
    "gemv": ["tg_kernel_gemv_w4.h", "tg_kernel.h"],
    "tiled": ["tg_kernel.h", "tg_sched.h"],
    "mx": ["tg_kernel_mx.h", "tg_kernel_dma_w4.h", "tg_kernel_dma.h", "tg_kernel.h", "tg_sched.h"],
    "sp24": ["tg_kernel_sp24.h", "tg_kernel_dma_w4.h", "tg_kernel_dma.h", "tg_kernel.h",
             "tg_sched.h"],
}


def kernel_family(config: str) -> str:
    if config.startswith("mx_"):
        return "mx"
    if config.startswith("sp24_"):
        return "sp24"
    if config.startswith("w4_") and "_dma" in config:
        return "dma_w4"
    if "_dma" in config:
        return "dma"
    if "_gemv" in config:
        return "gemv"
    return "tiled"


def source_hash(config: str) -> str:
    """Hash of the HIP sources the kernel of `config` is built from."""
    h = hashlib.sha256()
    for name in _FAMILY_SOURCES[kernel_family(config)]:
        with open(os.path.join(HERE, "csrc", name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def workload_launch(workload: str) -> tuple:
    """(configuration, swizzle group) the library launches for the workload
    (aligned operands).  The group decides which tiles share an XCD's L2, so
    a traffic record holds for one group only."""
    from . import binding, synth

    w = synth.WORKLOADS[workload]
    op = {"gemm": 0, "dequant_w4": 1, "mx": 2, "sp24": 3}[w.op]
    q = binding.query_config(op, w.M, w.N, w.K, w.dtype).split()
    group = [int(x.split("=")[1]) for x in q if x.startswith("group=")]
    return q[0], (group[0] if group else 0)


def workload_config(workload: str) -> str:
    """The configuration the library launches for the workload (aligned operands)."""
    return workload_launch(workload)[0]


COLD_BYTES = 1 << 30


def _rotated(tensors, cold: bool):
    """The operand sets launches cycle through: the tensors themselves, or
    (cold) enough copies that together they exceed COLD_BYTES."""
    if not cold:
        return [tensors]
    per = sum(x.numel() * x.element_size() for x in tensors)
    copies = max(4, -(-COLD_BYTES // per))
    return [tuple(x.clone() for x in tensors) for _ in range(copies)]


def run(workload: str, launches: int, cold: bool = False) -> None:
    """The program profiled: one calibration copy, then the workload's kernel."""
    import numpy as np
    import torch

    from . import binding, synth

    dev = torch.device("cuda:0")
    # calibration: one elementwise kernel that reads COPY_BYTES and writes
    # COPY_BYTES (the runtime's own copy engine path is not seen by FETCH_SIZE)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    dst = torch.mul(src, 1.0)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()

    w = synth.WORKLOADS[workload]
    inp = synth.make_inputs(w, integer=False)
    epi = "relu" if w.relu else None
    if w.op == "gemm":
        tdt = {synth.F32: torch.float32, synth.F16: torch.float16, synth.BF16: torch.bfloat16}
        view = np.int32 if w.dtype == synth.F32 else np.int16
        A = torch.from_numpy(inp["A"].view(view)).view(tdt[w.dtype]).to(dev)
        B = torch.from_numpy(inp["B"].view(view)).view(tdt[w.dtype]).to(dev)
        sets = _rotated((A, B), cold)
        for i in range(launches):
            binding.gemm(*sets[i % len(sets)], epilogue=epi)
    elif w.op == "mx":
        t = tuple(torch.from_numpy(inp[k]).to(dev) for k in ("Aq", "As", "Wq", "Ws"))
        sets = _rotated(t, cold)
        for i in range(launches):
            binding.gemm_mx(w.dtype, *sets[i % len(sets)], epilogue=epi)
    elif w.op == "sp24":
        tdt = {synth.F16: torch.float16, synth.BF16: torch.bfloat16}[w.dtype]
        Ac = torch.from_numpy(inp["Ac"].view(np.int16)).view(tdt).to(dev)
        B = torch.from_numpy(inp["B"].view(np.int16)).view(tdt).to(dev)
        Ai = torch.from_numpy(inp["Ai"]).to(dev)
        sets = _rotated((Ac, Ai, B), cold)
        for i in range(launches):
            binding.gemm_sp24(*sets[i % len(sets)], epilogue=epi)
    else:
        A = torch.from_numpy(inp["A"].view(np.int16)).view(torch.bfloat16).to(dev)
        Wq = torch.from_numpy(inp["Wq"]).to(dev)
        Ws = torch.from_numpy(inp["Ws"]).to(dev)
        sets = _rotated((A, Wq, Ws), cold)
        for i in range(launches):
            binding.dequant_gemm_w4(*sets[i % len(sets)], epilogue=epi)
    torch.cuda.synchronize()
    print("traffic run done: %s x%d%s" % (workload, launches, " cold" if cold else ""))


def _read(path: str, counter: str):
    """(calibration KiB, [kernel KiB per launch]) from a counter_collection CSV.
    The calibration kernel is the elementwise multiply of run(); the runtime's
    small host-to-device copies also appear and are ignored."""
    other, kern = [], []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter:
                continue
            v = float(r["Counter_Value"])
            if "tg::" in r["Kernel_Name"]:
                kern.append(v)
            else:
                other.append((r["Kernel_Name"], v))
    calib = [o for o in other if "elementwise" in o[0]]
    if len(calib) != 1:
        raise SystemExit("expected exactly one calibration kernel, found: %s" % other)
    return calib[0][1], kern


def commands(workload: str, launches: int, cold: bool) -> list:
    """The command lines that make a record (OUT: the output folder)."""
    run = "python3 -m tiled_dense_gemm_07_amd.traffic run --workload %s --launches %d%s" % (
        workload, launches, " --cold" if cold else "")
    return [
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/f -o f -- " + run,
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/w -o w -- " + run,
        "python3 -m tiled_dense_gemm_07_amd.traffic summarize --workload %s "
        "--fetch OUT/f/f_counter_collection.csv --write OUT/w/w_counter_collection.csv "
        "--out profiles/traffic_%s.json%s" % (workload, workload, " --cold" if cold else ""),
    ]


def summarize(workload: str, fetch_csv: str, write_csv: str, out: str, cold: bool = False) -> dict:
    from . import synth

    w = synth.WORKLOADS[workload]
    f_copy, f_k = _read(fetch_csv, "FETCH_SIZE")
    w_copy, w_k = _read(write_csv, "WRITE_SIZE")
    if not f_k or not w_k or f_copy is None or w_copy is None:
        raise SystemExit("counter files lack the copy or the kernel rows")
    f_factor = COPY_BYTES / (f_copy * 1024.0)
    w_factor = COPY_BYTES / (w_copy * 1024.0)
    fetch = f_factor * 1024.0 * sum(f_k) / len(f_k)
    write = w_factor * 1024.0 * sum(w_k) / len(w_k)
    config, group = workload_launch(workload)
    rec = {
        "workload": workload,
        "config": config,
        "group_m": group,
        "source_hash": source_hash(config),
        "copy_bytes": COPY_BYTES,
        "fetch_size_kib_copy": f_copy, "write_size_kib_copy": w_copy,
        "fetch_factor": f_factor, "write_factor": w_factor,
        "fetch_size_kib_per_launch": sum(f_k) / len(f_k),
        "write_size_kib_per_launch": sum(w_k) / len(w_k),
        "cold": cold,
        "fabric_fetch_bytes_per_launch": fetch,
        "fabric_write_bytes_per_launch": write,
        "fabric_bytes_per_launch": fetch + write,
        "algorithmic_bytes_per_launch": w.algorithmic_bytes(),
        "traffic_over_algorithmic": (fetch + write) / w.algorithmic_bytes(),
        "launches": len(f_k),
        "commands": commands(workload, len(f_k), cold),
    }
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("run")
    r.add_argument("--workload", required=True)
    r.add_argument("--launches", type=int, default=3)
    r.add_argument("--cold", action="store_true")
    s = sub.add_parser("summarize")
    s.add_argument("--workload", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--cold", action="store_true")
    args = ap.parse_args(argv)
    if args.cmd == "run":
        run(args.workload, args.launches, args.cold)
    else:
        print(json.dumps(summarize(args.workload, args.fetch, args.write, args.out, args.cold),
                         indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
