"""Offline sweep over the compiled tile / stage / wave / swizzle configurations.

The pages tune tiles by trying a small grid of configurations on the target GPU
and keeping the fastest ("TileLang ... 一个高效 GEMM 内核", mhpq.cn, sections 4.2
and 4.3: tune BK first, try a 3 x 3 x 3 grid, retune per GPU; the gtnt.cn page's
tuning_config with tile_sizes [32, 64, 128]).  Here every configuration is a
compiled instantiation of the kernel template; the sweep times each one on each
requested shape with HIP events on the launch stream, appends every result to a
JSON-lines log (a rerun skips shapes already measured), picks the fastest per
shape and regenerates the selection table compiled into the library
(csrc/tg_tuned.inc).  Rebuild the library afterwards.

    python -m tiled_dense_gemm_07_amd.sweep --log sweep.jsonl --write-table
"""

from __future__ import annotations

import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "tg_tuned.inc")


WARM_MS = 40.0  # back-to-back work before a configuration's timed launches


def time_config(fn, stream, launches: int = 20, warmup: int = 3) -> float:
    """Median launch time (ms) over `launches` event-timed launches, after at
    least `warmup` launches and WARM_MS of back-to-back work: the card leaves
    its idle clocks only after tens of milliseconds of load."""
    import torch

    for _ in range(warmup):
        fn()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        fn()
    b.record(stream)
    stream.synchronize()
    once_ms = max(a.elapsed_time(b) / 5, 1e-3)
    for _ in range(min(int(WARM_MS / once_ms) + 1, 5000)):
        fn()
    stream.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    stream.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return ts[len(ts) // 2]


def sweep_shape(op: int, dtype: int, M: int, N: int, K: int, relu: bool, done: set, log):
    import torch

    from . import binding, synth

    key = (op, dtype, M, N, K)
    if key in done:
        return
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    tdt = {synth.F32: torch.float32, synth.F16: torch.float16, synth.BF16: torch.bfloat16}
    g = torch.Generator(device=dev).manual_seed(1234)
    if op == binding.TG_OP_GEMM:
        A = torch.randn((M, K), generator=g, device=dev).to(tdt[dtype])
        B = torch.randn((K, N), generator=g, device=dev).to(tdt[dtype])
        C = torch.empty((M, N), dtype=tdt[dtype], device=dev)
    elif op == binding.TG_OP_SP24:
        A = torch.randn((M, K // 2), generator=g, device=dev).to(tdt[dtype])
        As = torch.randint(0, 256, (M, K // 8), generator=g, device=dev, dtype=torch.uint8)
        B = torch.randn((K, N), generator=g, device=dev).to(tdt[dtype])
        C = torch.empty((M, N), dtype=tdt[dtype], device=dev)
    elif op == binding.TG_OP_MX:
        # dtype carries the activation format; codes uniform, scales 2^-4 .. 2^0
        kq = K // 2 if dtype == binding.TG_MX_E2M1 else K
        A = torch.randint(0, 256, (M, kq), generator=g, device=dev, dtype=torch.uint8)
        if dtype == binding.TG_MX_E4M3:
            A[(A & 0x7F) == 0x7F] = 0x38  # no NaN codes
        As = torch.randint(123, 128, (M, K // 32), generator=g, device=dev, dtype=torch.uint8)
        Wq = torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.uint8)
        Ws = torch.randint(123, 128, (N, K // 32), generator=g, device=dev, dtype=torch.uint8)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    else:
        A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
        Wq = torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.uint8)
        Ws = torch.randint(123, 128, (N, K // 32), generator=g, device=dev, dtype=torch.uint8)
        C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    epi = "relu" if relu else None
    names = binding.list_configs(op, dtype)
    for idx, name in enumerate(names):
        if name.endswith("_narrow"):
            continue  # element-load variants serve unaligned operands only
        if op == binding.TG_OP_MX and not name.startswith("mx_" + synth.MX_NAMES[dtype]):
            continue  # the other activation format
        if op == binding.TG_OP_GEMM:
            fn = lambda: binding.gemm_with_config(idx, A, B, C=C, epilogue=epi, stream=stream)
        elif op == binding.TG_OP_MX:
            fn = lambda: binding.gemm_mx(dtype, A, As, Wq, Ws, C=C, epilogue=epi, stream=stream,
                                         config=idx)
        elif op == binding.TG_OP_SP24:
            fn = lambda: binding.gemm_sp24(A, As, B, C=C, epilogue=epi, stream=stream, config=idx)
        else:
            fn = lambda: binding.dequant_gemm_w4_with_config(idx, A, Wq, Ws, C=C, epilogue=epi,
                                                             stream=stream)
        try:
            fn()
        except binding.TileGemmError:
            continue  # not for this call (operand layout, alignment, K multiple)
        ms = time_config(fn, stream)
        rec = {"op": op, "dtype": dtype, "M": M, "N": N, "K": K, "config": name, "ms": ms,
               "tflops": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
        log.write(json.dumps(rec) + "\n")
        log.flush()
        print("sweep %s %dx%dx%d %-40s %8.4f ms %8.1f TFLOP/s" % (
            ("gemm", "w4", "mx", "sp24")[op], M, N, K, name, ms, rec["tflops"]), flush=True)
    del A, C
    torch.cuda.empty_cache()


def best_per_shape(records):
    best = {}
    for r in records:
        key = (r["op"], r["dtype"], r["M"], r["N"], r["K"])
        if key not in best or r["ms"] < best[key]["ms"]:
            best[key] = r
    return best


def write_table(best, path: str = TABLE):
    lines = [
        "// Best kernel configuration per measured shape, written by",
        "// tiled_dense_gemm_07_amd/sweep.py from timings on MI355X.  Shapes not listed",
        "// fall back to the built-in heuristic.  The last entry is a sentinel.",
        "static const TunedEntry kTuned[] = {",
    ]
    for key in sorted(best):
        r = best[key]
        lines.append('    {%d, %d, %d, %d, %d, "%s"},  // %.4f ms, %.1f TFLOP/s' % (
            r["op"], r["dtype"], r["M"], r["N"], r["K"], r["config"], r["ms"], r["tflops"]))
    lines.append("    {0, 0, 0, 0, 0, nullptr},")
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--log", default="sweep.jsonl", help="JSON-lines results (appended)")
    ap.add_argument("--shapes", default="workloads",
                    help="'workloads' or a comma list of op:dtype:MxNxK[:relu]")
    ap.add_argument("--write-table", action="store_true",
                    help="regenerate csrc/tg_tuned.inc from the log")
    ap.add_argument("--table", default=TABLE)
    args = ap.parse_args(argv)

    from . import synth

    shapes = []
    if args.shapes == "workloads":
        for w in synth.WORKLOADS.values():
            shapes.append(({"gemm": 0, "dequant_w4": 1, "mx": 2, "sp24": 3}[w.op], w.dtype, w.M,
                           w.N, w.K, w.relu))
    elif args.shapes:
        for item in args.shapes.split(","):
            parts = item.split(":")
            M, N, K = (int(x) for x in parts[2].split("x"))
            shapes.append((int(parts[0]), int(parts[1]), M, N, K, len(parts) > 3))

    records = []
    if os.path.exists(args.log):
        with open(args.log) as f:
            records = [json.loads(l) for l in f if l.strip()]
    done = {(r["op"], r["dtype"], r["M"], r["N"], r["K"]) for r in records}

    if shapes:
        import torch

        if not torch.cuda.is_available():
            print("the sweep times kernels and needs a GPU", file=sys.stderr)
            return 1
        with open(args.log, "a") as log:
            for s in shapes:
                sweep_shape(*s, done=done, log=log)
        with open(args.log) as f:
            records = [json.loads(l) for l in f if l.strip()]

    best = best_per_shape(records)
    for key, r in sorted(best.items()):
        print("best %s: %s %.4f ms %.1f TFLOP/s" % (key, r["config"], r["ms"], r["tflops"]))
    if args.write_table:
        write_table(best, args.table)
        print("wrote", args.table)
    return 0


if __name__ == "__main__":
    sys.exit(main())
