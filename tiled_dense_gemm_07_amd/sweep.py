"""Offline sweep: time the compiled configurations on a grid of shapes and
write the selection table compiled into the library (csrc/tg_tuned.inc).

The pages tune by trying candidate tilings on the target GPU and keeping the
fastest, per shape and per GPU ("TileLang ... 一个高效 GEMM 内核", mhpq.cn,
sections 4.2 and 4.3; the gtnt.cn page's tuning_config).  The candidates are
every configuration the library compiled (tiled_dense_gemm_07_amd/configgen.py
generates the GEMM families from the LDS and register budgets).  For each
shape of the grid below the sweep times every configuration that can run it,
then the swizzle group of the fastest few, and records:

  * for the workload shapes (synth.WORKLOADS): the fastest configuration and
    swizzle group of exactly that shape;
  * for every grid shape: the TOP fastest configurations with their times and
    their workgroups per compute unit.  A grid shape represents the bucket of
    calls nearest to it in log2(M), log2(N), log2(K); the library prices each
    of its configurations at the call's shape (measured time scaled by the
    number of tile rounds and by K) and launches the cheapest.

Timing: back-to-back launches on the launch stream between one pair of HIP
events (an event pair per launch adds microseconds to every launch), after a
warm-up that brings the card to its sustained clock.

    python -m tiled_dense_gemm_07_amd.sweep --log sweep.jsonl --write-table
"""

from __future__ import annotations

import argparse
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
TABLE = os.path.join(HERE, "csrc", "tg_tuned.inc")

OP_GEMM, OP_W4, OP_MX, OP_SP24 = 0, 1, 2, 3
TOP = 4              # configurations kept per grid shape
GROUPS = (1, 2, 4, 8, 16)  # swizzle groups tried for the fastest configurations
# A group other than the compiled one must be this much faster: narrower groups
# spread a round's tiles over more rows and columns, which costs fabric traffic
# (up to 1.8x), while 3 ms timings differ by 1-2%.
GROUP_MARGIN = 0.03
TIMED_MS = 3.0       # back-to-back work timed per configuration and shape


def grid():
    """(op, dtype, M, N, K) of the representative shapes."""
    out = []
    for dt in (2, 1):  # bf16, fp16
        for m in (256, 512, 1024, 2048, 4096, 8192):
            for n in (256, 512, 1024, 2048, 4096, 8192):
                for k in (512, 2048, 8192):
                    out.append((OP_GEMM, dt, m, n, k))
    for m in (256, 512, 1024, 2048, 4096):
        for n in (256, 512, 1024, 2048, 4096):
            for k in (512, 2048, 8192):
                out.append((OP_GEMM, 0, m, n, k))
    for m in (1, 16, 64, 256, 1024):
        for n in (4096, 8192):
            for k in (4096, 8192):
                out.append((OP_W4, 2, m, n, k))
    for fmt in (0, 1):
        for mn in (2048, 4096, 8192):
            for k in (2048, 8192):
                out.append((OP_MX, fmt, mn, mn, k))
    for dt in (2, 1):
        for mn in (1024, 2048, 4096, 8192):
            for k in (2048, 8192):
                out.append((OP_SP24, dt, mn, mn, k))
    return out


def workload_shapes():
    from . import synth

    return [({"gemm": 0, "dequant_w4": 1, "mx": 2, "sp24": 3}[w.op], w.dtype, w.M, w.N, w.K)
            for w in synth.WORKLOADS.values()]


def _inputs(op, dtype, M, N, K, dev):
    import torch

    g = torch.Generator(device=dev).manual_seed(1234)
    tdt = {0: torch.float32, 1: torch.float16, 2: torch.bfloat16}
    if op == OP_GEMM:
        A = torch.randn((M, K), generator=g, device=dev).to(tdt[dtype])
        B = torch.randn((K, N), generator=g, device=dev).to(tdt[dtype])
        return (A, B, torch.empty((M, N), dtype=tdt[dtype], device=dev))
    if op == OP_SP24:
        A = torch.randn((M, K // 2), generator=g, device=dev).to(tdt[dtype])
        Ai = torch.randint(0, 256, (M, K // 8), generator=g, device=dev, dtype=torch.uint8)
        B = torch.randn((K, N), generator=g, device=dev).to(tdt[dtype])
        return (A, Ai, B, torch.empty((M, N), dtype=tdt[dtype], device=dev))
    if op == OP_MX:
        kq = K // 2 if dtype == 0 else K
        A = torch.randint(0, 256, (M, kq), generator=g, device=dev, dtype=torch.uint8)
        if dtype == 1:
            A[(A & 0x7F) == 0x7F] = 0x38  # no NaN codes
        As = torch.randint(123, 128, (M, K // 32), generator=g, device=dev, dtype=torch.uint8)
        Wq = torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.uint8)
        Ws = torch.randint(123, 128, (N, K // 32), generator=g, device=dev, dtype=torch.uint8)
        return (A, As, Wq, Ws, torch.empty((M, N), dtype=torch.bfloat16, device=dev))
    A = torch.randn((M, K), generator=g, device=dev).to(torch.bfloat16)
    Wq = torch.randint(0, 256, (N, K // 2), generator=g, device=dev, dtype=torch.uint8)
    Ws = torch.randint(123, 128, (N, K // 32), generator=g, device=dev, dtype=torch.uint8)
    return (A, Wq, Ws, torch.empty((M, N), dtype=torch.bfloat16, device=dev))


def _launcher(op, dtype, idx, t, stream):
    from . import binding

    if op == OP_GEMM:
        A, B, C = t
        return lambda: binding.gemm_with_config(idx, A, B, C=C, stream=stream)
    if op == OP_MX:
        A, As, Wq, Ws, C = t
        return lambda: binding.gemm_mx(dtype, A, As, Wq, Ws, C=C, stream=stream, config=idx)
    if op == OP_SP24:
        A, Ai, B, C = t
        return lambda: binding.gemm_sp24(A, Ai, B, C=C, stream=stream, config=idx)
    A, Wq, Ws, C = t
    return lambda: binding.dequant_gemm_w4_with_config(idx, A, Wq, Ws, C=C, stream=stream)


def time_back_to_back(fn, stream) -> float:
    """Mean launch time (ms) of back-to-back launches worth about TIMED_MS,
    after two launches (the card is kept busy by the sweep, so its clock is
    already up)."""
    import torch

    fn()
    fn()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    fn()
    b.record(stream)
    stream.synchronize()
    n = int(min(200, max(5, TIMED_MS / max(a.elapsed_time(b), 1e-3))))
    a.record(stream)
    for _ in range(n):
        fn()
    b.record(stream)
    stream.synchronize()
    return a.elapsed_time(b) / n


def warm_card(dev):
    """About 100 ms of matrix work, so the sweep starts at the sustained clock."""
    import torch

    x = torch.randn((4096, 4096), device=dev, dtype=torch.bfloat16)
    for _ in range(800):
        torch.matmul(x, x)
    torch.cuda.synchronize()


def sweep_shape(op, dtype, M, N, K, log):
    import torch

    from . import binding

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    t = _inputs(op, dtype, M, N, K, dev)
    names = binding.list_configs(op, dtype)
    results = []
    for idx, name in enumerate(names):
        if name.endswith("_narrow"):
            continue  # element-load variants serve unaligned operands only
        if op == OP_MX and not name.startswith("mx_" + ("e2m1", "e4m3")[dtype]):
            continue
        fn = _launcher(op, dtype, idx, t, stream)
        try:
            fn()
        except binding.TileGemmError:
            continue  # not for this call (operand layout, alignment, K multiple)
        results.append([time_back_to_back(fn, stream), idx, name, 0])
    results.sort()
    # the swizzle group of the fastest few: the compiled group (0) and every
    # other, timed in two interleaved passes, the faster of each group's two
    # timings kept (a group timed right after another config's run read up
    # to 8% slow in one pass)
    for r in results[:TOP]:
        fn = _launcher(op, dtype, r[1], t, stream)
        best_of = {}
        for _ in range(2):
            for gm in (0,) + GROUPS:
                binding.set_swizzle_override(gm)
                try:
                    ms = time_back_to_back(fn, stream)
                finally:
                    binding.set_swizzle_override(0)
                best_of[gm] = min(best_of.get(gm, ms), ms)
        best = (best_of[0], 0)
        for gm in GROUPS:
            if best_of[gm] < best[0] * (1.0 - GROUP_MARGIN):
                best = (best_of[gm], gm)
        r[0], r[3] = best
    results.sort()
    for ms, idx, name, gm in results:
        rec = {"op": op, "dtype": dtype, "M": M, "N": N, "K": K, "config": name, "ms": ms,
               "group_m": gm, "per_cu": binding.config_occupancy(op, dtype, idx),
               "tflops": 2.0 * M * N * K / (ms * 1e-3) / 1e12}
        log.write(json.dumps(rec) + "\n")
    log.flush()
    if results:
        ms, _, name, gm = results[0]
        print("sweep %s/%d %dx%dx%d: %d configs, best %s g%d %.4f ms" % (
            ("gemm", "w4", "mx", "sp24")[op], dtype, M, N, K, len(results), name, gm, ms),
            flush=True)
    del t
    torch.cuda.empty_cache()


def best_per_shape(records):
    """{(op, dtype, M, N, K): [records sorted by time]}."""
    by = {}
    for r in records:
        by.setdefault((r["op"], r["dtype"], r["M"], r["N"], r["K"]), []).append(r)
    for v in by.values():
        v.sort(key=lambda r: r["ms"])
    return by


def write_table(by, exact_keys, grid_keys, path: str = TABLE):
    lines = [
        "// Selection table written by tiled_dense_gemm_07_amd/sweep.py from timings on",
        "// MI355X: {op, dtype, M, N, K, configuration, swizzle group (0: the",
        "// configuration's own), ms, workgroups per compute unit, exact}.  exact = 1:",
        "// the fastest for exactly this shape; exact = 0: the fastest few at a",
        "// representative shape of the bucket grid.  The last entry is a sentinel.",
        "static const TunedEntry kTuned[] = {",
    ]

    def row(r, exact):
        return '    {%d, %d, %d, %d, %d, "%s", %d, %.5f, %d, %d},  // %.1f TFLOP/s' % (
            r["op"], r["dtype"], r["M"], r["N"], r["K"], r["config"], r["group_m"], r["ms"],
            max(1, r["per_cu"]), exact, r["tflops"])

    for key in sorted(set(exact_keys)):
        if key in by:
            lines.append(row(by[key][0], 1))
    for key in sorted(set(grid_keys)):
        if key in by:
            for r in by[key][:TOP]:
                lines.append(row(r, 0))
    lines.append('    {0, 0, 0, 0, 0, nullptr, 0, 0.0, 0, 0},')
    lines.append("};")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--log", default="sweep.jsonl", help="JSON-lines results (appended)")
    ap.add_argument("--only", default=None,
                    help="comma list of ops to sweep (gemm, w4, mx, sp24); default all")
    ap.add_argument("--write-table", action="store_true",
                    help="regenerate csrc/tg_tuned.inc from the log")
    ap.add_argument("--table", default=TABLE)
    ap.add_argument("--no-run", action="store_true", help="only rewrite the table from the log")
    args = ap.parse_args(argv)

    exact = workload_shapes()
    grid_keys = grid()
    shapes = exact + grid_keys
    if args.only:
        keep = {("gemm", "w4", "mx", "sp24").index(x) for x in args.only.split(",")}
        shapes = [s for s in shapes if s[0] in keep]

    records = []
    if os.path.exists(args.log):
        with open(args.log) as f:
            records = [json.loads(l) for l in f if l.strip()]
    done = {(r["op"], r["dtype"], r["M"], r["N"], r["K"]) for r in records}

    if not args.no_run:
        import torch

        from . import binding

        if not torch.cuda.is_available():
            print("the sweep times kernels and needs a GPU", file=sys.stderr)
            return 1
        binding.load_library()
        warm_card(torch.device("cuda:0"))
        with open(args.log, "a") as log:
            for s in shapes:
                if s not in done:
                    sweep_shape(*s, log=log)
                    done.add(s)
        with open(args.log) as f:
            records = [json.loads(l) for l in f if l.strip()]

    by = best_per_shape(records)
    if args.write_table:
        write_table(by, exact, grid_keys, args.table)
        print("wrote", args.table)
    return 0


if __name__ == "__main__":
    sys.exit(main())
