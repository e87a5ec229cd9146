"""Sustained matrix-core clock and the MFMA ceilings on this card.

Runs the probe kernel of csrc/tg_probe.hip (the bf16 GEMM's 256-workgroup
grid and exact MFMA count at 4096^3, on register operands, with no memory
traffic in the loop) once on random N(0, 1) bf16 operands and once on zeros,
and reports TFLOP/s (HIP events on the launch stream) and the average shader
clock that workgroup 0 measured (s_memtime ticks over 100 MHz s_memrealtime
ticks).  This is the throughput the chip sustains for the GEMM's MFMA work
alone under its power limit; the GEMM kernel cannot exceed it.

measure_mx() does the same for the MX-format GEMM at 8192^3 (E2M1 or E4M3
activations times E2M1 weights, the kernel's grid and scaled-MFMA count), on
random codes (no E4M3 NaN) or zeros.

    python -m tiled_dense_gemm_07_amd.clockprobe
"""

from __future__ import annotations

import ctypes
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
PROBE_LIB = os.path.join(HERE, "libtgprobe.so")
GRID = 256          # tiles of the 4096^3 bf16 GEMM at 256 x 256
STRIPS = 128        # 4096 / 32
FLOPS = 2.0 * 4096 ** 3


def load():
    if not os.path.exists(PROBE_LIB):
        raise RuntimeError("libtgprobe.so is missing: run python -m tiled_dense_gemm_07_amd.build")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.tgp_operand_words.argtypes = [ctypes.c_int]
    lib.tgp_operand_words.restype = ctypes.c_int
    lib.tgp_mfma_ceiling.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int, ctypes.c_int,
                                                             ctypes.c_void_p]
    lib.tgp_mfma_ceiling.restype = ctypes.c_int
    lib.tgp_mfma16_ceiling.argtypes = lib.tgp_mfma_ceiling.argtypes
    lib.tgp_mfma16_ceiling.restype = ctypes.c_int
    lib.tgp_mx_operand_words.argtypes = [ctypes.c_int]
    lib.tgp_mx_operand_words.restype = ctypes.c_int
    lib.tgp_mx_ceiling.argtypes = [ctypes.c_int] + [ctypes.c_void_p] * 3 + [
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.tgp_mx_ceiling.restype = ctypes.c_int
    return lib


def measure(data: str = "random", launches: int = 20, warmup: int = 3, shape: int = 32) -> dict:
    """shape 32: v_mfma_f32_32x32x16_bf16; 16: v_mfma_f32_16x16x32_bf16."""
    import torch

    lib = load()
    entry = lib.tgp_mfma_ceiling if shape == 32 else lib.tgp_mfma16_ceiling
    dev = torch.device("cuda:0")
    words = lib.tgp_operand_words(GRID)
    g = torch.Generator(device=dev).manual_seed(20260001)
    if data == "random":
        src = torch.randn((words * 8,), generator=g, device=dev).to(torch.bfloat16)
    else:
        src = torch.zeros((words * 8,), dtype=torch.bfloat16, device=dev)
    out = torch.empty((GRID * 256,), dtype=torch.float32, device=dev)
    clk = torch.zeros((2,), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = ctypes.c_void_p(stream.cuda_stream)

    def launch():
        rc = entry(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                   ctypes.c_void_p(clk.data_ptr()), GRID, STRIPS, s)
        if rc != 0:
            raise RuntimeError("probe launch failed (%d)" % rc)

    for _ in range(warmup):
        launch()
    stream.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for a, b in evs:
        a.record(stream)
        launch()
        b.record(stream)
    stream.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    med = ts[len(ts) // 2]
    ticks, real = clk.cpu().tolist()
    return {"mfma": "%dx%d" % (shape, shape), "data": data, "median_ms": round(med, 5),
            "tflops": round(FLOPS / med / 1e9, 1),
            "clock_ghz": round(ticks / (real * 10.0), 3) if real > 0 else None}


MX_GRID = {0: 1024, 1: 2048}   # 8192^3 tiles at 256 x 256 (E2M1) / 128 x 256 (E4M3)
MX_STRIPS = 64                 # 8192 / 128
MX_FLOPS = 2.0 * 8192 ** 3


def measure_mx(fmt: int, data: str = "random", launches: int = 10, warmup: int = 2) -> dict:
    import torch

    lib = load()
    dev = torch.device("cuda:0")
    grid = MX_GRID[fmt]
    nbytes = lib.tgp_mx_operand_words(grid) * 32
    g = torch.Generator(device=dev).manual_seed(20260002)
    if data == "random":
        src = torch.randint(0, 256, (nbytes,), generator=g, device=dev, dtype=torch.uint8)
        src[(src & 0x7F) == 0x7F] = 0x38  # no E4M3 NaN codes
    else:
        src = torch.zeros((nbytes,), dtype=torch.uint8, device=dev)
    out = torch.empty((grid * 256,), dtype=torch.float32, device=dev)
    clk = torch.zeros((2,), dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    s = ctypes.c_void_p(stream.cuda_stream)

    def launch():
        rc = lib.tgp_mx_ceiling(fmt, ctypes.c_void_p(src.data_ptr()),
                                ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clk.data_ptr()),
                                grid, MX_STRIPS, s)
        if rc != 0:
            raise RuntimeError("probe launch failed (%d)" % rc)

    for _ in range(warmup):
        launch()
    stream.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(launches)]
    for a, b in evs:
        a.record(stream)
        launch()
        b.record(stream)
    stream.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    med = ts[len(ts) // 2]
    ticks, real = clk.cpu().tolist()
    return {"kind": "mx_e2m1" if fmt == 0 else "mx_e4m3", "data": data,
            "median_ms": round(med, 5), "tflops": round(MX_FLOPS / med / 1e9, 1),
            "clock_ghz": round(ticks / (real * 10.0), 3) if real > 0 else None}


def main():
    for shape in (32, 16):
        for data in ("random", "zeros"):
            print(json.dumps(measure(data, shape=shape)), flush=True)
    for fmt in (0, 1):
        for data in ("random", "zeros"):
            print(json.dumps(measure_mx(fmt, data)), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
