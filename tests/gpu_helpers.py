"""Shared helpers for the GPU parity tests: moving storage words between numpy
and torch, running the library, and comparing with the oracle."""

from __future__ import annotations

import sys

import numpy as np

F32, F16, BF16 = 0, 1, 2


def say(msg: str):
    """Name the case before its GPU step (flushed, so it survives a crash)."""
    sys.stdout.write("[gpu] %s\n" % msg)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch

    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]


def to_device(bits: np.ndarray, dtype: int, dev):
    import torch

    if dtype == F32:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).view(torch.float32)
    else:
        t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch_dtype(dtype))
    return t.to(dev)


def to_host_bits(t, dtype: int) -> np.ndarray:
    import torch

    if dtype == F32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def bits_to_f64(bits: np.ndarray, dtype: int) -> np.ndarray:
    if dtype == F32:
        return bits.view(np.float32).astype(np.float64)
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def tol_report(got: np.ndarray, want: np.ndarray) -> dict:
    err = np.abs(got - want)
    rel = err / np.maximum(np.abs(want), 1e-30)
    fro = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    return {"max_abs": float(err.max(initial=0.0)), "max_rel": float(rel.max(initial=0.0)),
            "rel_fro": fro}


def assert_close_16(got: np.ndarray, want: np.ndarray, atol=1e-2, rtol=1e-2):
    """The fp16 / bf16 / 4-bit bound: |got - want| <= atol + rtol * |want| elementwise."""
    bad = np.abs(got - want) > atol + rtol * np.abs(want)
    assert not bad.any(), "%d of %d outside atol %g + rtol %g: %s" % (
        int(bad.sum()), bad.size, atol, rtol, tol_report(got, want))


def assert_fro_32(got: np.ndarray, want: np.ndarray, bound=1e-5):
    """The fp32 bound: relative Frobenius error <= 1e-5."""
    r = tol_report(got, want)
    assert r["rel_fro"] <= bound, r


def sample_entries(M: int, N: int, count: int, seed: int):
    """Random entries plus the four corners and the last row / column edges."""
    r = np.random.Generator(np.random.PCG64(seed))
    rows = list(r.integers(0, M, size=count))
    cols = list(r.integers(0, N, size=count))
    for m in (0, M - 1):
        for n in range(0, N, max(1, N // 64)):
            rows.append(m)
            cols.append(n)
        rows.append(m)
        cols.append(N - 1)
    for n in (0, N - 1):
        for m in range(0, M, max(1, M // 64)):
            rows.append(m)
            cols.append(n)
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)
