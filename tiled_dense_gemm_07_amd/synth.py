"""Seeded synthetic inputs for the GEMM and dequant-GEMM workloads.

This module only draws random numbers and stores them in the operand formats.
It holds none of the GEMM arithmetic: the tests and the benchmark feed the same
arrays to the HIP library and to the CPU oracle, and neither side imports the
other.

The pages benchmark on random matrices only (``torch.randn`` inputs in the
mhpq.cn page, section 3.2; ``assert_close`` checks in the blog.hotdry.top
page), so every workload here is synthetic:

* floating inputs: numpy ``Generator(PCG64(seed)).standard_normal`` in float64,
  rounded to float32, then rounded (nearest-even) to the operand type;
* integer inputs: uniform on {-4, ..., 4}, exact in every operand type;
  operands of several GiB take the same range from a hash of (row, column,
  seed) instead (:func:`hashed_ints`), so they can be filled on the device;
* 4-bit weights: uniform bytes (so both nibbles are uniform on 0..15),
  E8M0 scale bytes 127 + uniform{-4..0}, i.e. scales 2^-4 .. 2^0;
* MX-format activations: E2M1 as the weights; E4M3 codes uniform over the 254
  non-NaN bytes; E8M0 scale bytes as for the weights;
* 2:4 sparse A: kept values drawn as the floating (or integer) inputs, the
  two kept positions of every group of 4 k uniform over the 6 pairs.

Seeds: ``20260000 + 100 * workload_index + {0: A, 1: B, 2: codes, 3: scales,
4: activation scales}``,
plus 50 for the integer-valued run.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

F32, F16, BF16 = 0, 1, 2
DTYPE_NAMES = {F32: "f32", F16: "f16", BF16: "bf16"}
STORAGE = {F32: np.uint32, F16: np.uint16, BF16: np.uint16}


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def normal_f32(shape, seed: int) -> np.ndarray:
    """N(0, 1) draws rounded to float32."""
    return rng(seed).standard_normal(shape).astype(np.float32)


def integers_f32(shape, seed: int, lo: int = -4, hi: int = 4) -> np.ndarray:
    """Uniform integers in [lo, hi] stored as float32 (exact)."""
    return rng(seed).integers(lo, hi + 1, size=shape).astype(np.float32)


def hashed_ints(r, c, seed: int, lo: int = -4, hi: int = 4):
    """Integers in [lo, hi] as a function of (row, column, seed): a 32-bit
    multiply / xor-shift mix of the index pair.

    `r` and `c` are broadcastable int64 arrays: numpy arrays, or torch tensors
    on any device (the same integer operators, so an operand of several GiB
    can be filled on the device while the oracle side evaluates the rows or
    columns it needs on the host).  Every product stays below 2^63.
    """
    m = 0xFFFFFFFF
    x = (r * 0x3C6EF35F + c * 0x1B873593 + seed * 0x61C88647) & m
    x = x ^ (x >> 16)
    x = (x * 0x7FEB352D) & m
    x = x ^ (x >> 15)
    x = (x * 0x2C1B3C6D) & m
    x = x ^ (x >> 16)
    return x % (hi - lo + 1) + lo


def to_storage(x: np.ndarray, dtype: int) -> np.ndarray:
    """float32 values -> raw storage words of the operand type (round to nearest even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F32:
        return x.view(np.uint32).copy()
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16).copy()
    if dtype == BF16:
        import torch  # CPU cast only

        t = torch.from_numpy(x).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError("unknown dtype %r" % (dtype,))


def w4_codes(N: int, K: int, seed: int) -> np.ndarray:
    """Packed E2M1 codes [N, K/2]: two uniform 4-bit codes per byte."""
    return rng(seed).integers(0, 256, size=(N, K // 2), dtype=np.uint8)


def w4_scales(N: int, K: int, seed: int, emin: int = -4, emax: int = 0) -> np.ndarray:
    """E8M0 scale bytes [N, K/32] for scales 2^emin .. 2^emax (uniform exponent)."""
    e = rng(seed).integers(emin, emax + 1, size=(N, K // 32))
    return (127 + e).astype(np.uint8)


def e4m3_codes(M: int, K: int, seed: int) -> np.ndarray:
    """E4M3 codes [M, K], uniform over the bytes that are not NaN (0x7F, 0xFF)."""
    v = rng(seed).integers(0, 254, size=(M, K))
    v = v + (v >= 0x7F)  # skip 0x7F; 253 -> 254; 0xFF is never drawn
    return v.astype(np.uint8)


def e4m3_codes_range(M: int, K: int, seed: int, efield_lo: int, efield_hi: int) -> np.ndarray:
    """E4M3 codes [M, K] with uniform sign, exponent field uniform in
    [efield_lo, efield_hi] and uniform 3-bit mantissa (never NaN for
    efield_hi <= 14)."""
    r = rng(seed)
    sign = r.integers(0, 2, size=(M, K))
    ef = r.integers(efield_lo, efield_hi + 1, size=(M, K))
    mant = r.integers(0, 8, size=(M, K))
    return ((sign << 7) | (ef << 3) | mant).astype(np.uint8)


MX_E2M1, MX_E4M3 = 0, 1
MX_NAMES = {MX_E2M1: "e2m1", MX_E4M3: "e4m3"}


def mx_inputs(fmt: int, M: int, N: int, K: int, seed_a: int, seed_as: int, seed_codes: int,
              seed_scales: int):
    """Activation codes (E2M1 [M, K/2] or E4M3 [M, K]), their scale bytes [M, K/32],
    packed weight codes [N, K/2] and weight scale bytes [N, K/32]."""
    Aq = w4_codes(M, K, seed_a) if fmt == MX_E2M1 else e4m3_codes(M, K, seed_a)
    return Aq, w4_scales(M, K, seed_as), w4_codes(N, K, seed_codes), w4_scales(N, K, seed_scales)


SP24_PAIRS = ((0, 1), (0, 2), (0, 3), (1, 2), (1, 3), (2, 3))


def sp24_meta(M: int, K: int, seed: int) -> np.ndarray:
    """Position nibbles [M, K/8]: group j's pair (p0, p1), uniform over the 6
    pairs, stored as p0 | p1 << 2 in byte j // 2 (low nibble for even j)."""
    pick = rng(seed).integers(0, 6, size=(M, K // 4))
    nib = np.array([p0 | (p1 << 2) for p0, p1 in SP24_PAIRS], dtype=np.uint8)[pick]
    return (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)


def sp24_inputs(M: int, N: int, K: int, dtype: int, seed_a: int, seed_meta: int, seed_b: int,
                integer: bool = False):
    """Kept values Ac [M, K/2] and B [K, N] as storage words, position nibbles
    Ai [M, K/8]."""
    draw = integers_f32 if integer else normal_f32
    Ac = to_storage(draw((M, K // 2), seed_a), dtype)
    B = to_storage(draw((K, N), seed_b), dtype)
    return Ac, sp24_meta(M, K, seed_meta), B


@dataclass(frozen=True)
class Workload:
    """One of the workload shapes; `index` keys the seeds."""

    name: str
    index: int
    op: str  # "gemm", "dequant_w4", "mx" or "sp24"
    dtype: int  # operand type; for "mx" the activation format (MX_E2M1 / MX_E4M3)
    M: int
    N: int
    K: int
    relu: bool

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K

    def algorithmic_bytes(self) -> int:
        """Read every operand once and write C once."""
        if self.op == "gemm":
            es = 4 if self.dtype == F32 else 2
            return es * (self.M * self.K + self.K * self.N + self.M * self.N)
        if self.op == "sp24":
            return 2 * (self.M * self.K // 2 + self.K * self.N + self.M * self.N) + self.M * self.K // 8
        if self.op == "mx":
            a = self.M * self.K // 2 if self.dtype == MX_E2M1 else self.M * self.K
            return (a + self.M * self.K // 32 + self.N * self.K // 2 + self.N * self.K // 32
                    + 2 * self.M * self.N)
        return 2 * self.M * self.K + self.N * self.K // 2 + self.N * self.K // 32 + 2 * self.M * self.N


WORKLOADS = {
    "f32_512": Workload("f32_512", 1, "gemm", F32, 512, 512, 512, False),
    "f16_1024": Workload("f16_1024", 2, "gemm", F16, 1024, 1024, 1024, False),
    "f32_4096": Workload("f32_4096", 3, "gemm", F32, 4096, 4096, 4096, False),
    "bf16_4096_relu": Workload("bf16_4096_relu", 4, "gemm", BF16, 4096, 4096, 4096, True),
    "bf16_4000x4032x4096_relu": Workload("bf16_4000x4032x4096_relu", 4, "gemm", BF16,
                                         4000, 4032, 4096, True),
    "w4_256x8192x8192": Workload("w4_256x8192x8192", 5, "dequant_w4", BF16, 256, 8192, 8192,
                                 False),
    # memory-bound probes of the same dequant entry (decode-like M)
    "w4_1x8192x8192": Workload("w4_1x8192x8192", 6, "dequant_w4", BF16, 1, 8192, 8192, False),
    "w4_16x8192x8192": Workload("w4_16x8192x8192", 7, "dequant_w4", BF16, 16, 8192, 8192, False),
    # the same weight format with block-format activations on the scaled MFMA
    "mx_e2m1_8192": Workload("mx_e2m1_8192", 8, "mx", MX_E2M1, 8192, 8192, 8192, False),
    "mx_e4m3_8192": Workload("mx_e4m3_8192", 9, "mx", MX_E4M3, 8192, 8192, 8192, False),
    # 2:4 structured-sparse A (the flops are the dense-equivalent 2 M N K)
    "sp24_bf16_4096_relu": Workload("sp24_bf16_4096_relu", 10, "sp24", BF16, 4096, 4096, 4096,
                                    True),
    # tile grids that are not whole waves of one tile per compute unit
    # (384 and 144 tiles of 256 x 256): the tail of the last wave
    "bf16_6144x4096x4096_relu": Workload("bf16_6144x4096x4096_relu", 11, "gemm", BF16,
                                         6144, 4096, 4096, True),
    "bf16_3072_relu": Workload("bf16_3072_relu", 12, "gemm", BF16, 3072, 3072, 3072, True),
}


def seeds(w: Workload, integer: bool = False) -> dict:
    base = 20260000 + 100 * w.index + (50 if integer else 0)
    return {"A": base + 0, "B": base + 1, "codes": base + 2, "scales": base + 3,
            "a_scales": base + 4}


def gemm_inputs(M: int, N: int, K: int, dtype: int, seed_a: int, seed_b: int,
                integer: bool = False):
    """Row-major A [M, K] and B [K, N] as storage words."""
    draw = integers_f32 if integer else normal_f32
    A = to_storage(draw((M, K), seed_a), dtype)
    B = to_storage(draw((K, N), seed_b), dtype)
    return A, B


def dequant_inputs(M: int, N: int, K: int, seed_a: int, seed_codes: int, seed_scales: int,
                   integer: bool = False):
    """bf16 activations [M, K], packed codes [N, K/2], scale bytes [N, K/32]."""
    draw = integers_f32 if integer else normal_f32
    A = to_storage(draw((M, K), seed_a), BF16)
    return A, w4_codes(N, K, seed_codes), w4_scales(N, K, seed_scales)


def make_inputs(w: Workload, integer: bool = False) -> dict:
    s = seeds(w, integer)
    if w.op == "gemm":
        A, B = gemm_inputs(w.M, w.N, w.K, w.dtype, s["A"], s["B"], integer)
        return {"A": A, "B": B, "seeds": s}
    if w.op == "mx":
        Aq, As, Wq, Ws = mx_inputs(w.dtype, w.M, w.N, w.K, s["A"], s["a_scales"], s["codes"],
                                   s["scales"])
        return {"Aq": Aq, "As": As, "Wq": Wq, "Ws": Ws, "seeds": s}
    if w.op == "sp24":
        Ac, Ai, B = sp24_inputs(w.M, w.N, w.K, w.dtype, s["A"], s["codes"], s["B"], integer)
        return {"Ac": Ac, "Ai": Ai, "B": B, "seeds": s}
    A, Wq, Ws = dequant_inputs(w.M, w.N, w.K, s["A"], s["codes"], s["scales"], integer)
    return {"A": A, "Wq": Wq, "Ws": Ws, "seeds": s}
