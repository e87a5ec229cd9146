"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each check takes an ``oracle.Oracle`` so the same checks can also be run
against deliberately broken copies of the oracle (tests/test_oracle_mutants.py)
to show that a plausible mistake in it is caught.

What pins what:
  * number codecs: exhaustive comparison with numpy / torch CPU casts, and an
    exact-rational (fractions.Fraction) round-to-nearest-even written here
    from the definition of a binary floating-point grid;
  * E2M1 / E8M0: the OCP MX v1.0 tables under tests/golden/, and torch's
    float8_e8m0fnu encoding;
  * GEMM: closed forms (identity, permutation, all ones, rank one, the 2 x 2
    textbook product) and brute force in exact rational arithmetic;
  * ReLU: y = max(sum, 0) with +0 for non-positive sums;
  * dequant GEMM: reductions to row sums, one-hot weights (nibble order and
    the k/32 scale index), per-group scales, and a weight decode done here from
    the golden table;
  * E4M3: the OCP MX v1.0 landmark values under tests/golden/ and torch's
    float8_e4m3fn decoding of all 256 codes;
  * MX-format GEMM: row sums, one-hot activations and weights (nibble order,
    E4M3 row stride, both k/32 scale indexes), NaN scales and codes, and exact
    rational brute force on operands decoded here (golden E2M1 table, torch
    E4M3, powers of two);
  * 2:4 sparse GEMM: a dense 2:4 matrix compressed here (values and position
    nibbles) must give the exact rational product of the dense matrix, in
    both the full and the entry-by-entry oracle; one-hot kept values pin the
    group stride, the value order and the nibble order; a repeated position
    must add both values.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

F32, F16, BF16 = 0, 1, 2
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------------------
# Independent helpers (written here, not taken from the oracle).
# ---------------------------------------------------------------------------

def rne_fraction(x: Fraction, ebits: int, fbits: int):
    """Nearest value of a binary floating-point grid, ties to even (exact).

    Returns a Fraction, or +-inf on overflow.
    """
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    bias = 2 ** (ebits - 1) - 1
    emin = 1 - bias
    emax = (2 ** ebits - 2) - bias
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = max(e, emin) - fbits
    scaled = a / (Fraction(2) ** q)
    n = math.floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * Fraction(2) ** q
    maxval = (2 - Fraction(1, 2 ** fbits)) * Fraction(2) ** emax
    if val > maxval:
        return sign * math.inf
    return sign * val


def storage_of(values, dtype: int) -> np.ndarray:
    """Exactly representable float values -> storage words via numpy / torch casts."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == F32:
        f = v.astype(np.float32)
        assert np.array_equal(f.astype(np.float64), v), "value not exact in fp32"
        return f.view(np.uint32)
    if dtype == F16:
        h = v.astype(np.float16)
        assert np.array_equal(h.astype(np.float64), v), "value not exact in fp16"
        return h.view(np.uint16)
    import torch

    t = torch.from_numpy(v).to(torch.bfloat16)
    assert np.array_equal(t.to(torch.float64).numpy(), v), "value not exact in bf16"
    return t.view(torch.int16).numpy().view(np.uint16)


def exact_product(A, B):
    """Exact rational A @ B for small float64 matrices."""
    M, K = A.shape
    _, N = B.shape
    out = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            for k in range(K):
                s += Fraction(float(A[i, k])) * Fraction(float(B[k, j]))
            out[i][j] = s
    return out


def load_e2m1_golden():
    tab = {}
    with open(os.path.join(GOLDEN, "e2m1_table.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            tab[int(code)] = float(val)
    assert sorted(tab) == list(range(16))
    return tab


def load_e8m0_golden():
    pts = {}
    with open(os.path.join(GOLDEN, "e8m0_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            e, lg = line.split()
            pts[int(e)] = None if lg == "nan" else int(lg)
    return pts


def load_e4m3_golden():
    pts = {}
    with open(os.path.join(GOLDEN, "e4m3_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, val = line.split()
            pts[int(code, 16)] = float(val)  # "nan" and "-0" parse as floats
    return pts


def decode_e4m3_torch(codes):
    """E4M3 codes -> float64 through torch's float8_e4m3fn (a library decoder)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8))
    return t.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def decode_mx_a_here(fmt, Aq, As):
    """Test-side activation decode (golden E2M1 table or torch E4M3, ldexp scales)."""
    Aq = np.asarray(Aq, dtype=np.uint8)
    if fmt == 0:
        tab = load_e2m1_golden()
        lut = np.array([tab[c] for c in range(16)], dtype=np.float64)
        M, half = Aq.shape
        codes = np.empty((M, 2 * half), dtype=np.uint8)
        codes[:, 0::2] = Aq & 0xF
        codes[:, 1::2] = Aq >> 4
        elem = lut[codes]
    else:
        elem = decode_e4m3_torch(Aq)
    scale = np.ldexp(1.0, np.asarray(As, dtype=np.int64) - 127)
    return elem * np.repeat(scale, 32, axis=1)


def decode_w4_here(Wq, Ws):
    """Test-side weight decode from the golden tables (independent of the oracle)."""
    tab = load_e2m1_golden()
    lut = np.array([tab[c] for c in range(16)], dtype=np.float64)
    Wq = np.asarray(Wq, dtype=np.uint8)
    N, half = Wq.shape
    K = 2 * half
    codes = np.empty((N, K), dtype=np.uint8)
    codes[:, 0::2] = Wq & 0xF
    codes[:, 1::2] = Wq >> 4
    scale = np.ldexp(1.0, np.asarray(Ws, dtype=np.int64) - 127)
    return lut[codes] * np.repeat(scale, 32, axis=1)


def _gemm_both(orc, A, B, dtype, relu=False):
    """Full-matrix and entry-by-entry oracle results (both must pass every pin)."""
    Y = orc.gemm_f64(A, B, dtype, relu)
    M, N = Y.shape
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Ye = orc.gemm_entries_f64(A, B, dtype, rr.ravel(), cc.ravel(), relu).reshape(M, N)
    return Y, Ye


def _dq_both(orc, A, Wq, Ws, relu=False):
    Y = orc.dequant_w4_f64(A, Wq, Ws, relu)
    M, N = Y.shape
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Ye = orc.dequant_w4_entries_f64(A, Wq, Ws, rr.ravel(), cc.ravel(), relu).reshape(M, N)
    return Y, Ye


def _mx_both(orc, fmt, Aq, As, Wq, Ws, relu=False):
    Y = orc.mx_gemm_f64(fmt, Aq, As, Wq, Ws, relu)
    M, N = Y.shape
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Ye = orc.mx_gemm_entries_f64(fmt, Aq, As, Wq, Ws, rr.ravel(), cc.ravel(), relu).reshape(M, N)
    return Y, Ye


def _same(x, y):
    """Bitwise equality of float64 arrays (distinguishes +0 and -0)."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    return x.shape == y.shape and np.array_equal(x.view(np.uint64), y.view(np.uint64))


# ---------------------------------------------------------------------------
# Codec pins.
# ---------------------------------------------------------------------------

def check_decode_f16_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.decode(F16, bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert _same(got[~nan], ref[~nan])


def check_decode_bf16_exhaustive(orc):
    import torch

    bits = np.arange(65536, dtype=np.uint16)
    got = orc.decode(BF16, bits)
    # bf16 is the upper half of a binary32 word
    ref = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref_t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert _same(got[~nan], ref[~nan])
    assert _same(ref_t[~nan], ref[~nan])


def check_decode_f32_sample(orc):
    r = np.random.Generator(np.random.PCG64(11))
    bits = r.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0, 0x80000000, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000, 0xFF800000]
    got = orc.decode(F32, bits)
    ref = bits.view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert _same(got[~nan], ref[~nan])


def _random_doubles(seed, n):
    r = np.random.Generator(np.random.PCG64(seed))
    x = r.standard_normal(n) * np.exp2(r.integers(-40, 40, size=n))
    return x


def check_encode_f16(orc):
    x = np.concatenate([
        _random_doubles(1, 100000) * 1e-3,
        np.random.Generator(np.random.PCG64(2)).standard_normal(100000) * 3e4,  # overflow side
        np.random.Generator(np.random.PCG64(3)).standard_normal(100000) * 1e-6,  # subnormals
    ])
    # constructed ties: midpoints between neighbouring fp16 values
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16).view(np.float16).astype(np.float64)
    h2 = (np.arange(0, 0x7BFF, 7, dtype=np.uint16) + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (h + h2) / 2, -(h + h2) / 2, [65504.0, 65519.99, 65520.0, 1e9, -1e9]])
    got = orc.encode(F16, x).view(np.float16).astype(np.float64)
    ref = x.astype(np.float16).astype(np.float64)  # numpy rounds float64 -> float16 once
    assert _same(got, ref)


def check_encode_f32(orc):
    x = np.concatenate([_random_doubles(4, 200000),
                        np.random.Generator(np.random.PCG64(5)).standard_normal(1000) * 1e-40,
                        [3.5e38, 3.4028235677973366e38, 1e39, -1e39]])
    got = orc.encode(F32, x).view(np.float32).astype(np.float64)
    ref = x.astype(np.float32).astype(np.float64)
    assert _same(got, ref)


def check_encode_bf16_from_f32(orc):
    import torch

    r = np.random.Generator(np.random.PCG64(6))
    f = r.standard_normal(200000).astype(np.float32)
    # constructed ties: exactly halfway between two bf16 neighbours
    hi = r.integers(0, 0x7F00, size=20000).astype(np.uint32) << 16
    ties = (hi | 0x8000).view(np.float32)
    f = np.concatenate([f, ties, -ties, np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8], np.float32)])
    got = orc.encode(BF16, f.astype(np.float64))
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # worked ties: 1 + 2^-8 -> 1.0 (even), 1 + 3*2^-8 -> 1 + 2^-6
    assert got[-2] == 0x3F80 and got[-1] == 0x3F82


def check_encode_exact_rational(orc):
    """Direct fp64 -> fp16 / bf16 / fp32 rounding against Fraction RNE (single rounding)."""
    x = _random_doubles(7, 1500)
    x = np.concatenate([x, [0.0, -0.0, 2.0 ** -140, 6e-8, -6e-8, 2.0 ** -25, 2.0 ** -24 * 1.5]])
    for dtype, eb, fb in ((F16, 5, 10), (BF16, 8, 7), (F32, 8, 23)):
        got = orc.decode(dtype, orc.encode(dtype, x))
        for xi, gi in zip(x, got):
            ref = rne_fraction(Fraction(float(xi)), eb, fb)
            if isinstance(ref, float):  # inf
                assert gi == ref, (dtype, xi, gi)
            else:
                assert Fraction(float(gi)) == ref, (dtype, xi, gi, ref)


def check_e2m1_table(orc):
    tab = load_e2m1_golden()
    for code, val in tab.items():
        got = orc.decode_e2m1(code)
        assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), (code, got)


def check_e8m0(orc):
    import torch

    for e, lg in load_e8m0_golden().items():
        got = orc.decode_e8m0(e)
        if lg is None:
            assert math.isnan(got)
        else:
            assert got == math.ldexp(1.0, lg), (e, got)
    # torch's float8_e8m0fnu encodes powers of two to the same byte
    for e in range(0, 255):
        v = orc.decode_e8m0(e)
        b = torch.tensor([v], dtype=torch.float32).to(torch.float8_e8m0fnu).view(torch.uint8)
        assert int(b.item()) == e, (e, v)


# ---------------------------------------------------------------------------
# GEMM pins.
# ---------------------------------------------------------------------------

def check_textbook_2x2(orc):
    for dtype in (F32, F16, BF16):
        A = storage_of([[1, 2], [3, 4]], dtype)
        B = storage_of([[5, 6], [7, 8]], dtype)
        for Y in _gemm_both(orc, A, B, dtype):
            assert _same(Y, [[19, 22], [43, 50]])


def check_identity(orc):
    r = np.random.Generator(np.random.PCG64(21))
    for dtype in (F32, F16, BF16):
        K, N = 24, 17
        Bv = r.integers(-100, 101, size=(K, N)) / 8.0
        B = storage_of(Bv, dtype)
        A = storage_of(np.eye(K), dtype)
        for Y in _gemm_both(orc, A, B, dtype):
            assert _same(Y + 0.0, Bv + 0.0)


def check_permutation(orc):
    r = np.random.Generator(np.random.PCG64(22))
    for dtype in (F32, BF16):
        K, N = 19, 13
        perm = r.permutation(K)
        P = np.zeros((K, K))
        P[np.arange(K), perm] = 1.0
        Bv = r.integers(-50, 51, size=(K, N)).astype(np.float64)
        for Y in _gemm_both(orc, storage_of(P, dtype), storage_of(Bv, dtype), dtype):
            assert _same(Y + 0.0, Bv[perm] + 0.0)


def check_all_ones(orc):
    for dtype in (F32, F16, BF16):
        for (M, N, K) in ((3, 5, 7), (1, 1, 1), (9, 4, 33)):
            A = storage_of(np.ones((M, K)), dtype)
            B = storage_of(np.ones((K, N)), dtype)
            for Y in _gemm_both(orc, A, B, dtype):
                assert _same(Y, np.full((M, N), float(K)))


def check_rank_one(orc):
    # A[m, k] = u_m * a_k, B[k, n] = b_k * v_n  ->  C = (a . b) u_m v_n.
    # Non-symmetric vectors: a transposed operand or a wrong index changes it.
    u = np.array([1, -2, 3, 0, 5, -1, 2], dtype=np.float64)
    a = np.array([2, 1, -3, 4, 1, -1, 3, 2, -2, 1, 1], dtype=np.float64)
    b = np.array([1, 3, 2, -1, 2, 2, -3, 1, 1, -2, 4], dtype=np.float64)
    v = np.array([3, -1, 2, 1, -2, 4, 1, 1, 2], dtype=np.float64)
    ab = float(a @ b)
    ref = ab * np.outer(u, v)
    for dtype in (F32, F16, BF16):
        A = storage_of(np.outer(u, a), dtype)
        B = storage_of(np.outer(b, v), dtype)
        for Y in _gemm_both(orc, A, B, dtype):
            assert _same(Y + 0.0, ref + 0.0)


def check_brute_force_dyadic(orc):
    r = np.random.Generator(np.random.PCG64(23))
    for trial in range(60):
        M, N, K = (int(x) for x in r.integers(1, 9, size=3))
        dtype = (F32, F16, BF16)[trial % 3]
        Av = r.integers(-64, 65, size=(M, K)) * np.exp2(r.integers(-6, 1, size=(M, K)))
        Bv = r.integers(-64, 65, size=(K, N)) * np.exp2(r.integers(-6, 1, size=(K, N)))
        ex = exact_product(Av, Bv)
        for relu in (False, True):
            for Y in _gemm_both(orc, storage_of(Av, dtype), storage_of(Bv, dtype), dtype, relu):
                for i in range(M):
                    for j in range(N):
                        want = ex[i][j]
                        if relu:
                            want = max(want, Fraction(0))
                        assert Fraction(float(Y[i, j])) == want, (M, N, K, i, j)


def check_brute_force_general(orc):
    """General fp32 inputs: the fp64 sum is within the standard accumulation bound."""
    r = np.random.Generator(np.random.PCG64(24))
    for _ in range(20):
        M, N, K = (int(x) for x in r.integers(1, 9, size=3))
        Af = r.standard_normal((M, K)).astype(np.float32)
        Bf = r.standard_normal((K, N)).astype(np.float32)
        ex = exact_product(Af.astype(np.float64), Bf.astype(np.float64))
        for Y in _gemm_both(orc, Af.view(np.uint32), Bf.view(np.uint32), F32):
            for i in range(M):
                for j in range(N):
                    mag = sum(abs(float(Af[i, k]) * float(Bf[k, j])) for k in range(K))
                    err = abs(Fraction(float(Y[i, j])) - ex[i][j])
                    assert err <= Fraction(K + 1) * Fraction(1, 2 ** 52) * Fraction(mag)


def check_relu(orc):
    r = np.random.Generator(np.random.PCG64(25))
    M, N, K = 7, 9, 5
    Av = r.integers(-4, 5, size=(M, K)).astype(np.float64)
    Bv = r.integers(-4, 5, size=(K, N)).astype(np.float64)
    for dtype in (F32, BF16):
        A, B = storage_of(Av, dtype), storage_of(Bv, dtype)
        Y0 = orc.gemm_f64(A, B, dtype, False)
        for Y in _gemm_both(orc, A, B, dtype, True):
            assert np.all(Y >= 0) and not np.any(np.signbit(Y))
            assert _same(Y, np.where(Y0 > 0, Y0, 0.0))
        assert np.any(Y0 < 0) and np.any(Y0 > 0)


def check_round_outputs(orc):
    """Integer sums below 2^24 encode exactly; fp16 overflow goes to inf."""
    y = np.array([0.0, 1.0, -3.0, 16384.0, 65504.0, 65520.0, 2.0 ** 23 + 1, -(2.0 ** 24)])
    assert np.array_equal(orc.decode(F32, orc.encode(F32, y)), y)
    f16 = orc.decode(F16, orc.encode(F16, y))
    assert f16[4] == 65504.0 and math.isinf(f16[5])
    assert np.array_equal(f16[:4], y[:4])


# ---------------------------------------------------------------------------
# Dequant GEMM pins.
# ---------------------------------------------------------------------------

def _bf16_ints(r, shape, lo=-4, hi=4):
    v = r.integers(lo, hi + 1, size=shape).astype(np.float64)
    return v, storage_of(v, BF16)


def check_dequant_row_sums(orc):
    r = np.random.Generator(np.random.PCG64(31))
    M, N, K = 5, 6, 64
    Av, A = _bf16_ints(r, (M, K))
    Wq = np.full((N, K // 2), 0x22, dtype=np.uint8)  # every code is 2 -> 1.0
    Ws = np.full((N, K // 32), 127, dtype=np.uint8)  # every scale 2^0
    for Y in _dq_both(orc, A, Wq, Ws):
        assert _same(Y + 0.0, np.repeat(Av.sum(axis=1, keepdims=True), N, axis=1) + 0.0)


def check_dequant_one_hot(orc):
    r = np.random.Generator(np.random.PCG64(32))
    tab = load_e2m1_golden()
    M, N, K = 4, 5, 96
    Av, A = _bf16_ints(r, (M, K))
    for (n0, k0, code, e) in ((0, 0, 7, 127), (1, 1, 3, 125), (2, 33, 13, 126),
                              (4, 95, 5, 123), (3, 64, 9, 130), (2, 62, 15, 124)):
        Wq = np.zeros((N, K // 2), dtype=np.uint8)
        Wq[n0, k0 // 2] = code << (4 * (k0 % 2))
        Ws = np.full((N, K // 32), 127, dtype=np.uint8)
        Ws[n0, k0 // 32] = e
        want = np.zeros((M, N))
        want[:, n0] = Av[:, k0] * tab[code] * 2.0 ** (e - 127)
        for Y in _dq_both(orc, A, Wq, Ws):
            assert _same(Y + 0.0, want + 0.0), (n0, k0, code, e)


def check_dequant_group_scales(orc):
    r = np.random.Generator(np.random.PCG64(33))
    M, N, K = 3, 4, 128
    Av, A = _bf16_ints(r, (M, K))
    Wq = np.full((N, K // 2), 0x44, dtype=np.uint8)  # every code 4 -> 2.0
    Ws = r.integers(120, 131, size=(N, K // 32)).astype(np.uint8)
    gsum = Av.reshape(M, K // 32, 32).sum(axis=2)  # [M, groups]
    want = 2.0 * gsum @ np.ldexp(1.0, Ws.astype(np.int64) - 127).T
    for Y in _dq_both(orc, A, Wq, Ws):
        assert _same(Y + 0.0, want + 0.0)


def check_dequant_random_vs_decoded(orc):
    r = np.random.Generator(np.random.PCG64(34))
    M, N, K = 6, 10, 96
    Av, A = _bf16_ints(r, (M, K))
    Wq = r.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    Ws = (127 + r.integers(-4, 1, size=(N, K // 32))).astype(np.uint8)
    W = decode_w4_here(Wq, Ws)
    assert _same(orc.w4_decode(Wq, Ws) + 0.0, W + 0.0)
    ex = exact_product(Av, W.T)
    for relu in (False, True):
        for Y in _dq_both(orc, A, Wq, Ws, relu):
            for i in range(M):
                for j in range(N):
                    want = max(ex[i][j], Fraction(0)) if relu else ex[i][j]
                    assert Fraction(float(Y[i, j])) == want


# ---------------------------------------------------------------------------
# E4M3 and the MX-format GEMM.
# ---------------------------------------------------------------------------

def check_e4m3_points(orc):
    for code, val in load_e4m3_golden().items():
        got = orc.decode_e4m3(code)
        if math.isnan(val):
            assert math.isnan(got), (code, got)
        else:
            assert got == val and math.copysign(1.0, got) == math.copysign(1.0, val), (code, got)


def check_e4m3_vs_torch(orc):
    ref = decode_e4m3_torch(np.arange(256))
    for code in range(256):
        got = orc.decode_e4m3(code)
        if math.isnan(ref[code]):
            assert math.isnan(got), (code, got)
        else:
            assert _same(got, ref[code]), (code, got, ref[code])


E2M1_ONE, E4M3_ONE = 0x2, 0x38  # the codes of 1.0


def _mx_ones(fmt, M, K):
    if fmt == 0:
        return np.full((M, K // 2), E2M1_ONE * 0x11, dtype=np.uint8)
    return np.full((M, K), E4M3_ONE, dtype=np.uint8)


def check_mx_row_sums(orc):
    # a == 1 everywhere: Y[m][n] = sum_k w(n, k), the decoded weight row sums
    r = np.random.Generator(np.random.PCG64(41))
    M, N, K = 3, 5, 96
    Wq = r.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    Ws = r.integers(124, 131, size=(N, K // 32)).astype(np.uint8)
    want = np.repeat(decode_w4_here(Wq, Ws).sum(axis=1)[None, :], M, axis=0)
    As = np.full((M, K // 32), 127, dtype=np.uint8)
    for fmt in (0, 1):
        for Y in _mx_both(orc, fmt, _mx_ones(fmt, M, K), As, Wq, Ws):
            assert _same(Y + 0.0, want + 0.0), fmt


def check_mx_one_hot(orc):
    # one nonzero activation and one nonzero weight at the same k: Y has a
    # single nonzero entry, the product of the two decoded values
    tab = load_e2m1_golden()
    M, N, K = 4, 3, 128
    cases = ((0, 0, 0, 0, 7, 0x3c, 127, 126), (1, 2, 33, 1, 3, 0x01, 125, 129),
             (3, 1, 62, 15, 13, 0xfe, 124, 130), (2, 0, 95, 6, 5, 0x4a, 128, 120),
             (1, 1, 127, 9, 1, 0x81, 131, 127))
    for fmt in (0, 1):
        for (m0, n0, k0, ca2, cw, ca8, ea, ew) in cases:
            ca = ca2 if fmt == 0 else ca8
            Aq = np.zeros((M, K // 2) if fmt == 0 else (M, K), dtype=np.uint8)
            if fmt == 0:
                Aq[m0, k0 // 2] = ca << (4 * (k0 % 2))
                av = tab[ca]
            else:
                Aq[m0, k0] = ca
                av = float(decode_e4m3_torch(np.array([ca]))[0])
            As = np.full((M, K // 32), 127, dtype=np.uint8)
            As[m0, k0 // 32] = ea
            Wq = np.zeros((N, K // 2), dtype=np.uint8)
            Wq[n0, k0 // 2] = cw << (4 * (k0 % 2))
            Ws = np.full((N, K // 32), 127, dtype=np.uint8)
            Ws[n0, k0 // 32] = ew
            want = np.zeros((M, N))
            want[m0, n0] = av * 2.0 ** (ea - 127) * tab[cw] * 2.0 ** (ew - 127)
            for Y in _mx_both(orc, fmt, Aq, As, Wq, Ws):
                assert _same(Y + 0.0, want + 0.0), (fmt, m0, n0, k0)


def check_mx_nan(orc):
    # a NaN scale (E8M0 255) or a NaN E4M3 code poisons exactly the results
    # that take one of its products
    M, N, K = 3, 4, 64
    Wq = np.full((N, K // 2), 0x22, dtype=np.uint8)
    Ws = np.full((N, K // 32), 127, dtype=np.uint8)
    for fmt in (0, 1):
        Aq = _mx_ones(fmt, M, K)
        As = np.full((M, K // 32), 127, dtype=np.uint8)
        As[1, 1] = 255
        for Y in _mx_both(orc, fmt, Aq, As, Wq, Ws):
            assert np.isnan(Y[1]).all() and not np.isnan(Y[[0, 2]]).any()
        As[1, 1] = 127
        Ws2 = Ws.copy()
        Ws2[2, 0] = 255
        for Y in _mx_both(orc, fmt, Aq, As, Wq, Ws2):
            assert np.isnan(Y[:, 2]).all() and not np.isnan(Y[:, [0, 1, 3]]).any()
    Aq = _mx_ones(1, M, K)
    Aq[2, 40] = 0xff
    for Y in _mx_both(orc, 1, Aq, np.full((M, K // 32), 127, dtype=np.uint8), Wq, Ws):
        assert np.isnan(Y[2]).all() and not np.isnan(Y[:2]).any()


def check_mx_random_vs_decoded(orc):
    r = np.random.Generator(np.random.PCG64(42))
    M, N, K = 5, 7, 128
    Wq = r.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    Ws = r.integers(118, 137, size=(N, K // 32)).astype(np.uint8)
    W = decode_w4_here(Wq, Ws)
    for fmt in (0, 1):
        if fmt == 0:
            Aq = r.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
        else:
            Aq = r.integers(0, 256, size=(M, K), dtype=np.uint8)
            Aq[(Aq & 0x7F) == 0x7F] = 0x3a  # no NaN codes here
        As = r.integers(118, 137, size=(M, K // 32)).astype(np.uint8)
        A = decode_mx_a_here(fmt, Aq, As)
        assert _same(orc.mx_decode_a(fmt, Aq, As) + 0.0, A + 0.0), fmt
        ex = exact_product(A, W.T)
        for relu in (False, True):
            for Y in _mx_both(orc, fmt, Aq, As, Wq, Ws, relu):
                for i in range(M):
                    for j in range(N):
                        want = max(ex[i][j], Fraction(0)) if relu else ex[i][j]
                        assert Fraction(float(Y[i, j])) == want, (fmt, relu, i, j)


# ---------------------------------------------------------------------------
# 2:4 structured-sparse GEMM.
# ---------------------------------------------------------------------------

def compress_sp24_here(A):
    """Dense [M, K] with at most two nonzeros per group of 4 k -> values
    [M, K/2] (float64) and metadata [M, K/8]: group j keeps (v0 at p0, v1 at
    p1), p0 < p1, the nibble p0 | p1 << 2 in byte j // 2 at bit 4 (j % 2).
    Groups with fewer nonzeros fill the remaining slots with zero values at
    unused positions."""
    A = np.asarray(A, dtype=np.float64)
    M, K = A.shape
    vals = np.zeros((M, K // 2))
    meta = np.zeros((M, K // 8), dtype=np.uint8)
    for m in range(M):
        for j in range(K // 4):
            g = A[m, 4 * j:4 * j + 4]
            pos = [p for p in range(4) if g[p] != 0]
            assert len(pos) <= 2, "not 2:4 sparse"
            for p in range(4):
                if len(pos) == 2:
                    break
                if p not in pos:
                    pos.append(p)
            p0, p1 = sorted(pos)
            vals[m, 2 * j], vals[m, 2 * j + 1] = g[p0], g[p1]
            meta[m, j // 2] |= (p0 | (p1 << 2)) << (4 * (j % 2))
    return vals, meta


def _sp24_both(orc, Ac, Ai, B, dtype, relu=False):
    Y = orc.gemm_sp24_f64(Ac, Ai, B, dtype, relu)
    M, N = Y.shape
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    Ye = orc.gemm_sp24_entries_f64(Ac, Ai, B, dtype, rr.ravel(), cc.ravel(), relu).reshape(M, N)
    return Y, Ye


def _random_sp24_dense(r, M, K, lo=-4, hi=4):
    A = np.zeros((M, K))
    for m in range(M):
        for j in range(K // 4):
            for p in r.choice(4, size=2, replace=False):
                A[m, 4 * j + p] = r.integers(lo, hi + 1) + 0.5 * r.integers(0, 2)
    return A


def check_sp24_brute_force(orc):
    r = np.random.Generator(np.random.PCG64(51))
    for dtype, (M, N, K) in ((BF16, (5, 7, 32)), (F16, (3, 9, 48)), (F32, (4, 6, 24))):
        A = _random_sp24_dense(r, M, K)
        B = r.integers(-4, 5, size=(K, N)).astype(np.float64) * 0.25
        vals, meta = compress_sp24_here(A)
        Ac, Bs = storage_of(vals, dtype), storage_of(B, dtype)
        assert _same(orc.sp24_densify(Ac, meta, dtype) + 0.0, A + 0.0), dtype
        ex = exact_product(A, B)
        for relu in (False, True):
            for Y in _sp24_both(orc, Ac, meta, Bs, dtype, relu):
                for i in range(M):
                    for j in range(N):
                        want = max(ex[i][j], Fraction(0)) if relu else ex[i][j]
                        assert Fraction(float(Y[i, j])) == want, (dtype, relu, i, j)


def check_sp24_one_hot(orc):
    # one kept value: Y[m0] = v * B[4 j + p], other rows zero
    r = np.random.Generator(np.random.PCG64(52))
    M, N, K = 3, 5, 32
    B = r.integers(-8, 9, size=(K, N)).astype(np.float64)
    Bs = storage_of(B, BF16)
    for (m0, j, t, p, v) in ((0, 0, 0, 0, 1.5), (1, 1, 1, 3, -2.0), (2, 6, 0, 2, 3.0),
                             (1, 7, 1, 1, 0.5), (0, 5, 1, 2, -1.0)):
        vals = np.zeros((M, K // 2))
        meta = np.zeros((M, K // 8), dtype=np.uint8)
        vals[m0, 2 * j + t] = v
        other = 0 if p != 0 else 1  # the other slot's position (its value is zero)
        nib = (p | (other << 2)) if t == 0 else (other | (p << 2))
        meta[m0, j // 2] = nib << (4 * (j % 2))
        want = np.zeros((M, N))
        want[m0] = v * B[4 * j + p]
        for Y in _sp24_both(orc, storage_of(vals, BF16), meta, Bs, BF16):
            assert _same(Y + 0.0, want + 0.0), (m0, j, t, p)


def check_sp24_repeated_position(orc):
    # both values of a group at one position: that element of A is their sum
    M, N, K = 2, 3, 16
    B = np.arange(K * N, dtype=np.float64).reshape(K, N) - 20.0
    vals = np.zeros((M, K // 2))
    meta = np.zeros((M, K // 8), dtype=np.uint8)
    vals[1, 2 * 3], vals[1, 2 * 3 + 1] = 2.0, 5.0  # group 3, both at position 1
    meta[1, 1] = (1 | (1 << 2)) << 4
    want = np.zeros((M, N))
    want[1] = 7.0 * B[4 * 3 + 1]
    for Y in _sp24_both(orc, storage_of(vals, F32), meta, storage_of(B, F32), F32):
        assert _same(Y + 0.0, want + 0.0)


# ---------------------------------------------------------------------------
# Operands stored transposed (C = op(A) op(B)).
# ---------------------------------------------------------------------------

LAYOUTS = ((0, 0), (0, 1), (1, 0), (1, 1))


def _stored(X, trans):
    """Storage of a logical matrix X: as is, or its transpose."""
    X = np.asarray(X, dtype=np.float64)
    return np.ascontiguousarray(X.T) if trans else X


def check_layout_textbook_2x2(orc):
    for dtype in (F32, F16, BF16):
        for ta, tb in LAYOUTS:
            A = storage_of(_stored([[1, 2], [3, 4]], ta), dtype)
            B = storage_of(_stored([[5, 6], [7, 8]], tb), dtype)
            Y = orc.gemm_layout_f64(A, ta, B, tb, dtype)
            assert _same(Y, [[19, 22], [43, 50]]), (ta, tb)
            e = orc.gemm_layout_entries_f64(A, ta, B, tb, dtype, [0, 0, 1, 1], [0, 1, 0, 1])
            assert _same(e, [19, 22, 43, 50]), (ta, tb)


def check_layout_brute_force(orc):
    """Random dyadic operands in every layout, against the exact rational
    product of the logical matrices (the stored arrays transposed here)."""
    r = np.random.Generator(np.random.PCG64(31))
    for trial in range(24):
        M, N, K = (int(x) for x in r.integers(1, 9, size=3))
        ta, tb = LAYOUTS[trial % 4]
        dtype = (F32, F16, BF16)[trial % 3]
        Av = r.integers(-64, 65, size=(M, K)) / 16.0
        Bv = r.integers(-64, 65, size=(K, N)) / 16.0
        A = storage_of(_stored(Av, ta), dtype)
        B = storage_of(_stored(Bv, tb), dtype)
        # dyadic inputs with small sums: the exact product is an fp64 value
        want = np.array([[float(x) for x in row] for row in exact_product(Av, Bv)])
        Y = orc.gemm_layout_f64(A, ta, B, tb, dtype)
        assert _same(Y + 0.0, want + 0.0), (M, N, K, ta, tb)
        rows = np.repeat(np.arange(M), N)
        cols = np.tile(np.arange(N), M)
        e = orc.gemm_layout_entries_f64(A, ta, B, tb, dtype, rows, cols)
        assert _same(e.reshape(M, N) + 0.0, want + 0.0), (M, N, K, ta, tb)


def check_layout_rank_one(orc):
    # Non-square, non-symmetric: a stride or index mix-up changes the result.
    u = np.array([1, -2, 3, 0, 5], dtype=np.float64)
    a = np.array([2, 1, -1, 3, 0, 1, -2], dtype=np.float64)
    b = np.array([1, 0, 2, -1, 1, 3, 1], dtype=np.float64)
    v = np.array([3, -1, 2], dtype=np.float64)
    Av, Bv = np.outer(u, a), np.outer(b, v)
    want = float(a @ b) * np.outer(u, v)
    for ta, tb in LAYOUTS:
        A = storage_of(_stored(Av, ta), BF16)
        B = storage_of(_stored(Bv, tb), BF16)
        assert _same(orc.gemm_layout_f64(A, ta, B, tb, BF16, relu=True) + 0.0,
                     np.maximum(want, 0.0) + 0.0), (ta, tb)


ALL_CHECKS = [
    check_decode_f16_exhaustive, check_decode_bf16_exhaustive, check_decode_f32_sample,
    check_encode_f16, check_encode_f32, check_encode_bf16_from_f32, check_encode_exact_rational,
    check_e2m1_table, check_e8m0, check_textbook_2x2, check_identity, check_permutation,
    check_all_ones, check_rank_one, check_brute_force_dyadic, check_brute_force_general,
    check_relu, check_round_outputs, check_dequant_row_sums, check_dequant_one_hot,
    check_dequant_group_scales, check_dequant_random_vs_decoded, check_layout_textbook_2x2,
    check_layout_brute_force, check_layout_rank_one, check_e4m3_points, check_e4m3_vs_torch,
    check_mx_row_sums, check_mx_one_hot, check_mx_nan, check_mx_random_vs_decoded,
    check_sp24_brute_force, check_sp24_one_hot, check_sp24_repeated_position,
]
