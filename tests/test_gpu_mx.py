"""GPU parity of the MX-format GEMM (tg_gemm_mx) against the CPU oracle.

The oracle is the exact sum.  The scaled matrix instruction does not form it
exactly: on gfx950 it adds each group of 8 consecutive products in fixed point
whose last bit is 2^(e_g - 13), e_g the largest exponent sum E(a) + E(w) of
the group's elements (subnormal and zero elements count with their format's
smallest normal exponent), truncating each product toward zero, and combines
the group sums in floating point (behaviour measured with in-bounds probes;
E2M1 x E2M1 products never reach the window, E4M3 x E2M1 products can).

Bars:
  * sums that are exact in that arithmetic and in fp32 (element and scale
    ranges chosen so that every product and partial sum is a multiple of a
    power of two inside the window and below 2^24 of it): bit-exact with one
    round-to-nearest-even of the exact fp64 sum;
  * full-range random codes and scales, E2M1 x E2M1: the stated 4-bit
    tolerance |C - Y| <= 1e-2 + 1e-2 |Y| on every entry, and the bound of the
    arithmetic without truncation, |C - Y| <= (1 + 2^-8) A + 2^-8 |Y| with
    A = (K / 8) 2^-24 S and S = sum_k |a(m, k) w(n, k)| (the fp32 roundings),
    then one bf16 rounding.  An E2M1 x E2M1 product is a multiple of 2^-3 and
    its group's window ends at 2^(4 - 13) or below, so it is never truncated;
  * full-range random codes and scales, E4M3 x E2M1: products can fall below
    the window, so the bound adds the truncation T = sum over groups of
    (nonzero products) * 2^(e_g - 13) * scales; and at least 99% of entries
    meet 1e-2 + 1e-2 |Y| (the truncation error is relative to each group's
    largest product, so only entries whose sum cancels to far below its terms
    miss it: about 0.3% in a CPU model of the arithmetic at 8192^3);
  * NaN scale bytes (E8M0 255) and NaN E4M3 codes: NaN exactly in the outputs
    whose sums take one of their products.
Full-size shapes run in the benchmark's launch configuration and are checked
on sampled entries the oracle sums one by one.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import BF16, bits_to_f64, say, sample_entries, to_host_bits
from tiled_dense_gemm_07_amd import binding, synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
FMTS = [synth.MX_E2M1, synth.MX_E4M3]
FNAME = synth.MX_NAMES


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def run_mx(fmt, Aq, As, Wq, Ws, relu=False, config=None):
    t = [torch.from_numpy(np.ascontiguousarray(x)).to(DEV) for x in (Aq, As, Wq, Ws)]
    Ct = binding.gemm_mx(fmt, *t, epilogue="relu" if relu else None, config=config)
    torch.cuda.synchronize()
    return to_host_bits(Ct, BF16)


def exact_inputs(fmt, M, N, K, seed):
    """Codes and scales whose sums are exact in fp32 at K <= 1024.

    E2M1 elements are multiples of 1/2 up to 6; with scales 2^-1 .. 2^1 each
    operand is a multiple of 1/4 up to 12, each product a multiple of 2^-4 up
    to 144, and a sum of 1024 of them needs at most 18 + 4 bits.  E4M3
    activations with exponent fields 6..9 are multiples of 2^-4 below 8; with
    scale 1 the products are multiples of 2^-6 up to 96: 17 + 6 bits."""
    Wq = synth.w4_codes(N, K, seed + 2)
    Ws = synth.w4_scales(N, K, seed + 3, emin=-1, emax=1)
    if fmt == synth.MX_E2M1:
        Aq = synth.w4_codes(M, K, seed)
        As = synth.w4_scales(M, K, seed + 1, emin=-1, emax=1)
    else:
        Aq = synth.e4m3_codes_range(M, K, seed, 6, 9)
        As = synth.w4_scales(M, K, seed + 1, emin=0, emax=0)
    return Aq, As, Wq, Ws


def abs_codes(fmt, Aq, Wq):
    """The same codes with every sign bit cleared."""
    a = Aq & (0x77 if fmt == synth.MX_E2M1 else 0x7F)
    return a, Wq & 0x77


def _exponents(v, emin):
    """floor(log2 |v|), at least emin (subnormals and zeros count as emin)."""
    a = np.abs(v)
    return np.maximum(np.floor(np.log2(np.where(a > 0, a, 1.0))), emin)


def truncation_bound(fmt, Aq, As, Wq, Ws, rows, cols):
    """T of the module docstring for the entries (rows[i], cols[i]); zero for
    E2M1 activations, whose products the window always holds."""
    if fmt == synth.MX_E2M1:
        return np.zeros(len(rows))
    ones_a = np.full_like(As, 127)
    ones_w = np.full_like(Ws, 127)
    ea = oracle.mx_decode_a(fmt, Aq, ones_a)        # unscaled elements
    ew = oracle.mx_decode_a(0, Wq, ones_w)
    Ea = _exponents(ea, -6 if fmt == synth.MX_E4M3 else 0)
    Ew = _exponents(ew, 0)
    sa = np.ldexp(1.0, As.astype(np.int64) - 127)   # [M, K/32]
    sw = np.ldexp(1.0, Ws.astype(np.int64) - 127)
    K = ea.shape[1]
    out = np.empty(len(rows))
    for lo in range(0, len(rows), 256):
        r, c = rows[lo:lo + 256], cols[lo:lo + 256]
        e = (Ea[r] + Ew[c]).reshape(len(r), K // 8, 8).max(axis=2)
        nz = ((ea[r] * ew[c]) != 0).reshape(len(r), K // 8, 8).sum(axis=2)
        scale = np.repeat(sa[r] * sw[c], 4, axis=1)  # per group of 8
        out[lo:lo + 256] = (nz * np.ldexp(1.0, (e - 13).astype(np.int64)) * scale).sum(axis=1)
    return out


def check_bound(got_bits, Y, S, T, K):
    got = bits_to_f64(got_bits, BF16)
    err = (1 + 2.0 ** -8) * (T + (K / 8) * 2.0 ** -24 * S)
    tol = err + 2.0 ** -8 * np.abs(Y)
    bad = ~(np.abs(got - Y) <= tol)
    assert not bad.any(), "%d of %d outside the bound (first at %s: got %r want %r tol %r)" % (
        int(bad.sum()), bad.size, np.argwhere(bad)[0].tolist(), got[bad][0], Y[bad][0],
        tol[bad][0])


E4M3_MIN_FRACTION = 0.99


def check_stated_tolerance(fmt, got_bits, Y):
    """The 4-bit path's stated tolerance |C - Y| <= 1e-2 + 1e-2 |Y|: on every
    entry for E2M1 activations; on at least E4M3_MIN_FRACTION of the entries
    for E4M3 activations (checked where there are 1000 entries or more)."""
    got = bits_to_f64(got_bits, BF16)
    ok = np.abs(got - Y) <= 1e-2 + 1e-2 * np.abs(Y)
    frac = float(ok.mean())
    say("mx %s: %.5f of %d entries within 1e-2 + 1e-2 |Y|" % (FNAME[fmt], frac, ok.size))
    if fmt == synth.MX_E2M1:
        assert ok.all(), "%d of %d outside 1e-2 + 1e-2 |Y|" % (int((~ok).sum()), ok.size)
    elif ok.size >= 1000:
        assert frac >= E4M3_MIN_FRACTION, frac


def full_bound_inputs(fmt, Aq, As, Wq, Ws, M, N):
    rr, cc = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    a_abs, w_abs = abs_codes(fmt, Aq, Wq)
    S = oracle.mx_gemm_f64(fmt, a_abs, As, w_abs, Ws)
    T = truncation_bound(fmt, Aq, As, Wq, Ws, rr.ravel(), cc.ravel()).reshape(M, N)
    return S, T


SHAPES = [(1, 1, 128), (3, 5, 128), (17, 31, 256), (65, 72, 256), (129, 257, 384),
          (256, 256, 128), (300, 520, 512), (130, 600, 1024)]


@pytest.mark.parametrize("relu", [False, True], ids=["none", "relu"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
def test_mx_exact(fmt, shape, relu):
    M, N, K = shape
    Aq, As, Wq, Ws = exact_inputs(fmt, M, N, K, 1200 + M + N)
    say("mx exact %s %s relu=%s" % (FNAME[fmt], shape, relu))
    got = run_mx(fmt, Aq, As, Wq, Ws, relu)
    want = oracle.encode(BF16, oracle.mx_gemm_f64(fmt, Aq, As, Wq, Ws, relu))
    diff = got != want
    assert not diff.any(), "%d of %d entries differ (first at %s)" % (
        int(diff.sum()), diff.size, np.argwhere(diff)[0].tolist())


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("fmt", FMTS, ids=lambda f: FNAME[f])
def test_mx_random(fmt, shape):
    M, N, K = shape
    Aq, As, Wq, Ws = synth.mx_inputs(fmt, M, N, K, 1300 + M, 1400 + N, 1500 + K, 1600)
    say("mx random %s %s" % (FNAME[fmt], shape))
    got = run_mx(fmt, Aq, As, Wq, Ws)
    Y = oracle.mx_gemm_f64(fmt, Aq, As, Wq, Ws)
    S, T = full_bound_inputs(fmt, Aq, As, Wq, Ws, M, N)
    check_bound(got, Y, S, T, K)
    check_stated_tolerance(fmt, got, Y)


def test_mx_wide_scale_range():
    """Scale bytes across [20, 230]: one scale per row keeps each sum a
    multiple of that row's and column's scales times 2^-4 (exact), so the
    result is bit-exact wherever every product and partial sum is a normal
    fp32 value and the result a normal bf16 value."""
    M, N, K = 64, 96, 256
    r = np.random.Generator(np.random.PCG64(91))
    for fmt in FMTS:
        Aq, _, Wq, _ = exact_inputs(fmt, M, N, K, 1700)
        ea = r.integers(20, 231, size=M)
        ew = r.integers(20, 231, size=N)
        ea[0], ew[0], ea[1], ew[1] = 20, 230, 230, 20
        As = np.repeat(ea[:, None], K // 32, axis=1).astype(np.uint8)
        Ws = np.repeat(ew[:, None], K // 32, axis=1).astype(np.uint8)
        say("mx scale range %s" % FNAME[fmt])
        got = run_mx(fmt, Aq, As, Wq, Ws)
        Y = oracle.mx_gemm_f64(fmt, Aq, As, Wq, Ws)
        a_abs, w_abs = abs_codes(fmt, Aq, Wq)
        S = oracle.mx_gemm_f64(fmt, a_abs, As, w_abs, Ws)
        # smallest nonzero product: 1/2 * 1/2 * both scales
        lo = ea[:, None] + ew[None, :] - 254 - 2 >= -126
        ok = lo & (S < 2.0 ** 126) & (np.abs(Y) >= 2.0 ** -126)
        assert ok.sum() > M * N // 4
        want = oracle.encode(BF16, Y)
        assert np.array_equal(got[ok], want[ok]), FNAME[fmt]


def test_mx_nan():
    M, N, K = 40, 72, 256
    for fmt in FMTS:
        Aq, As, Wq, Ws = exact_inputs(fmt, M, N, K, 1800)
        As[3, 2] = 255
        Ws[5, 7] = 255
        if fmt == synth.MX_E4M3:
            Aq[9, 100] = 0xFF
            Aq[10, 200] = 0x7F
        say("mx nan %s" % FNAME[fmt])
        got = bits_to_f64(run_mx(fmt, Aq, As, Wq, Ws), BF16)
        Y = oracle.mx_gemm_f64(fmt, Aq, As, Wq, Ws)
        assert np.array_equal(np.isnan(got), np.isnan(Y)), FNAME[fmt]
        assert np.isnan(Y[3]).all() and np.isnan(Y[:, 5]).all()


def test_mx_zero_k_and_empty():
    for fmt in FMTS:
        say("mx K=0 %s" % FNAME[fmt])
        e = torch.empty((0,), dtype=torch.uint8, device=DEV)
        C = torch.full((5, 7), 3.0, dtype=torch.bfloat16, device=DEV)
        out = binding.gemm_mx(fmt, e.view(5, 0), e.view(5, 0), e.view(7, 0), e.view(7, 0), C=C)
        torch.cuda.synchronize()
        assert (out.float() == 0).all()
        C0 = torch.empty((0, 7), dtype=torch.bfloat16, device=DEV)
        binding.gemm_mx(fmt, e.view(0, 0), e.view(0, 0), e.view(7, 0), e.view(7, 0), C=C0)


@pytest.mark.parametrize("shape", [(300, 264, 384), (300, 264, 512), (200, 136, 1536),
                                   (64, 72, 2560),
                                   # 4-strip scale chunks on three stages: 12 + 4 strips;
                                   # 256-k strips: one and two loop passes
                                   (130, 200, 2048), (130, 264, 1024)],
                         ids=lambda s: "x".join(map(str, s)))
def test_mx_every_config(shape):
    """Every configuration, forced: bit-exact where it runs; the other activation
    format, chunked scale staging at K % 512 != 0 and 256-k strips at K % 1024
    != 0 refuse the call."""
    M, N, K = shape
    for fmt in FMTS:
        Aq, As, Wq, Ws = exact_inputs(fmt, M, N, K, 1900 + K)
        want = oracle.encode(BF16, oracle.mx_gemm_f64(fmt, Aq, As, Wq, Ws, relu=True))
        for idx, name in enumerate(binding.list_configs(binding.TG_OP_MX)):
            bk = int(name.split("_")[2].split("x")[2])
            if (not name.startswith("mx_" + FNAME[fmt]) or
                    (name.endswith(("_sc8", "_sc4")) and K % 512) or (bk == 256 and K % 1024)):
                with pytest.raises(binding.TileGemmError):
                    run_mx(fmt, Aq, As, Wq, Ws, relu=True, config=idx)
                continue
            say("mx config %d %s %s" % (idx, name, shape))
            got = run_mx(fmt, Aq, As, Wq, Ws, relu=True, config=idx)
            assert np.array_equal(got, want), name


def test_mx_deterministic():
    w = synth.WORKLOADS["mx_e4m3_8192"]
    Aq, As, Wq, Ws = synth.mx_inputs(w.dtype, 1024, 2048, 2048, 11, 12, 13, 14)
    t = [torch.from_numpy(x).to(DEV) for x in (Aq, As, Wq, Ws)]
    say("mx determinism")
    first = binding.gemm_mx(w.dtype, *t).clone()
    for _ in range(4):
        assert torch.equal(binding.gemm_mx(w.dtype, *t).view(torch.int16), first.view(torch.int16))


@pytest.mark.parametrize("name", ["mx_e2m1_8192", "mx_e4m3_8192"])
def test_mx_workload(name):
    """The full-size benchmark workloads, default selection, sampled entries."""
    w = synth.WORKLOADS[name]
    inp = synth.make_inputs(w)
    say("mx workload %s seeds=%s" % (name, inp["seeds"]))
    got = run_mx(w.dtype, inp["Aq"], inp["As"], inp["Wq"], inp["Ws"], w.relu).reshape(w.M, w.N)
    rows, cols = sample_entries(w.M, w.N, 4000, seed=w.index * 7)
    Y = oracle.mx_gemm_entries_f64(w.dtype, inp["Aq"], inp["As"], inp["Wq"], inp["Ws"], rows, cols,
                                   w.relu)
    a_abs, w_abs = abs_codes(w.dtype, inp["Aq"], inp["Wq"])
    S = oracle.mx_gemm_entries_f64(w.dtype, a_abs, inp["As"], w_abs, inp["Ws"], rows, cols)
    T = truncation_bound(w.dtype, inp["Aq"], inp["As"], inp["Wq"], inp["Ws"], rows, cols)
    check_bound(got[rows, cols], Y, S, T, w.K)
    check_stated_tolerance(w.dtype, got[rows, cols], Y)
    assert np.isfinite(bits_to_f64(got, BF16)).all()
