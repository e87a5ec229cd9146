"""GPU parity of the split-K entry (tg_gemm_splitk) against the CPU oracle.

Same bars as the plain GEMM: bit-exact on integer-valued inputs (every partial
sum, and every sum of split partials, is an integer below 2^24, so exact in
fp32), the workload tolerances on random inputs.  Also: the caller's workspace
is reused across calls of different shapes and split counts without clearing
(the counters return to zero), the result does not depend on the order in
which a tile's workgroups finish (bitwise repeatable), and every configuration
that can split K runs forced.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import BF16, F16, F32, say, to_device, to_host_bits
from test_gpu_parity import DNAME, DTYPES, check_full
from tiled_dense_gemm_07_amd import binding, synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def run_splitk(A, B, dtype, relu, splits=0, workspace=None, config=None):
    At, Bt = to_device(A, dtype, DEV), to_device(B, dtype, DEV)
    Ct = binding.gemm_splitk(At, Bt, epilogue="relu" if relu else None, splits=splits,
                             workspace=workspace, config=config)
    torch.cuda.synchronize()
    return to_host_bits(Ct, dtype)


def split_names(dtype):
    return [(i, n) for i, n in enumerate(binding.list_configs(0, dtype))
            if n.split("_")[3].count("x") == 2]  # three wave counts: k-slice groups


SHAPES = [(256, 256, 4096), (64, 96, 2048), (100, 72, 1000), (33, 40, 777), (256, 256, 96),
          (1, 8, 4096)]


@pytest.mark.parametrize("integer", [True, False], ids=["int", "rand"])
@pytest.mark.parametrize("splits", [0, 2, 3, 16])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_splitk_shapes(dtype, shape, splits, integer):
    M, N, K = shape
    A, B = synth.gemm_inputs(M, N, K, dtype, 3101 + M, 3202 + N, integer)
    say("splitk %s %s splits=%d int=%s" % (DNAME[dtype], shape, splits, integer))
    got = run_splitk(A, B, dtype, relu=True, splits=splits)
    check_full(got, oracle.gemm_f64(A, B, dtype, relu=True), dtype, integer)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_every_split_config(dtype):
    """Each configuration with k-slice groups, forced, split 4 ways on a ragged shape."""
    M, N, K = 136, 200, 1800
    A, B = synth.gemm_inputs(M, N, K, dtype, 3303, 3404, integer=True)
    want = oracle.encode(dtype, oracle.gemm_f64(A, B, dtype))
    names = split_names(dtype)
    assert len(names) >= 2
    for idx, name in names:
        say("split config %d %s" % (idx, name))
        got = run_splitk(A, B, dtype, relu=False, splits=4, config=idx)
        assert np.array_equal(got, want), name


def test_split_config_refuses_plain_configs():
    A = torch.zeros((64, 256), dtype=torch.bfloat16, device=DEV)
    B = torch.zeros((256, 64), dtype=torch.bfloat16, device=DEV)
    split = {i for i, _ in split_names(BF16)}
    plain = [i for i in range(len(binding.list_configs(0, BF16))) if i not in split]
    with pytest.raises(binding.TileGemmError) as ei:
        binding.gemm_splitk(A, B, splits=2, config=plain[0])
    assert ei.value.status == 6


def test_workspace_reuse():
    """One workspace, calls of different shapes and split counts in a row: the
    per-tile counters are back at zero after each call."""
    dtype = BF16
    shapes = [(256, 256, 4096, 0), (64, 64, 8192, 16), (128, 96, 2048, 3), (256, 256, 4096, 5),
              (32, 32, 1024, 2)]
    need = max(binding.splitk_workspace_size(M, N, K, dtype, s) for M, N, K, s in shapes)
    ws = torch.zeros((need,), dtype=torch.uint8, device=DEV)
    for M, N, K, s in shapes:
        A, B = synth.gemm_inputs(M, N, K, dtype, 3505 + K, 3606 + N, integer=True)
        say("reuse %dx%dx%d splits=%d" % (M, N, K, s))
        got = run_splitk(A, B, dtype, relu=False, splits=s, workspace=ws)
        assert np.array_equal(got, oracle.encode(dtype, oracle.gemm_f64(A, B, dtype)))
        # the counters lead the workspace and are zero again (counted here for
        # the largest tile, 64 x 64, whose counters are the fewest)
        tiles = ((M + 63) // 64) * ((N + 63) // 64)
        assert not ws[: tiles * 4].any().item()


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_splitk_repeatable(dtype):
    """Random inputs: repeated calls give identical bits (partials are summed in
    split order whichever workgroup finishes last)."""
    M, N, K = 128, 128, 8192
    A, B = synth.gemm_inputs(M, N, K, dtype, 3707, 3808)
    At, Bt = to_device(A, dtype, DEV), to_device(B, dtype, DEV)
    ws = binding.splitk_workspace(M, N, K, dtype, 0, device=DEV)
    first = binding.gemm_splitk(At, Bt, workspace=ws)
    for _ in range(5):
        again = binding.gemm_splitk(At, Bt, workspace=ws)
        assert torch.equal(first.view(torch.int16 if dtype != F32 else torch.int32),
                           again.view(torch.int16 if dtype != F32 else torch.int32))
    torch.cuda.synchronize()
    check_full(to_host_bits(first, dtype), oracle.gemm_f64(A, B, dtype), dtype, integer=False)


@pytest.mark.parametrize("dtype", DTYPES, ids=lambda d: DNAME[d])
def test_splitk_equals_plain_on_integers(dtype):
    """Integer-valued inputs: the split result is tg_gemm's, bit for bit."""
    M, N, K = 192, 160, 6000
    A, B = synth.gemm_inputs(M, N, K, dtype, 3909, 4010, integer=True)
    got = run_splitk(A, B, dtype, relu=True)
    At, Bt = to_device(A, dtype, DEV), to_device(B, dtype, DEV)
    plain = binding.gemm(At, Bt, epilogue="relu")
    torch.cuda.synchronize()
    assert np.array_equal(got, to_host_bits(plain, dtype))


def test_splitk_unaligned_and_k0():
    """Operands that are not 16-byte aligned run the plain kernel (no workspace
    needed); K = 0 gives zeros."""
    M, N, K = 37, 45, 2000
    A, B = synth.gemm_inputs(M, N, K, F16, 4111, 4212, integer=True)
    got = run_splitk(A, B, F16, relu=False, splits=4, workspace=None)
    assert np.array_equal(got, oracle.encode(F16, oracle.gemm_f64(A, B, F16)))
    A0 = torch.zeros((64, 0), dtype=torch.float32, device=DEV)
    B0 = torch.zeros((0, 64), dtype=torch.float32, device=DEV)
    C = torch.full((64, 64), 7.0, dtype=torch.float32, device=DEV)
    binding.gemm_splitk(A0, B0, C=C, splits=4)
    torch.cuda.synchronize()
    assert not C.any().item()


def test_splitk_workload_256x256x8192():
    """bf16 256 x 256 x 8192 + ReLU (a few output tiles, long K) in full."""
    M, N, K = 256, 256, 8192
    A, B = synth.gemm_inputs(M, N, K, BF16, 4313, 4414)
    say("splitk workload %dx%dx%d" % (M, N, K))
    got = run_splitk(A, B, BF16, relu=True)
    check_full(got, oracle.gemm_f64(A, B, BF16, relu=True), BF16, integer=False)
