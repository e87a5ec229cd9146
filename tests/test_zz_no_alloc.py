"""The allocation-free split-K entry point (tg_gemm_splitk_noalloc) against the
split-K entry point with a caller workspace (tg_gemm_splitk), through the C ABI.

Both run the same kernels with the same split plan, so their outputs must be
identical bit for bit; integer-valued inputs are also checked against the
oracle.  Two calls in a row, the second on a smaller input, check that the
shared scratch array's counters are cleared between calls; a split that needs
more than the array holds is refused.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from gpu_helpers import BF16, F16, F32, say, to_device, to_host_bits
from tiled_dense_gemm_07_amd import binding, synth

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
DNAME = {F32: "f32", F16: "f16", BF16: "bf16"}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    binding.load_library()


def _pair(M, N, K, dtype, integer, seed, splits=0, relu=True):
    """(no-alloc output bits, workspace output bits, oracle bits or None)."""
    A, B = synth.gemm_inputs(M, N, K, dtype, seed, seed + 1, integer)
    At, Bt = to_device(A, dtype, DEV), to_device(B, dtype, DEV)
    epi = "relu" if relu else None
    assert binding.splitk_workspace_size(M, N, K, dtype, splits) > 0, "the call must split"
    C1 = torch.empty((M, N), dtype=At.dtype, device=DEV)
    binding.gemm_splitk_noalloc(At, Bt, C1, epilogue=epi, splits=splits)
    C2 = binding.gemm_splitk(At, Bt, epilogue=epi, splits=splits)
    torch.cuda.synchronize()
    want = oracle.encode(dtype, oracle.gemm_f64(A, B, dtype, relu)) if integer else None
    return to_host_bits(C1, dtype), to_host_bits(C2, dtype), want


@pytest.mark.parametrize("integer", [True, False], ids=["int", "rand"])
@pytest.mark.parametrize("dtype", [BF16, F16, F32], ids=lambda d: DNAME[d])
def test_noalloc_matches_workspace_entry(dtype, integer):
    """Two calls in a row, the second smaller: same bits as tg_gemm_splitk."""
    for (M, N, K), seed in (((256, 256, 8192), 41), ((100, 72, 3000), 43)):
        say("noalloc split-K %s %dx%dx%d int=%s" % (DNAME[dtype], M, N, K, integer))
        got, ref, want = _pair(M, N, K, dtype, integer, seed)
        assert np.array_equal(got, ref), "differs from tg_gemm_splitk"
        if want is not None:
            assert np.array_equal(got, want), "differs from the oracle"


def test_noalloc_explicit_splits_then_smaller():
    """Explicit split counts, a large tile count first, then a small one."""
    for (M, N, K), splits, seed in (((512, 512, 8192), 8, 51), ((64, 64, 2048), 2, 53)):
        say("noalloc split-K bf16 %dx%dx%d splits=%d" % (M, N, K, splits))
        got, ref, want = _pair(M, N, K, BF16, True, seed, splits=splits)
        assert np.array_equal(got, ref)
        assert np.array_equal(got, want)


def test_noalloc_refuses_beyond_scratch():
    """A split whose partial tiles exceed the array: TG_ERR_SCRATCH, C untouched."""
    M, N, K = 2048, 2048, 8192
    need = binding.splitk_workspace_size(M, N, K, BF16, 16)
    assert need > binding.TG_SPLITK_SCRATCH_BYTES
    A = torch.ones((M, K), dtype=torch.bfloat16, device=DEV)
    B = torch.ones((K, N), dtype=torch.bfloat16, device=DEV)
    C = torch.full((M, N), 3.0, dtype=torch.bfloat16, device=DEV)
    say("noalloc split-K beyond the scratch array (%d bytes)" % need)
    with pytest.raises(binding.TileGemmError) as e:
        binding.gemm_splitk_noalloc(A, B, C, splits=16)
    assert e.value.status == 10
    torch.cuda.synchronize()
    assert (C.float() == 3.0).all()
