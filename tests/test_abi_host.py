"""Host-side checks of the C ABI (no GPU needed, no kernel launched).

* the library loads and exports every entry point include/tilegemm.h declares;
* every invalid-argument path returns its status before any HIP call;
* the block-swizzled tile order is a bijection and keeps each XCD's tiles
  in one contiguous run of the grouped raster order.
"""

import ctypes
import os
import re

import numpy as np
import pytest

from tiled_dense_gemm_07_amd import binding, synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, NULLP, SHAPE, DTYPE, EPI, ALIAS, NOCFG, HIP, BADL, WSP, SCRATCH = range(11)

# fake, well-separated device addresses: validation never dereferences them
PA, PB, PC, PS = 0x10000000, 0x20000000, 0x30000000, 0x40000000


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def declared_functions():
    text = open(os.path.join(ROOT, "include", "tilegemm.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tg_[a-z0-9_]+)\s*\(", text)))


def test_exports_match_header(lib):
    declared = declared_functions()
    assert declared == sorted(binding.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(11):
        text = binding.status_str(s)
        assert text.startswith("TG_")
    assert "unknown" in binding.status_str(99)


def test_gemm_argument_errors(lib):
    g = lib.tg_gemm
    assert g(-1, 4, 4, 2, PA, PB, PC, 0, None) == SHAPE
    assert g(4, -1, 4, 2, PA, PB, PC, 0, None) == SHAPE
    assert g(4, 4, -1, 2, PA, PB, PC, 0, None) == SHAPE
    assert g(4, 4, 1 << 31, 2, PA, PB, PC, 0, None) == SHAPE
    assert g(4, 4, 1 << 23, 2, PA, PB, PC, 0, None) == SHAPE  # 256*K*2 > 2^31
    assert g(4, 1 << 23, 4, 2, PA, PB, PC, 0, None) == SHAPE  # 128*N*2 > 2^31
    assert g(4, 4, 4, 3, PA, PB, PC, 0, None) == DTYPE
    assert g(4, 4, 4, -1, PA, PB, PC, 0, None) == DTYPE
    assert g(4, 4, 4, 2, PA, PB, PC, 2, None) == EPI
    assert g(4, 4, 4, 2, None, PB, PC, 0, None) == NULLP
    assert g(4, 4, 4, 2, PA, None, PC, 0, None) == NULLP
    assert g(4, 4, 4, 2, PA, PB, None, 0, None) == NULLP
    # C overlapping A or B
    assert g(4, 4, 4, 2, PA, PB, PA + 8, 0, None) == ALIAS
    assert g(4, 4, 4, 0, PA, PB, PB - 8, 0, None) == ALIAS
    # empty outputs are a no-op, even with NULL pointers
    assert g(0, 4, 4, 2, None, None, None, 0, None) == OK
    assert g(4, 0, 4, 2, None, None, None, 0, None) == OK
    # K == 0 needs only C
    assert g(4, 4, 0, 2, None, None, None, 0, None) == NULLP


def test_dequant_argument_errors(lib):
    d = lib.tg_dequant_gemm_w4
    assert d(4, 4, 48, PA, PB, PS, PC, 0, None) == SHAPE  # K % 32
    assert d(4, 4, -32, PA, PB, PS, PC, 0, None) == SHAPE
    assert d(4, 4, 64, PA, PB, PS, PC, 7, None) == EPI
    assert d(4, 4, 64, PA, PB, None, PC, 0, None) == NULLP
    assert d(4, 4, 64, PA, PB, PS, PB + 4, 0, None) == ALIAS
    assert d(4, 4, 64, PA, PB, PS, PS, 0, None) == ALIAS
    assert d(0, 4, 64, None, None, None, None, 0, None) == OK


def test_forced_config_errors(lib):
    n = lib.tg_config_count(0, 2)
    assert n > 0
    assert lib.tg_gemm_config(n, 4, 4, 4, 2, PA, PB, PC, 0, None) == NOCFG
    assert lib.tg_gemm_config(-1, 4, 4, 4, 2, PA, PB, PC, 0, None) == NOCFG
    nw = lib.tg_config_count(1, 2)
    assert nw > 0
    assert lib.tg_dequant_gemm_w4_config(nw, 4, 4, 64, PA, PB, PS, PC, 0, None) == NOCFG
    # a 16-byte-load configuration refuses operands that are not 16-byte aligned
    names = binding.list_configs(0, 2)
    for name in ("gemm_bf16_256x256x32_w2x2_s4_g4_dma", "gemm_bf16_128x128x64_w2x2_s2_g8_deep"):
        wide = names.index(name)
        assert lib.tg_gemm_config(wide, 4, 4, 4, 2, PA + 2, PB, PC, 0, None) == NOCFG
        # rows that are not whole 16-byte chunks (K % 8 != 0) are refused too
        assert lib.tg_gemm_config(wide, 4, 4, 12, 2, PA, PB, PC, 0, None) == NOCFG


def test_forced_dequant_config_requirements(lib):
    """The DMA dequant kernel needs whole 128- or 256-wide strips and 4-byte aligned
    scale bytes; the weight-streaming kernel needs K % bk == 0.  A forced
    configuration that cannot run the call is refused before any HIP call."""
    names = binding.list_configs(1, 2)
    d = lib.tg_dequant_gemm_w4_config
    for name in names:
        idx = names.index(name)
        if name.endswith("_dma") or name.startswith("w4_bf16_16x32x128_"):
            assert d(idx, 64, 64, 96, PA, PB, PS, PC, 0, None) == NOCFG, name
        if name.endswith("_dma"):
            assert d(idx, 64, 64, 256, PA, PB, PS + 2, PC, 0, None) == NOCFG, name
        if name.endswith("_sc16") or name.endswith("_sc8"):
            # scale blocks: K % 512 == 0 and 16-byte aligned scale rows
            assert d(idx, 64, 64, 256, PA, PB, PS, PC, 0, None) == NOCFG, name
            assert d(idx, 64, 64, 512, PA, PB, PS + 4, PC, 0, None) == NOCFG, name
        if "x256_" in name and name.startswith("w4_bf16_64x128x256_"):
            # 256-k strips: K % 256 == 0
            assert d(idx, 64, 64, 640, PA, PB, PS, PC, 0, None) == NOCFG, name


def test_gemm_ex_argument_errors(lib):
    g = lib.tg_gemm_ex
    BADL = 8
    assert g(4, 4, 4, 2, PA, 2, PB, 0, PC, 0, None) == BADL
    assert g(4, 4, 4, 2, PA, 0, PB, -1, PC, 0, None) == BADL
    assert g(-1, 4, 4, 2, PA, 1, PB, 1, PC, 0, None) == SHAPE
    assert g(1 << 25, 4, 8, 2, PA, 1, PB, 0, PC, 0, None) == SHAPE  # 64 * M * 2 > 2^31
    assert g(1 << 23, 4, 8, 2, PA, 1, PB, 0, PC, 0, None) == SHAPE  # 128 * M * 2 > 2^31
    assert g(4, 4, 4, 2, None, 1, PB, 0, PC, 0, None) == NULLP
    assert g(4, 4, 4, 2, PA, 1, PB, 0, PA + 4, 0, None) == ALIAS
    assert g(0, 4, 4, 2, None, 1, None, 1, None, 0, None) == OK
    # a forced configuration compiled for another operand layout
    gc = lib.tg_gemm_ex_config
    for dt in (0, 1, 2):
        for idx, name in enumerate(binding.list_configs(0, dt)):
            lay = next((c for c in ("_nt", "_tn", "_tt") if c in name), "")
            for ta, tb, code in ((0, 0, ""), (0, 1, "_nt"), (1, 0, "_tn"), (1, 1, "_tt")):
                if code != lay:
                    assert gc(idx, 64, 64, 64, dt, PA, ta, PB, tb, PC, 0, None) == NOCFG, name
    buf = ctypes.create_string_buffer(128)
    assert lib.tg_query_config_ex(1, 4, 64, 64, 2, 1, 0, buf, 128) == BADL
    assert lib.tg_query_config_ex(0, 4096, 4096, 4096, 2, 1, 1, buf, 128) == OK
    assert buf.value.decode().startswith("gemm_bf16_256x256x32_w2x2_s4_g4_dma_tt")
    # every dtype and alignment has a configuration in every layout
    for dt in (0, 1, 2):
        for ta, tb, code in ((0, 1, "_nt"), (1, 0, "_tn"), (1, 1, "_tt")):
            for M, N, K in ((4096, 4096, 4096), (37, 45, 29)):
                assert lib.tg_query_config_ex(0, M, N, K, dt, ta, tb, buf, 128) == OK
                name = buf.value.decode()
                assert code in name, (dt, ta, tb, M, name)


def _ws_size(lib, M, N, K, dt, splits):
    out = ctypes.c_size_t(12345)
    st = lib.tg_gemm_splitk_workspace_size(M, N, K, dt, splits, ctypes.byref(out))
    return st, out.value


def test_splitk_workspace_size(lib):
    st, n = _ws_size(lib, 256, 256, 8192, 2, 0)
    assert st == OK and n > 0
    # counters plus one fp32 partial tile per split, for the largest candidate plan
    assert n >= 256 * 256 * 4 * 2
    assert _ws_size(lib, 256, 256, 8192, 2, 1) == (OK, 0)      # no split
    assert _ws_size(lib, 0, 256, 8192, 2, 0) == (OK, 0)        # nothing to do
    assert _ws_size(lib, 8192, 8192, 64, 2, 0) == (OK, 0)      # one strip: no split
    st4, n4 = _ws_size(lib, 256, 256, 8192, 2, 4)
    st8, n8 = _ws_size(lib, 256, 256, 8192, 2, 8)
    assert st4 == st8 == OK and 0 < n4 < n8
    assert _ws_size(lib, 4, 4, 4, 7, 0)[0] == DTYPE
    assert _ws_size(lib, 4, 4, -1, 2, 0)[0] == SHAPE
    assert _ws_size(lib, 4, 4, 4, 2, -1)[0] == SHAPE
    assert lib.tg_gemm_splitk_workspace_size(4, 4, 4, 2, 0, None) == NULLP


def test_splitk_argument_errors(lib):
    g = lib.tg_gemm_splitk
    M, N, K = 256, 256, 8192
    _, need = _ws_size(lib, M, N, K, 2, 0)
    PW = 0x50000000
    # (M, N, K, dtype, A, B, C, epi, splits, workspace, bytes, stream)
    assert g(M, N, K, 2, PA, PB, PC, 0, -1, PW, need, None) == SHAPE
    assert g(M, N, K, 3, PA, PB, PC, 0, 0, PW, need, None) == DTYPE
    assert g(M, N, K, 2, PA, PB, PC, 5, 0, PW, need, None) == EPI
    assert g(M, N, K, 2, None, PB, PC, 0, 0, PW, need, None) == NULLP
    assert g(M, N, K, 2, PA, PB, PA + 64, 0, 0, PW, need, None) == ALIAS
    assert g(M, N, K, 2, PA, PB, PC, 0, 0, PC + 64, need, None) == ALIAS  # workspace over C
    assert g(M, N, K, 2, PA, PB, PC, 0, 0, None, 0, None) == WSP
    assert g(M, N, K, 2, PA, PB, PC, 0, 0, PW, need - 1, None) == WSP
    assert g(M, N, K, 2, PA, PB, PC, 0, 0, PW + 8, need, None) == WSP    # misaligned
    assert g(0, N, K, 2, None, None, None, 0, 0, None, 0, None) == OK
    # forced configurations: a plain one cannot split, an index out of range
    c = lib.tg_gemm_splitk_config
    names = binding.list_configs(0, 2)
    plain = next(i for i, n in enumerate(names) if n.split("_")[3].count("x") == 1)
    assert c(plain, M, N, K, 2, PA, PB, PC, 0, 2, PW, need, None) == NOCFG
    assert c(len(names), M, N, K, 2, PA, PB, PC, 0, 2, PW, need, None) == NOCFG
    split = [i for i, n in enumerate(names) if n.split("_")[3].count("x") == 2]
    assert split
    for i in split:
        assert c(i, M, N, K, 2, PA, PB, PC, 0, 4, None, 0, None) == WSP


def test_splitk_noalloc_argument_errors(lib):
    """Argument errors, and a split beyond the fixed scratch array, are refused
    before any HIP call (no device here)."""
    g = lib.tg_gemm_splitk_noalloc
    M, N, K = 256, 256, 8192
    # (M, N, K, dtype, A, B, C, epi, splits, stream)
    assert g(M, N, K, 2, PA, PB, PC, 0, -1, None) == SHAPE
    assert g(M, N, K, 3, PA, PB, PC, 0, 0, None) == DTYPE
    assert g(M, N, K, 2, PA, PB, PC, 5, 0, None) == EPI
    assert g(M, N, K, 2, None, PB, PC, 0, 0, None) == NULLP
    assert g(M, N, K, 2, PA, PB, PA + 64, 0, 0, None) == ALIAS
    assert g(0, N, K, 2, None, None, None, 0, 0, None) == OK
    big = (2048, 2048, 8192)
    assert _ws_size(lib, *big, 2, 16)[1] > binding.TG_SPLITK_SCRATCH_BYTES
    assert g(*big, 2, PA, PB, PC, 0, 16, None) == SCRATCH
    # the automatic split of every dtype fits the array at these long-K shapes:
    # the call gets past the size check to the device lookup (no device here)
    for dt in (0, 1, 2):
        for shape in ((256, 256, 8192), (64, 4096, 4096), (512, 512, 8192), (128, 128, 16384)):
            assert g(*shape, dt, PA, PB, PC, 0, 0, None) == HIP, shape


def test_mx_argument_errors(lib):
    g = lib.tg_gemm_mx
    PQ = 0x50000000
    # (M, N, K, fmt, Aq, As, Wq, Ws, C, epi, stream)
    assert g(4, 4, 128, 2, PA, PS, PB, PQ, PC, 0, None) == DTYPE
    assert g(4, 4, 128, -1, PA, PS, PB, PQ, PC, 0, None) == DTYPE
    assert g(4, 4, 128, 0, PA, PS, PB, PQ, PC, 2, None) == EPI
    assert g(4, 4, 96, 0, PA, PS, PB, PQ, PC, 0, None) == SHAPE  # K % 128
    assert g(4, 4, -128, 1, PA, PS, PB, PQ, PC, 0, None) == SHAPE
    assert g(4, 4, 1 << 23, 1, PA, PS, PB, PQ, PC, 0, None) == SHAPE  # 256 K > 2^31
    assert g(4, 4, 128, 0, None, PS, PB, PQ, PC, 0, None) == NULLP
    assert g(4, 4, 128, 1, PA, None, PB, PQ, PC, 0, None) == NULLP
    assert g(4, 4, 128, 0, PA, PS, PB, None, PC, 0, None) == NULLP
    assert g(4, 4, 128, 0, PA, PS, PB, PQ, None, 0, None) == NULLP
    assert g(4, 4, 128, 1, PA, PS, PB, PQ, PA + 100, 0, None) == ALIAS  # inside Aq (E4M3)
    assert g(4, 4, 128, 0, PA, PS, PB, PQ, PS + 8, 0, None) == ALIAS   # inside As
    assert g(0, 4, 128, 0, None, None, None, None, None, 0, None) == OK
    # unaligned codes or scale rows: no configuration
    assert g(4, 4, 128, 0, PA + 8, PS, PB, PQ, PC, 0, None) == NOCFG
    assert g(4, 4, 128, 0, PA, PS + 2, PB, PQ, PC, 0, None) == NOCFG
    assert g(4, 4, 128, 1, PA, PS, PB, PQ + 1, PC, 0, None) == NOCFG
    # forced configurations of the other activation format, or out of range
    names = binding.list_configs(binding.TG_OP_MX)
    c = lib.tg_gemm_mx_config
    for idx, name in enumerate(names):
        other = 1 if name.startswith("mx_e2m1") else 0
        assert c(idx, 4, 4, 128, other, PA, PS, PB, PQ, PC, 0, None) == NOCFG, name
    assert c(len(names), 4, 4, 128, 0, PA, PS, PB, PQ, PC, 0, None) == NOCFG
    # chunked scale staging needs K % 512 == 0 and 16-byte aligned scale rows
    for idx, name in enumerate(names):
        if name.endswith(("_sc8", "_sc4")):
            fmt = 0 if name.startswith("mx_e2m1") else 1
            assert c(idx, 4, 4, 384, fmt, PA, PS, PB, PQ, PC, 0, None) == NOCFG, name
            assert c(idx, 4, 4, 512, fmt, PA, PS + 4, PB, PQ, PC, 0, None) == NOCFG, name
    assert c(-1, 4, 4, 128, 0, PA, PS, PB, PQ, PC, 0, None) == NOCFG
    buf = ctypes.create_string_buffer(128)
    # (the workload shapes' exact table entries: test_tuned_table_selects_its_configurations)
    assert lib.tg_query_config_ex(2, 8192, 8192, 8192, 0, 0, 0, buf, 128) == OK
    assert buf.value.decode().startswith("mx_e2m1_")
    assert lib.tg_query_config_ex(2, 8192, 8192, 8192, 1, 0, 0, buf, 128) == OK
    assert buf.value.decode().startswith("mx_e4m3_")
    assert lib.tg_query_config_ex(2, 300, 200, 256, 1, 0, 0, buf, 128) == OK
    got = buf.value.decode().split()[0]
    assert got.startswith("mx_e4m3_") and not got.endswith(("_sc8", "_sc4")), got  # K % 512
    assert lib.tg_query_config_ex(2, 64, 64, 64, 0, 0, 0, buf, 128) == SHAPE
    assert lib.tg_query_config_ex(2, 64, 64, 128, 3, 0, 0, buf, 128) == DTYPE
    assert lib.tg_query_config_ex(2, 64, 64, 128, 0, 1, 0, buf, 128) == BADL


def test_sp24_argument_errors(lib):
    g = lib.tg_gemm_sp24
    # (M, N, K, dtype, Ac, Ai, B, C, epi, stream)
    assert g(4, 8, 32, 0, PA, PS, PB, PC, 0, None) == DTYPE       # fp32 has no sparse kernel
    assert g(4, 8, 32, 5, PA, PS, PB, PC, 0, None) == DTYPE
    assert g(4, 8, 32, 2, PA, PS, PB, PC, 3, None) == EPI
    assert g(4, 8, 48, 2, PA, PS, PB, PC, 0, None) == SHAPE       # K % 32
    assert g(-4, 8, 32, 1, PA, PS, PB, PC, 0, None) == SHAPE
    assert g(4, 8, 32, 2, None, PS, PB, PC, 0, None) == NULLP
    assert g(4, 8, 32, 2, PA, None, PB, PC, 0, None) == NULLP
    assert g(4, 8, 32, 2, PA, PS, None, PC, 0, None) == NULLP
    assert g(4, 8, 32, 2, PA, PS, PB, None, 0, None) == NULLP
    assert g(4, 8, 32, 2, PA, PS, PB, PB + 64, 0, None) == ALIAS
    assert g(0, 8, 32, 2, None, None, None, None, 0, None) == OK
    assert g(4, 8, 32, 2, PA + 8, PS, PB, PC, 0, None) == NOCFG   # unaligned values
    assert g(4, 12, 32, 2, PA, PS, PB, PC, 0, None) == NOCFG      # N % 8
    assert g(4, 8, 32, 2, PA, PS + 1, PB, PC, 0, None) == NOCFG   # unaligned metadata
    c = lib.tg_gemm_sp24_config
    n = lib.tg_config_count(3, 2)
    assert n >= 1 and c(n, 4, 8, 32, 2, PA, PS, PB, PC, 0, None) == NOCFG
    assert c(0, 4, 8, 32, 0, PA, PS, PB, PC, 0, None) == DTYPE
    buf = ctypes.create_string_buffer(128)
    assert lib.tg_query_config_ex(3, 4096, 4096, 4096, 2, 0, 0, buf, 128) == OK
    assert buf.value.decode().startswith("sp24_bf16_")
    assert lib.tg_query_config_ex(3, 64, 64, 48, 2, 0, 0, buf, 128) == SHAPE
    assert lib.tg_query_config_ex(3, 64, 64, 64, 0, 0, 0, buf, 128) == DTYPE
    assert lib.tg_query_config_ex(3, 64, 64, 64, 2, 0, 1, buf, 128) == BADL


def test_launch_failure_is_reported(lib, monkeypatch):
    # TG_FAULT=launch makes the launcher report a HIP failure after validation
    # and before any HIP call.
    monkeypatch.setenv("TG_FAULT", "launch")
    assert lib.tg_gemm(4, 4, 4, 2, PA, PB, PC, 0, None) == HIP
    assert lib.tg_dequant_gemm_w4(4, 4, 64, PA, PB, PS, PC, 0, None) == HIP
    assert lib.tg_gemm_mx(4, 4, 128, 0, PA, PS, PB, PS + 64, PC, 0, None) == HIP
    assert lib.tg_gemm_sp24(4, 8, 32, 2, PA, PS, PB, PC, 0, None) == HIP
    with pytest.raises(binding.TileGemmError) as ei:
        binding._check(HIP)
    assert ei.value.status == HIP


def test_query_config(lib):
    s = binding.query_config(0, 4096, 4096, 4096, binding.TG_BF16)
    assert s.startswith("gemm_bf16_") and "grid=" in s
    s = binding.query_config(1, 256, 8192, 8192)
    assert s.startswith("w4_bf16_")
    s = binding.query_config(0, 17, 31, 33, binding.TG_F16)
    assert " threads=256 " in s and "_narrow" in s and " group=" in s
    buf = ctypes.create_string_buffer(8)
    assert lib.tg_query_config(0, 64, 64, 64, 2, buf, 8) == OK  # truncates
    assert len(buf.value) == 7
    assert lib.tg_query_config(5, 64, 64, 64, 2, buf, 8) == NOCFG
    assert lib.tg_query_config(0, 64, 64, 64, 2, None, 8) == NULLP
    assert lib.tg_query_config(1, 64, 64, 40, 2, buf, 8) == SHAPE


def test_tuned_table_selects_its_configurations(lib):
    """Every shape of the generated selection table resolves to the configuration
    it names (names are looked up in a table formatted once per process), and
    configuration names are unique within each list."""
    table = os.path.join(os.path.dirname(binding.__file__), "csrc", "tg_tuned.inc")
    rows = re.findall(r"\{(\d+), (\d+), (\d+), (\d+), (\d+), \"([^\"]+)\", (\d+), "
                      r"([0-9.]+), (\d+), ([01])\}", open(table).read())
    assert rows
    entries = [r[:6] for r in rows if r[9] == "1"]
    assert entries
    for op, dt, M, N, K, name in entries:
        got = binding.query_config(int(op), int(M), int(N), int(K), int(dt)).split()[0]
        assert got == name, (op, dt, M, N, K, got, name)
    # every named configuration exists
    for op, dt, M, N, K, name, *_ in rows:
        assert name in binding.list_configs(int(op), int(dt)), name
    for op, dts in ((0, (0, 1, 2)), (1, (2,)), (2, (0, 1)), (3, (1, 2))):
        for dt in dts:
            names = binding.list_configs(op, dt)
            assert len(names) == len(set(names)), (op, dt)
    # repeated lookups give the same answer
    for _ in range(3):
        assert binding.query_config(1, 256, 8192, 8192).split()[0] == [
            e[5] for e in entries if e[:5] == ("1", "2", "256", "8192", "8192")][0]


def _table_rows():
    table = os.path.join(os.path.dirname(binding.__file__), "csrc", "tg_tuned.inc")
    rows = re.findall(r"\{(\d+), (\d+), (\d+), (\d+), (\d+), \"([^\"]+)\", (\d+), "
                      r"([0-9.]+), (\d+), ([01])\}", open(table).read())
    return [(int(r[0]), int(r[1]), int(r[2]), int(r[3]), int(r[4]), r[5], int(r[6]),
             float(r[7]), int(r[8]), int(r[9])) for r in rows]


def _nearest_bucket(op, dt, M, N, K):
    import math

    reps = {(r[2], r[3], r[4]) for r in _table_rows() if r[0] == op and r[1] == dt and not r[9]}
    lg = lambda x: math.log2(max(x, 1))
    return min(reps, key=lambda s: abs(lg(M) - lg(s[0])) + abs(lg(N) - lg(s[1])) +
               abs(lg(K) - lg(s[2])))


def test_selection_by_bucket_and_tile_rounds():
    """Shapes off the measured grid take a configuration measured at their
    nearest grid shape, priced by tile rounds: 3072^3 and 6144 x 4096 x 4096
    fill whole rounds of 256 workgroups with 192-row tiles (192 and 512
    tiles, against 144 and 384 of 256 x 256), 8192^3 takes 256 x 256 tiles
    (four whole rounds), and small grids with long K take k-slice groups."""
    q = lambda M, N, K, dt=binding.TG_BF16: binding.query_config(0, M, N, K, dt).split()[0]
    assert q(3072, 3072, 3072).startswith("gemm_bf16_192x256x64")
    assert q(6144, 4096, 4096).startswith("gemm_bf16_192x256x64")
    assert q(8192, 8192, 8192).startswith("gemm_bf16_256x256x")
    assert "x4_s2" in q(512, 512, 8192) or "x2_s2" in q(512, 512, 8192)
    assert q(512, 512, 8192).endswith("_deep")
    for op, dt, M, N, K in ((0, 2, 3000, 5000, 3000), (0, 1, 1536, 1536, 6144),
                            (0, 0, 768, 768, 768), (0, 2, 12288, 12288, 4096),
                            (1, 2, 100, 8192, 8192), (3, 2, 6144, 6144, 4096)):
        rep = _nearest_bucket(op, dt, M, N, K)
        listed = {r[5] for r in _table_rows() if r[:5] == (op, dt) + rep and not r[9]}
        got = binding.query_config(op, M, N, K, dt).split()[0]
        assert got in listed, (op, dt, M, N, K, rep, got, listed)


def test_config_lists(lib):
    for op, dt in ((0, 0), (0, 1), (0, 2), (1, 2)):
        names = binding.list_configs(op, dt)
        assert len(names) == len(set(names)) and names
        # each list has a narrow (element-load) configuration for unaligned operands
        assert any(n.endswith("_narrow") for n in names)
    for dt in (1, 2):
        sp = binding.list_configs(binding.TG_OP_SP24, dt)
        assert sp and len(sp) == len(set(sp)) and all(n.startswith("sp24_") for n in sp)
    assert binding.list_configs(binding.TG_OP_SP24, 0) == []
    mx = binding.list_configs(binding.TG_OP_MX)
    assert len(mx) == len(set(mx)) and mx == binding.list_configs(binding.TG_OP_MX, 1)
    assert any(n.startswith("mx_e2m1_") for n in mx) and any(n.startswith("mx_e4m3_") for n in mx)


def _raster_reference(tiles_m, tiles_n, group_m, logical):
    """Grouped raster order written out directly: groups of group_m tile rows,
    each walked column by column, top to bottom within a column."""
    order = []
    for first in range(0, tiles_m, group_m):
        rows = range(first, min(first + group_m, tiles_m))
        for n in range(tiles_n):
            for m in rows:
                order.append((m, n))
    return order[logical]


@pytest.mark.parametrize("tm,tn,gm", [(1, 1, 1), (3, 5, 2), (16, 16, 4), (16, 16, 8), (7, 9, 4),
                                      (4, 64, 4), (64, 2, 8), (17, 16, 16), (1, 37, 4), (33, 1, 8)])
def test_tile_map_bijection_and_xcd_runs(tm, tn, gm):
    om, on = binding.tile_map(tm, tn, gm)
    total = tm * tn
    pairs = set(zip(om.tolist(), on.tolist()))
    assert len(pairs) == total
    assert all(0 <= m < tm and 0 <= n < tn for m, n in pairs)
    # ids dealt to one XCD (w mod 8) take one contiguous run of the raster order
    q, r = divmod(total, 8)
    start = 0
    for x in range(8):
        ids = list(range(x, total, 8))
        assert len(ids) == q + (1 if x < r else 0)
        for j, w in enumerate(ids):
            assert (int(om[w]), int(on[w])) == _raster_reference(tm, tn, gm, start + j)
        start += len(ids)


def test_tile_map_errors(lib):
    a = np.empty(4, dtype=np.int32)
    p = a.ctypes.data_as(ctypes.c_void_p)
    assert lib.tg_tile_map(0, 4, 1, p, p) == SHAPE
    assert lib.tg_tile_map(2, 2, 0, p, p) == SHAPE
    assert lib.tg_tile_map(2, 2, 1, None, p) == NULLP


def test_hashed_ints_numpy_and_torch_agree():
    """The index-hash generator used for multi-GiB operands: values in range,
    roughly uniform, and the same on numpy arrays and torch tensors."""
    import torch

    r, c = np.arange(300)[:, None], np.arange(500)[None, :]
    h = synth.hashed_ints(r, c, 7)
    assert h.min() == -4 and h.max() == 4
    counts = np.bincount((h + 4).ravel(), minlength=9)
    assert counts.min() > 0.9 * h.size / 9 and counts.max() < 1.1 * h.size / 9
    t = synth.hashed_ints(torch.arange(300)[:, None], torch.arange(500)[None, :], 7)
    assert np.array_equal(t.numpy(), h)
    assert not np.array_equal(synth.hashed_ints(r, c, 8), h)
    # the largest indices an operand can have: int64 arrays give what Python's
    # unbounded integers give, so no product wrapped
    big = 0x7FFFFFFF
    want = synth.hashed_ints(big, big, big)  # Python ints
    got = synth.hashed_ints(np.array([[big]], dtype=np.int64), np.array([[big]], dtype=np.int64),
                            big)
    assert int(got[0, 0]) == want
