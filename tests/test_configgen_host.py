"""The generated kernel configurations (tiled_dense_gemm_07_amd/configgen.py),
checked on the host:

* every generated candidate satisfies the budgets and divisibility rules the
  generator states (recomputed here from the definitions, not through the
  generator's filters), and the pruning keeps the deepest ring per choice of
  tile, waves and BK;
* the compiled library lists exactly the generated configurations;
* every compiled instantiation of a generated configuration stays within the
  register budget its occupancy allows and uses no scratch (no spills), read
  from the code object metadata of the built objects.
"""

from __future__ import annotations

import os
import re
import subprocess

import pytest

from tiled_dense_gemm_07_amd import binding, configgen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BUILD = os.path.join(ROOT, "tiled_dense_gemm_07_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"

DTYPES = (configgen.F32, configgen.F16, configgen.BF16)


@pytest.mark.parametrize("dt", DTYPES, ids=("f32", "f16", "bf16"))
def test_candidates_fit_the_budgets(dt):
    cands = configgen.candidates(dt)
    assert cands
    for c in cands:
        es = 4 if dt == configgen.F32 else 2
        wtm, wtn = c.bm // c.wgm, c.bn // c.wgn
        assert wtm % 32 == 0 and wtn % 32 == 0, c
        assert max(wtm, wtn) <= (2 if c.family == "dma" else 1) * min(wtm, wtn), c
        nw = c.wgm * c.wgn * c.ks
        assert 4 <= nw <= 16 and nw * 64 <= 1024, c
        if c.family == "dma":
            assert dt != configgen.F32
            lds = c.stages * (c.bm + c.bn) * c.bk * 2
            assert (c.bm * c.bk * 2) % (1024 * nw) == 0 and (c.bn * c.bk * 2) % (1024 * nw) == 0
            assert 128 <= c.bn * 2 <= 1024  # n-contiguous LDS rows
            assert 2 <= c.stages <= 4 and c.bk in (32, 64, 128)
        else:
            lds = max(2 * (c.bm + c.bn) * c.bk * es, (c.ks - 1) * c.bm * c.bn * 4)
            nslab = c.bk // (2 * (4 if dt == configgen.F32 else 8))
            assert nslab % c.ks == 0 and (nslab // c.ks) % 2 == 0 and nslab // c.ks >= 2, c
        assert lds == c.lds and lds <= 160 * 1024, c
        assert c.regs <= 512 // c.occupancy, c
        # LDS leaves room for enough workgroups to fill the compiled occupancy
        assert (160 * 1024 // lds) * nw >= 4 * c.occupancy, c


@pytest.mark.parametrize("dt", DTYPES, ids=("f32", "f16", "bf16"))
def test_prune_keeps_the_deepest_ring(dt):
    gen = configgen.dma_candidates if dt != configgen.F32 else configgen.deep_candidates
    kept = {(c.bm, c.bn, c.wgm, c.wgn, c.ks, c.bk): c for c in configgen.candidates(dt)
            if c.family == ("dma" if dt != configgen.F32 else "deep")}
    for c in gen(dt):
        k = (c.bm, c.bn, c.wgm, c.wgn, c.ks, c.bk)
        if k in kept:
            assert kept[k].stages >= c.stages


def test_library_lists_the_generated_configurations():
    binding.load_library()
    for dt in DTYPES:
        names = binding.list_configs(0, dt)
        gen = configgen.listed_order(dt)
        assert names[:len(gen)] == gen, dt


_ARGS = re.compile(r"L([ib])(\d+)E")


def _kernel_args(sym):
    """Template arguments of a mangled gemm_dma_kernel / gemm_kernel symbol."""
    body = sym.split("kernelI", 1)[1]
    return [int(v) for _, v in _ARGS.findall(body)]


def _metadata(obj):
    """{kernel symbol: (vgpr, agpr, private segment bytes)} from a built object."""
    tmp = obj + ".meta"
    os.makedirs(tmp, exist_ok=True)
    fb, co = os.path.join(tmp, "fb.bin"), os.path.join(tmp, "gfx950.co")
    subprocess.run([os.path.join(LLVM, "llvm-objcopy"), "--dump-section", ".hip_fatbin=" + fb,
                    obj], check=True, capture_output=True)
    subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                    "--input=" + fb, "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                    "--output=" + co], check=True, capture_output=True)
    notes = subprocess.run([os.path.join(LLVM, "llvm-readelf"), "--notes", co], check=True,
                           capture_output=True, text=True).stdout
    out, cur = {}, {}
    for line in notes.splitlines():
        line = line.strip().lstrip("- ")
        m = re.match(r"\.(name|vgpr_count|agpr_count|private_segment_fixed_size):\s+(\S+)", line)
        if not m:
            continue
        cur[m.group(1)] = m.group(2)
        if all(k in cur for k in ("name", "vgpr_count", "agpr_count",
                                  "private_segment_fixed_size")):
            out[cur["name"]] = (int(cur["vgpr_count"]), int(cur["agpr_count"]),
                                int(cur["private_segment_fixed_size"]))
            cur = {}
    return out


@pytest.mark.parametrize("dt", DTYPES, ids=("f32", "f16", "bf16"))
def test_compiled_registers_and_no_spills(dt):
    tools = ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")
    if not all(os.path.exists(os.path.join(LLVM, t)) for t in tools):
        pytest.skip("ROCm LLVM tools not installed")
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in configgen.generated_sources()
            if "_%s_" % configgen.DNAME[dt] in s]
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library not built (run the build first)")
    meta = {}
    for o in objs:
        meta.update(_metadata(o))
    want = {}
    for c in configgen.candidates(dt):
        if c.family == "dma":
            key = ("gemm_dma_kernel", (dt, 0, 0, c.bm, c.bn, c.wgm, c.wgn, c.stages, c.group_m, c.bk))
        else:
            key = ("gemm_kernel", (dt, 0, c.bm, c.bn, c.bk, c.wgm, c.wgn, 2, c.group_m, 1, 1, 0, 0,
                                   c.ks))
        want[key] = c
    found = 0
    for sym, (vgpr, agpr, scratch) in meta.items():
        kind = "gemm_dma_kernel" if "gemm_dma_kernel" in sym else (
            "gemm_kernel" if "gemm_kernel" in sym else None)
        if kind is None:
            continue
        c = want.get((kind, tuple(_kernel_args(sym))))
        if c is None:
            continue
        found += 1
        # gfx950 metadata: vgpr_count is the unified total (AGPRs included)
        assert scratch == 0, (c.name(), "spills", scratch)
        assert agpr <= vgpr <= 512 // c.occupancy, (c.name(), vgpr, agpr, c.occupancy)
    assert found == len(want), (found, len(want))
