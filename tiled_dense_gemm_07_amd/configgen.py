"""Kernel configurations generated from the hardware budgets.

The pages tune a GEMM by searching a small grid of tile sizes and pipeline
depths on the target GPU ("TileLang ... 一个高效 GEMM 内核", mhpq.cn, sections
4.2 and 4.3: tune BK first, then a 3 x 3 x 3 grid of tiles, and retune per
GPU; the gtnt.cn page's tuning_config with tile_sizes [32, 64, 128]; the
blog.hotdry.top page: num_stages 2-4).  Here the grid is the cross product
of the kernel templates' structural parameters, and a candidate is kept only
if it fits one MI355X compute unit:

  * LDS: the stage ring (and the k-slice groups' partial tiles) within the
    160 KiB a compute unit has;
  * registers: a per-lane estimate of accumulators, fragments, staging and
    addressing within the 512 VGPR + AGPR a SIMD lane has, divided by the
    waves per SIMD the kernel is compiled for;
  * occupancy: every configuration keeps at least one wave on each of the
    four SIMDs, and its LDS leaves room for enough workgroups to reach the
    waves per SIMD it is compiled for;
  * the templates' own divisibility rules (whole 1 KiB copies per wave,
    whole 32 x 32 MFMA blocks per wave, even slab counts, ...), mirrored here
    from their static_asserts.

The swizzle group is not part of a configuration: it is a launch parameter,
tuned by the sweep per shape bucket.

    python -m tiled_dense_gemm_07_amd.configgen          # write csrc/tg_gen_*.inc
    python -m tiled_dense_gemm_07_amd.configgen --list   # print the candidates

The build regenerates the .inc files before compiling.  The host tests check
every compiled kernel's register count and scratch use (from the code object
metadata) against the budgets assumed here.
"""

from __future__ import annotations

import argparse
import os
from dataclasses import dataclass

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")

LDS_BYTES = 160 * 1024   # per compute unit
REGS_PER_LANE = 512      # VGPR + AGPR per SIMD lane
SIMDS = 4                # per compute unit
MAX_THREADS = 1024       # per workgroup

F32, F16, BF16 = 0, 1, 2
ES = {F32: 4, F16: 2, BF16: 2}    # bytes per element
VEC = {F32: 4, F16: 8, BF16: 8}   # elements per 16-byte chunk
DT_NAME = {F32: "DT_F32", F16: "DT_F16", BF16: "DT_BF16"}


@dataclass(frozen=True)
class Cand:
    family: str     # "dma": LDS-DMA kernel (16-bit); "deep": register-staged deep pipeline
    dtype: int
    bm: int
    bn: int
    bk: int
    wgm: int
    wgn: int
    stages: int
    ks: int         # k-slice wave groups (deep family)
    group_m: int    # default swizzle group (a launch may override it)
    occupancy: int  # waves per SIMD the kernel is compiled for
    regs: int       # estimated VGPR + AGPR per lane
    lds: int        # LDS bytes

    @property
    def waves(self) -> int:
        return self.wgm * self.wgn * self.ks

    def name(self) -> str:
        """The name the C ABI's config_name prints for this configuration."""
        wav = ("w%dx%dx%d" % (self.wgm, self.wgn, self.ks) if self.ks > 1
               else "w%dx%d" % (self.wgm, self.wgn))
        pipe = "_dma" if self.family == "dma" else "_deep"
        return "gemm_%s_%dx%dx%d_%s_s%d_g%d%s" % (
            {F32: "f32", F16: "f16", BF16: "bf16"}[self.dtype], self.bm, self.bn, self.bk, wav,
            self.stages, self.group_m, pipe)

    def macro(self) -> str:
        if self.family == "dma":
            return "TG_CONFIG_DMA_BK(%s, false, false, %d, %d, %d, %d, %d, %d, %d)" % (
                DT_NAME[self.dtype], self.bm, self.bn, self.wgm, self.wgn, self.stages,
                self.group_m, self.bk)
        return "TG_CONFIG_KS(%s, %d, %d, %d, %d, %d, %d, %d)" % (
            DT_NAME[self.dtype], self.bm, self.bn, self.bk, self.wgm, self.wgn, self.group_m,
            self.ks)


def default_group(bm: int, bn: int) -> int:
    """Default swizzle group: 4 tile rows for tiles of 192 rows or more, else 8."""
    return 4 if bm >= 192 else 8


# ---------------------------------------------------------------------------
# LDS-DMA GEMM (DmaGemm in tg_kernel_dma.h): 16-bit operands, A row-major
# (k-contiguous LDS rows), B row-major (n-contiguous LDS rows read by the
# transposing LDS read), 32, 64 or 128 k per strip, 2-4 stages, 4 or 8 waves.
# ---------------------------------------------------------------------------
DMA_BM = (64, 128, 192, 256)
DMA_BN = (64, 128, 256)
DMA_BK = (32, 64, 128)
DMA_WAVES = ((2, 2), (2, 4), (4, 2))
DMA_STAGES = (2, 3, 4)


def dma_regs(bm, bn, bk, wgm, wgn) -> int:
    """Per-lane registers: accumulators (one fp32 per 64 outputs of the wave
    tile), two fragment sets (A: 4 per 32-row block, B: 4 per 32-column block),
    copy and read offsets, and a fixed allowance for addresses, loop state and
    the epilogue.  Calibrated on the compiled 256 x 256 x 64 eight-wave kernel
    (228 estimated and compiled)."""
    nw = wgm * wgn
    wtm, wtn = bm // wgm, bn // wgn
    fm, fn = wtm // 32, wtn // 32
    ja = bm * bk * 2 // 1024 // nw
    jb = bn * bk * 2 // 1024 // nw
    sl = bk // 16
    return wtm * wtn // 64 + 2 * (4 * fm + 4 * fn) + (2 * ja + jb + sl + fn + 10) + 24


def dma_occupancy(bm, bn, nw, lds) -> int:
    """Waves per SIMD (DmaOcc): one on four waves for the largest tiles and for
    rings of more than half the LDS (no second workgroup fits), else two."""
    return 1 if nw <= 4 and (bm * bn >= 256 * 128 or 2 * lds > LDS_BYTES) else 2


def dma_candidates(dtype: int):
    for bm in DMA_BM:
        for bn in DMA_BN:
            for bk in DMA_BK:
                for wgm, wgn in DMA_WAVES:
                    for ns in DMA_STAGES:
                        nw = wgm * wgn
                        wtm, wtn = bm // wgm, bn // wgn
                        if bm % wgm or bn % wgn or wtm % 32 or wtn % 32:
                            continue  # whole 32 x 32 MFMA blocks per wave
                        sa, sb = bm * bk * 2, bn * bk * 2
                        if sa % (1024 * nw) or sb % (1024 * nw):
                            continue  # whole 1 KiB copies per wave
                        if not 8 <= bn // 8 <= 64:
                            continue  # n-contiguous LDS rows of 128 to 1024 bytes
                        lds = ns * (sa + sb)
                        if lds > LDS_BYTES:
                            continue
                        occ = dma_occupancy(bm, bn, nw, lds)
                        regs = dma_regs(bm, bn, bk, wgm, wgn)
                        if regs > REGS_PER_LANE // occ:
                            continue
                        if (LDS_BYTES // lds) * nw < occ * SIMDS:
                            continue  # the ring leaves LDS for too few workgroups
                        yield Cand("dma", dtype, bm, bn, bk, wgm, wgn, ns, 1,
                                   default_group(bm, bn), occ, regs, lds)


# ---------------------------------------------------------------------------
# Register-staged deep pipeline with k-slice groups (GemmKernel<..., PIPE 1,
# KS> in tg_kernel.h): any operand type, strips loaded to registers two strips
# ahead and transposed into LDS, two LDS stages; KS groups of WGM x WGN waves
# share each strip's slabs.  For grids of a few hundred tiles or fewer (and
# the fp32 GEMM, which has no LDS-DMA kernel).
# ---------------------------------------------------------------------------
DEEP_TILES = (32, 64, 128)
DEEP_BK = {F32: (32, 64, 128), F16: (64, 128, 256), BF16: (64, 128, 256)}
DEEP_WAVES = ((1, 1), (1, 2), (2, 1), (2, 2))
DEEP_KS = (1, 2, 4)


def deep_layout_ok(dt, bm, bn, bk, nt) -> bool:
    """The register-staged operand loaders' divisibility rules (KOp / XOp)."""
    vec, es = VEC[dt], ES[dt]
    cpr = bk // vec
    if (bm * cpr) % nt or bm * cpr // nt < 1:
        return False  # A strip: whole 16-byte chunks per thread
    uw_raw = cpr * bn // nt
    uw = min(uw_raw, vec)
    if uw < 1 or uw & (uw - 1) or uw * es < 4:
        return False
    if (cpr * (bn // uw)) % nt or cpr * (bn // uw) // nt < 1:
        return False  # B strip: whole transposition units per thread
    return True


def deep_regs(dt, bm, bn, bk, wgm, wgn, ks) -> int:
    """Per-lane registers: accumulators, two staging sets of the A and B strip
    chunks (4 per 16-byte chunk), two fragment sets (4 per 32-row or 32-column
    block) and a fixed allowance for addresses and loop state."""
    nt = wgm * wgn * ks * 64
    vec = VEC[dt]
    cpr = bk // vec
    wtm, wtn = bm // wgm, bn // wgn
    fm, fn = wtm // 32, wtn // 32
    a_chunks = bm * cpr // nt
    uw = min(cpr * bn // nt, vec)
    b_regs = (cpr * (bn // uw) // nt) * vec  # u32x4 registers per thread, as XOp::NREG
    return wtm * wtn // 64 + 2 * 4 * (a_chunks + b_regs) + 2 * 4 * (fm + fn) + 40


def deep_candidates(dtype: int):
    for bm in DEEP_TILES:
        for bn in DEEP_TILES:
            for bk in DEEP_BK[dtype]:
                for wgm, wgn in DEEP_WAVES:
                    for ks in DEEP_KS:
                        nw = wgm * wgn * ks
                        nt = nw * 64
                        wtm, wtn = bm // wgm, bn // wgn
                        if bm % wgm or bn % wgn or wtm % 32 or wtn % 32:
                            continue
                        if nt > MAX_THREADS or nw < SIMDS:
                            continue  # at least one wave per SIMD
                        nslab = bk // (2 * VEC[dtype])
                        if nslab % ks or (nslab // ks) < 2 or (nslab // ks) % 2:
                            continue  # each group's slabs alternate fragment sets in pairs
                        if not deep_layout_ok(dtype, bm, bn, bk, nt):
                            continue
                        ring = 2 * (bm + bn) * bk * ES[dtype]
                        red = (ks - 1) * bm * bn * 4
                        lds = max(ring, red)
                        if lds > LDS_BYTES:
                            continue
                        occ = -(-nw // SIMDS)
                        regs = deep_regs(dtype, bm, bn, bk, wgm, wgn, ks)
                        if regs > REGS_PER_LANE // occ:
                            continue
                        if (LDS_BYTES // lds) * nw < occ * SIMDS:
                            continue  # the ring leaves LDS for too few workgroups
                        yield Cand("deep", dtype, bm, bn, bk, wgm, wgn, 2, ks,
                                   default_group(bm, bn), occ, regs, lds)


# Configurations the register estimate admits but the compiler spills (the
# host tests read every compiled kernel's scratch use; these are the ones
# they found): four waves on a 256 x 256 x 64 tile hold 256 accumulators and
# two 64-k fragment sets per lane.
COMPILER_SPILLS = {("dma", 256, 256, 64, 2, 2)}


def prune(cands, max_aspect: int):
    """Two rules cut the cross product to what is worth compiling and timing.
    Wave tiles no more than `max_aspect` times longer one way than the other:
    an MFMA block reads one A and one B fragment, so for a given number of
    blocks a square wave tile reads the fewest fragments.  And for each tile
    shape, wave layout, k-slice count and strip depth BK only the deepest
    ring that fits: more stages keep more copies in flight at no cost in
    MFMA work.  BK itself stays a free choice (the pages tune it first)."""
    best = {}
    for c in cands:
        if (c.family, c.bm, c.bn, c.bk, c.wgm, c.wgn) in COMPILER_SPILLS:
            continue
        wtm, wtn = c.bm // c.wgm, c.bn // c.wgn
        if max(wtm, wtn) > max_aspect * min(wtm, wtn):
            continue
        key = (c.family, c.bm, c.bn, c.wgm, c.wgn, c.ks, c.bk)
        if key not in best or c.stages > best[key].stages:
            best[key] = c
    return list(best.values())


def candidates(dtype: int):
    """Every generated configuration of `dtype`: the LDS-DMA family (16-bit
    only), then the register-staged family, largest tiles first in each."""
    out = []
    if dtype in (F16, BF16):
        out += sorted(prune(dma_candidates(dtype), 2),
                      key=lambda c: (-c.bm * c.bn, -c.bk, c.stages, c.wgm))
    out += sorted(prune(deep_candidates(dtype), 1),
                  key=lambda c: (-c.bm * c.bn, -c.bk, c.ks, c.wgm))
    return out


# The generated configurations of a dtype are compiled in SHARDS translation
# units (csrc/tg_gemm_gen_<dtype>_<i>.hip, each including its .inc), so that
# the build compiles them in parallel.  Candidate j goes to shard j % SHARDS.
SHARDS = {F32: 2, F16: 4, BF16: 4}
DNAME = {F32: "f32", F16: "f16", BF16: "bf16"}


def inc_path(dtype: int, shard: int) -> str:
    return os.path.join(CSRC, "tg_gen_%s_%d.inc" % (DNAME[dtype], shard))


def render(dtype: int, shard: int) -> str:
    lines = ["// Generated by tiled_dense_gemm_07_amd/configgen.py: the configurations",
             "// that fit one MI355X compute unit's LDS and registers (shard %d of %d)."
             % (shard, SHARDS[dtype]), "// Do not edit."]
    for j, c in enumerate(candidates(dtype)):
        if j % SHARDS[dtype] == shard:
            lines.append("    %s,  // %s: %d regs/lane at %d wave(s)/SIMD, %d B LDS" % (
                c.macro(), c.name(), c.regs, c.occupancy, c.lds))
    return "\n".join(lines) + "\n"


def shard_source(dtype: int, shard: int) -> str:
    return "tg_gemm_gen_%s_%d.hip" % (DNAME[dtype], shard)


def render_shard_tu(dtype: int, shard: int) -> str:
    d = DNAME[dtype]
    return """// %s GEMM configurations generated from the hardware budgets (shard %d of %d);
// generated by tiled_dense_gemm_07_amd/configgen.py.  Do not edit.
#include "tg_configs.h"
#include "tg_kernel.h"
#include "tg_kernel_dma.h"

namespace tg {

static const Config kGen[] = {
#include "tg_gen_%s_%d.inc"
};

ConfigList configs_gen_%s_%d() { return {kGen, (int)(sizeof(kGen) / sizeof(kGen[0]))}; }

}  // namespace tg
""" % (d, shard, SHARDS[dtype], d, shard, d, shard)


def render_lists() -> str:
    lines = ["// Generated by tiled_dense_gemm_07_amd/configgen.py: the shard lists of the",
             "// generated GEMM configurations.  Do not edit.", "#pragma once", "",
             '#include "tg_configs.h"', "", "namespace tg {", ""]
    for dt in (F32, F16, BF16):
        for sh in range(SHARDS[dt]):
            lines.append("ConfigList configs_gen_%s_%d();" % (DNAME[dt], sh))
    lines.append("")
    for dt in (F32, F16, BF16):
        lines.append("#define TG_GEN_%s_SHARDS %s" % (
            DNAME[dt].upper(), ", ".join("configs_gen_%s_%d()" % (DNAME[dt], sh)
                                         for sh in range(SHARDS[dt]))))
    lines += ["", "}  // namespace tg", ""]
    return "\n".join(lines)


def generated_sources() -> list:
    """The shard translation units the build compiles (file names in csrc/)."""
    return [shard_source(dt, sh) for dt in (F32, F16, BF16) for sh in range(SHARDS[dt])]


def write_all() -> list:
    """Write every generated file whose content changed (the shards' .inc and
    translation units, the list header); returns the paths written."""
    files = {os.path.join(CSRC, "tg_gen_lists.h"): render_lists()}
    for dt in (F32, F16, BF16):
        for sh in range(SHARDS[dt]):
            files[inc_path(dt, sh)] = render(dt, sh)
            files[os.path.join(CSRC, shard_source(dt, sh))] = render_shard_tu(dt, sh)
    written = []
    for path, text in files.items():
        if os.path.exists(path) and open(path).read() == text:
            continue
        with open(path, "w") as f:
            f.write(text)
        written.append(path)
    return written


def listed_order(dtype: int) -> list:
    """Generated names in the order the library lists them (shard 0's, then
    shard 1's, ...)."""
    c = candidates(dtype)
    return [x.name() for sh in range(SHARDS[dtype]) for j, x in enumerate(c)
            if j % SHARDS[dtype] == sh]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--list", action="store_true")
    args = ap.parse_args(argv)
    if args.list:
        for dt in (F32, F16, BF16):
            for c in candidates(dt):
                print("%-44s regs %3d occ %d lds %6d" % (c.name(), c.regs, c.occupancy, c.lds))
    else:
        for path in write_all():
            print("wrote", path)
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
