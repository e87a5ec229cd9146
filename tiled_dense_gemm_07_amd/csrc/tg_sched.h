// Block-swizzled tile scheduler: workgroup id -> output tile.
//
// The pages turn on a block "swizzle" so that blocks running at the same time
// touch the same A rows and B columns and hit in L2 ("使用 Tilelang DSL 开发
// GPU/CPU/加速器高性能内核", blog.hotdry.top, the parameter checklist), in place
// of the plain row-major order pid_m = pid / tiles_n, pid_n = pid % tiles_n of
// the mhpq.cn page's GEMM kernel (section 3.2).
//
// On MI355X the hardware deals consecutive workgroup ids round-robin over the
// 8 XCDs, and each XCD has its own 4 MiB L2.  So the map works in two steps:
//   1. regroup ids so that the ids one XCD receives (w mod 8 == x) become one
//      contiguous run of logical tile numbers;
//   2. walk logical numbers in groups of `group_m` tile rows, column by column,
//      so each XCD's run covers a compact group_m x (run / group_m) patch.
// Both steps are bijections for any grid size, including partial edge tiles.
#pragma once

#ifndef __HIPCC__
#define TG_HD
#else
#define TG_HD __host__ __device__
#endif

namespace tg {

constexpr int kNumXcd = 8;

struct TileCoord {
    int m;
    int n;
};

TG_HD inline TileCoord tile_of(int wg, int tiles_m, int tiles_n, int group_m)
{
    const int total = tiles_m * tiles_n;
    // step 1: XCD regrouping (XCD x receives ids x, x + 8, x + 16, ...)
    const int x = wg % kNumXcd;
    const int j = wg / kNumXcd;
    const int q = total / kNumXcd;
    const int r = total % kNumXcd;
    const int logical = x * q + (x < r ? x : r) + j;
    // step 2: grouped raster over tile rows
    const int per_group = group_m * tiles_n;
    const int g = logical / per_group;
    const int first_m = g * group_m;
    const int rows_here = (tiles_m - first_m) < group_m ? (tiles_m - first_m) : group_m;
    const int within = logical - g * per_group;
    TileCoord t;
    t.m = first_m + within % rows_here;
    t.n = within / rows_here;
    return t;
}

}  // namespace tg
