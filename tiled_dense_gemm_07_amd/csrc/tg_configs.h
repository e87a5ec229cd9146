// Compiled kernel configurations and the launch table shared by the
// per-dtype translation units and the C ABI.
#pragma once

#include <stdint.h>

namespace tg {

struct Config {
    int op;     // 0 = GEMM, 1 = 4-bit dequant GEMM, 2 = MX-format GEMM, 3 = 2:4 sparse GEMM
    int dtype;  // 0 = fp32, 1 = fp16, 2 = bf16 (MX: activation format, 0 = E2M1, 1 = E4M3)
    int bm, bn, bk;
    int wgm, wgn;  // waves along M and N (64 threads each)
    int stages;    // LDS ring depth
    int group_m;   // swizzle group (tile rows)
    bool wide;     // 16-byte global loads (aligned operands) vs element loads
    bool ta, tb;   // operand layouts: A stored [K][M] / B stored [N][K] (else [M][K] / [K][N])
    int pipe;      // 0: single staging set; 1: deep pipeline; 2: LDS-DMA pipeline;
                   // 3: weight-streaming dequant kernel for few rows (K % bk == 0)
    const void* kernel;
    bool chunked_scales = false;  // MX: scale bytes staged 8 strips at a time
                                  // (K % 512 == 0, 16-byte aligned scale rows)
    int ks = 1;                   // k-slice wave groups (WGM x WGN waves each)
    bool runs = false;            // weight-streaming dequant: k assigned in contiguous
                                  // 64-byte row runs (for several activation rows)
};

struct ConfigList {
    const Config* items;
    int count;
};

ConfigList configs_gemm_f32();
ConfigList configs_gemm_f16();
ConfigList configs_gemm_bf16();
ConfigList configs_dequant_w4();
ConfigList configs_mx();
ConfigList configs_sp24(int dtype);

}  // namespace tg

#define TG_CONFIG(OP, DT, BMODE, BM, BN, BK, WGM, WGN, ST, GM, WIDE, PIPE)                      \
    tg::Config                                                                                 \
    {                                                                                          \
        OP, DT, BM, BN, BK, WGM, WGN, ST, GM, WIDE, false, false, PIPE,                        \
            (const void*)&tg::gemm_kernel<DT, BMODE, BM, BN, BK, WGM, WGN, ST, GM, WIDE, PIPE> \
    }

// The same with transposed operand layouts compiled in (TA: A stored [K][M],
// TB: B stored [N][K]).
#define TG_CONFIG_T(DT, BM, BN, BK, WGM, WGN, ST, GM, WIDE, PIPE, TA, TB)                      \
    tg::Config                                                                                \
    {                                                                                         \
        0, DT, BM, BN, BK, WGM, WGN, ST, GM, WIDE, TA, TB, PIPE,                              \
            (const void*)&tg::gemm_kernel<DT, B_KN, BM, BN, BK, WGM, WGN, ST, GM, WIDE, PIPE, \
                                          TA, TB>                                             \
    }

// Register-staged kernel with KS k-slice wave groups (plain layouts, 16-byte
// loads, deep pipeline): small shapes whose tile grid leaves compute units idle.
#define TG_CONFIG_KS(DT, BM, BN, BK, WGM, WGN, GM, KS)                                         \
    tg::Config                                                                                \
    {                                                                                         \
        0, DT, BM, BN, BK, WGM, WGN, 2, GM, true, false, false, 1,                            \
            (const void*)&tg::gemm_kernel<DT, B_KN, BM, BN, BK, WGM, WGN, 2, GM, true, 1,     \
                                          false, false, KS>,                                  \
            false, KS                                                                         \
    }

// Configurations of the LDS-DMA kernel (16-bit operands, 32 k per strip, NS
// stages; TG_CONFIG_DMA_BK: BK k per strip).
#define TG_CONFIG_DMA_BK(DT, TA, TB, BM, BN, WGM, WGN, NS, GM, BK)                           \
    tg::Config                                                                             \
    {                                                                                      \
        0, DT, BM, BN, BK, WGM, WGN, NS, GM, true, TA, TB, 2,                              \
            (const void*)&tg::gemm_dma_kernel<DT, TA, TB, BM, BN, WGM, WGN, NS, GM, BK>    \
    }
#define TG_CONFIG_DMA(DT, TA, TB, BM, BN, WGM, WGN, NS, GM) \
    TG_CONFIG_DMA_BK(DT, TA, TB, BM, BN, WGM, WGN, NS, GM, 32)
