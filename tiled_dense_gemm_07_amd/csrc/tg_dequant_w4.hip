// Weight-only 4-bit dequant GEMM configurations: the bf16 tiled kernel with its
// B strip read as packed E2M1 codes + E8M0 scales and expanded to bf16 in LDS.
#include "tg_configs.h"
#include "tg_kernel.h"
#include "tg_kernel_gemv_w4.h"
#include "tg_kernel_dma_w4.h"

namespace tg {

static const Config kCfg[] = {
    // few activation rows: weight-streaming kernel (bk = the K multiple it
    // needs; lane ranges, then contiguous row runs)
    tg::Config{1, DT_BF16, 16, 32, 128, 16, 1, 1, 1, true, false, false, 3,
               (const void*)&gemv_w4_kernel<true, false>},
    tg::Config{1, DT_BF16, 16, 32, 32, 16, 1, 1, 1, true, false, false, 3,
               (const void*)&gemv_w4_kernel<false, false>},
    tg::Config{1, DT_BF16, 16, 32, 128, 16, 1, 1, 1, true, false, false, 3,
               (const void*)&gemv_w4_kernel<true, true>, false, 1, true},
    tg::Config{1, DT_BF16, 16, 32, 32, 16, 1, 1, 1, true, false, false, 3,
               (const void*)&gemv_w4_kernel<false, true>, false, 1, true},
    // many rows: LDS-DMA pipeline, codes dequantised in registers (K % 128 == 0)
    tg::Config{1, DT_BF16, 64, 128, 128, 2, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 4, 4>},
    tg::Config{1, DT_BF16, 64, 128, 128, 2, 2, 4, 8, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 4, 8>},
    tg::Config{1, DT_BF16, 64, 256, 128, 2, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 256, 2, 2, 4, 4>},
    // k-slice groups: every wave covers the whole tile (1 x 1 x 4) or half
    // of it (1 x 2 x 2, 2 x 1 x 2) over its share of each strip's k
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 1, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 1, 4, 4, 4>, false, 4},
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 2, 4, 4, 2>, false, 2},
    tg::Config{1, DT_BF16, 64, 128, 128, 2, 1, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 1, 4, 4, 2>, false, 2},
    tg::Config{1, DT_BF16, 128, 64, 128, 1, 1, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<128, 64, 1, 1, 4, 4, 4>, false, 4},
    // scale bytes staged 16 strips at a time (K % 512 == 0, 16-byte aligned scale rows)
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 2, 4, 4, 2, 16>, true, 2},
    tg::Config{1, DT_BF16, 64, 128, 128, 2, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 4, 4, 1, 16>, true, 1},
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 1, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 1, 4, 4, 4, 16>, true, 4},
    // 256-k strips on a three-stage ring, scale blocks of 8 strips (K % 512 == 0,
    // 16-byte aligned scale rows): half the barriers, whole 128-byte code rows
    tg::Config{1, DT_BF16, 64, 128, 256, 1, 2, 3, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 2, 3, 4, 2, 8, 256>, true, 2},
    tg::Config{1, DT_BF16, 64, 128, 256, 2, 2, 3, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 3, 4, 2, 8, 256>, true, 2},
    tg::Config{1, DT_BF16, 64, 128, 256, 1, 1, 3, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 1, 3, 4, 4, 8, 256>, true, 4},
    tg::Config{1, DT_BF16, 64, 128, 256, 2, 2, 3, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 3, 4, 1, 8, 256>, true, 1},
    // eight waves (two per SIMD): one wave's MFMAs run while the other waits
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 2, 4, 4, 4, 16>, true, 4},
    tg::Config{1, DT_BF16, 64, 128, 128, 2, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 4, 4, 2, 16>, true, 2},
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 2, 4, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 2, 4, 4, 4>, false, 4},
    // six-stage rings: more copy bytes in flight per compute unit
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 2, 6, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 2, 6, 4, 2>, false, 2},
    tg::Config{1, DT_BF16, 64, 128, 128, 2, 2, 6, 8, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 2, 2, 6, 8>},
    tg::Config{1, DT_BF16, 64, 128, 128, 1, 1, 6, 4, true, false, false, 2, (const void*)&dma_w4_kernel<64, 128, 1, 1, 6, 4, 4>, false, 4},
    TG_CONFIG(1, DT_BF16, B_W4, 256, 64, 128, 4, 1, 2, 4, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 128, 128, 128, 2, 2, 2, 4, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 256, 128, 64, 2, 2, 2, 4, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 128, 64, 128, 2, 2, 2, 4, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 64, 64, 128, 2, 2, 2, 8, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 32, 128, 128, 1, 4, 2, 8, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 32, 64, 128, 1, 2, 2, 8, true, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 64, 64, 128, 2, 2, 2, 8, false, 0),
    TG_CONFIG(1, DT_BF16, B_W4, 128, 64, 128, 2, 2, 2, 4, true, 1),
    TG_CONFIG(1, DT_BF16, B_W4, 64, 64, 128, 2, 2, 2, 8, true, 1),
    TG_CONFIG(1, DT_BF16, B_W4, 32, 64, 128, 1, 2, 2, 8, true, 1),
};

ConfigList configs_dequant_w4() { return {kCfg, (int)(sizeof(kCfg) / sizeof(kCfg[0]))}; }

}  // namespace tg
