// fp16 GEMM kernel configurations (instantiations of the tiled kernel template).
#include "tg_configs.h"
#include "tg_kernel.h"
#include "tg_kernel_dma.h"

namespace tg {

static const Config kCfg[] = {
    // 64 k per strip: whole 128-byte row segments of A, two stages
    TG_CONFIG_DMA_BK(DT_F16, false, false, 256, 256, 2, 2, 2, 4, 64),
    TG_CONFIG_DMA_BK(DT_F16, false, false, 256, 256, 2, 2, 2, 8, 64),
    // eight waves, two per SIMD (128 x 64 wave tiles)
    TG_CONFIG_DMA_BK(DT_F16, false, false, 256, 256, 2, 4, 2, 4, 64),
    TG_CONFIG_DMA_BK(DT_F16, false, false, 256, 256, 4, 2, 2, 4, 64),
    TG_CONFIG_DMA(DT_F16, false, false, 256, 256, 2, 4, 3, 4),
    // 192-row tiles: grids that divide into whole waves of 256 workgroups
    TG_CONFIG_DMA_BK(DT_F16, false, false, 192, 256, 2, 4, 2, 4, 64),
    TG_CONFIG_DMA_BK(DT_F16, false, false, 192, 256, 2, 2, 2, 4, 64),
    TG_CONFIG_DMA(DT_F16, false, false, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_F16, false, false, 256, 256, 2, 2, 4, 8),
    TG_CONFIG_DMA(DT_F16, false, false, 256, 256, 2, 2, 3, 4),
    TG_CONFIG_DMA(DT_F16, false, false, 256, 256, 2, 2, 5, 4),
    TG_CONFIG_DMA(DT_F16, false, false, 256, 128, 2, 2, 4, 8),
    TG_CONFIG_DMA(DT_F16, false, false, 128, 128, 2, 2, 4, 8),
    // transposed-operand layouts (A stored [K][M] and/or B stored [N][K])
    TG_CONFIG_DMA(DT_F16, false, true, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_F16, true, false, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_F16, true, true, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_F16, false, true, 128, 128, 2, 2, 4, 8),
    TG_CONFIG_DMA(DT_F16, true, false, 128, 128, 2, 2, 4, 8),
    TG_CONFIG_DMA(DT_F16, true, true, 128, 128, 2, 2, 4, 8),
    TG_CONFIG(0, DT_F16, B_KN, 256, 256, 64, 2, 4, 2, 4, true, 0),
    TG_CONFIG(0, DT_F16, B_KN, 128, 128, 64, 2, 2, 2, 8, true, 0),
    TG_CONFIG(0, DT_F16, B_KN, 128, 64, 64, 2, 2, 2, 8, true, 0),
    TG_CONFIG(0, DT_F16, B_KN, 64, 64, 64, 2, 2, 2, 8, true, 0),
    TG_CONFIG(0, DT_F16, B_KN, 64, 64, 64, 2, 2, 2, 8, false, 0),
    // unaligned transposed layouts: element loads
    TG_CONFIG_T(DT_F16, 64, 64, 64, 2, 2, 2, 8, false, 0, false, true),
    TG_CONFIG_T(DT_F16, 64, 64, 64, 2, 2, 2, 8, false, 0, true, false),
    TG_CONFIG_T(DT_F16, 64, 64, 64, 2, 2, 2, 8, false, 0, true, true),
    TG_CONFIG(0, DT_F16, B_KN, 128, 128, 64, 2, 2, 2, 8, true, 1),
    TG_CONFIG(0, DT_F16, B_KN, 64, 64, 64, 2, 2, 2, 8, true, 1),
    // k-slice wave groups for grids of a few hundred tiles or less
    TG_CONFIG_KS(DT_F16, 64, 64, 128, 2, 2, 8, 2),
    TG_CONFIG_KS(DT_F16, 64, 64, 128, 1, 1, 8, 4),
    TG_CONFIG_KS(DT_F16, 32, 64, 128, 1, 2, 8, 2),
    TG_CONFIG_KS(DT_F16, 32, 32, 256, 1, 1, 8, 4),
};

ConfigList configs_gemm_f16() { return {kCfg, (int)(sizeof(kCfg) / sizeof(kCfg[0]))}; }

}  // namespace tg
