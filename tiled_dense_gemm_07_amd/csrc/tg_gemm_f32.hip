// fp32 GEMM kernel configurations (instantiations of the tiled kernel template).
// The first one is the pages' own tile: 128 x 128 x 32 (mhpq.cn, section 3.2).
#include "tg_configs.h"
#include "tg_kernel.h"

namespace tg {

static const Config kCfg[] = {
    TG_CONFIG(0, DT_F32, B_KN, 128, 128, 32, 2, 2, 2, 8, true, 0),
    TG_CONFIG(0, DT_F32, B_KN, 128, 128, 32, 2, 2, 3, 8, true, 0),
    TG_CONFIG(0, DT_F32, B_KN, 256, 128, 32, 2, 2, 2, 4, true, 0),
    TG_CONFIG(0, DT_F32, B_KN, 256, 256, 32, 2, 2, 2, 4, true, 0),
    TG_CONFIG(0, DT_F32, B_KN, 64, 64, 32, 2, 2, 2, 8, true, 0),
    TG_CONFIG(0, DT_F32, B_KN, 64, 64, 32, 2, 2, 2, 8, false, 0),
    TG_CONFIG(0, DT_F32, B_KN, 256, 256, 32, 2, 2, 2, 4, true, 1),
    TG_CONFIG(0, DT_F32, B_KN, 128, 128, 32, 2, 2, 2, 8, true, 1),
    TG_CONFIG(0, DT_F32, B_KN, 64, 64, 32, 2, 2, 2, 8, true, 1),
    // k-slice wave groups for grids of a few hundred tiles or less
    TG_CONFIG_KS(DT_F32, 32, 32, 128, 1, 1, 8, 4),
    TG_CONFIG_KS(DT_F32, 32, 32, 64, 1, 1, 8, 2),
    TG_CONFIG_KS(DT_F32, 32, 64, 128, 1, 2, 8, 4),
    TG_CONFIG_KS(DT_F32, 64, 64, 64, 2, 2, 8, 2),
    // transposed-operand layouts (A stored [K][M] and/or B stored [N][K])
    TG_CONFIG_T(DT_F32, 128, 128, 32, 2, 2, 2, 8, true, 1, false, true),
    TG_CONFIG_T(DT_F32, 128, 128, 32, 2, 2, 2, 8, true, 1, true, false),
    TG_CONFIG_T(DT_F32, 128, 128, 32, 2, 2, 2, 8, true, 1, true, true),
    TG_CONFIG_T(DT_F32, 64, 64, 32, 2, 2, 2, 8, true, 1, false, true),
    TG_CONFIG_T(DT_F32, 64, 64, 32, 2, 2, 2, 8, true, 1, true, false),
    TG_CONFIG_T(DT_F32, 64, 64, 32, 2, 2, 2, 8, true, 1, true, true),
    TG_CONFIG_T(DT_F32, 64, 64, 32, 2, 2, 2, 8, false, 0, false, true),
    TG_CONFIG_T(DT_F32, 64, 64, 32, 2, 2, 2, 8, false, 0, true, false),
    TG_CONFIG_T(DT_F32, 64, 64, 32, 2, 2, 2, 8, false, 0, true, true),
};

ConfigList configs_gemm_f32() { return {kCfg, (int)(sizeof(kCfg) / sizeof(kCfg[0]))}; }

}  // namespace tg
