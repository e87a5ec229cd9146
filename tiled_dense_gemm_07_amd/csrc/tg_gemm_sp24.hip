// 2:4 structured-sparse GEMM configurations (sparse matrix instruction,
// 64 dense k per strip, 3 LDS stages; K % 32 == 0, the metadata-chunk ones
// K % 256 == 0).
#include "tg_configs.h"
#include "tg_kernel_sp24.h"

namespace tg {

#define TG_CONFIG_SP24(DT, BM, BN, GM)                                                  \
    tg::Config                                                                          \
    {                                                                                   \
        3, DT, BM, BN, 64, 2, 2, 3, GM, true, false, false, 2,                          \
            (const void*)&tg::gemm_sp24_kernel<DT, BM, BN, 2, 2, 3, GM>                 \
    }
// eight waves, two per SIMD (WGM x WGN = 2 x 4 or 4 x 2)
#define TG_CONFIG_SP24_W(DT, BM, BN, WGM, WGN, GM)                                      \
    tg::Config                                                                          \
    {                                                                                   \
        3, DT, BM, BN, 64, WGM, WGN, 3, GM, true, false, false, 2,                      \
            (const void*)&tg::gemm_sp24_kernel<DT, BM, BN, WGM, WGN, 3, GM>             \
    }

// metadata copied in chunks of 4 strips (K % 256 == 0, 16-byte aligned rows)
#define TG_CONFIG_SP24_C(DT, BM, BN, WGM, WGN, GM)                                      \
    tg::Config                                                                          \
    {                                                                                   \
        3, DT, BM, BN, 64, WGM, WGN, 3, GM, true, false, false, 2,                      \
            (const void*)&tg::gemm_sp24_kernel<DT, BM, BN, WGM, WGN, 3, GM, true>, true \
    }

static const Config kCfgBf16[] = {
    TG_CONFIG_SP24_C(DT_BF16, 256, 256, 2, 4, 4),
    TG_CONFIG_SP24_C(DT_BF16, 256, 128, 2, 2, 4),
    TG_CONFIG_SP24_C(DT_BF16, 128, 256, 2, 2, 4),
    TG_CONFIG_SP24_C(DT_BF16, 128, 128, 2, 2, 8),
    TG_CONFIG_SP24_W(DT_BF16, 256, 256, 2, 4, 4),
    TG_CONFIG_SP24(DT_BF16, 256, 128, 4),
    TG_CONFIG_SP24(DT_BF16, 256, 128, 8),
    TG_CONFIG_SP24(DT_BF16, 128, 256, 4),
    TG_CONFIG_SP24(DT_BF16, 128, 128, 8),
};
static const Config kCfgF16[] = {
    TG_CONFIG_SP24_C(DT_F16, 256, 256, 2, 4, 4),
    TG_CONFIG_SP24_C(DT_F16, 256, 128, 2, 2, 4),
    TG_CONFIG_SP24_C(DT_F16, 128, 256, 2, 2, 4),
    TG_CONFIG_SP24_C(DT_F16, 128, 128, 2, 2, 8),
    TG_CONFIG_SP24_W(DT_F16, 256, 256, 2, 4, 4),
    TG_CONFIG_SP24(DT_F16, 256, 128, 4),
    TG_CONFIG_SP24(DT_F16, 256, 128, 8),
    TG_CONFIG_SP24(DT_F16, 128, 256, 4),
    TG_CONFIG_SP24(DT_F16, 128, 128, 8),
};

ConfigList configs_sp24(int dtype)
{
    if (dtype == DT_BF16)
        return {kCfgBf16, (int)(sizeof(kCfgBf16) / sizeof(kCfgBf16[0]))};
    if (dtype == DT_F16)
        return {kCfgF16, (int)(sizeof(kCfgF16) / sizeof(kCfgF16[0]))};
    return {nullptr, 0};
}

}  // namespace tg
