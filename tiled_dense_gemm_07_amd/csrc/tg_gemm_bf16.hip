// bf16 GEMM configurations: the generated ones (tg_gemm_gen_bf16_*.hip,
// from the LDS and register budgets) and, listed here by hand, the operand
// layouts the generator does not cover: operands stored transposed and
// operands that are not 16-byte aligned (element loads).
#include <vector>

#include "tg_configs.h"
#include "tg_gen_lists.h"
#include "tg_kernel.h"
#include "tg_kernel_dma.h"

namespace tg {

static const Config kCfg[] = {
    // transposed-operand layouts (A stored [K][M] and/or B stored [N][K])
    TG_CONFIG_DMA(DT_BF16, false, true, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_BF16, true, false, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_BF16, true, true, 256, 256, 2, 2, 4, 4),
    TG_CONFIG_DMA(DT_BF16, false, true, 128, 128, 2, 2, 4, 8),
    TG_CONFIG_DMA(DT_BF16, true, false, 128, 128, 2, 2, 4, 8),
    TG_CONFIG_DMA(DT_BF16, true, true, 128, 128, 2, 2, 4, 8),
    // unaligned operands: element loads
    TG_CONFIG(0, DT_BF16, B_KN, 64, 64, 64, 2, 2, 2, 8, false, 0),
    TG_CONFIG_T(DT_BF16, 64, 64, 64, 2, 2, 2, 8, false, 0, false, true),
    TG_CONFIG_T(DT_BF16, 64, 64, 64, 2, 2, 2, 8, false, 0, true, false),
    TG_CONFIG_T(DT_BF16, 64, 64, 64, 2, 2, 2, 8, false, 0, true, true),
};

ConfigList configs_gemm_bf16()
{
    // generated shards first (plain layouts), then the list above; the order
    // is fixed, so configuration indices are stable within a build
    static const std::vector<Config> all = [] {
        std::vector<Config> v;
        for (ConfigList L : {TG_GEN_BF16_SHARDS, ConfigList{kCfg, (int)(sizeof(kCfg) / sizeof(kCfg[0]))}})
            v.insert(v.end(), L.items, L.items + L.count);
        return v;
    }();
    return {all.data(), (int)all.size()};
}

}  // namespace tg
