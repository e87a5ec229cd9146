// MX-format GEMM configurations: E2M1 or E4M3 activations with E8M0 block
// scales times E2M1 weights with E8M0 block scales, on the scaled matrix
// instruction (K % 128 == 0; the chunked-scale variants K % 512 == 0).
// Config dtype = the activation format (0: E2M1, 1: E4M3).
#include "tg_configs.h"
#include "tg_kernel_mx.h"

namespace tg {

#define TG_CONFIG_MX(FMT, BM, BN, GM, CS)                                                    \
    tg::Config                                                                               \
    {                                                                                        \
        2, (FMT) == MX_E2M1 ? 0 : 1, BM, BN, 128, 2, 2, 4, GM, true, false, false, 2,         \
            (const void*)&tg::gemm_mx_kernel<FMT, BM, BN, 2, 2, 4, GM, CS>, CS                \
    }

static const Config kCfg[] = {
    // scale bytes staged 8 strips at a time (K % 512 == 0)
    TG_CONFIG_MX(MX_E2M1, 256, 256, 4, true),
    TG_CONFIG_MX(MX_E2M1, 256, 256, 8, true),
    TG_CONFIG_MX(MX_E2M1, 128, 128, 8, true),
    TG_CONFIG_MX(MX_E4M3, 128, 256, 4, true),
    TG_CONFIG_MX(MX_E4M3, 128, 256, 8, true),
    TG_CONFIG_MX(MX_E4M3, 128, 128, 8, true),
    // scale bytes staged per strip (any K % 128 == 0)
    TG_CONFIG_MX(MX_E2M1, 256, 256, 4, false),
    TG_CONFIG_MX(MX_E2M1, 256, 256, 8, false),
    TG_CONFIG_MX(MX_E2M1, 128, 128, 8, false),
    TG_CONFIG_MX(MX_E4M3, 128, 256, 4, false),
    TG_CONFIG_MX(MX_E4M3, 128, 256, 8, false),
    TG_CONFIG_MX(MX_E4M3, 128, 128, 8, false),
};

ConfigList configs_mx() { return {kCfg, (int)(sizeof(kCfg) / sizeof(kCfg[0]))}; }

}  // namespace tg
