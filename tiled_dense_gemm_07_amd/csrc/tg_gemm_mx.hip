// MX-format GEMM configurations: E2M1 or E4M3 activations with E8M0 block
// scales times E2M1 weights with E8M0 block scales, on the scaled matrix
// instruction (K % 128 == 0).  Config dtype = the activation format
// (0: E2M1, 1: E4M3).
#include "tg_configs.h"
#include "tg_kernel_mx.h"

namespace tg {

#define TG_CONFIG_MX(FMT, BM, BN, GM)                                                        \
    tg::Config                                                                               \
    {                                                                                        \
        2, (FMT) == MX_E2M1 ? 0 : 1, BM, BN, 128, 2, 2, 4, GM, true, false, false, 2,         \
            (const void*)&tg::gemm_mx_kernel<FMT, BM, BN, 2, 2, 4, GM>                       \
    }

static const Config kCfg[] = {
    TG_CONFIG_MX(MX_E2M1, 256, 256, 4),
    TG_CONFIG_MX(MX_E2M1, 256, 256, 8),
    TG_CONFIG_MX(MX_E2M1, 128, 128, 8),
    TG_CONFIG_MX(MX_E4M3, 128, 256, 4),
    TG_CONFIG_MX(MX_E4M3, 128, 256, 8),
    TG_CONFIG_MX(MX_E4M3, 128, 128, 8),
};

ConfigList configs_mx() { return {kCfg, (int)(sizeof(kCfg) / sizeof(kCfg[0]))}; }

}  // namespace tg
