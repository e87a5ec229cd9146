// MX-format GEMM configurations: E2M1 or E4M3 activations with E8M0 block
// scales times E2M1 weights with E8M0 block scales, on the scaled matrix
// instruction (K % 128 == 0; the chunked-scale variants K % 512 == 0).
// Config dtype = the activation format (0: E2M1, 1: E4M3).
#include "tg_configs.h"
#include "tg_kernel_mx.h"
#include "tg_kernel_mx2.h"

namespace tg {

#define TG_CONFIG_MX(FMT, BM, BN, GM, CS)                                                    \
    tg::Config                                                                               \
    {                                                                                        \
        2, (FMT) == MX_E2M1 ? 0 : 1, BM, BN, 128, 2, 2, 4, GM, true, false, false, 2,         \
            (const void*)&tg::gemm_mx_kernel<FMT, BM, BN, 2, 2, 4, GM, CS>, CS                \
    }

// WGM x WGN waves and NS stages
#define TG_CONFIG_MX_W(FMT, BM, BN, WGM, WGN, NS, GM, CS)                                    \
    tg::Config                                                                               \
    {                                                                                        \
        2, (FMT) == MX_E2M1 ? 0 : 1, BM, BN, 128, WGM, WGN, NS, GM, true, false, false, 2,    \
            (const void*)&tg::gemm_mx_kernel<FMT, BM, BN, WGM, WGN, NS, GM, CS>, CS           \
    }

// 256-k strips on a two-stage ring, scales in 4-strip chunks (K % 1024 == 0)
#define TG_CONFIG_MX2(FMT, BM, BN, WGM, WGN, GM)                                             \
    tg::Config                                                                               \
    {                                                                                        \
        2, (FMT) == MX_E2M1 ? 0 : 1, BM, BN, 256, WGM, WGN, 2, GM, true, false, false, 2,    \
            (const void*)&tg::gemm_mx2_kernel<FMT, BM, BN, WGM, WGN, GM>, true               \
    }

static const Config kCfg[] = {
    TG_CONFIG_MX2(MX_E2M1, 256, 256, 2, 2, 4),
    TG_CONFIG_MX2(MX_E2M1, 256, 256, 2, 4, 4),
    TG_CONFIG_MX2(MX_E4M3, 128, 256, 2, 2, 4),
    // eight waves (two per SIMD) with per-strip scale copies; E4M3 on
    // 256 x 256 tiles takes three stages (150 KiB of LDS). Eight waves with
    // 8-strip scale chunks on four stages, and E4M3 256 x 256 on four waves
    // and four stages, compile with spills or accumulator copies in the main
    // loop and are left out.
    TG_CONFIG_MX_W(MX_E2M1, 256, 256, 2, 4, 4, 4, false),
    TG_CONFIG_MX_W(MX_E4M3, 256, 256, 2, 4, 3, 4, false),
    // three stages with scale chunks of 4 strips (16 bytes per row; E4M3
    // 256 x 256: 160 KiB of LDS)
    TG_CONFIG_MX_W(MX_E4M3, 256, 256, 2, 4, 3, 4, true),
    TG_CONFIG_MX_W(MX_E2M1, 256, 256, 2, 4, 3, 4, true),
    TG_CONFIG_MX_W(MX_E2M1, 256, 256, 2, 2, 3, 4, true),
    TG_CONFIG_MX_W(MX_E4M3, 128, 256, 2, 4, 4, 4, false),
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
