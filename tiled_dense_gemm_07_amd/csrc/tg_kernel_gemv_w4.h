// Weight-only 4-bit dequant GEMM for few activation rows (M <= 16 per
// workgroup): the memory-bound, decode-like end of the dequant entry.
//
// The operation is the pages' weight-only low-bit GEMM ("WFP4" GEMM in
// "TileLang架构深度剖析", the performance section; "Dequant GEMM" in
// "使用 Tilelang DSL 开发 GPU/CPU/加速器高性能内核"): C[m][n] = sum_k A[m][k] W[n][k],
// W given as E2M1 codes two per byte with one E8M0 scale per 32 k.  With so
// few rows the run time is the time to stream the packed weights from HBM
// once, so this kernel is built around that stream instead of around an LDS
// tile:
//  * a workgroup owns 32 weight rows (two groups of 16) and all of K; its 16
//    waves split K into rounds of 512 (wave w takes rounds w, w+16, ...);
//  * in a round, lane (n = l % 16, g = l / 16) loads 4 x 16 bytes of codes of
//    row n covering k in [512 r + 128 g, +128) and the 4 scale bytes of those
//    k, for each row group: every byte of a 128-byte line is used, and a wave
//    keeps 8 KiB of weights in flight;
//  * the codes are expanded to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4
//    applies the scale exactly) and fed straight to v_mfma_f32_16x16x32_bf16
//    as the 16-row operand; the activation fragment of the same k (rows m of
//    A, zero past M) is the other operand;
//  * the 16 waves' 16 x 32 partial sums are added in LDS in a fixed order (so
//    results do not depend on timing), then ReLU, one rounding and the store.
// The k order inside a round is permuted the same way for A and W, which only
// reorders the sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel.h"

namespace tg {

typedef __attribute__((ext_vector_type(4))) float f32x4v;

template <bool DWORD_SCALES>
struct GemvW4 {
    static constexpr int NWAVE = 16;
    static constexpr int ROWS = 32;     // weight rows per workgroup
    static constexpr int NG = ROWS / 16;
    static constexpr int ROUND = 512;   // k per wave round
    static constexpr int MB = 16;       // activation rows per workgroup

    static __device__ __forceinline__ void run(const GemmParams& p)
    {
        __shared__ __attribute__((aligned(16))) float red[NWAVE][NG * 256];
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int mb = blockIdx.x % p.tiles_m;
        const int nb = blockIdx.x / p.tiles_m;
        const int m0 = mb * MB;
        const int n0 = nb * ROWS;
        const int ln = lane & 15;  // row within a 16-row group (W) / activation row (A)
        const int g = lane >> 4;   // k quarter of the round
        const int K = p.K;
        const int rowb = K / 2;    // code bytes per weight row
        const int srow = K / 32;   // scale bytes per weight row

        // weight codes and scales of rows n0 .., activations of rows m0 ..
        const auto wrs = make_rsrc((const char*)p.B + (int64_t)n0 * rowb,
                                   clamp_bytes((int64_t)(p.N - n0) * rowb));
        const auto srs = make_rsrc((const char*)p.Bs + (int64_t)n0 * srow,
                                   clamp_bytes((int64_t)(p.N - n0) * srow));
        const auto ars = make_rsrc((const char*)p.A + (int64_t)m0 * K * 2,
                                   clamp_bytes((int64_t)(p.M - m0) * K * 2));
        const bool arow = m0 + ln < p.M;

        f32x4v acc[NG];
#pragma unroll
        for (int q = 0; q < NG; ++q)
            acc[q] = f32x4v{0.0f, 0.0f, 0.0f, 0.0f};

        const int rounds = (K + ROUND - 1) / ROUND;
        for (int r = w; r < rounds; r += NWAVE) {
            const int kq = r * ROUND + 128 * g;  // this lane's first k
            const bool kv = kq < K;              // K is a multiple of 32; kq, +32, ... may pass it
            // issue all weight loads of the round first (8 KiB per wave in flight)
            u32x4 code[NG][4];
            u32 sc[NG];
#pragma unroll
            for (int q = 0; q < NG; ++q) {
                const u32 rowoff = (u32)((16 * q + ln) * rowb);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool v = kq + 32 * c < K;
                    code[q][c] = buf_load16(wrs, v ? rowoff + (u32)(kq + 32 * c) / 2 : kOob);
                }
                const u32 soff = (u32)((16 * q + ln) * srow + kq / 32);
                if (DWORD_SCALES) {
                    sc[q] = buf_load4(srs, kv ? soff : kOob);
                } else {
                    u32 s4 = 0;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        s4 |= buf_load1(srs, kq + 32 * c < K ? soff + c : kOob) << (8 * c);
                    sc[q] = s4;
                }
            }
            // activation fragments: 16 bytes of row m0 + ln at the same k
            u32x4 af[16];
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int k = kq + 8 * j;
                af[j] = buf_load16(ars, (arow && k < K) ? (u32)(ln * K + k) * 2u : kOob);
            }
            // every load of the round is in flight before the first is consumed
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int q = 0; q < NG; ++q) {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    // a scale byte only multiplies codes of k < K (zeros past it)
                    const u32 e = (sc[q] >> (8 * c)) & 0xFFu;
                    const float s = e8m0_to_f32(kq + 32 * c < K ? e : 127u);
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const u32 packed = code[q][c][h];  // 8 codes: k = kq + 32c + 8h ..
                        u32x4 b;
                        b[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 0));
                        b[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 1));
                        b[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 2));
                        b[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 3));
                        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, af[4 * c + h]),
                            acc[q], 0, 0, 0);
                    }
                }
            }
        }

        // lane holds m = ln, n = 16 q + 4 g + i (i = 0..3) of the workgroup's rows
#pragma unroll
        for (int q = 0; q < NG; ++q)
            *(f32x4v*)&red[w][q * 256 + lane * 4] = acc[q];
        __syncthreads();
        if (tid < NG * 256) {
            float s = 0.0f;
#pragma unroll
            for (int v = 0; v < NWAVE; ++v)
                s += red[v][tid];
            const int q = tid >> 8, l = (tid >> 2) & 63, i = tid & 3;
            const int m = m0 + (l & 15);
            const int n = n0 + 16 * q + 4 * (l >> 4) + i;
            if (m < p.M && n < p.N) {
                if (p.relu && !(s > 0.0f))
                    s = 0.0f;
                ((uint16_t*)p.C)[(int64_t)m * p.N + n] = cvt1(s, DT_BF16);
            }
        }
    }
};

template <bool DWORD_SCALES>
__global__ __attribute__((amdgpu_flat_work_group_size(1024, 1024))) void gemv_w4_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    GemvW4<DWORD_SCALES>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
