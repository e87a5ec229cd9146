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
//  * a round is 16 MFMA steps of 32 k.  Two assignments of k to lanes, a
//    template parameter chosen by the activation row count:
//    - lane ranges (RUNS = false): lane (n = l % 16, g = l / 16) takes the
//      128 k of [512 r + 128 g, +128) (4 x 16 bytes of codes of row n and the
//      4 scale bytes of those k); step (c, h) multiplies k = 512 r + 128 g +
//      32 c + 8 h + 0..7 in group g.  Few VALU operations per code, and the
//      activation loads of one row are cheap; with 16 rows each activation
//      load touches 64 scattered 16-byte pieces, and those loads bound it;
//    - contiguous runs (RUNS = true): step (c, h) takes k = 512 r + 128 c +
//      32 h + 8 g + 0..7 in group g, so the four groups of one row read one
//      contiguous 64-byte run for each activation load (16 runs per load).
//      The codes are loaded the same way (load c: lane (n, g) takes the 16
//      bytes of k in [512 r + 128 c + 32 g, +32)), which puts the codes of
//      step (c, h) in dword g of group h; a 4 x 4 transpose across the lane
//      groups (two rounds of lane-row swaps) moves them to dword h of group
//      g.  The 16 scale bytes of a row's round are one 16-byte load;
//  * the codes are expanded to bf16 in registers (v_cvt_scalef32_pk_bf16_fp4
//    applies the scale exactly) and fed straight to v_mfma_f32_16x16x32_bf16
//    as the 16-row operand; the activation fragment of the same k (rows m of
//    A, zero past M) is the other operand;
//  * the 16 waves' 16 x 32 partial sums are added in LDS in a fixed order (so
//    results do not depend on timing), then ReLU, one rounding and the store.
// The k order inside an MFMA step is permuted the same way for A and W, which
// only reorders the sum.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel.h"

namespace tg {

typedef __attribute__((ext_vector_type(4))) float f32x4v;

// 4 x 4 transpose across the four 16-lane groups: afterwards d[h] of group g
// is what d[g] of group h was.  A swap of lane halves (groups 2, 3 of one
// register with groups 0, 1 of another), then a swap of odd and even groups.
__device__ __forceinline__ void transpose4(u32 (&d)[4])
{
    const auto s02 = __builtin_amdgcn_permlane32_swap(d[0], d[2], false, false);
    const auto s13 = __builtin_amdgcn_permlane32_swap(d[1], d[3], false, false);
    const auto s01 = __builtin_amdgcn_permlane16_swap(s02[0], s13[0], false, false);
    const auto s23 = __builtin_amdgcn_permlane16_swap(s02[1], s13[1], false, false);
    d[0] = s01[0];
    d[1] = s01[1];
    d[2] = s23[0];
    d[3] = s23[1];
}

// Eight E2M1 codes (low nibble first) to eight bf16 values times scale s.
__device__ __forceinline__ u32x4 expand8(u32 packed, float s)
{
    u32x4 b;
    b[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 0));
    b[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 1));
    b[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 2));
    b[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, s, 3));
    return b;
}

template <bool DWORD_SCALES, bool RUNS>
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

        if constexpr (RUNS) {
            const int rounds = (K + ROUND - 1) / ROUND;
            for (int r = w; r < rounds; r += NWAVE) {
                const int kr = r * ROUND;
                // every code load of the round is issued before the first is
                // consumed (8 KiB per wave in flight), after the activation
                // fragments of steps 0 and 1 (16 bytes of row m0 + ln per
                // lane) and the scales: vector loads complete in order, so
                // steps 0 and 1 wait only for their own codes, not for the
                // whole round.
                u32x4 code[NG][4];  // [group][c]: codes of k in [kr + 128 c + 32 g, +32)
                u32x4 sc[NG];       // the row's 16 scale bytes of the round, block 4 c + h
                u32x4 af[16];
                const auto load_af = [&](int c) {
#pragma unroll
                    for (int h = 0; h < 4; ++h) {
                        const int k = kr + 128 * c + 32 * h + 8 * g;
                        af[4 * c + h] =
                            buf_load16(ars, (arow && k < K) ? (u32)(ln * K + k) * 2u : kOob);
                    }
                };
                const auto load_codes = [&](int c) {
#pragma unroll
                    for (int q = 0; q < NG; ++q) {
                        const u32 rowoff = (u32)((16 * q + ln) * rowb);
                        const int k = kr + 128 * c + 32 * g;  // K is a multiple of 32
                        code[q][c] = buf_load16(wrs, k < K ? rowoff + (u32)k / 2 : kOob);
                    }
                };
                load_af(0);
                load_af(1);
                if constexpr (DWORD_SCALES) {
#pragma unroll
                    for (int q = 0; q < NG; ++q) {
                        const u32 soff = (u32)((16 * q + ln) * srow + kr / 32);
                        if (kr + ROUND <= K) {
                            sc[q] = buf_load16(srs, soff);  // 4-byte aligned rows
                        } else {
                            // the last, partial round: dword i (blocks 4 i ..) only
                            // while inside the row (K % 128 == 0 for aligned rows)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                sc[q][i] = buf_load4(srs, kr + 128 * i < K ? soff + 4 * i : kOob);
                        }
                    }
                }
                // (byte-aligned scale rows: their bytes are loaded per step below)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    load_codes(c);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    // the activation fragments of step c + 2 are loaded during
                    // step c (all sixteen at once would not fit the 128
                    // registers of a wave)
                    if (c + 2 < 4)
                        load_af(c + 2);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int q = 0; q < NG; ++q) {
                        if (!DWORD_SCALES) {
                            const u32 soff = (u32)((16 * q + ln) * srow + kr / 32 + 4 * c);
                            u32 b = 0;
#pragma unroll
                            for (int h = 0; h < 4; ++h)
                                b |= buf_load1(srs, kr + 32 * (4 * c + h) < K ? soff + h : kOob)
                                     << (8 * h);
                            sc[q][c] = b;
                        }
                        // group g holds dword e = codes of step (c, g), lanes 8 e ..;
                        // step (c, h) wants, in group g, the dword g of group h
                        u32 d[4] = {code[q][c][0], code[q][c][1], code[q][c][2], code[q][c][3]};
                        transpose4(d);
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            const int blk = 4 * c + h;  // 32-k block of the round
                            const u32 e = (sc[q][blk >> 2] >> (8 * (blk & 3))) & 0xFFu;
                            // a scale byte only multiplies codes of k < K (zeros past it)
                            const float s = e8m0_cvt_scale(kr + 32 * blk < K ? e : 127u);
                            const u32 packed = d[h];  // 8 codes: k = kr + 128 c + 32 h + 8 g ..
                            const u32x4 b = expand8(packed, s);
                            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, af[blk]),
                                acc[q], 0, 0, 0);
                        }
                    }
                }
            }
        } else {
            const int rounds = (K + ROUND - 1) / ROUND;
            for (int r = w; r < rounds; r += NWAVE) {
                const int kq = r * ROUND + 128 * g;  // this lane's first k
                const bool kv = kq < K;              // K is a multiple of 32; kq, +32, ... may pass it
                // every load of the round is issued before the first is
                // consumed (8 KiB of codes per wave in flight), in the order
                // the steps consume them: vector loads complete in order, so a
                // step waits only for its own loads and those before them.
                // The activation fragments (16 bytes of row m0 + ln at the
                // lane's k, mostly from L2) and the scales come first, then
                // the codes of group 0, then those of group 1.
                u32x4 af[16];
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int k = kq + 8 * j;
                    af[j] = buf_load16(ars, (arow && k < K) ? (u32)(ln * K + k) * 2u : kOob);
                }
                u32 sc[NG];
#pragma unroll
                for (int q = 0; q < NG; ++q) {
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
                u32x4 code[NG][4];
#pragma unroll
                for (int q = 0; q < NG; ++q) {
                    const u32 rowoff = (u32)((16 * q + ln) * rowb);
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const bool v = kq + 32 * c < K;
                        code[q][c] = buf_load16(wrs, v ? rowoff + (u32)(kq + 32 * c) / 2 : kOob);
                    }
                }
                // every load of the round is in flight before the first is consumed
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int q = 0; q < NG; ++q) {
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        // a scale byte only multiplies codes of k < K (zeros past it)
                        const u32 e = (sc[q] >> (8 * c)) & 0xFFu;
                        const float s = e8m0_cvt_scale(kq + 32 * c < K ? e : 127u);
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            const u32 packed = code[q][c][h];  // 8 codes: k = kq + 32c + 8h ..
                            const u32x4 b = expand8(packed, s);
                            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, af[4 * c + h]),
                                acc[q], 0, 0, 0);
                        }
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

template <bool DWORD_SCALES, bool RUNS>
__global__ __attribute__((amdgpu_flat_work_group_size(1024, 1024))) void gemv_w4_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    GemvW4<DWORD_SCALES, RUNS>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
