// Weight-only 4-bit dequant GEMM, LDS-DMA pipeline (many activation rows).
//
// The operation is the pages' weight-only low-bit GEMM ("WFP4" GEMM in
// "TileLang架构深度剖析", the performance section; "Dequant GEMM" in
// "使用 Tilelang DSL 开发 GPU/CPU/加速器高性能内核"), tiled as their dense GEMM
// is ("TileLang ... 一个高效 GEMM 内核", mhpq.cn, sections 2.1, 3.2, 3.3):
// C[m][n] = sum_k A[m][k] W[n][k], W stored as E2M1 codes two per byte with an
// E8M0 scale per 32 k.
//
// MI355X mapping:
//  * BM x BN x 128 strips, four waves in a 2 x 2 grid, NS-stage LDS ring filled
//    by LDS-DMA copies (no VGPR staging): A as [BM][128] bf16 (256-byte rows),
//    the packed codes as [BN][64 bytes] and the scale bytes as [BN][4].  The
//    codes stay packed in LDS (a quarter of the bf16 bytes); each wave expands
//    its own B fragments in registers (v_cvt_scalef32_pk_bf16_fp4, exact)
//    right before the MFMA that consumes them.
//  * Inside a strip the k order is permuted the same way on both operands:
//    MFMA slab s (0..7) takes, in lane half h, k = 64 h + 8 s .. + 7.  A lane's
//    codes for the whole strip are then one contiguous 32-byte run of its row
//    (two ds_read_b128), and its A fragment of slab s is 16-byte chunk 8 h + s.
//  * Chunk swizzles keep the fragment reads free of bank conflicts: A chunks
//    are XORed with row & 15, code chunks with the 64-byte-row swizzle.
//  * Strips are whole (K % 128 == 0; other K use the register-staged kernel);
//    out-of-range rows (m >= M, n >= N) and the strips padded past K copy
//    zeros.  The barrier/copy schedule is the one of the 16-bit DMA kernel:
//    one barrier per strip after its first MFMA, copies of strip t + NS - 1
//    staggered across the waves and MFMA slots.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel.h"
#include "tg_kernel_dma.h"

namespace tg {

// 4-byte-per-lane copy global -> LDS: lane l's dword lands at LDS byte lds + 4 l.
__device__ __forceinline__ void dma4(u32 lds, u32 voff, __amdgpu_buffer_rsrc_t rs)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds" ::"s"(lds),
                 "v"(voff), "s"(rs)
                 : "memory");
}

template <int BM, int BN, int WGM, int WGN, int NS, int GROUP_M>
struct DmaW4 {
    static constexpr int BK = 128;
    static constexpr int NW = WGM * WGN;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr int NM = FM * FN;      // MFMAs per slab
    static constexpr int SLOTS = 8 * NM;    // MFMAs per strip
    static constexpr int A_STAGE = BM * BK * 2;
    static constexpr int W_STAGE = BN * BK / 2;
    static constexpr int S_STAGE = BN * 4;
    static constexpr int W_REGION = NS * A_STAGE;
    static constexpr int S_REGION = W_REGION + NS * W_STAGE;
    static constexpr int LDS_BYTES = S_REGION + NS * S_STAGE;
    static constexpr int JA = A_STAGE / 1024 / NW;  // A copies per wave per strip
    static constexpr int JW = W_STAGE / 1024 / NW;  // code copies per wave per strip
    static constexpr int NSC = S_STAGE / 256;       // scale copies per strip (waves 0 .. NSC-1)

    static_assert(NW == 4, "four waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of 32x32 blocks");
    static_assert(JA >= 1 && JW >= 1 && A_STAGE % (1024 * NW) == 0 && W_STAGE % (1024 * NW) == 0,
                  "strips split into whole 1 KiB copies per wave");
    static_assert(NSC >= 1 && NSC <= NW && S_STAGE % 256 == 0, "one scale copy per wave at most");
    static_assert(NS == 4, "four stages (code registers alternate per strip)");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    template <int W>
    struct Copies {
        static constexpr int N = JA + JW + (W < NSC ? 1 : 0);
        static constexpr int AHEAD = (NS - 3) * N;
    };
    static constexpr int NCMAX = JA + JW + 1;

    struct Lane {
        u32 a_off[JA];
        u32 w_off[JW];
        u32 s_off;
        u32 a_rd[8];  // A fragment read offset of slab s (stage 0, fm 0)
        u32 w_rd[2];  // code chunk 2h, 2h+1 of this lane's row (stage 0, fn 0)
        u32 s_rd;     // scale bytes 2h, 2h+1 of this lane's row (stage 0, fn 0)
    };

    struct Regs {
        u32x4 code[FN][2];  // 32 bytes = 64 codes per n-block
        u32 sc[FN];         // two scale bytes (k groups 2h, 2h+1)
    };

    static __device__ __forceinline__ int swz16(int r) { return r & 15; }

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn)
    {
        const int K = p.K;
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int row = (w * JA + j) * 4 + (lane >> 4);
            const int c = (lane & 15) ^ swz16(row);
            L.a_off[j] = (m0 + row < p.M) ? (u32)(row * K + c * 8) * 2u : kOob;
        }
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int row = (w * JW + j) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz_a(row);
            L.w_off[j] = (n0 + row < p.N) ? (u32)(row * (K / 2) + c * 16) : kOob;
        }
        {
            const int row = w * 64 + lane;
            L.s_off = (w < NSC && n0 + row < p.N) ? (u32)(row * (K / 32)) : kOob;
        }
        const int h = lane >> 5;
        const int ar = wm * WTM + (lane & 31);
#pragma unroll
        for (int s = 0; s < 8; ++s)
            L.a_rd[s] = ar * (BK * 2) + (((8 * h + s) ^ swz16(ar)) << 4);
        const int nr = wn * WTN + (lane & 31);
        L.w_rd[0] = W_REGION + nr * 64 + (((2 * h) ^ swz_a(nr)) << 4);
        L.w_rd[1] = W_REGION + nr * 64 + (((2 * h + 1) ^ swz_a(nr)) << 4);
        L.s_rd = S_REGION + nr * 4 + 2 * h;
    }

    struct StripRes {
        __amdgpu_buffer_rsrc_t a, w, s;
        bool valid;
    };

    static __device__ __forceinline__ StripRes strip_res(const GemmParams& p, int m0, int n0,
                                                         int strip)
    {
        const int K = p.K;
        const int k0 = strip * BK;
        StripRes r;
        r.valid = k0 < K;
        r.a = make_rsrc((const char*)p.A + ((int64_t)m0 * K + k0) * 2,
                        clamp_bytes(((int64_t)(p.M - m0 - 1) * K + (K - k0)) * 2));
        r.w = make_rsrc((const char*)p.B + (int64_t)n0 * (K / 2) + k0 / 2,
                        clamp_bytes((int64_t)(p.N - n0 - 1) * (K / 2) + (K - k0) / 2));
        r.s = make_rsrc((const char*)p.Bs + (int64_t)n0 * (K / 32) + k0 / 32,
                        clamp_bytes((int64_t)(p.N - n0 - 1) * (K / 32) + (K - k0) / 32));
        return r;
    }

    template <int ST, int W>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const StripRes& r, int d,
                                                      u32 smem0)
    {
        if (d < JA)
            dma16(smem0 + ST * A_STAGE + (W * JA + d) * 1024, r.valid ? L.a_off[d] : kOob, r.a);
        else if (d < JA + JW)
            dma16(smem0 + W_REGION + ST * W_STAGE + (W * JW + d - JA) * 1024,
                  r.valid ? L.w_off[d - JA] : kOob, r.w);
        else
            dma4(smem0 + S_REGION + ST * S_STAGE + W * 256, r.valid ? L.s_off : kOob, r.s);
    }

    template <int ST, int W>
    static __device__ __forceinline__ void issue_copies(const Lane& L, const GemmParams& p,
                                                        int m0, int n0, int strip, u32 smem0)
    {
        const StripRes r = strip_res(p, m0, n0, strip);
#pragma unroll
        for (int d = 0; d < Copies<W>::N; ++d)
            issue_copy<ST, W>(L, r, d, smem0);
    }

    template <int ST>
    static __device__ __forceinline__ void read_codes(Regs& R, const Lane& L, lds_char* sm)
    {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            R.code[fn][0] = *(const lds_u32x4*)(sm + L.w_rd[0] + ST * W_STAGE + fn * 32 * 64);
            R.code[fn][1] = *(const lds_u32x4*)(sm + L.w_rd[1] + ST * W_STAGE + fn * 32 * 64);
            R.sc[fn] = *(const __attribute__((address_space(3))) uint16_t*)(sm + L.s_rd +
                                                                            ST * S_STAGE +
                                                                            fn * 32 * 4);
        }
    }

    template <int ST>
    static __device__ __forceinline__ void read_a(u32x4 (&af)[FM], const Lane& L, lds_char* sm,
                                                  int s)
    {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            af[fm] = *(const lds_u32x4*)(sm + L.a_rd[s] + ST * A_STAGE + fm * 32 * BK * 2);
    }

    // B fragment of n-block fn, slab s: codes 8 s .. 8 s + 7 of the lane's 64.
    static __device__ __forceinline__ bf16x8 dequant(const Regs& R, int fn, int s)
    {
        const u32 packed = R.code[fn][s >> 2][s & 3];
        const float sc = e8m0_to_f32((R.sc[fn] >> (8 * (s >> 2))) & 0xFFu);
        u32x4 b;
        b[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 0));
        b[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 1));
        b[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 2));
        b[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 3));
        return __builtin_bit_cast(bf16x8, b);
    }

    // A fragments are read PF slabs ahead into a 4-deep ring (slab s of any
    // strip lives in AF[s % 4]).
    static constexpr int PF = 3;

    // One strip (stage ST) of wave W.  Slot i = MFMA (fm, fn) of slab s with
    // s = i / NM.  Before slot 0: codes of this strip in R[ST & 1], A slabs
    // 0 .. PF-1 in the ring.  Slot 0 waits for strip t + 1's copies and
    // barriers, then reads strip t + 1's codes into R[(ST + 1) & 1]; the last
    // slot of slab s reads A slab s + PF (of strip t + 1 past slab 7); the
    // copies of strip t + NS - 1 are staggered over the slots.
    template <int ST, int W>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Regs (&R)[2],
                                                 u32x4 (&AF)[4][FM], const Lane& L, lds_char* sm,
                                                 const GemmParams& p, int m0, int n0, int t,
                                                 u32 smem0)
    {
        constexpr int NXT = (ST + 1) % NS;
        constexpr int CPY = (ST + NS - 1) % NS;
        constexpr int CUR = ST & 1;
        StripRes r;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int s = i / NM, fm = (i % NM) / FN, fn = i % FN;
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant(R[CUR], fn, s),
                                                                  __builtin_bit_cast(bf16x8, AF[s & 3][fm]),
                                                                  acc[fm][fn], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (i == 0) {
                wait_copies_barrier<Copies<W>::AHEAD>();
                __builtin_amdgcn_sched_barrier(0);
                r = strip_res(p, m0, n0, t + NS - 1);
                read_codes<NXT>(R[CUR ^ 1], L, sm);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (i % NM == NM - 1) {
                if (s + PF < 8)
                    read_a<ST>(AF[(s + PF) & 3], L, sm, s + PF);
                else
                    read_a<NXT>(AF[(s + PF) & 3], L, sm, s + PF - 8);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int d = 0; d < Copies<W>::N; ++d) {
                if (((d * NW + W) * SLOTS) / (NCMAX * NW) == i) {
                    issue_copy<CPY, W>(L, r, d, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    template <int W>
    static __device__ __forceinline__ void main_loop(f32x16 (&acc)[FM][FN], const Lane& L,
                                                     lds_char* sm, const GemmParams& p, int m0,
                                                     int n0, int KT, u32 smem0)
    {
        issue_copies<0, W>(L, p, m0, n0, 0, smem0);
        issue_copies<1, W>(L, p, m0, n0, 1, smem0);
        issue_copies<2 % NS, W>(L, p, m0, n0, 2, smem0);
        static_assert(NS == 4, "prologue and loop written for four stages");
        wait_copies_barrier<(NS - 2) * Copies<W>::N>();
        Regs R[2];
        u32x4 AF[4][FM];
        read_codes<0>(R[0], L, sm);
#pragma unroll
        for (int s = 0; s < PF; ++s)
            read_a<0>(AF[s], L, sm, s);
        // The strip count is rounded up to a multiple of NS: strips at or past
        // KT copy only zeros, which add exactly nothing.
        for (int t = 0; t < KT; t += NS) {
            strip<0, W>(acc, R, AF, L, sm, p, m0, n0, t, smem0);
            strip<1, W>(acc, R, AF, L, sm, p, m0, n0, t + 1, smem0);
            strip<2, W>(acc, R, AF, L, sm, p, m0, n0, t + 2, smem0);
            strip<3, W>(acc, R, AF, L, sm, p, m0, n0, t + 3, smem0);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    static __device__ __forceinline__ void run(const GemmParams& p)
    {
        __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
        lds_char* sm = (lds_char*)smem;
        const u32 smem0 = lds_offset(smem);
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm = w / WGN;
        const int wn = w % WGN;
        const TileCoord tc = tile_of(blockIdx.x, p.tiles_m, p.tiles_n, GROUP_M);
        const int m0 = tc.m * BM;
        const int n0 = tc.n * BN;
        const int KT = p.K / BK;

        Lane L;
        setup(L, p, m0, n0, w, lane, wm, wn);
        f32x16 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[fm][fn][r] = 0.0f;
        switch (w) {
        case 0:
            main_loop<0>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        case 1:
            main_loop<1>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        case 2:
            main_loop<2>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        default:
            main_loop<3>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        }
        if ((p.N & 7) == 0 && ((uintptr_t)p.C & 15) == 0 && NW * WTM * WTN * 2 <= LDS_BYTES) {
            wait_all_barrier();  // every wave's copies landed and reads done
            store_tile_staged<DT_BF16, WTM, WTN, FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN,
                                                        lane, sm + w * (WTM * WTN * 2));
            return;
        }
        // epilogue: same lane layout as the 16-bit DMA kernel (m = lane % 32,
        // four consecutive n per accumulator quad)
        const int lr = lane & 31;
        const int g = lane >> 5;
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int m = m0 + wm * WTM + fm * 32 + lr;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int n = n0 + wn * WTN + fn * 32 + 8 * q + 4 * g;
                    float v[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float x = acc[fm][fn][4 * q + e];
                        v[e] = (p.relu && !(x > 0.0f)) ? 0.0f : x;
                    }
                    const int64_t idx = (int64_t)m * p.N + n;
                    if (p.c_vec && n + 3 < p.N) {
                        *(u32x2*)(C + idx) = u32x2{pack2(v[0], v[1], DT_BF16), pack2(v[2], v[3], DT_BF16)};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N)
                                C[idx + e] = cvt1(v[e], DT_BF16);
                    }
                }
            }
        }
    }
};

template <int BM, int BN, int WGM, int WGN, int NS, int GROUP_M>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * 64, WGM * WGN * 64))) void
dma_w4_kernel(GemmParams p)
{
    DmaW4<BM, BN, WGM, WGN, NS, GROUP_M>::run(p);
}

}  // namespace tg
