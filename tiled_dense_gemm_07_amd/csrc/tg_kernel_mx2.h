// MX-format GEMM (E2M1 or E4M3 activations x E2M1 weights) on 256-k strips
// and a two-stage LDS ring.
//
// The same product as tg_kernel_mx.h (the pages' "WFP4" GEMM, "TileLang架构
// 深度剖析", the performance section, with both operands in OCP MX blocks):
// C[m][n] = sum_k a(m, k) w(n, k), each 32 k of a row sharing one E8M0 scale,
// fp32 accumulation, one rounding to bf16, on v_mfma_scale_f32_32x32x64_f8f6f4.
// What differs is the strip: 256 k instead of 128, so a row's E2M1 codes for
// a strip are one whole 128-byte line (E4M3: two).  An LDS-DMA copy then
// covers whole lines (8 rows x 128 bytes, or 4 x 256) where the 128-k
// kernel's E2M1 copies cover 16 rows x 64 bytes (16 half lines), and the
// address path, which spends its cycles per line, has half the work per
// byte; the strip also carries twice the MFMAs per barrier.  The price is the
// ring: a 256 x 256 E2M1 tile's (or 128 x 256 E4M3 tile's) strip is 64 KiB,
// so two stages fill 128 KiB of the 160 KiB LDS, and the scale chunks the
// rest.
//  * four 64-k steps per strip; fragment reads of step q: E2M1 lane (row r,
//    half h) reads 16-byte chunk 2 q + h of its row (128-byte rows, chunk c
//    at position c ^ swz8(r)); E4M3 lane (r, h) reads chunks 4 q + h and
//    4 q + 2 + h (256-byte rows, chunk c at position c ^ (r & 15)); the
//    copies place the chunks there, and the reads are conflict-free;
//  * scales in chunks of 4 strips (32 bytes per row: strips 0, 1 in one
//    16-byte half, 2, 3 in the other, the halves swapped for rows with bit 3
//    set), copied with 16-byte copies into one of two buffers during strip
//    4 c + 1 (chunk c + 1); a lane reads its row's 8 scale bytes of a strip
//    with one 8-byte read and shifts them per step and lane half;
//  * the two-stage schedule of the 16-bit LDS-DMA kernel: the barrier sits
//    at the start of the last step, after every wave has waited for all its
//    copies (strip t + 1's) and LDS reads; after it strip t + 1 is visible,
//    its scales and first fragments are read, and the copies of strip t + 2
//    go into the stage strip t used, spread over the last step of t and the
//    first step of t + 1;
//  * K % 1024 == 0 (whole scale chunks; the loop runs 4 strips at a time so
//    that the stage and the place in the chunk are compile-time constants),
//    16-byte aligned operand and scale rows.  Rows past M or N copy zeros.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel_mx.h"

namespace tg {

template <int AFMT, int BM, int BN, int WGM, int WGN, int GROUP_M>
struct DmaMx2 {
    static constexpr int BK = 256;
    static constexpr bool A8 = AFMT == MX_E4M3;
    static constexpr int SL = 4;      // 64-k steps per strip
    static constexpr int CH = 4;      // strips per scale chunk
    static constexpr int NW = WGM * WGN;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr int ROWB = BK / 2;  // code bytes per row per strip (E2M1)
    static constexpr int A_ROWB = A8 ? BK : ROWB;
    static constexpr int A_STAGE = BM * A_ROWB;
    static constexpr int W_STAGE = BN * ROWB;
    static constexpr int W_REGION = 2 * A_STAGE;
    static constexpr int SA_REGION = W_REGION + 2 * W_STAGE;
    static constexpr int SA_BUF = BM * 32;  // one chunk of A scales (32 bytes per row)
    static constexpr int SW_BUF = BN * 32;
    static constexpr int SW_REGION = SA_REGION + 2 * SA_BUF;
    static constexpr int LDS_BYTES = SW_REGION + 2 * SW_BUF;
    static constexpr int JA = A_STAGE / 1024 / NW;  // A copies per wave per strip
    static constexpr int JW = W_STAGE / 1024 / NW;
    static constexpr int NCOPY = JA + JW;
    static constexpr int NCA = BM / 32;             // chunk copies of A scales (32 rows each)
    static constexpr int NCW = BN / 32;
    static constexpr int JS = (NCA + NCW) / NW;     // chunk copies per wave
    static constexpr int NM = FM * FN;              // MFMAs per step
    static constexpr int NRD_A = FM * (A8 ? 2 : 1);
    static constexpr int NRD = NRD_A + FN;          // fragment reads per step
    static constexpr int STEPS = NM > NRD ? NM : NRD;  // slots per step
    static constexpr int SLOTS = SL * STEPS;
    static constexpr int CSLOTS = 2 * STEPS;        // copy window: last step of t, first of t + 1

    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of 32x32 blocks");
    static_assert(JA >= 1 && JW >= 1 && A_STAGE % (1024 * NW) == 0 && W_STAGE % (1024 * NW) == 0,
                  "strips split into whole 1 KiB copies per wave");
    static_assert((NCA + NCW) % NW == 0 && JS >= 1 && 2 * JS <= STEPS, "chunk copies split evenly");
    static_assert(SA_REGION % 1024 == 0 && SW_REGION % 1024 == 0,
                  "scale buffers 1 KiB aligned (the chunk halves are selected by an xor)");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    struct Lane {
        u32 a_off[JA];
        u32 w_off[JW];
        u32 s_off[JS];    // chunk copies: row offset + 16-byte half
        u32 a_rd[SL][A8 ? 2 : 1];  // [step][part]: this lane's code chunk (stage 0, fm 0)
        u32 w_rd[SL];     // [step] (stage 0, fn 0)
        u32 sa_rd, sw_rd; // this lane's row in scale buffer 0 (strips 0, 1; 2, 3 at ^ 16)
        u32 sh[2];        // 8 * lane half (+ 16 for odd steps): byte to byte 0
    };

    struct Frag {  // one 64-k step
        u32x4 a[FM][A8 ? 2 : 1];
        u32x4 w[FN];
    };

    // A chunk swizzle: 128-byte rows (E2M1) as the 16-bit kernel's, 256-byte
    // rows (E4M3) by the row's low 4 bits
    static __device__ __forceinline__ int swz_arow(int r) { return A8 ? (r & 15) : swz8(r); }
    struct Scales {  // one strip: a row's 8 scale bytes per block, as read
        u32x2 a[FM];
        u32x2 w[FN];
    };

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn)
    {
        const int K = p.K;
        // copy j: rows 8 j' .. + 7, lane l -> row 8 j' + l / 8, LDS 16-byte
        // position l & 7, which holds code chunk (l & 7) ^ swz8(row); E4M3 A:
        // rows 4 j' .., lane l -> row 4 j' + l / 16, position l & 15
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            constexpr int CPR = A8 ? 16 : 8;  // 16-byte chunks per row
            const int row = (w * JA + j) * (64 / CPR) + lane / CPR;
            const int c = (lane % CPR) ^ swz_arow(row);
            L.a_off[j] = (m0 + row < p.M) ? (u32)(row * (A8 ? K : K / 2) + c * 16) : kOob;
        }
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int row = (w * JW + j) * 8 + (lane >> 3);
            const int c = (lane & 7) ^ swz8(row);
            L.w_off[j] = (n0 + row < p.N) ? (u32)(row * (K / 2) + c * 16) : kOob;
        }
        // chunk copy g: 32 rows x 32 bytes, lane l -> row 32 g' + l / 2 at
        // position l & 1, which holds the row's half (l & 1) ^ bit 3 of the row
#pragma unroll
        for (int d = 0; d < JS; ++d) {
            const int g = w * JS + d;
            const bool isa = g < NCA;
            const int row = (isa ? g : g - NCA) * 32 + (lane >> 1);
            const int half = (lane & 1) ^ ((row >> 3) & 1);
            const bool ok = isa ? (m0 + row < p.M) : (n0 + row < p.N);
            L.s_off[d] = ok ? (u32)(row * (K / 32) + half * 16) : kOob;
        }
        const int h = lane >> 5;
        const int ar = wm * WTM + (lane & 31);
        const int nr = wn * WTN + (lane & 31);
#pragma unroll
        for (int q = 0; q < SL; ++q) {
            if constexpr (A8) {
                // bytes 0..15: k = 64 q + 16 h; bytes 16..31: k = 64 q + 32 + 16 h
                L.a_rd[q][0] = ar * A_ROWB + (((4 * q + h) ^ swz_arow(ar)) << 4);
                L.a_rd[q][1] = ar * A_ROWB + (((4 * q + 2 + h) ^ swz_arow(ar)) << 4);
            } else {
                // 32 codes of step q, lane half h: k = 64 q + 32 h
                L.a_rd[q][0] = ar * A_ROWB + (((2 * q + h) ^ swz_arow(ar)) << 4);
            }
            L.w_rd[q] = W_REGION + nr * ROWB + (((2 * q + h) ^ swz8(nr)) << 4);
        }
        L.sa_rd = SA_REGION + ar * 32 + (((ar >> 3) & 1) << 4);
        L.sw_rd = SW_REGION + nr * 32 + (((nr >> 3) & 1) << 4);
        L.sh[0] = 8 * h;
        L.sh[1] = 8 * h + 16;
    }

    struct Res {
        __amdgpu_buffer_rsrc_t a, w, sa, sw;
    };
    struct StripOff {
        u32 a, w;  // byte offsets of the strip in a row of A codes, of W codes
        bool valid;
    };

    static __device__ __forceinline__ Res band_res(const GemmParams& p, int m0, int n0)
    {
        using Base = DmaMx<MX_E2M1, BM, BN, 2, 2, 4, GROUP_M, false>;
        const int K = p.K;
        Res r;
        r.a = Base::band(p.A, m0, p.M - m0, A8 ? K : K / 2);
        r.w = Base::band(p.B, n0, p.N - n0, K / 2);
        r.sa = Base::band(p.As, m0, p.M - m0, K / 32);
        r.sw = Base::band(p.Bs, n0, p.N - n0, K / 32);
        return r;
    }

    static __device__ __forceinline__ StripOff strip_off(const GemmParams& p, int strip)
    {
        const int k0 = strip * BK;
        return StripOff{(u32)(A8 ? k0 : k0 / 2), (u32)(k0 / 2), k0 < p.K};
    }

    // Copy d of wave W for strip offset o into stage ST.
    template <int ST, int W>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const Res& r,
                                                      const StripOff& o, int d, u32 smem0)
    {
        if (d < JA)
            dma16(smem0 + ST * A_STAGE + (W * JA + d) * 1024, o.valid ? L.a_off[d] + o.a : kOob,
                  r.a);
        else
            dma16(smem0 + W_REGION + ST * W_STAGE + (W * JW + d - JA) * 1024,
                  o.valid ? L.w_off[d - JA] + o.w : kOob, r.w);
    }

    // Chunk copy d of wave W: the scale bytes of strips 4 c .. 4 c + 3 into
    // buffer c & 1 (K % 1024 == 0: a chunk is inside the rows or past K).
    template <int W>
    static __device__ __forceinline__ void issue_chunk(const Lane& L, const Res& r,
                                                       const GemmParams& p, int c, int d,
                                                       u32 smem0)
    {
        const int g = W * JS + d;
        const u32 buf = (u32)(c & 1);
        const u32 off = 1024 * c < p.K ? L.s_off[d] + (u32)(c * 32) : kOob;
        if (g < NCA)
            dma16(smem0 + SA_REGION + buf * SA_BUF + g * 1024, off, r.sa);
        else
            dma16(smem0 + SW_REGION + buf * SW_BUF + (g - NCA) * 1024, off, r.sw);
    }

    // Fragment read i of step Q of stage ST: A blocks, then W blocks.
    template <int ST, int Q>
    static __device__ __forceinline__ void read_one(Frag& F, const Lane& L, lds_char* sm, int i)
    {
        if (i < NRD_A) {
            const int fm = A8 ? (i >> 1) : i, part = A8 ? (i & 1) : 0;
            F.a[fm][part] = *(const lds_u32x4*)(sm + L.a_rd[Q][part] + ST * A_STAGE +
                                                fm * 32 * A_ROWB);
        } else {
            F.w[i - NRD_A] =
                *(const lds_u32x4*)(sm + L.w_rd[Q] + ST * W_STAGE + (i - NRD_A) * 32 * ROWB);
        }
    }

    // Scale bytes of strip u, its place P in the chunk at compile time.
    template <int P>
    static __device__ __forceinline__ void read_scales(Scales& S, const Lane& L, lds_char* sm,
                                                       int u)
    {
        typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
        const u32 buf = (u32)((u >> 2) & 1);
        const u32 hx = (u32)((P >> 1) << 4);
        const u32 ra = (L.sa_rd ^ hx) + buf * SA_BUF + (P & 1) * 8;
        const u32 rw = (L.sw_rd ^ hx) + buf * SW_BUF + (P & 1) * 8;
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            S.a[fm] = *(const lds_u32x2*)(sm + ra + fm * 32 * 32);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            S.w[fn] = *(const lds_u32x2*)(sm + rw + fn * 32 * 32);
    }

    // MFMA i of step Q; the scale words are shifted at their first use.
    template <int Q>
    static __device__ __forceinline__ void mfma_one(f32x16 (&acc)[FM][FN], const Frag& F,
                                                    const Scales& S, const Lane& L, int i)
    {
        const int fm = i / FN, fn = i % FN;
        const u32x4 wv = F.w[fn], lo = F.a[fm][0], hi = F.a[fm][A8 ? 1 : 0];
        const i32x8 wop = {(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3], 0, 0, 0, 0};
        const i32x8 aop = A8 ? i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                     (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]}
                             : i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            wop, aop, acc[fm][fn], MX_E2M1, AFMT, 0, (int)(S.w[fn][Q >> 1] >> L.sh[Q & 1]), 0,
            (int)(S.a[fm][Q >> 1] >> L.sh[Q & 1]));
    }

    static constexpr int cpos(int d, int W) { return ((d * NW + W) * CSLOTS) / (NCOPY * NW); }

    // Slot SLOT of strip t (stage ST, place P in its scale chunk, scale set
    // CUR) of wave W, then the following slots.  Step s = SLOT / STEPS uses
    // fragment set F[s & 1] and reads the next step's into the other (the
    // last step reads step 0 of strip t + 1 into F[0], after the barrier).
    template <int ST, int P, int CUR, int W, int SLOT>
    static __device__ __forceinline__ void slots(f32x16 (&acc)[FM][FN], Frag (&F)[2],
                                                 Scales (&SC)[2], const Lane& L, const Res& res,
                                                 lds_char* sm, const GemmParams& p, int t,
                                                 const StripOff& r2, const StripOff& r1,
                                                 u32 smem0)
    {
        constexpr int S = SLOT / STEPS, I = SLOT % STEPS;
        constexpr int NXT = ST ^ 1;
        if constexpr (I < NM) {
            mfma_one<S>(acc, F[S & 1], SC[CUR], L, I);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (S == SL - 1 && I == 0) {
            // strip t + 1's copies landed, every wave is done with strip t's
            // stage (its last step is in registers)
            wait_all_barrier();
            __builtin_amdgcn_sched_barrier(0);
            read_scales<(P + 1) % CH>(SC[CUR ^ 1], L, sm, t + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (I < NRD) {
            if constexpr (S + 1 < SL)
                read_one<ST, S + 1>(F[(S + 1) & 1], L, sm, I);
            else
                read_one<NXT, 0>(F[0], L, sm, I);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (P == 1 && S == 1) {
            // scale chunk c + 1 into the buffer chunk c - 1 used
#pragma unroll
            for (int d = 0; d < JS; ++d) {
                if (I == 2 * d + 1) {
                    issue_chunk<W>(L, res, p, t / CH + 1, d, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        // copy window: positions < STEPS in the last step (strip t + 2 into
        // this strip's stage, after the barrier), the rest in step 0 (strip
        // t + 1 into the other stage)
#pragma unroll
        for (int d = 0; d < NCOPY; ++d) {
            constexpr int LAST = (SL - 1) * STEPS;
            if (cpos(d, W) < STEPS && LAST + cpos(d, W) == SLOT) {
                issue_copy<ST, W>(L, res, r2, d, smem0);
                __builtin_amdgcn_sched_barrier(0);
            } else if (cpos(d, W) >= STEPS && cpos(d, W) - STEPS == SLOT) {
                issue_copy<NXT, W>(L, res, r1, d, smem0);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        if constexpr (SLOT + 1 < SLOTS)
            slots<ST, P, CUR, W, SLOT + 1>(acc, F, SC, L, res, sm, p, t, r2, r1, smem0);
    }

    template <int ST, int P, int W>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Frag (&F)[2],
                                                 Scales (&SC)[2], const Lane& L, const Res& res,
                                                 lds_char* sm, const GemmParams& p, int t,
                                                 u32 smem0)
    {
        const StripOff r2 = strip_off(p, t + 2);
        const StripOff r1 = strip_off(p, t + 1);
        slots<ST, P, P & 1, W, 0>(acc, F, SC, L, res, sm, p, t, r2, r1, smem0);
    }

    template <int W>
    static __device__ __forceinline__ void main_loop(f32x16 (&acc)[FM][FN], const Lane& L,
                                                     lds_char* sm, const GemmParams& p, int m0,
                                                     int n0, int KT, u32 smem0)
    {
        const Res res = band_res(p, m0, n0);
#pragma unroll
        for (int d = 0; d < JS; ++d)
            issue_chunk<W>(L, res, p, 0, d, smem0);
        {
            // strip 0 whole; of strip 1 the part the first strip's window
            // leaves to strip -1's last step
            const StripOff o0 = strip_off(p, 0), o1 = strip_off(p, 1);
#pragma unroll
            for (int d = 0; d < NCOPY; ++d) {
                issue_copy<0, W>(L, res, o0, d, smem0);
                if (cpos(d, W) < STEPS)
                    issue_copy<1, W>(L, res, o1, d, smem0);
            }
        }
        wait_all_barrier();
        Frag F[2];
        Scales SC[2];
        read_scales<0>(SC[0], L, sm, 0);
#pragma unroll
        for (int i = 0; i < NRD; ++i)
            read_one<0, 0>(F[0], L, sm, i);
        // K % 1024 == 0: whole groups of 4 strips
        for (int t = 0; t < KT; t += 4) {
            strip<0, 0, W>(acc, F, SC, L, res, sm, p, t, smem0);
            strip<1, 1, W>(acc, F, SC, L, res, sm, p, t + 1, smem0);
            strip<0, 2, W>(acc, F, SC, L, res, sm, p, t + 2, smem0);
            strip<1, 3, W>(acc, F, SC, L, res, sm, p, t + 3, smem0);
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
        const TileCoord tc = tile_of(blockIdx.x, p.tiles_m, p.tiles_n, group_of(p, GROUP_M));
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
        case 3:
            main_loop<3>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        case 4:
            main_loop<4 % NW>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        case 5:
            main_loop<5 % NW>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        case 6:
            main_loop<6 % NW>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        default:
            main_loop<7 % NW>(acc, L, sm, p, m0, n0, KT, smem0);
            break;
        }
        if ((p.N & 7) == 0 && ((uintptr_t)p.C & 15) == 0 && NW * WTM * WTN * 2 <= LDS_BYTES) {
            wait_all_barrier();  // every wave's copies landed and reads done
            store_tile_staged<DT_BF16, WTM, WTN, FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN,
                                                        lane, sm + w * (WTM * WTN * 2));
            return;
        }
        mx_store_direct<FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane);
    }
};

template <int AFMT, int BM, int BN, int WGM, int WGN, int GROUP_M>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * 64, WGM * WGN * 64),
                          amdgpu_waves_per_eu(WGM * WGN > 4 ? 2 : 1,
                                              WGM * WGN > 4 ? 2 : 1))) void
gemm_mx2_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    DmaMx2<AFMT, BM, BN, WGM, WGN, GROUP_M>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
