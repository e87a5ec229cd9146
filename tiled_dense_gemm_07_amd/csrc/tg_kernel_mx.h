// MX-format GEMM: both operands in OCP microscaling blocks, multiplied by the
// gfx950 scaled matrix instruction with no dequantisation step.
//
// The pages' weight-only low-bit GEMM ("WFP4" GEMM in "TileLang架构深度剖析",
// the performance section; "Dequant GEMM" in "使用 Tilelang DSL 开发
// GPU/CPU/加速器高性能内核") with the activations also in a block format:
//   C[m][n] = sum_k a(m, k) w(n, k),
//   a(m, k) = elemA(m, k) * 2^(SA[m][k/32] - 127)   (E2M1 or E4M3 elements),
//   w(n, k) = e2m1(n, k)  * 2^(SW[n][k/32] - 127),
// fp32 accumulation, one rounding to bf16.  v_mfma_scale_f32_32x32x64_f8f6f4
// multiplies 64 k of a 32x32 block per instruction and applies both scales
// itself.  Its lane layout (measured on the GPU with an in-bounds probe):
//   * lane l supplies row (or column) l % 32 and the scale byte of k-block
//     l / 32 of the instruction's 64 k (byte 0 of the scale operand, or the
//     byte op_sel names);
//   * E2M1: lane l's 32 codes are k = 32 (l / 32) + 0 .. 31, low nibble first;
//   * E4M3: lane l's bytes 0..15 are k = 16 (l / 32) + 0 .. 15 and bytes
//     16..31 are k = 32 + 16 (l / 32) + 0 .. 15.
// MI355X mapping (as the other LDS-DMA kernels here):
//  * BM x BN x 128 strips, four waves in a 2 x 2 grid, NS-stage LDS ring filled
//    by LDS-DMA copies: the codes as stored (E2M1: 64 bytes per row per strip,
//    E4M3: 128 bytes) and the four scale bytes of each row (dword copies);
//  * per 64-k step a wave reads, per 32-row block, one ds_read_b128 of E2M1
//    codes or two of E4M3 codes (chunk swizzles keep them conflict-free) and
//    issues one scaled MFMA per block pair;
//  * a row's four scale bytes are read once per strip and shifted per lane
//    half and k-step, so byte 0 of the scale operand is always the block the
//    lane supplies;
//  * scale bytes reach LDS either per strip (one dword per row: 64 rows per
//    copy, each in its own cache line) or, when K % 512 == 0, in chunks of 8
//    strips (32 bytes per row, 16 per lane: 32 rows per copy; 4 strips and 16
//    bytes per row on a three-stage ring), double buffered; the chunks cut
//    the cache-line accesses of the scale copies four- to eightfold, and those
//    accesses, not the bytes, are what the address unit spends its cycles on;
//  * one barrier per strip after its first MFMA publishes strip t + 1 and frees
//    strip t - 1; copies of strip t + NS - 1 are staggered across waves and
//    slots.  K must be a multiple of 128 and the scale rows 4-byte aligned;
//    rows past M or N and strips padded past K copy zeros.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel.h"
#include "tg_kernel_dma.h"
#include "tg_kernel_dma_w4.h"

namespace tg {

typedef __attribute__((ext_vector_type(8))) int i32x8;

enum MxFmt { MX_E4M3 = 0, MX_E2M1 = 4 };  // the instruction's format codes

// Result blocks of one wave stored straight from the accumulators (C rows
// that are not whole 16-byte runs): lane l holds row l % 32 and, for element
// 4 q + e, column 8 q + 4 (l / 32) + e of its 32 x 32 block; ReLU, one
// rounding to bf16.
template <int FM, int FN>
__device__ __forceinline__ void mx_store_direct(const f32x16 (&acc)[FM][FN], const GemmParams& p,
                                                int mw0, int nw0, int lane)
{
    const int lr = lane & 31;
    const int g = lane >> 5;
    uint16_t* C = (uint16_t*)p.C;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int m = mw0 + fm * 32 + lr;
        if (m >= p.M)
            continue;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = nw0 + fn * 32 + 8 * q + 4 * g;
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = acc[fm][fn][4 * q + e];
                    v[e] = (p.relu && !(x > 0.0f)) ? 0.0f : x;
                }
                const int64_t idx = (int64_t)m * p.N + n;
                if (p.c_vec && n + 3 < p.N) {
                    *(u32x2*)(C + idx) =
                        u32x2{pack2(v[0], v[1], DT_BF16), pack2(v[2], v[3], DT_BF16)};
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

template <int AFMT, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M, bool CS>
struct DmaMx {
    static constexpr int BK = 128;
    static constexpr int NW = WGM * WGN;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr bool A8 = AFMT == MX_E4M3;
    static constexpr int A_ROWB = A8 ? 128 : 64;  // code bytes per row per strip
    static constexpr int A_STAGE = BM * A_ROWB;
    static constexpr int W_STAGE = BN * 64;
    // CS: strips per scale chunk (8, or 4 on a three-stage ring, whose LDS
    // has room for 16 bytes per row only), scale bytes per row and chunk, and
    // the lanes and rows one 16-byte chunk copy covers
    static constexpr int CH = CS ? (NS == 3 ? 4 : 8) : 1;
    static constexpr int RB = 4 * CH;
    static constexpr int LPR = CS ? RB / 16 : 1;
    static constexpr int RPC = 64 / LPR;
    static constexpr int SA_STAGE = CS ? BM * RB : BM * 4;  // bytes per scale buffer
    static constexpr int SW_STAGE = CS ? BN * RB : BN * 4;
    static constexpr int NSB = CS ? 2 : NS;                 // scale buffers
    static constexpr int W_REGION = NS * A_STAGE;
    static constexpr int SA_REGION = W_REGION + NS * W_STAGE;
    static constexpr int SW_REGION = SA_REGION + NSB * SA_STAGE;
    static constexpr int LDS_BYTES = SW_REGION + NSB * SW_STAGE;
    static constexpr int JA = A_STAGE / 1024 / NW;
    static constexpr int JW = W_STAGE / 1024 / NW;
    static constexpr int NSA = CS ? 0 : BM * 4 / 256;   // per-strip dword scale copies of A
    static constexpr int NSW = CS ? 0 : BN * 4 / 256;
    static constexpr int NCA = CS ? BM / RPC : 0;       // chunk copies of A scales (CS)
    static constexpr int NCW = CS ? BN / RPC : 0;
    static constexpr int JS = (NCA + NCW) / NW;         // chunk copies per wave
    static constexpr int NM = FM * FN;          // MFMAs per 64-k step
    static constexpr int SLOTS = 2 * NM;        // MFMAs per strip

    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of 32x32 blocks");
    static_assert(JA >= 1 && JW >= 1 && A_STAGE % (1024 * NW) == 0 && W_STAGE % (1024 * NW) == 0,
                  "strips split into whole 1 KiB copies per wave");
    static_assert(CS || (NSA >= 1 && NSA <= NW && NSW >= 1 && NSW <= NW),
                  "scale copies: one per wave at most");
    static_assert(!CS || ((NCA + NCW) % NW == 0 && JS >= 1), "chunk copies split evenly");
    static_assert(NS == 4 || NS == 3, "three or four stages");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(SA_REGION % 32 == 0 && SW_REGION % 32 == 0 && SA_STAGE % 32 == 0,
                  "scale regions 32-byte aligned (the chunk halves are selected by an xor)");

    template <int W>
    struct Copies {
        static constexpr int N = JA + JW + (W < NSA ? 1 : 0) + (W < NSW ? 1 : 0);
        static constexpr int AHEAD = (NS - 3) * N;
    };
    static constexpr int NCMAX = JA + JW + (CS ? 0 : 2);

    struct Lane {
        u32 a_off[JA];
        u32 w_off[JW];
        u32 sa_off, sw_off;       // per-strip scale copies (!CS)
        u32 s_off[CS ? JS : 1];   // chunk copies (CS): row offset + 16-byte half
        u32 s_half[CS ? JS : 1];  //   and that half (0, 1; always 0 for 4-strip chunks)
        u32 a_rd[2][A8 ? 2 : 1];  // [k-step][part]: code chunks of this lane (stage 0, fm 0)
        u32 w_rd[2];              // [k-step] (stage 0, fn 0)
        u32 sa_rd, sw_rd;         // this lane's row of scale bytes (buffer 0, block 0;
                                  // 8-strip chunks: strips 0-3, strips 4-7 at ^ 16)
        u32 sh[2];                // [k-step]: 8 * lane half + 16 * k-step, the shift that
                                  // brings the lane's scale byte to byte 0
    };

    struct Frag {  // one 64-k step
        u32x4 a[FM][A8 ? 2 : 1];
        u32x4 w[FN];
    };
    struct Scales {  // one strip: a row's four scale bytes per block, as read
        u32 a[FM];
        u32 w[FN];
    };

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn)
    {
        const int K = p.K;
        const int arow_b = A8 ? K : K / 2;  // code bytes per stored A row
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            if constexpr (A8) {
                const int row = (w * JA + j) * 8 + (lane >> 3);
                const int c = (lane & 7) ^ swz8(row);
                L.a_off[j] = (m0 + row < p.M) ? (u32)(row * arow_b + c * 16) : kOob;
            } else {
                const int row = (w * JA + j) * 16 + (lane >> 2);
                const int c = (lane & 3) ^ swz_a(row);
                L.a_off[j] = (m0 + row < p.M) ? (u32)(row * arow_b + c * 16) : kOob;
            }
        }
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int row = (w * JW + j) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz_a(row);
            L.w_off[j] = (n0 + row < p.N) ? (u32)(row * (K / 2) + c * 16) : kOob;
        }
        {
            const int row = w * 64 + lane;
            L.sa_off = (w < NSA && m0 + row < p.M) ? (u32)(row * (K / 32)) : kOob;
            L.sw_off = (w < NSW && n0 + row < p.N) ? (u32)(row * (K / 32)) : kOob;
        }
        if constexpr (CS) {
            // chunk copy g of 8-strip chunks: 32 rows x 32 bytes, lane l -> row
            // g' * 32 + l / 2 at LDS 16-byte position l & 1, which holds the
            // row's half (l & 1) ^ bit 3 of the row (two-way bank spread for the
            // reads); of 4-strip chunks: 64 rows x 16 bytes, lane l -> row
            // g' * 64 + l
#pragma unroll
            for (int d = 0; d < JS; ++d) {
                const int g = w * JS + d;
                const bool isa = g < NCA;
                const int row = (isa ? g : g - NCA) * RPC + lane / LPR;
                const int half = LPR == 2 ? (lane & 1) ^ ((row >> 3) & 1) : 0;
                const bool ok = isa ? (m0 + row < p.M) : (n0 + row < p.N);
                L.s_off[d] = ok ? (u32)(row * (K / 32) + half * 16) : kOob;
                L.s_half[d] = (u32)half;
            }
        }
        const int h = lane >> 5;
        const int ar = wm * WTM + (lane & 31);
        const int nr = wn * WTN + (lane & 31);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            if constexpr (A8) {
                // bytes 0..15: k = 64 q + 16 h; bytes 16..31: k = 64 q + 32 + 16 h
                L.a_rd[q][0] = ar * A_ROWB + (((4 * q + h) ^ swz8(ar)) << 4);
                L.a_rd[q][1] = ar * A_ROWB + (((4 * q + 2 + h) ^ swz8(ar)) << 4);
            } else {
                // 32 codes: k = 64 q + 32 h
                L.a_rd[q][0] = ar * A_ROWB + (((2 * q + h) ^ swz_a(ar)) << 4);
            }
            L.w_rd[q] = W_REGION + nr * 64 + (((2 * q + h) ^ swz_a(nr)) << 4);
        }
        if constexpr (CS && CH == 8) {
            const int xa = (ar >> 3) & 1, xw = (nr >> 3) & 1;
            L.sa_rd = SA_REGION + ar * 32 + (xa << 4);
            L.sw_rd = SW_REGION + nr * 32 + (xw << 4);
        } else if constexpr (CS) {
            L.sa_rd = SA_REGION + ar * 16;
            L.sw_rd = SW_REGION + nr * 16;
        } else {
            L.sa_rd = SA_REGION + ar * 4;
            L.sw_rd = SW_REGION + nr * 4;
        }
        L.sh[0] = 8 * h;
        L.sh[1] = 8 * h + 16;
    }

    // One buffer resource per array for the workgroup's whole row band (all
    // of K); a strip adds its byte offset to the lane offsets.  Offsets of
    // rows past M or N are kOob and stay out of range after the addition; so
    // do the offsets of strips past K.  (Per-strip resources would cost
    // scalar registers this kernel does not have to spare.)
    struct Res {
        __amdgpu_buffer_rsrc_t a, w, sa, sw;
    };
    struct StripOff {
        u32 a, w, s;  // byte offsets of strip t in a row of A codes, W codes, scales
        bool valid;
    };

    // Resource of `rows` rows of `row_bytes` bytes from base + row0 * row_bytes.
    // The copies take it as a scalar operand; the 64-bit range arithmetic may
    // be done on the vector ALU, so its parts are read back as wave-uniform
    // scalars explicitly.
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t band(const void* base, int row0,
                                                                  int rows, int row_bytes)
    {
        const uint64_t a = (uint64_t)((const char*)base + (int64_t)row0 * row_bytes);
        const u32 lo = __builtin_amdgcn_readfirstlane((u32)a);
        const u32 hi = __builtin_amdgcn_readfirstlane((u32)(a >> 32));
        const u32 n = __builtin_amdgcn_readfirstlane(clamp_bytes((int64_t)rows * row_bytes));
        return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), n);
    }

    static __device__ __forceinline__ Res band_res(const GemmParams& p, int m0, int n0)
    {
        const int K = p.K;
        Res r;
        r.a = band(p.A, m0, p.M - m0, A8 ? K : K / 2);
        r.w = band(p.B, n0, p.N - n0, K / 2);
        r.sa = band(p.As, m0, p.M - m0, K / 32);
        r.sw = band(p.Bs, n0, p.N - n0, K / 32);
        return r;
    }

    static __device__ __forceinline__ StripOff strip_off(const GemmParams& p, int strip)
    {
        const int k0 = strip * BK;
        StripOff o;
        o.valid = k0 < p.K;
        o.a = (u32)(A8 ? k0 : k0 / 2);
        o.w = (u32)(k0 / 2);
        o.s = (u32)(k0 / 32);
        return o;
    }

    // Copy d of wave W for strip offsets o into stage ST.
    template <int ST, int W>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const Res& r,
                                                      const StripOff& o, int d, u32 smem0)
    {
        if (d < JA)
            dma16(smem0 + ST * A_STAGE + (W * JA + d) * 1024, o.valid ? L.a_off[d] + o.a : kOob,
                  r.a);
        else if (d < JA + JW)
            dma16(smem0 + W_REGION + ST * W_STAGE + (W * JW + d - JA) * 1024,
                  o.valid ? L.w_off[d - JA] + o.w : kOob, r.w);
        else if (W < NSA && d == JA + JW)
            dma4(smem0 + SA_REGION + ST * SA_STAGE + W * 256, o.valid ? L.sa_off + o.s : kOob,
                 r.sa);
        else
            dma4(smem0 + SW_REGION + ST * SW_STAGE + W * 256, o.valid ? L.sw_off + o.s : kOob,
                 r.sw);
    }

    // Chunk copies (CS) of wave W: the scale bytes of strips CH c .. CH c +
    // CH - 1 into buffer c & 1.  A lane's 16 bytes (four strips) are inside its
    // row or past its end as a whole (K % 512 == 0); past the end they read as
    // zeros.
    template <int W>
    static __device__ __forceinline__ void issue_chunk(const Lane& L, const Res& r,
                                                       const GemmParams& p, int c, int d,
                                                       u32 smem0)
    {
        const int g = W * JS + d;
        const u32 buf = (u32)(c & 1);
        const bool ok = (u32)(c * (CH / 4)) + L.s_half[d] < (u32)(p.K / 512);
        const u32 off = ok ? L.s_off[d] + (u32)(c * RB) : kOob;
        if (g < NCA)
            dma16(smem0 + SA_REGION + buf * SA_STAGE + g * 1024, off, r.sa);
        else
            dma16(smem0 + SW_REGION + buf * SW_STAGE + (g - NCA) * 1024, off, r.sw);
    }

    template <int ST, int W>
    static __device__ __forceinline__ void issue_copies(const Lane& L, const Res& r,
                                                        const GemmParams& p, int strip, u32 smem0)
    {
        const StripOff o = strip_off(p, strip);
#pragma unroll
        for (int d = 0; d < Copies<W>::N; ++d)
            issue_copy<ST, W>(L, r, o, d, smem0);
    }

    // LDS reads of k-step Q of stage ST: A blocks, then W blocks.
    static constexpr int NRD_A = FM * (A8 ? 2 : 1);
    static constexpr int NRD = NRD_A + FN;

    template <int ST, int Q>
    static __device__ __forceinline__ void read_one(Frag& F, const Lane& L, lds_char* sm, int i)
    {
        if (i < NRD_A) {
            const int fm = A8 ? (i >> 1) : i, part = A8 ? (i & 1) : 0;
            F.a[fm][part] = *(const lds_u32x4*)(sm + L.a_rd[Q][part] + ST * A_STAGE +
                                                fm * 32 * A_ROWB);
        } else {
            const int fn = i - NRD_A;
            F.w[fn] = *(const lds_u32x4*)(sm + L.w_rd[Q] + ST * W_STAGE + fn * 32 * 64);
        }
    }

    // Scale bytes of strip u (SL = u % 4 at compile time).
    template <int SL>
    static __device__ __forceinline__ void read_scales(Scales& S, const Lane& L, lds_char* sm,
                                                       int u)
    {
        typedef __attribute__((address_space(3))) u32 lds_u32;
        u32 ra, rw;
        if constexpr (CS && CH == 8) {
            // strips 4-7 of the chunk: the other 16-byte half of the row (the
            // regions and rows are 32-byte aligned, so an xor selects it)
            const u32 hi = (u32)(u & 4) << 2;
            const u32 buf = (u32)((u >> 3) & 1);
            ra = (L.sa_rd ^ hi) + buf * SA_STAGE + SL * 4;
            rw = (L.sw_rd ^ hi) + buf * SW_STAGE + SL * 4;
        } else if constexpr (CS) {
            const u32 buf = (u32)((u >> 2) & 1);
            ra = L.sa_rd + buf * SA_STAGE + SL * 4;
            rw = L.sw_rd + buf * SW_STAGE + SL * 4;
        } else {
            ra = L.sa_rd + SL * SA_STAGE;
            rw = L.sw_rd + SL * SW_STAGE;
        }
        constexpr int RA = CS ? RB : 4;  // LDS bytes per scale row
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            S.a[fm] = *(const lds_u32*)(sm + ra + fm * 32 * RA);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            S.w[fn] = *(const lds_u32*)(sm + rw + fn * 32 * RA);
    }

    // MFMA i of k-step Q.  The scale words are shifted here, at their first
    // use, so the wait for their LDS read falls a strip after it was issued.
    template <int Q>
    static __device__ __forceinline__ void mfma_one(f32x16 (&acc)[FM][FN], const Frag& F,
                                                    const Scales& S, const Lane& L, int i)
    {
        const int fm = i / FN, fn = i % FN;
        const u32x4 wv = F.w[fn];
        const i32x8 wop = {(int)wv[0], (int)wv[1], (int)wv[2], (int)wv[3], 0, 0, 0, 0};
        i32x8 aop;
        if constexpr (A8) {
            const u32x4 lo = F.a[fm][0], hi = F.a[fm][A8 ? 1 : 0];  // A8: two parts
            aop = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                        (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        } else {
            const u32x4 lo = F.a[fm][0];
            aop = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], 0, 0, 0, 0};
        }
        // first operand: weights (rows n of the result block), second:
        // activations (columns m); scale byte 0 of each
        acc[fm][fn] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            wop, aop, acc[fm][fn], MX_E2M1, AFMT, 0, (int)(S.w[fn] >> L.sh[Q]), 0,
            (int)(S.a[fm] >> L.sh[Q]));
    }

    // One strip (stage ST) of wave W: k-step 0 with fragments F0, then k-step 1
    // with F1.  Slot 0 waits for strip t + 1's copies and barriers; k-step 0's
    // slots read k-step 1 into F1; k-step 1's slots read strip t + 1's scales
    // (into SC[(ST + 1) & 1]) and k-step 0 (into F0); copies of strip
    // t + NS - 1 are staggered over the slots.  CS: strip CH c + 1 also copies
    // scale chunk c + 1 (into the buffer chunk c - 1 used, whose last reads
    // were before strip CH c - 1).  On four stages the wait of strip CH c + 2
    // leaves those copies in flight too, and chunk c + 1 has landed by strip
    // CH c + 3; on three stages every strip's wait takes all copies, so it has
    // landed by strip CH c + 2.  P is
    // the strip's place in its chunk (CS) as a compile-time constant: a
    // run-time test there would split the strip into branches, and the
    // compiler then sinks the MFMAs of whole strips past them, away from the
    // copies and reads they are meant to hide.
    template <int ST, int CUR, int W, int P = 0>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Frag& F0, Frag& F1,
                                                 Scales (&SC)[2], const Lane& L, const Res& res,
                                                 lds_char* sm, const GemmParams& p, int t,
                                                 u32 smem0)
    {
        constexpr int NXT = (ST + 1) % NS;
        constexpr int CPY = (ST + NS - 1) % NS;
        // scale slot of strip t + 1: its position in the chunk (CS, NS == 4)
        // or its stage
        constexpr int SNX = CS ? (P + 1) & 3 : (ST + 1) % NS;
        constexpr int STEPS = NM > NRD ? NM : NRD;
        StripOff o;
#pragma unroll
        for (int slot = 0; slot < 2 * STEPS; ++slot) {
            const int i = slot % STEPS;
            if (slot < STEPS) {
                if (i < NM) {
                    mfma_one<0>(acc, F0, SC[CUR], L, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (i < NRD) {
                    read_one<ST, 1>(F1, L, sm, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                if (i < NM) {
                    mfma_one<1>(acc, F1, SC[CUR], L, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (i == 0) {
                    read_scales<SNX>(SC[CUR ^ 1], L, sm, t + 1);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (i < NRD) {
                    read_one<NXT, 0>(F0, L, sm, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (slot == 0) {
                if constexpr (CS && NS == 4 && P == 2)
                    wait_copies_barrier<Copies<W>::AHEAD + JS>();
                else
                    wait_copies_barrier<Copies<W>::AHEAD>();
                __builtin_amdgcn_sched_barrier(0);
                o = strip_off(p, t + NS - 1);
            }
            if constexpr (CS && P == 1) {
#pragma unroll
                for (int d = 0; d < JS; ++d) {
                    if (slot == 2 * d + 1) {
                        issue_chunk<W>(L, res, p, t / CH + 1, d, smem0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < Copies<W>::N; ++d) {
                if (((d * NW + W) * 2 * STEPS) / (NCMAX * NW) == slot) {
                    issue_copy<CPY, W>(L, res, o, d, smem0);
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
        const Res res = band_res(p, m0, n0);
        if constexpr (CS) {
#pragma unroll
            for (int d = 0; d < JS; ++d)
                issue_chunk<W>(L, res, p, 0, d, smem0);
        }
        // strips 0 .. NS-2 into stages 0 .. NS-2
        issue_copies<0, W>(L, res, p, 0, smem0);
        issue_copies<1, W>(L, res, p, 1, smem0);
        if constexpr (NS > 3)
            issue_copies<2, W>(L, res, p, 2, smem0);
        wait_copies_barrier<(NS - 2) * Copies<W>::N>();
        Frag F0, F1;
        Scales SC[2];
        read_scales<0>(SC[0], L, sm, 0);
#pragma unroll
        for (int i = 0; i < NRD; ++i)
            read_one<0, 0>(F0, L, sm, i);
        // The strip count is rounded up to a whole number of loop bodies (NS
        // strips, 6 for NS == 3 so that the scale registers alternate per
        // strip): strips at or past KT copy only zeros, which add nothing.
        if constexpr (CS && NS == 3) {
            // 12 strips (stage, place in the 4-strip chunk and scale register
            // set all repeat), then the 4 or 8 left (K % 512 == 0)
            int t = 0;
            for (; t + 12 <= KT; t += 12) {
                strip<0, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t, smem0);
                strip<1, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 1, smem0);
                strip<2, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 2, smem0);
                strip<0, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 3, smem0);
                strip<1, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t + 4, smem0);
                strip<2, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 5, smem0);
                strip<0, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 6, smem0);
                strip<1, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 7, smem0);
                strip<2, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t + 8, smem0);
                strip<0, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 9, smem0);
                strip<1, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 10, smem0);
                strip<2, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 11, smem0);
            }
            if (t + 4 <= KT) {
                strip<0, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t, smem0);
                strip<1, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 1, smem0);
                strip<2, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 2, smem0);
                strip<0, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 3, smem0);
                if (t + 8 <= KT) {
                    strip<1, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t + 4, smem0);
                    strip<2, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 5, smem0);
                    strip<0, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 6, smem0);
                    strip<1, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 7, smem0);
                }
            }
        } else if constexpr (CS) {
            // whole chunks of 8 strips, then 4 (K % 512 == 0)
            int t = 0;
            for (; t + 8 <= KT; t += 8) {
                strip<0, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t, smem0);
                strip<1, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 1, smem0);
                strip<2, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 2, smem0);
                strip<3, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 3, smem0);
                strip<0, 0, W, 4>(acc, F0, F1, SC, L, res, sm, p, t + 4, smem0);
                strip<1, 1, W, 5>(acc, F0, F1, SC, L, res, sm, p, t + 5, smem0);
                strip<2, 0, W, 6>(acc, F0, F1, SC, L, res, sm, p, t + 6, smem0);
                strip<3, 1, W, 7>(acc, F0, F1, SC, L, res, sm, p, t + 7, smem0);
            }
            if (t < KT) {
                strip<0, 0, W, 0>(acc, F0, F1, SC, L, res, sm, p, t, smem0);
                strip<1, 1, W, 1>(acc, F0, F1, SC, L, res, sm, p, t + 1, smem0);
                strip<2, 0, W, 2>(acc, F0, F1, SC, L, res, sm, p, t + 2, smem0);
                strip<3, 1, W, 3>(acc, F0, F1, SC, L, res, sm, p, t + 3, smem0);
            }
        } else if constexpr (NS == 4) {
            for (int t = 0; t < KT; t += 4) {
                strip<0, 0, W>(acc, F0, F1, SC, L, res, sm, p, t, smem0);
                strip<1, 1, W>(acc, F0, F1, SC, L, res, sm, p, t + 1, smem0);
                strip<2, 0, W>(acc, F0, F1, SC, L, res, sm, p, t + 2, smem0);
                strip<3, 1, W>(acc, F0, F1, SC, L, res, sm, p, t + 3, smem0);
            }
        } else {
            for (int t = 0; t < KT; t += 6) {
                strip<0, 0, W>(acc, F0, F1, SC, L, res, sm, p, t, smem0);
                strip<1, 1, W>(acc, F0, F1, SC, L, res, sm, p, t + 1, smem0);
                strip<2, 0, W>(acc, F0, F1, SC, L, res, sm, p, t + 2, smem0);
                strip<0, 1, W>(acc, F0, F1, SC, L, res, sm, p, t + 3, smem0);
                strip<1, 0, W>(acc, F0, F1, SC, L, res, sm, p, t + 4, smem0);
                strip<2, 1, W>(acc, F0, F1, SC, L, res, sm, p, t + 5, smem0);
            }
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

// Waves per SIMD: two with eight waves or for the small E2M1 tile (its
// fragments fit in 128 registers), else one.
template <int AFMT, int BM, int BN, int NW>
struct MxOcc {
    static constexpr int value = (NW > 4 || (AFMT == MX_E2M1 && BM * BN <= 128 * 128)) ? 2 : 1;
};

template <int AFMT, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M, bool CS>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * 64, WGM * WGN * 64),
                          amdgpu_waves_per_eu(MxOcc<AFMT, BM, BN, WGM * WGN>::value,
                                              MxOcc<AFMT, BM, BN, WGM * WGN>::value))) void
gemm_mx_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    DmaMx<AFMT, BM, BN, WGM, WGN, NS, GROUP_M, CS>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
