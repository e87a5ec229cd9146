// 2:4 structured-sparse GEMM on the gfx950 sparse matrix instruction.
//
// The sparse GEMM the blog.hotdry.top page names for 2:4 sparsity (its
// monitoring-and-debugging paragraph: skip the dense work): A [M][K] keeps at
// most two values in every group of four consecutive k.  It arrives
// compressed: Ac [M][K/2] (the two kept values of group j at 2j, 2j + 1) and
// Ai [M][K/8] (group j's nibble p0 | p1 << 2 in byte j / 2, low nibble for even
// j).  C[m][n] = sum_j sum_t Ac[m][2j + t] * B[4j + p_t][n], B [K][N] row-major,
// fp32 accumulation, optional ReLU, one rounding to the operand type.
//
// v_smfmac_f32_32x32x32_{bf16,f16} multiplies a 32 x 32 block of A, given as
// 16 kept values per row, by a dense 32 x 32 block of B.  Its lane layout
// (measured on the GPU with an in-bounds probe):
//   * A: lane l supplies row l % 32, kept values of k 16 (l / 32) .. + 15
//     (8 values, 4 groups), and their positions in bits 0..15 of the index
//     operand, 2 bits per value in value order - exactly the 16 bits of Ai
//     for those 4 groups;
//   * B: lane l supplies column l % 32, elements 0..7 = k 8 (l / 32) + 0..7 and
//     8..15 = k 16 + 8 (l / 32) + 0..7 - the dense kernel's fragments of two
//     consecutive 16-k slabs.
// MI355X mapping (the LDS-DMA GEMM's, adapted):
//  * BM x BN x 64 strips (two 32-k steps), four waves in 2 x 2 or eight in
//    2 x 4 (two per SIMD: 256 x 256 tiles, 128 x 64 wave tiles), a 3-stage
//    LDS ring filled by LDS-DMA: Ac rows of 64 bytes (swizzle swz_a), the two
//    metadata dwords of each row as two [BM][4] blocks (dword copies), B as
//    [64 k][BN] (the dense kernel's x-contiguous operand, transposing reads);
//  * per k-step a wave reads per 32-row block one ds_read_b128 of kept values
//    and its metadata dword (shifted by lane half: one ds_read_b32, or with CS
//    one ds_read_b128 of four dwords every second strip), and per 32-column
//    block the two slab fragments of B; one sparse MFMA per block pair;
//  * one barrier per strip after its first MFMA; copies of strip t + 2 into
//    the stage strip t - 1 used, spread over the strip;
//  * CS (K % 256 == 0, 16-byte aligned metadata rows): the metadata of 4
//    strips (32 bytes per row) is copied as one chunk with 16-byte copies
//    (32 rows per copy) into one of two LDS buffers, instead of 4 bytes per
//    row per strip (64 rows, 64 cache lines per copy): the address path
//    spends its cycles per line, and the per-strip copies cost a fifth of the
//    kernel.  Chunk c + 1 is copied during strip 4 c + 1 into the buffer
//    chunk c - 1 used; each strip's barrier waits for every copy, so it has
//    landed by strip 4 c + 2.  The strip's place in its chunk and its stage
//    are compile-time constants (a loop of 12 strips, then 4 or 8): a
//    run-time test would split the strip into branches past which the
//    compiler sinks the MFMAs.
// K % 32 == 0: a strip past K copies zeros (values and B), so whatever
// positions its metadata holds, its products are zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel.h"
#include "tg_kernel_dma.h"
#include "tg_kernel_dma_w4.h"

namespace tg {

typedef __attribute__((ext_vector_type(16))) __bf16 bf16x16;
typedef __attribute__((ext_vector_type(16))) _Float16 f16x16;

template <int DT, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M, bool CS>
struct DmaSp24 {
    static_assert(DT == DT_BF16 || DT == DT_F16, "16-bit operands only");
    static constexpr int BK = 64;  // dense k per strip
    static constexpr int NW = WGM * WGN;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    using OB = DmaOperand<false, BN, WTN, FN, NW, BK>;
    static constexpr int A_STAGE = BM * 64;  // 32 kept values per row per strip
    static constexpr int I_STAGE = BM * 8;   // two metadata dwords per row per strip
    static constexpr int CH = 4;             // strips per metadata chunk (CS)
    static constexpr int I_CHUNK = BM * 32;  // one chunk buffer (CS)
    static constexpr int B_STAGE = OB::STAGE;
    static constexpr int I_REGION = NS * A_STAGE;
    static constexpr int B_REGION = I_REGION + (CS ? 2 * I_CHUNK : NS * I_STAGE);
    static constexpr int LDS_BYTES = B_REGION + NS * B_STAGE;
    static constexpr int JA = A_STAGE / 1024 / NW;   // value copies per wave per strip
    static constexpr int NIC = CS ? 0 : I_STAGE / 256;  // metadata dword copies per strip
    static constexpr int JI = NIC / NW;              // ... per wave
    static constexpr int NCC = CS ? BM / 32 : 0;     // chunk copies per chunk (CS)
    static constexpr int JC = NCC / NW;              // ... per wave
    static constexpr int NCOPY = JA + JI + OB::J;    // copies per wave per strip
    static constexpr int NM = FM * FN;               // MFMAs per 32-k step
    static constexpr int NRD = 2 * FM + 4 * FN;      // LDS reads per 32-k step

    static_assert(NW == 4 || NW == 8, "four or eight waves");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of 32x32 blocks");
    static_assert(JA >= 1 && A_STAGE % (1024 * NW) == 0, "value copies split evenly");
    static_assert(CS ? (JC >= 1 && NCC % NW == 0) : (JI >= 1 && NIC % NW == 0),
                  "metadata copies split evenly");
    static_assert(I_REGION % 1024 == 0, "chunk buffers 1 KiB aligned (the halves are selected by an xor)");
    static_assert(NS == 3, "three stages: the barrier publishes strip t + 1 while t - 1 is free");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    struct Lane {
        u32 a_off[JA];        // value copies: row offset + chunk (kOob past M)
        u32 i_off[CS ? JC : JI];  // metadata copies: row offset + dword, or (CS) row
                                  // offset + 16-byte half of the chunk (kOob past M)
        int a_c;              // chunk this lane copies: dense k 16 a_c .. of the strip,
                              // the same for all JA copies (rows 16 apart share swz_a)
        u32 a_rd[2];          // [k-step]: this lane's 16 bytes of kept values (stage 0, fm 0)
        u32 i_rd;             // this lane's metadata dword of k-step 0 (stage 0, fm 0);
                              // k-step 1's is BM * 4 bytes further.  CS: its row in
                              // chunk buffer 0 (strips 0, 1 of the chunk; 2, 3 at ^ 16)
        int h16;              // 16 * lane half
        typename OB::Lane b;
    };

    typedef __attribute__((ext_vector_type(16))) short s16x16;

    struct Frag {  // one 32-k step
        u32x4 a[FM];
        u32 idx[FM];
        s16x16 b[FN];  // quarters: slab 2q (k 8h ..), two reads; slab 2q + 1 (k 16 + 8h ..)
    };

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn)
    {
        const int K = p.K;
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int row = (w * JA + j) * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz_a(row);
            L.a_off[j] = (m0 + row < p.M) ? (u32)(row * K + c * 16) : kOob;  // K/2 values x 2 B
        }
        if constexpr (CS) {
            // chunk copy g: rows 32 g .., lane l -> row 32 g + l / 2 at LDS 16-byte
            // position l & 1, which holds the row's half (l & 1) ^ bit 3 of the row
#pragma unroll
            for (int j = 0; j < JC; ++j) {
                const int row = (w * JC + j) * 32 + (lane >> 1);
                const int half = (lane & 1) ^ ((row >> 3) & 1);
                L.i_off[j] = (m0 + row < p.M) ? (u32)(row * (K / 8) + half * 16) : kOob;
            }
        } else {
#pragma unroll
            for (int j = 0; j < JI; ++j) {
                const int g = w * JI + j;           // dword copy index: block (g / (BM / 64)), rows ...
                const int blk = g / (BM / 64);      // metadata dword 0 or 1 of the strip
                const int row = (g % (BM / 64)) * 64 + lane;
                L.i_off[j] = (m0 + row < p.M) ? (u32)(row * (K / 8) + blk * 4) : kOob;
            }
        }
        // swz_a depends on row bits 1-3 only, and rows of one lane differ by 16
        L.a_c = (lane & 3) ^ swz_a(lane >> 2);
        const int h = lane >> 5;
        const int ar = wm * WTM + (lane & 31);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            L.a_rd[q] = ar * 64 + (((2 * q + h) ^ swz_a(ar)) << 4);
        }
        L.i_rd = CS ? I_REGION + ar * 32 + (((ar >> 3) & 1) << 4) : I_REGION + ar * 4;
        L.h16 = 16 * h;
        OB::setup(L.b, n0, p.N, p.N, w, lane, wn * WTN, B_REGION, p.B, p.K);
    }

    // Resources of the tile's row band (values, metadata) for all of K, and
    // of B's strip; a strip adds its byte offset to the value and metadata
    // lane offsets.
    struct Res {
        __amdgpu_buffer_rsrc_t a, i;
    };
    struct StripRes {
        typename OB::Strip b;
        u32 ao, io;  // strip byte offsets in a row of values / metadata
        int krem;    // valid dense k within the strip
    };

    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t band(const void* base, int row0,
                                                                  int rows, int row_bytes)
    {
        const uint64_t a = (uint64_t)((const char*)base + (int64_t)row0 * row_bytes);
        const u32 lo = __builtin_amdgcn_readfirstlane((u32)a);
        const u32 hi = __builtin_amdgcn_readfirstlane((u32)(a >> 32));
        const u32 n = __builtin_amdgcn_readfirstlane(clamp_bytes((int64_t)rows * row_bytes));
        return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), n);
    }

    static __device__ __forceinline__ Res band_res(const GemmParams& p, int m0)
    {
        Res r;
        r.a = band(p.A, m0, p.M - m0, p.K);      // K/2 values of 2 bytes per row
        r.i = band(p.As, m0, p.M - m0, p.K / 8);
        return r;
    }

    static __device__ __forceinline__ StripRes strip_res(const GemmParams& p, int n0, int strip)
    {
        const int k0 = strip * BK;
        StripRes r;
        r.b.rs = OB::strip_rsrc(p.B, n0, p.N, p.N, p.K, k0);
        r.b.so = 0u;
        r.ao = (u32)k0;      // k0 / 2 values x 2 bytes
        r.io = (u32)(k0 / 8);
        r.krem = p.K - k0;
        return r;
    }

    // Copy d of wave W into stage ST: values, then metadata, then B.
    template <int ST, int W>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const Res& res,
                                                      const StripRes& r, int d, u32 smem0)
    {
        if (d < JA) {
            dma16(smem0 + ST * A_STAGE + (W * JA + d) * 1024,
                  16 * L.a_c < r.krem ? L.a_off[d] + r.ao : kOob, res.a);
        } else if (d < JA + JI) {
            const int j = d - JA;
            const int g = W * JI + j;
            const int blk = g / (BM / 64);  // metadata dword of the strip: dense k 32 blk ..
            const int rb = g % (BM / 64);
            dma4(smem0 + I_REGION + ST * I_STAGE + blk * BM * 4 + rb * 256,
                 32 * blk < r.krem ? L.i_off[j] + r.io : kOob, res.i);
        } else {
            OB::template copy<ST>(L.b, r.b, r.krem, d - JA - JI, W, smem0 + B_REGION);
        }
    }

    template <int ST, int W>
    static __device__ __forceinline__ void issue_copies(const Lane& L, const Res& res,
                                                        const GemmParams& p, int n0, int strip,
                                                        u32 smem0)
    {
        const StripRes r = strip_res(p, n0, strip);
#pragma unroll
        for (int d = 0; d < NCOPY; ++d)
            issue_copy<ST, W>(L, res, r, d, smem0);
    }

    // Chunk copy j of wave W (CS): the metadata of strips 4 c .. 4 c + 3 into
    // buffer c & 1.  Past K (K % 256 == 0) a chunk copies zeros.
    template <int W>
    static __device__ __forceinline__ void issue_chunk(const Lane& L, const Res& r,
                                                       const GemmParams& p, int c, int j,
                                                       u32 smem0)
    {
        const u32 off = 256 * c < p.K ? L.i_off[j] + (u32)(c * 32) : kOob;
        dma16(smem0 + I_REGION + (u32)(c & 1) * I_CHUNK + (W * JC + j) * 1024, off, r.i);
    }

    // Read i (0 .. NRD-1) of k-step Q of stage ST: values and metadata per
    // row block, then the B fragments (two slabs) per column block.  SP: the
    // strip's place in its metadata chunk and ib the chunk buffer's offset (CS).
    template <int ST, int Q, int SP>
    static __device__ __forceinline__ void read_one(Frag& F, u32x4 (&meta)[FM], const Lane& L,
                                                    lds_char* sm, int i, u32 ib)
    {
        typedef __attribute__((address_space(3))) u32 lds_u32;
        if (i < FM) {
            F.a[i] = *(const lds_u32x4*)(sm + L.a_rd[Q] + ST * A_STAGE + i * 32 * 64);
        } else if (i < 2 * FM) {
            const int fm = i - FM;
            if constexpr (CS) {
                // The row's 16-byte half SP / 2 of the chunk holds the
                // metadata of strips SP & ~1 and SP | 1 (dword 2 (SP % 2) + Q).
                // It is read whole at k-step 0 of an even place and kept for
                // the four k-steps of the pair: rows 32 bytes apart with the
                // half flipped by row bit 3 put a 16-lane pass of 16 rows on
                // 16 different 16-byte bank groups, where dword reads of 32
                // rows met two to a bank.
                if constexpr (Q == 0 && (SP & 1) == 0) {
                    const u32 a = (L.i_rd ^ (u32)((SP >> 1) << 4)) + ib + fm * 32 * 32;
                    meta[fm] = *(const lds_u32x4*)(sm + a);
                }
                F.idx[fm] = meta[fm][2 * (SP & 1) + Q] >> L.h16;
            } else {
                F.idx[fm] = *(const lds_u32*)(sm + L.i_rd + Q * BM * 4 + ST * I_STAGE +
                                              fm * 32 * 4) >>
                            L.h16;
            }
        } else {
            // B: quarter u of column block f holds 4 consecutive k of slab
            // 2 Q + u / 2 (the transposing read of the dense kernel's operand)
            const int j = i - 2 * FM;  // 0 .. 4 FN - 1
            const int f = j >> 2, u = j & 3;
            const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(sm + L.b.rd[f] + ST * B_STAGE +
                             (16 * (2 * Q + (u >> 1)) + 4 * (u & 1)) * (BN * 2)));
            if (u == 0)
                F.b[f].s0123 = v;
            else if (u == 1)
                F.b[f].s4567 = v;
            else if (u == 2)
                F.b[f].s89ab = v;
            else
                F.b[f].scdef = v;
        }
    }

    static __device__ __forceinline__ void mfma_one(f32x16 (&acc)[FM][FN], const Frag& F, int i)
    {
        const int fm = i / FN, fn = i % FN;
        const s16x8 a8 = __builtin_bit_cast(s16x8, F.a[fm]);
        const s16x16 b16 = F.b[fn];
        // first operand: the sparse A block (rows m), second: B (columns n),
        // so the result block is laid out as the other kernels' transposed
        // one: lane l holds column n = l % 32 ... of rows m.  The epilogue
        // below reads it that way.
        if constexpr (DT == DT_BF16)
            acc[fm][fn] = __builtin_amdgcn_smfmac_f32_32x32x32_bf16(
                __builtin_bit_cast(bf16x8, a8), __builtin_bit_cast(bf16x16, b16), acc[fm][fn],
                (int)F.idx[fm], 0, 0);
        else
            acc[fm][fn] = __builtin_amdgcn_smfmac_f32_32x32x32_f16(
                __builtin_bit_cast(f16x8, a8), __builtin_bit_cast(f16x16, b16), acc[fm][fn],
                (int)F.idx[fm], 0, 0);
    }

    // One strip (stage ST) of wave W: k-step 0 with F0, k-step 1 with F1.
    // Slot i of a k-step issues MFMA i, then the reads of the next k-step
    // (k-step 1 of this strip into F1, or k-step 0 of strip t + 1 into F0)
    // spread evenly over the NM slots; slot 0 waits for strip t + 1's copies
    // and barriers; copies of strip t + 2 are spread over the strip.
    // CS: P is the strip's place in its metadata chunk; strip 4 c + 1 also
    // copies chunk c + 1.
    template <int ST, int W, int P = 0>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Frag& F0, Frag& F1,
                                                 u32x4 (&meta)[FM],
                                                 const Lane& L, const Res& res, lds_char* sm,
                                                 const GemmParams& p, int n0, int t, u32 smem0)
    {
        constexpr int NXT = (ST + 1) % NS;
        constexpr int CPY = (ST + NS - 1) % NS;
        constexpr int SLOTS = 2 * NM;
        constexpr int PN = (P + 1) % CH;  // place of strip t + 1
        // chunk buffers of strips t and t + 1
        const u32 ib = CS ? (u32)((t >> 2) & 1) * I_CHUNK : 0u;
        const u32 ibn = CS ? (u32)(((t + 1) >> 2) & 1) * I_CHUNK : 0u;
        StripRes r;
#pragma unroll
        for (int slot = 0; slot < SLOTS; ++slot) {
            const int i = slot % NM;
            const int lo = (i * NRD) / NM, hi = ((i + 1) * NRD) / NM;
            if (slot < NM) {
                mfma_one(acc, F0, i);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rd = lo; rd < hi; ++rd)
                    read_one<ST, 1, P>(F1, meta, L, sm, rd, ib);
            } else {
                mfma_one(acc, F1, i);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int rd = lo; rd < hi; ++rd)
                    read_one<NXT, 0, PN>(F0, meta, L, sm, rd, ibn);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (slot == 0) {
                wait_copies_barrier<0>();
                __builtin_amdgcn_sched_barrier(0);
                r = strip_res(p, n0, t + NS - 1);
            }
            if constexpr (CS && P == 1) {
#pragma unroll
                for (int j = 0; j < JC; ++j) {
                    if (slot == 2 * j + 1) {
                        issue_chunk<W>(L, res, p, (t >> 2) + 1, j, smem0);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                }
            }
#pragma unroll
            for (int d = 0; d < NCOPY; ++d) {
                if (((d * NW + W) * SLOTS) / (NCOPY * NW) == slot) {
                    issue_copy<CPY, W>(L, res, r, d, smem0);
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
        const Res res = band_res(p, m0);
        if constexpr (CS) {
#pragma unroll
            for (int j = 0; j < JC; ++j)
                issue_chunk<W>(L, res, p, 0, j, smem0);
        }
        issue_copies<0, W>(L, res, p, n0, 0, smem0);
        issue_copies<1, W>(L, res, p, n0, 1, smem0);
        wait_copies_barrier<NCOPY>();  // chunk 0 and strip 0 landed and visible
        Frag F0, F1;
        u32x4 meta[FM];  // CS: each row block's metadata for two strips (see read_one)
#pragma unroll
        for (int i = 0; i < NRD; ++i)
            read_one<0, 0, 0>(F0, meta, L, sm, i, 0u);
        if constexpr (CS) {
            // 12 strips (the stage and the place in the chunk both repeat),
            // then the 4 or 8 left (K % 256 == 0)
            int t = 0;
            for (; t + 12 <= KT; t += 12) {
                strip<0, W, 0>(acc, F0, F1, meta, L, res, sm, p, n0, t, smem0);
                strip<1, W, 1>(acc, F0, F1, meta, L, res, sm, p, n0, t + 1, smem0);
                strip<2, W, 2>(acc, F0, F1, meta, L, res, sm, p, n0, t + 2, smem0);
                strip<0, W, 3>(acc, F0, F1, meta, L, res, sm, p, n0, t + 3, smem0);
                strip<1, W, 0>(acc, F0, F1, meta, L, res, sm, p, n0, t + 4, smem0);
                strip<2, W, 1>(acc, F0, F1, meta, L, res, sm, p, n0, t + 5, smem0);
                strip<0, W, 2>(acc, F0, F1, meta, L, res, sm, p, n0, t + 6, smem0);
                strip<1, W, 3>(acc, F0, F1, meta, L, res, sm, p, n0, t + 7, smem0);
                strip<2, W, 0>(acc, F0, F1, meta, L, res, sm, p, n0, t + 8, smem0);
                strip<0, W, 1>(acc, F0, F1, meta, L, res, sm, p, n0, t + 9, smem0);
                strip<1, W, 2>(acc, F0, F1, meta, L, res, sm, p, n0, t + 10, smem0);
                strip<2, W, 3>(acc, F0, F1, meta, L, res, sm, p, n0, t + 11, smem0);
            }
            if (t + 4 <= KT) {
                strip<0, W, 0>(acc, F0, F1, meta, L, res, sm, p, n0, t, smem0);
                strip<1, W, 1>(acc, F0, F1, meta, L, res, sm, p, n0, t + 1, smem0);
                strip<2, W, 2>(acc, F0, F1, meta, L, res, sm, p, n0, t + 2, smem0);
                strip<0, W, 3>(acc, F0, F1, meta, L, res, sm, p, n0, t + 3, smem0);
                if (t + 8 <= KT) {
                    strip<1, W, 0>(acc, F0, F1, meta, L, res, sm, p, n0, t + 4, smem0);
                    strip<2, W, 1>(acc, F0, F1, meta, L, res, sm, p, n0, t + 5, smem0);
                    strip<0, W, 2>(acc, F0, F1, meta, L, res, sm, p, n0, t + 6, smem0);
                    strip<1, W, 3>(acc, F0, F1, meta, L, res, sm, p, n0, t + 7, smem0);
                }
            }
        } else {
            // The strip count is rounded up to a multiple of NS: strips at or
            // past KT copy only zeros, which add exactly nothing.
            for (int t = 0; t < KT; t += NS) {
                strip<0, W>(acc, F0, F1, meta, L, res, sm, p, n0, t, smem0);
                strip<1, W>(acc, F0, F1, meta, L, res, sm, p, n0, t + 1, smem0);
                strip<2, W>(acc, F0, F1, meta, L, res, sm, p, n0, t + 2, smem0);
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
        const int KT = (p.K + BK - 1) / BK;

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
        if (((uintptr_t)p.C & 15) == 0 && NW * WTM * WTN * 2 <= LDS_BYTES) {  // N % 8 == 0 always
            wait_all_barrier();  // every wave's copies landed and reads done
            store_tile_staged_t<DT, WTM, WTN, FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane,
                                                     sm + w * (WTM * WTN * 2));
            return;
        }
        // epilogue: the result block of MFMA (fm, fn) has rows m (A) and
        // columns n (B): lane l holds column n = l % 32 of rows
        // 8 (r / 4) + 4 (l / 32) + r % 4 for element r
        const int lc = lane & 31;
        const int g = lane >> 5;
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = n0 + wn * WTN + fn * 32 + lc;
            if (n >= p.N)
                continue;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int m = m0 + wm * WTM + fm * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                    if (m < p.M) {
                        const float x = acc[fm][fn][r];
                        C[(int64_t)m * p.N + n] =
                            cvt1((p.relu && !(x > 0.0f)) ? 0.0f : x, DT);
                    }
                }
            }
        }
    }
};

// Waves per SIMD: one with four waves (all registers of a lane), two with eight.
template <int WGM, int WGN>
struct Sp24Occ {
    static constexpr int value = WGM * WGN > 4 ? 2 : 1;
};

template <int DT, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M, bool CS = false>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * 64, WGM * WGN * 64),
                          amdgpu_waves_per_eu(Sp24Occ<WGM, WGN>::value,
                                              Sp24Occ<WGM, WGN>::value))) void
gemm_sp24_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    DmaSp24<DT, BM, BN, WGM, WGN, NS, GROUP_M, CS>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
