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
//  * BM x BN x BK strips (BK = 128 or 256), WGM x WGN x KS waves (four or
//    eight), an NS-stage LDS ring filled by LDS-DMA copies (no VGPR
//    staging): A as [BM][BK] bf16 (256- or 512-byte rows), the packed codes as
//    [BN][BK / 2 bytes] and the scale bytes as [BN][4] (BK = 128; or SB
//    strips at a time, below).  The
//    codes stay packed in LDS (a quarter of the bf16 bytes); each wave expands
//    its own B fragments in registers (v_cvt_scalef32_pk_bf16_fp4, exact)
//    right before the MFMA that consumes them.  One buffer resource per operand
//    covers the tile's row band for the whole K; a strip adds its byte offset
//    to the lane offsets.
//  * Inside a strip the k order is permuted the same way on both operands:
//    MFMA slab s (0 .. BK/16 - 1) takes, in lane half h, k = (BK/2) h + 8 s
//    .. + 7.  A lane's codes for the whole strip are then one contiguous run
//    of its row (BK/4 bytes: 32 or 64), and its A fragment of slab s is
//    16-byte chunk (BK/16) h + s.
//  * Chunk swizzles keep the fragment reads free of bank conflicts: A chunks
//    are XORed with row & 15, code chunks with the 64- or 128-byte-row
//    swizzle.
//  * K-slice variant (KS = 2 or 4): the waves form KS groups of
//    WGM x WGN waves that all cover the whole tile; group q multiplies slabs
//    q (BK/16)/KS .. of every strip (a lane's codes are then a half or a
//    quarter of the run), so each A fragment feeds more MFMAs and every
//    code is expanded once per tile instead of once per wave row.  The KS
//    partial accumulators are added through LDS after the main loop in group
//    order 0, 1, ..., KS-1, and group q stores its share of the tile.
//  * Scale blocks (SB > 1): the scale bytes of SB strips (64 bytes per
//    weight row: SB = 16 strips of 128 k or 8 of 256 k) are copied together
//    with 16-byte copies into one of two LDS buffers, in the middle of the
//    previous block, so a strip needs no 4-byte-per-lane scale copies (a
//    third of the cache-line requests for 2% of the bytes).  Needs
//    K % 512 == 0 and 16-byte aligned scale rows; 16-byte pieces past a
//    row's end copy zeros.  A row's 16-byte chunk c sits at position
//    c ^ ((row >> 2) & 3).  Each strip a lane reads the whole 16-byte chunk
//    that holds its bytes (ds_read_b128, which serves 16 lanes at a time:
//    16 consecutive rows hit 16 distinct chunk positions of the banks) and
//    picks its bytes in registers; a one- or two-byte read by all 32 rows of
//    a wave would meet rows 16 apart on the same bank.
//  * Strips are whole (K % BK == 0; other K use the register-staged kernel);
//    out-of-range rows (m >= M, n >= N) and the strips past K copy zeros.
//    The barrier/copy schedule is the one of the 16-bit DMA kernel: one
//    barrier per strip after its first MFMA, copies of strip t + NS - 1
//    staggered across the waves and MFMA slots (on a three-stage ring over
//    the first half of the slots, so the last copy still has half a strip
//    before the barrier that waits for it).  The two code register sets
//    alternate per strip; with an odd ring the loop covers 2 NS strips per
//    iteration and the last strips run one by one.
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

// The same with a wave-uniform byte offset added to every lane's address.
__device__ __forceinline__ void dma4_so(u32 lds, u32 voff, __amdgpu_buffer_rsrc_t rs, u32 soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds" ::"s"(lds),
                 "v"(voff), "s"(rs), "s"(soff)
                 : "memory");
}

template <int BM, int BN, int WGM, int WGN, int NS, int GROUP_M, int KS = 1, int SB = 1,
          int BK_ = 128>
struct DmaW4 {
    static constexpr int BK = BK_;
    static constexpr int NSL = BK / 16;     // MFMA slabs of a strip
    static constexpr int NWG = WGM * WGN;   // waves of one k-slice group
    static constexpr int NW = NWG * KS;     // waves of the workgroup
    static constexpr int SPW = NSL / KS;    // MFMA slabs of a strip per wave
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr int NM = FM * FN;      // MFMAs per slab
    static constexpr int SLOTS = SPW * NM;  // MFMAs per strip and wave
    static constexpr int NB = FM * FN;      // 32 x 32 blocks of a wave tile
    static constexpr int A_STAGE = BM * BK * 2;
    static constexpr int W_STAGE = BN * BK / 2;
    static constexpr int S_STAGE = BN * 4;       // one strip's scale bytes (SB == 1, BK == 128)
    static constexpr int SROW = 64;              // SB > 1: a row's bytes of one scale block
    static constexpr int S_BUF = BN * SROW;      // one block of SB strips' scale bytes
    static constexpr int W_REGION = NS * A_STAGE;
    static constexpr int S_REGION = W_REGION + NS * W_STAGE;
    static constexpr int RING_BYTES = S_REGION + (SB == 1 ? NS * S_STAGE : 2 * S_BUF);
    // k-slice groups add their partial tiles through LDS: one 4 KiB region
    // per wave and block, reusing the ring after the main loop
    static constexpr int RED_BYTES = KS > 1 ? NW * NB * 4096 : 0;
    static constexpr int LDS_BYTES = RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;
    static constexpr int JA = A_STAGE / 1024 / NW;  // A copies per wave per strip
    static constexpr int JW = W_STAGE / 1024 / NW;  // code copies per wave per strip
    static constexpr int NSC = SB == 1 ? S_STAGE / 256 : 0;  // scale copies per strip (waves 0 .. NSC-1)
    static constexpr int JS = SB == 1 ? 0 : S_BUF / 1024 / NW;  // 16-byte scale-block copies per wave
    static constexpr int SCPR = SROW / 16;          // 16-byte chunks of a row's block
    static constexpr int CPRA = BK * 2 / 16;        // 16-byte chunks of an A row
    static constexpr int CPRW = BK / 2 / 16;        // 16-byte chunks of a code row
    static constexpr int LB = SPW * 4;              // a lane's code bytes per strip and block
    static constexpr int NWR = LB >= 16 ? LB / 16 : 1;  // its 16-byte code reads (or one 8-byte)
    static constexpr int SPL = SPW >= 4 ? SPW / 4 : 1;  // its scale bytes per strip and block

    static_assert(BK == 128 || BK == 256, "128- or 256-k strips");
    static_assert(NW == 4 || NW == 8, "one or two waves per SIMD");
    static_assert(KS == 1 || KS == 2 || KS == 4, "k-slice groups split the slabs of a strip");
    static_assert(SPW >= 2 && LB <= 64, "a lane's codes: 8 to 64 contiguous bytes");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of 32x32 blocks");
    static_assert(JA >= 1 && JW >= 1 && A_STAGE % (1024 * NW) == 0 && W_STAGE % (1024 * NW) == 0,
                  "strips split into whole 1 KiB copies per wave");
    static_assert(SB > 1 || (BK == 128 && NSC >= 1 && NSC <= NW && S_STAGE % 256 == 0),
                  "per-strip scale copies: 128-k strips, one copy per wave at most");
    static_assert(SB == 1 || (SB * BK / 32 == SROW && JS >= 1 && S_BUF % (1024 * NW) == 0),
                  "scale blocks of 64 bytes per row, split into whole 1 KiB copies per wave");
    static_assert(NS >= 3 && (NS % 2 == 0 || BK == 256),
                  "three stages (256-k strips) or an even ring of four or more");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    // A scale block is issued in the middle of the block before it (strip
    // t % SB == SB / 2) and first read SB / 2 strips later; the per-strip wait
    // leaves (NS - 3) strips of copies in flight, so it covers the block only
    // if at least that many strips' copies were issued after it.
    static_assert(SB == 1 || NS <= SB / 2 + 2,
                  "the strip wait must cover the scale block issued half a block earlier");
    static_assert(SB == 1 || BK == 256 || NS == 4,
                  "128-k strips with scale blocks: four stages (a strip's place in its block "
                  "chunk is its stage)");

    template <int W>
    struct Copies {
        static constexpr int N = JA + JW + (W < NSC ? 1 : 0);
        static constexpr int AHEAD = (NS - 3) * N;
    };
    static constexpr int NCMAX = JA + JW + (SB == 1 ? 1 : 0);
    // MFMA slots over which a strip's copies are staggered: all of them on
    // rings of four or more stages, the first half on three
    static constexpr int CSPAN = NS == 3 ? SLOTS / 2 : SLOTS;

    struct Lane {
        u32 a_off[JA];
        u32 w_off[JW];
        u32 s_off;
        u32 sb_off[JS > 0 ? JS : 1];  // SB > 1: this lane's 16 scale bytes of block 0
        u32 sb_c[JS > 0 ? JS : 1];    // and their byte position within a row's block
        u32 s_sw;                     // SB > 1: this lane's row's chunk swizzle, in bytes
        u32 a_rd[SPW];  // A fragment read offset of the wave's slab j (stage 0, fm 0)
        u32 w_rd[NWR];  // this lane's code pieces (stage 0, fn 0)
        u32 s_rd;       // SB == 1: scale byte(s) of this lane's row (stage 0, fn 0);
                        // SB > 1: the row's start in a block buffer
        __amdgpu_buffer_rsrc_t ra, rw, rs;  // row bands of A, codes, scales
    };

    struct Regs {
        u32 code[FN][SPW];  // 8 codes per slab and n-block
        u32 sc[FN];         // SB == 1: the lane's scale byte(s) of the strip
        u32x4 scw[SB > 1 ? FN : 1];  // SB > 1: the block chunk holding them
    };

    static __device__ __forceinline__ int swz16(int r) { return r & 15; }
    static __device__ __forceinline__ int swzw(int r) { return BK == 128 ? swz_a(r) : swz8(r); }

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn, int q)
    {
        const int K = p.K;
        L.ra = band(p.A, m0, p.M - m0, K * 2);
        L.rw = band(p.B, n0, p.N - n0, K / 2);
        L.rs = band(p.Bs, n0, p.N - n0, K / 32);
        // a 1 KiB copy covers 64 / CPRA rows of A and 64 / CPRW rows of codes
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int row = (w * JA + j) * (64 / CPRA) + lane / CPRA;
            const int c = (lane % CPRA) ^ swz16(row);
            L.a_off[j] = (m0 + row < p.M) ? (u32)(row * K + c * 8) * 2u : kOob;
        }
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int row = (w * JW + j) * (64 / CPRW) + lane / CPRW;
            const int c = (lane % CPRW) ^ swzw(row);
            L.w_off[j] = (n0 + row < p.N) ? (u32)(row * (K / 2) + c * 16) : kOob;
        }
        {
            const int row = w * 64 + lane;
            L.s_off = (w < NSC && n0 + row < p.N) ? (u32)(row * (K / 32)) : kOob;
        }
        if constexpr (SB > 1) {
#pragma unroll
            for (int i = 0; i < JS; ++i) {
                const int idx = (w * JS + i) * 64 + lane;
                const int row = idx / SCPR;
                const int c = (idx % SCPR) ^ ((row >> 2) & (SCPR - 1));  // global chunk
                L.sb_c[i] = (u32)c * 16u;
                L.sb_off[i] = n0 + row < p.N ? (u32)(row * (K / 32) + c * 16) : kOob;
            }
        }
        const int h = lane >> 5;
        const int ar = wm * WTM + (lane & 31);
#pragma unroll
        for (int j = 0; j < SPW; ++j)
            L.a_rd[j] = ar * (BK * 2) + ((((CPRA / 2) * h + q * SPW + j) ^ swz16(ar)) << 4);
        const int nr = wn * WTN + (lane & 31);
        L.s_sw = SB > 1 ? (u32)(((nr >> 2) & (SCPR - 1)) << 4) : 0u;
        // the lane's codes: bytes (BK/4) h + q LB .. + LB of its row
        const int cb = (BK / 4) * h + q * LB;
#pragma unroll
        for (int i = 0; i < NWR; ++i)
            L.w_rd[i] = W_REGION + nr * (BK / 2) + ((((cb >> 4) + i) ^ swzw(nr)) << 4) + (cb & 15);
        if constexpr (SB == 1)
            L.s_rd = S_REGION + nr * 4 + cb / 16;  // its first 32-k block: (BK/4 h + q LB) / 16
        else
            L.s_rd = S_REGION + nr * SROW;
    }

    // Byte offsets of one strip inside a row of A, of the codes and of the
    // scale bytes.  The buffer resources cover the tile's whole row bands
    // (set up once, in Lane); the offsets are the copies' scalar offsets,
    // added to the lane offsets by the address unit.  Rows past M or N have
    // kOob lane offsets, which stay out of range with the offset added
    // (offsets within a band stay below 2^31, so the sum cannot wrap);
    // strips past K copy kOob.
    struct StripRes {
        u32 a, w, s;
        bool valid;
    };

    static __device__ __forceinline__ StripRes strip_res(const GemmParams& p, int, int, int strip)
    {
        const int k0 = strip * BK;
        StripRes r;
        r.valid = k0 < p.K;
        r.a = (u32)k0 * 2u;
        r.w = (u32)k0 / 2u;
        r.s = (u32)k0 / 32u;
        return r;
    }

    // Resource of `rows` rows of `row_bytes` bytes from base + row0 * row_bytes,
    // its parts read back as wave-uniform scalars (the 64-bit range arithmetic
    // may be done on the vector ALU).
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t band(const void* base, int row0,
                                                                  int rows, int row_bytes)
    {
        const uint64_t a = (uint64_t)((const char*)base + (int64_t)row0 * row_bytes);
        const u32 lo = __builtin_amdgcn_readfirstlane((u32)a);
        const u32 hi = __builtin_amdgcn_readfirstlane((u32)(a >> 32));
        const u32 n = __builtin_amdgcn_readfirstlane(clamp_bytes((int64_t)rows * row_bytes));
        return make_rsrc((const void*)(((uint64_t)hi << 32) | lo), n);
    }

    template <int ST, int W>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const StripRes& r, int d,
                                                      u32 smem0)
    {
        // the strip's byte offsets go in as the copies' scalar offsets, so a
        // copy costs no vector address arithmetic
        if (d < JA)
            dma16_so(smem0 + ST * A_STAGE + (W * JA + d) * 1024, r.valid ? L.a_off[d] : kOob, L.ra,
                     r.a);
        else if (d < JA + JW)
            dma16_so(smem0 + W_REGION + ST * W_STAGE + (W * JW + d - JA) * 1024,
                     r.valid ? L.w_off[d - JA] : kOob, L.rw, r.w);
        else
            dma4_so(smem0 + S_REGION + ST * S_STAGE + W * 256, r.valid ? L.s_off : kOob, L.rs, r.s);
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

    // SB > 1: the scale bytes of strips blk SB .. blk SB + SB - 1 into buffer
    // blk % 2.  Pieces past a row's end (or of rows past N) copy zeros.
    template <int W>
    static __device__ __forceinline__ void issue_scale_block(const Lane& L, const GemmParams& p,
                                                             int blk, u32 smem0)
    {
        const u32 b0 = (u32)blk * (u32)SROW;
        const u32 rowb = (u32)(p.K / 32);
#pragma unroll
        for (int i = 0; i < JS; ++i)
            dma16(smem0 + S_REGION + (blk & 1) * S_BUF + (W * JS + i) * 1024,
                  b0 + L.sb_c[i] < rowb ? L.sb_off[i] + b0 : kOob, L.rs);
    }

    template <int ST>
    static __device__ __forceinline__ void read_codes(Regs& R, const Lane& L, lds_char* sm,
                                                      int strip)
    {
        typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
        typedef __attribute__((address_space(3))) uint16_t lds_u16;
        typedef __attribute__((address_space(3))) uint8_t lds_u8;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int wo = ST * W_STAGE + fn * 32 * (BK / 2);
            if constexpr (LB >= 16) {
#pragma unroll
                for (int i = 0; i < NWR; ++i) {
                    const u32x4 c = *(const lds_u32x4*)(sm + L.w_rd[i] + wo);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        R.code[fn][4 * i + e] = c[e];
                }
            } else {
                const u32x2 c = *(const lds_u32x2*)(sm + L.w_rd[0] + wo);
                R.code[fn][0] = c[0];
                R.code[fn][1] = c[1];
            }
            if constexpr (SB == 1) {
                const int so = ST * S_STAGE + fn * 32 * 4;
                if constexpr (SPL == 2)
                    R.sc[fn] = *(const lds_u16*)(sm + L.s_rd + so);
                else
                    R.sc[fn] = *(const lds_u8*)(sm + L.s_rd + so);
            } else {
                // the 16-byte chunk of the row's block that holds this strip's
                // bytes (rows 32 apart share the chunk swizzle)
                const int off = (strip % SB) * (BK / 32);
                const int so = ((strip / SB) & 1) * S_BUF + (int)(((u32)(off >> 4) << 4) ^ L.s_sw) +
                               fn * 32 * SROW;
                R.scw[fn] = *(const lds_u32x4*)(sm + L.s_rd + so);
            }
        }
    }

    template <int ST>
    static __device__ __forceinline__ void read_a(u32x4 (&af)[FM], const Lane& L, lds_char* sm,
                                                  int j)
    {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            af[fm] = *(const lds_u32x4*)(sm + L.a_rd[j] + ST * A_STAGE + fm * 32 * BK * 2);
    }

    // The lane's scale bytes of n-block fn in this strip (the low SPL bytes;
    // its 32-k blocks in k order).  SB > 1: they sit at byte
    // (strip % SB) BK/32 + (BK/4 h + q LB) / 16 of the row's block; for
    // 128-k strips the strip is the ring stage modulo 4 (SB = 16, NS = 4 or
    // 6 and the block chunk holds four strips), for 256-k strips its parity.
    template <int ST, int P>
    static __device__ __forceinline__ u32 scale_bytes(const Regs& R, int fn, int lane, int q)
    {
        if constexpr (SB == 1) {
            return R.sc[fn];
        } else {
            const int h = lane >> 5;
            constexpr int SPS = BK / 32;                       // bytes per strip
            constexpr int F = BK == 128 ? (ST % 4) * SPS : P * SPS;  // strip's byte in the chunk
            const int b = F + (((BK / 4) * h + q * LB) >> 4);  // lane's first byte
            const u32 d0 = R.scw[fn][F >> 2];
            const u32 d1 = R.scw[fn][(F >> 2) + (SPS > 4 ? 1 : 0)];
            const u32 d = ((b >> 2) != (F >> 2)) ? d1 : d0;
            return d >> (8 * (b & 3));
        }
    }

    // B fragment of n-block fn, the wave's slab j: its 8 codes, scaled.
    static __device__ __forceinline__ bf16x8 dequant(const Regs& R, u32 sbytes, int fn, int j)
    {
        const u32 packed = R.code[fn][j];
        const u32 sbyte = (sbytes >> (8 * (j >> 2))) & 0xFFu;  // 4 slabs per 32-k block
        const float sc = e8m0_cvt_scale(sbyte);
        u32x4 b;
        b[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 0));
        b[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 1));
        b[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 2));
        b[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 3));
        return __builtin_bit_cast(bf16x8, b);
    }

    // A fragments are read PF slabs ahead into a 4-deep ring: the wave's slab
    // j of stage ST lives in AF[(ST SPW + j) % 4].  PF <= SPW, so a read never
    // reaches past strip t + 1, which slot 0's barrier has published.
    static constexpr int PF = SPW < 3 ? SPW : 3;
    static_assert((NS * SPW) % 4 == 0, "the A ring wraps with the stage cycle");

    // One strip (stage ST, code registers R[P]) of wave W.  Slot i = MFMA
    // (fm, fn) of the wave's slab j = i / NM.  Before slot 0: codes of this
    // strip in R[P], A slabs 0 .. PF-1 in the ring.  Slot 0 waits for strip
    // t + 1's copies and barriers, then reads strip t + 1's codes into
    // R[P ^ 1]; the last slot of slab j reads A slab j + PF (of strip t + 1
    // past the wave's last slab); the copies of strip t + NS - 1 are
    // staggered over the first CSPAN slots.
    template <int ST, int P, int W>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Regs (&R)[2],
                                                 u32x4 (&AF)[4][FM], const Lane& L, lds_char* sm,
                                                 const GemmParams& p, int m0, int n0, int t,
                                                 u32 smem0, int lane)
    {
        constexpr int NXT = (ST + 1) % NS;
        constexpr int CPY = (ST + NS - 1) % NS;
        constexpr int Q = W / NWG;
        u32 sb[FN];
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
            sb[fn] = scale_bytes<ST, P>(R[P], fn, lane, Q);
        StripRes r;
#pragma unroll
        for (int i = 0; i < SLOTS; ++i) {
            const int j = i / NM, fm = (i % NM) / FN, fn = i % FN;
            const int g = ST * SPW + j;
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dequant(R[P], sb[fn], fn, j),
                                                                  __builtin_bit_cast(bf16x8, AF[g & 3][fm]),
                                                                  acc[fm][fn], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            if (i == 0) {
                wait_copies_barrier<Copies<W>::AHEAD>();
                __builtin_amdgcn_sched_barrier(0);
                r = strip_res(p, m0, n0, t + NS - 1);
                read_codes<NXT>(R[P ^ 1], L, sm, t + 1);
                if constexpr (SB > 1) {
                    if (t % SB == SB / 2)
                        issue_scale_block<W>(L, p, t / SB + 1, smem0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            if (i % NM == NM - 1) {
                if (j + PF < SPW)
                    read_a<ST>(AF[(g + PF) & 3], L, sm, j + PF);
                else
                    read_a<NXT>(AF[(g + PF) & 3], L, sm, j + PF - SPW);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int d = 0; d < Copies<W>::N; ++d) {
                if (((d * NW + W) * CSPAN) / (NCMAX * NW) == i) {
                    issue_copy<CPY, W>(L, r, d, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // Copies of strips 0 .. NS-2 into stages 0 .. NS-2.
    template <int S, int W>
    static __device__ __forceinline__ void prologue_copies(const Lane& L, const GemmParams& p,
                                                           int m0, int n0, u32 smem0)
    {
        if constexpr (S < NS - 1) {
            issue_copies<S, W>(L, p, m0, n0, S, smem0);
            prologue_copies<S + 1, W>(L, p, m0, n0, smem0);
        }
    }

    // Strips t + I .. t + G - 1 of one loop iteration: G = NS strips on an
    // even ring, 2 NS on an odd one (the code registers alternate per strip).
    static constexpr int G = NS % 2 == 0 ? NS : 2 * NS;
    template <int I, int W>
    static __device__ __forceinline__ void strips(f32x16 (&acc)[FM][FN], Regs (&R)[2],
                                                  u32x4 (&AF)[4][FM], const Lane& L, lds_char* sm,
                                                  const GemmParams& p, int m0, int n0, int t,
                                                  u32 smem0, int lane)
    {
        strip<I % NS, I & 1, W>(acc, R, AF, L, sm, p, m0, n0, t + I, smem0, lane);
        if constexpr (I + 1 < G)
            strips<I + 1, W>(acc, R, AF, L, sm, p, m0, n0, t, smem0, lane);
    }

    // The last n < G strips of an odd ring, from the loop's state at t.
    template <int I, int W>
    static __device__ __forceinline__ void tail(f32x16 (&acc)[FM][FN], Regs (&R)[2],
                                                u32x4 (&AF)[4][FM], const Lane& L, lds_char* sm,
                                                const GemmParams& p, int m0, int n0, int t, int n,
                                                u32 smem0, int lane)
    {
        if constexpr (I + 1 < G) {
            if (I < n) {
                strip<I % NS, I & 1, W>(acc, R, AF, L, sm, p, m0, n0, t + I, smem0, lane);
                tail<I + 1, W>(acc, R, AF, L, sm, p, m0, n0, t, n, smem0, lane);
            }
        }
    }

    template <int W>
    static __device__ __forceinline__ void main_loop(f32x16 (&acc)[FM][FN], const Lane& L,
                                                     lds_char* sm, const GemmParams& p, int m0,
                                                     int n0, int KT, u32 smem0, int lane)
    {
        if constexpr (SB > 1)
            issue_scale_block<W>(L, p, 0, smem0);
        prologue_copies<0, W>(L, p, m0, n0, smem0);
        wait_copies_barrier<(NS - 2) * Copies<W>::N>();
        Regs R[2];
        u32x4 AF[4][FM];
        read_codes<0>(R[0], L, sm, 0);
#pragma unroll
        for (int s = 0; s < PF; ++s)
            read_a<0>(AF[s], L, sm, s);
        if constexpr (NS % 2 == 0) {
            // The strip count is rounded up to a multiple of NS: strips at or
            // past KT copy only zeros, which add exactly nothing.
            for (int t = 0; t < KT; t += NS)
                strips<0, W>(acc, R, AF, L, sm, p, m0, n0, t, smem0, lane);
        } else {
            int t = 0;
            for (; t + G <= KT; t += G)
                strips<0, W>(acc, R, AF, L, sm, p, m0, n0, t, smem0, lane);
            tail<0, W>(acc, R, AF, L, sm, p, m0, n0, t, KT - t, smem0, lane);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // Direct (unstaged) store of a wave's MFMA-layout result blocks: lane l
    // holds row l % 32 and, for element 4 q + e, column 8 q + 4 (l / 32) + e of
    // its block.  For C rows that are not whole 16-byte chunks.
    template <int OFM, int OFN>
    static __device__ __forceinline__ void store_direct(const f32x16 (&acc)[OFM][OFN],
                                                        const GemmParams& p, int mw0, int nw0,
                                                        int lane)
    {
        const int lr = lane & 31;
        const int g = lane >> 5;
        uint16_t* C = (uint16_t*)p.C;
#pragma unroll
        for (int fm = 0; fm < OFM; ++fm) {
            const int m = mw0 + fm * 32 + lr;
            if (m >= p.M)
                continue;
#pragma unroll
            for (int fn = 0; fn < OFN; ++fn) {
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

    static __device__ __forceinline__ bool staged_ok(const GemmParams& p)
    {
        return (p.N & 7) == 0 && ((uintptr_t)p.C & 15) == 0;
    }

    // k-slice groups: how a wave tile's FM x FN blocks are shared out for the
    // final sum and store.  Group q owns OFM x OFN blocks, block rows
    // (q / KSN) OFM .. and block columns (q % KSN) OFN ..
    static constexpr int KSM = FM < KS ? FM : KS;
    static constexpr int KSN = KS / KSM;
    static constexpr int OFM = FM / KSM;
    static constexpr int OFN = FN / KSN;
    static_assert(KS == 1 || (FM % KSM == 0 && FN % KSN == 0 && KSM * KSN == KS),
                  "the wave tile's blocks divide among the k-slice groups");
    static_assert(RED_BYTES <= 160 * 1024, "partial tiles fit in LDS");

    // Partial block b of wave (group qq, position r) in LDS: four 1 KiB
    // chunks, chunk c holding elements 4c .. 4c+3 of every lane.
    typedef __attribute__((address_space(3))) f32x4 lds_f32x4;
    static __device__ __forceinline__ int red_off(int r, int qq, int b, int lane)
    {
        return ((r * KS + qq) * NB + b) * 4096 + lane * 16;
    }

    // After the main loop of wave W (group Q): every wave writes the partial
    // blocks the other groups own, then sums its own blocks over the groups in
    // order 0 .. KS-1 and stores them.
    template <int W>
    static __device__ __forceinline__ void reduce_store(const f32x16 (&acc)[FM][FN],
                                                        const GemmParams& p, int m0, int n0,
                                                        int lane, lds_char* sm)
    {
        constexpr int Q = W / NWG;
        constexpr int R = W % NWG;
        constexpr int WM = R / WGN, WN = R % WGN;
        constexpr int FM0 = (Q / KSN) * OFM, FN0 = (Q % KSN) * OFN;
        wait_all_barrier();  // every wave's copies landed and ring reads done
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const bool own = fm >= FM0 && fm < FM0 + OFM && fn >= FN0 && fn < FN0 + OFN;
                if (own)
                    continue;
                const int o = red_off(R, Q, fm * FN + fn, lane);
                // (float vectors throughout: a bit cast of a single vector
                // element would read element 0)
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    *(lds_f32x4*)(sm + o + c * 1024) =
                        f32x4{acc[fm][fn][4 * c], acc[fm][fn][4 * c + 1], acc[fm][fn][4 * c + 2],
                              acc[fm][fn][4 * c + 3]};
            }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        f32x16 sum[OFM][OFN];
#pragma unroll
        for (int a = 0; a < OFM; ++a)
#pragma unroll
            for (int b = 0; b < OFN; ++b) {
                const int fm = FM0 + a, fn = FN0 + b;
#pragma unroll
                for (int qq = 0; qq < KS; ++qq) {
                    f32x16 part;
                    if (qq == Q) {
                        part = acc[fm][fn];
                    } else {
                        const int o = red_off(R, qq, fm * FN + fn, lane);
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const f32x4 v = *(const lds_f32x4*)(sm + o + c * 1024);
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                part[4 * c + e] = v[e];
                        }
                    }
                    if (qq == 0)
                        sum[a][b] = part;
                    else
                        sum[a][b] += part;
                }
            }
        const int mw0 = m0 + WM * WTM + FM0 * 32;
        const int nw0 = n0 + WN * WTN + FN0 * 32;
        if (staged_ok(p)) {
            // the staging regions overlap the partials other waves still read
            asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
            store_tile_staged<DT_BF16, OFM * 32, OFN * 32, OFM, OFN>(
                sum, p, mw0, nw0, lane, sm + W * (OFM * 32 * OFN * 32 * 2));
            return;
        }
        store_direct<OFM, OFN>(sum, p, mw0, nw0, lane);
    }

    template <int W>
    static __device__ __forceinline__ void body(f32x16 (&acc)[FM][FN], const Lane& L,
                                                lds_char* sm, const GemmParams& p, int m0,
                                                int n0, int KT, u32 smem0, int lane, int wm,
                                                int wn)
    {
        main_loop<W>(acc, L, sm, p, m0, n0, KT, smem0, lane);
        if constexpr (KS > 1) {
            reduce_store<W>(acc, p, m0, n0, lane, sm);
        } else {
            if (staged_ok(p) && NW * WTM * WTN * 2 <= LDS_BYTES) {
                wait_all_barrier();  // every wave's copies landed and reads done
                store_tile_staged<DT_BF16, WTM, WTN, FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN,
                                                            lane, sm + W * (WTM * WTN * 2));
                return;
            }
            store_direct<FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane);
        }
    }

    // The wave index as a template argument (copy schedule, k-slice group).
    template <int W>
    static __device__ __forceinline__ void dispatch(int w, f32x16 (&acc)[FM][FN], const Lane& L,
                                                    lds_char* sm, const GemmParams& p, int m0,
                                                    int n0, int KT, u32 smem0, int lane, int wm,
                                                    int wn)
    {
        if constexpr (W + 1 < NW) {
            if (w != W) {
                dispatch<W + 1>(w, acc, L, sm, p, m0, n0, KT, smem0, lane, wm, wn);
                return;
            }
        }
        body<W>(acc, L, sm, p, m0, n0, KT, smem0, lane, wm, wn);
    }

    static __device__ __forceinline__ void run(const GemmParams& p)
    {
        __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
        lds_char* sm = (lds_char*)smem;
        const u32 smem0 = lds_offset(smem);
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int q = w / NWG;
        const int wm = (w % NWG) / WGN;
        const int wn = (w % NWG) % WGN;
        const TileCoord tc = tile_of(blockIdx.x, p.tiles_m, p.tiles_n, group_of(p, GROUP_M));
        const int m0 = tc.m * BM;
        const int n0 = tc.n * BN;
        const int KT = p.K / BK;

        Lane L;
        setup(L, p, m0, n0, w, lane, wm, wn, q);
        f32x16 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[fm][fn][r] = 0.0f;
        dispatch<0>(w, acc, L, sm, p, m0, n0, KT, smem0, lane, wm, wn);
    }
};

template <int BM, int BN, int WGM, int WGN, int NS, int GROUP_M, int KS = 1, int SB = 1,
          int BK = 128>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * KS * 64, WGM * WGN * KS * 64))) void
dma_w4_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    DmaW4<BM, BN, WGM, WGN, NS, GROUP_M, KS, SB, BK>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
