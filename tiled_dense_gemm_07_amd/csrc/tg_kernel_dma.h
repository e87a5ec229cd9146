// Large-tile 16-bit GEMM for CDNA4 (gfx950): every strip goes global -> LDS by
// DMA, and the row-major B operand is transposed by the LDS read itself.
//
// The method is the pages' tiled GEMM ("TileLang ... 一个高效 GEMM 内核",
// mhpq.cn, sections 2.1, 2.3 and 3.2): a workgroup owns a BM x BN tile of C,
// stages BM x BK strips of A and BK x BN strips of B in on-chip memory, keeps
// the fp32 accumulator in registers and overlaps the copy of later strips with
// the math on the current one (section 3.3; blog.hotdry.top: num_stages 2-4).
// How that maps onto MI355X here:
//  * Copies are buffer_load_dwordx4 ... lds: each wave instruction moves 1 KiB
//    from global memory straight into LDS, so no VGPRs stage the strips and no
//    ds_write is issued.  Out-of-range lanes (rows past M, columns past N, k
//    past K) get an offset beyond the buffer and the hardware writes zeros.
//  * A stage holds A as [BM][BK] (k contiguous, 64-byte rows) and B as
//    [BK][BN] (n contiguous, as in memory).  A fragments are one ds_read_b128
//    per lane; B fragments are two ds_read_b64_tr_b16, which hand each lane
//    four k-consecutive values of one column n.
//  * 16-byte chunks are XOR-swizzled by row on both layouts so that the MFMA
//    fragment reads hit distinct banks; the DMA writes whole 1 KiB blocks in
//    lane order, so the swizzle is applied to the global addresses instead.
//  * NS LDS stages (BK = 32): the copy of strip t + NS - 1 is issued while
//    strip t is multiplied.  One barrier per strip, placed in the middle of
//    the strip's MFMAs, both publishes strip t + 1 and frees the stage of
//    strip t - 1.  The first fragments of strip t + 1 are read during the
//    second half of strip t, so the matrix cores never wait on a barrier.
//  * Instruction order inside a strip is fixed with scheduling barriers:
//    MFMAs alternate with LDS reads and DMA issues, one wave per SIMD.
//  * The copies and the waits on them are inline assembly: the compiler does
//    not know that these loads write LDS, so it inserts no conservative waits
//    before the transposing reads; the kernel waits on vmcnt itself.  The
//    copies set M0 (the LDS destination); no other code in this kernel uses M0.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tg_kernel.h"

#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"

namespace tg {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;

__device__ __forceinline__ u32 lds_offset(const void* p)
{
    return (u32)(size_t)(const lds_char*)p;
}

// One 16-byte-per-lane copy global -> LDS: lane l's 16 bytes at `voff` of the
// buffer land at LDS byte lds + 16 l.  An LDS-DMA load that reads M0 needs one
// wait state after the instruction that writes M0.
__device__ __forceinline__ void dma16(u32 lds, u32 voff, __amdgpu_buffer_rsrc_t rs)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds),
                 "v"(voff), "s"(rs)
                 : "memory");
}

// The same with a wave-uniform byte offset added to every lane's address
// (the strip's place in a row band that one buffer resource covers).
__device__ __forceinline__ void dma16_so(u32 lds, u32 voff, __amdgpu_buffer_rsrc_t rs, u32 soff)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds" ::"s"(lds),
                 "v"(voff), "s"(rs), "s"(soff)
                 : "memory");
}

// Wait until at most N copies of this wave are in flight, then barrier.
template <int N>
__device__ __forceinline__ void wait_copies_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Wait until every copy and every LDS read of this wave has completed, then
// barrier: afterwards the copies of all waves are visible and no wave still
// reads the LDS it read before.
__device__ __forceinline__ void wait_all_barrier()
{
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Chunk swizzles.  A rows are 64 bytes (4 chunks): rows r, r+2, r+4, r+6 and
// rows r, r+4, r+8, r+12 each get four different chunk positions.  B rows are
// at least 256 bytes: the four k-rows one transposing read touches get chunk
// masks 0, 6, 10, 12, distinct in bits 1-2 and in bits 2-3.
__device__ __forceinline__ int swz_a(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }
__device__ __forceinline__ int swz_b(int k) { return ((k & 1) * 6) ^ ((k & 2) * 5); }
// x-contiguous rows of 128 bytes (64 columns): two rows share a 256-byte bank
// line, so of the four k-rows one half of a transposing read touches (32
// columns = 4 chunks each), rows k and k + 2 must take complementary chunk
// halves: chunk mask 4 on rows with k & 2.
__device__ __forceinline__ int swz_b8(int k) { return (k & 2) * 2; }

// 128-byte rows (8 chunks): chunk c of row r goes to position c ^ swz8(r).  Only
// the low five bits of r enter, so rows 32 apart (the 32-row blocks of a wave
// tile) share a swizzle and one lane offset serves every block; any 16
// consecutive rows of a 32-row block then read 16 distinct 16-byte bank groups.
__device__ __forceinline__ int swz8(int r) { return (r ^ ((r >> 3) & 3)) & 7; }

// One operand of the 16-bit DMA kernel: X (BM or BN) output rows/columns by
// BK (32, 64 or 128) k per strip.  In global memory the operand is either
// k-contiguous (KMAJ: each of its X rows holds consecutive k; leading
// dimension K) or x-contiguous (each k row holds consecutive x; leading
// dimension = the operand's full extent).  The LDS stage keeps the global
// orientation:
//  * KMAJ: [X][BK k], rows of 64 bytes (chunk swizzle swz_a), 128 bytes
//    (swz8) or 256 bytes; an MFMA fragment (8 consecutive k of one row per lane) is one
//    ds_read_b128.  A copy moves whole row segments of 2 BK bytes; 128-byte
//    segments are whole cache lines and copy about 1.4x faster than 64-byte
//    ones;
//  * x-contiguous: [BK k][X], chunk swizzle swz_b; a fragment is two
//    ds_read_b64_tr_b16 (4 consecutive k of one column each).
// Both give the MFMA the same operand layout: lane l holds 8 consecutive k of
// index l % 32 of a 32-wide block, starting at k = 16 s + 8 (l / 32) in slab s.
template <bool KMAJ, int X, int WX, int FX, int NW, int BK>
struct DmaOperand {
    static_assert(BK == 32 || BK == 64 || BK == 128, "strips of 32, 64 or 128 k");
    static constexpr int SL = BK / 16;                // MFMA slabs per strip
    static constexpr int STAGE = X * BK * 2;          // bytes per LDS stage
    static constexpr int J = STAGE / 1024 / NW;       // 1 KiB copies per wave per strip
    static constexpr int LPR = KMAJ ? BK / 8 : X / 8;  // 16-byte chunks per LDS row
    static constexpr int RPB = 64 / LPR;              // LDS rows per 1 KiB copy
    static constexpr int NRD = KMAJ ? FX : 2 * FX;    // LDS reads per slab
    static_assert(J >= 1 && STAGE % (1024 * NW) == 0, "strips split into whole 1 KiB copies per wave");
    static_assert(KMAJ || (LPR >= 8 && LPR <= 64), "x-contiguous rows of 128 to 1024 bytes");

    // k-contiguous rows of 64, 128 or 256 bytes (256: chunk c of row r at
    // position c ^ (r & 15), so any 16 consecutive rows read 16 distinct
    // positions and rows 32 apart share the swizzle)
    static __device__ __forceinline__ int kswz(int row)
    {
        return BK == 32 ? swz_a(row) : (BK == 64 ? swz8(row) : (row & 15));
    }
    static __device__ __forceinline__ int xswz(int k) { return LPR == 8 ? swz_b8(k) : swz_b(k); }

    struct Lane {
        u32 off[J];   // copy offsets within a strip (out of range past the x extent)
        int kk[KMAJ ? J : 1];  // KMAJ: k (within the strip) of the data each copy lane moves
        int lr;       // x-contiguous: the lane's k row within a copy (k = copy row + lr)
        u32 rd[KMAJ ? SL : FX];  // fragment read offsets (stage 0)
        __amdgpu_buffer_rsrc_t band;  // the tile's rows (KMAJ) or columns over the whole K
        bool use_band;  // x-contiguous: the band's offsets fit 31 bits (KMAJ: always)
    };
    // Where one strip's copies read: the tile's band (its rows over the whole
    // K, or its columns over all K rows) and the strip's byte offset in it,
    // set up once per tile, so a strip costs one scalar multiply.  An
    // x-contiguous band spans K rows of the full matrix width; where that
    // passes 31 bits of offset, each strip gets a resource rebased to its
    // first k row instead (uniform per workgroup, decided at setup).
    struct Strip {
        __amdgpu_buffer_rsrc_t rs;
        u32 so;
    };
    struct Frag {
        u32x4 v[KMAJ ? FX : 1];
        s16x4 t[KMAJ ? 1 : FX][2];
    };

    // x0: first row/column of the tile; xtot: the operand's full extent;
    // ld: leading dimension in elements; wx0: first row/column of this wave.
    static __device__ __forceinline__ void setup(Lane& L, int x0, int xtot, int ld, int w,
                                                 int lane, int wx0, u32 region, const void* base,
                                                 int K)
    {
        L.band = strip_rsrc(base, x0, xtot, ld, K, 0);
        L.use_band = KMAJ || (int64_t)(K - 1) * ld * 2 + (int64_t)(xtot - x0) * 2 < 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < J; ++j) {
            const int blk = w * J + j;
            const int row = blk * RPB + lane / LPR;
            if constexpr (KMAJ) {
                const int c = (lane % LPR) ^ kswz(row);
                L.kk[j] = c * 8;
                L.off[j] = (x0 + row < xtot) ? (u32)(row * ld + c * 8) * 2u : kOob;
            } else {
                const int c = (lane % LPR) ^ xswz(row);
                L.off[j] = (x0 + c * 8 < xtot) ? (u32)(row * ld + c * 8) * 2u : kOob;
            }
        }
        L.lr = lane / LPR;
        if constexpr (KMAJ) {
#pragma unroll
            for (int s = 0; s < SL; ++s) {
                const int row = wx0 + (lane & 31);
                const int c = 2 * s + (lane >> 5);
                L.rd[s] = region + row * (BK * 2) + ((c ^ kswz(row)) << 4);
            }
        } else {
            const int g = lane >> 4, t = lane & 15;
            const int k = 8 * (g >> 1) + (t >> 2);
#pragma unroll
            for (int f = 0; f < FX; ++f) {
                const int x = wx0 + f * 32 + 16 * (g & 1) + 4 * (t & 3);
                L.rd[f] = region + k * (X * 2) + (((x >> 3) ^ xswz(k)) << 4) + (x & 7) * 2;
            }
        }
    }

    // Descriptor of one strip (k0 .. k0 + BK - 1), rebased so offsets fit 31 bits.
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t strip_rsrc(const void* base, int x0,
                                                                        int xtot, int ld, int K,
                                                                        int k0)
    {
        if constexpr (KMAJ)
            return make_rsrc((const char*)base + ((int64_t)x0 * ld + k0) * 2,
                             clamp_bytes(((int64_t)(xtot - x0 - 1) * ld + (K - k0)) * 2));
        else
            return make_rsrc((const char*)base + ((int64_t)k0 * ld + x0) * 2,
                             clamp_bytes(((int64_t)(K - k0 - 1) * ld + (xtot - x0)) * 2));
    }

    template <bool BAND>
    static __device__ __forceinline__ Strip strip(const Lane& L, const void* base, int x0,
                                                  int xtot, int ld, int K, int k0)
    {
        Strip s;
        if constexpr (KMAJ) {
            s.rs = L.band;
            s.so = (u32)k0 * 2u;
        } else if constexpr (BAND) {
            s.rs = L.band;
            s.so = (u32)k0 * (u32)ld * 2u;
        } else {
            s.rs = strip_rsrc(base, x0, xtot, ld, K, k0);
            s.so = 0u;
        }
        return s;
    }

    template <int ST>
    static __device__ __forceinline__ void copy(const Lane& L, const Strip& sr, int krem, int d,
                                                int w, u32 region_lds)
    {
        const int kk = KMAJ ? L.kk[KMAJ ? d : 0] : (w * J + d) * RPB + L.lr;
        const u32 lds = region_lds + ST * STAGE + (w * J + d) * 1024;
        dma16_so(lds, kk < krem ? L.off[d] : kOob, sr.rs, sr.so);
    }

    // LDS read i (0 .. NRD-1) of slab S of stage ST.
    template <int ST, int S>
    static __device__ __forceinline__ void read(Frag& F, const Lane& L, lds_char* sm, int i)
    {
        if constexpr (KMAJ) {
            F.v[i] = *(const lds_u32x4*)(sm + L.rd[S] + ST * STAGE + i * 32 * (BK * 2));
        } else {
            const int f = i >> 1, h = i & 1;
            F.t[f][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)(sm + L.rd[f] + ST * STAGE + (16 * S + 4 * h) * (X * 2)));
        }
    }

    // The MFMA operand of block f (8 k per lane, 16-bit words).
    static __device__ __forceinline__ s16x8 frag(const Frag& F, int f)
    {
        if constexpr (KMAJ)
            return __builtin_bit_cast(s16x8, F.v[f]);
        else
            return __builtin_shufflevector(F.t[f][0], F.t[f][1], 0, 1, 2, 3, 4, 5, 6, 7);
    }
};

// As store_tile_staged, for result blocks in the other MFMA orientation: lane
// l holds column l % 32 and, for element r, row 8 (r / 4) + 4 (l / 32) + r % 4
// of its block (the first MFMA operand supplied the rows).
template <int DT, int WTM, int WTN, int FM, int FN>
__device__ __forceinline__ void store_tile_staged_t(const f32x16 (&acc)[FM][FN],
                                                    const GemmParams& p, int mw0, int nw0,
                                                    int lane, lds_char* st)
{
    constexpr int ROWB = WTN * 2;
    constexpr int CH = ROWB / 16;
    static_assert(CH >= 4 && CH <= 64 && (CH & (CH - 1)) == 0, "rows of 64 to 1024 bytes");
    typedef __attribute__((address_space(3))) uint16_t lds_u16;
    const int lc = lane & 31;
    const int g = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int col = fn * 32 + lc;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = fm * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const float x = acc[fm][fn][r];
                *(lds_u16*)(st + row * ROWB + (((col >> 3) ^ (row & (CH - 1))) << 4) +
                            (col & 7) * 2) = cvt1((p.relu && !(x > 0.0f)) ? 0.0f : x, DT);
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own region: no barrier needed
    constexpr int RPI = 64 / CH;
    store_rows_through<WTM, RPI, CH, 2>(st, p, mw0, nw0, lane);
}

// TA: A stored [K][M] (C = A^T-stored x B); TB: B stored [N][K].  BK: k per
// strip (32, 64 or 128); NS: LDS stages (2 .. 5).
template <int DT, bool TA, bool TB, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M,
          int BK>
struct DmaGemm {
    static_assert(DT == DT_BF16 || DT == DT_F16, "16-bit operands only");
    static constexpr int SL = BK / 16;  // MFMA slabs per strip
    static constexpr int NW = WGM * WGN;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    using OA = DmaOperand<!TA, BM, WTM, FM, NW, BK>;
    using OB = DmaOperand<TB, BN, WTN, FN, NW, BK>;
    static constexpr int A_STAGE = OA::STAGE;
    static constexpr int B_STAGE = OB::STAGE;
    static constexpr int A_REGION = NS * A_STAGE;
    static constexpr int LDS_BYTES = NS * (A_STAGE + B_STAGE);
    static constexpr int NREAD = OA::NRD + OB::NRD;  // LDS reads per slab
    // Fragment sets: a ring of RF, each slab reading the one PFD = RF - 1
    // slabs ahead.  Two sets for most tiles; four for wave tiles of one or
    // two MFMA blocks on rings of three or more stages and strips of four or
    // more slabs, whose one or two MFMAs per slab would not cover the LDS
    // read latency of the next slab.  (Two stages keep two sets: their
    // barrier sits in the last slab, so no earlier slab may read the next
    // strip.  With SL >= 4 the first reads of the next strip come after the
    // barrier in slot 0.)
    static constexpr int RF = (NS >= 3 && SL >= 4 && FM * FN <= 2) ? 4 : 2;
    static constexpr int PFD = RF - 1;
    static_assert((NS * SL) % RF == 0 && PFD < SL, "the fragment ring wraps with the stage cycle");
    static constexpr int NCOPY = OA::J + OB::J;      // copies per wave per strip
    static constexpr int VM_AHEAD = NS >= 3 ? (NS - 3) * NCOPY : 0;  // copies in flight at the barrier

    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of whole 32x32 blocks");
    static_assert(NS >= 2 && NS <= 5, "two to five stages");
    static_assert(NW <= 8, "the main loop is instantiated for up to eight waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    struct Frag {
        typename OA::Frag a;
        typename OB::Frag b;
    };

    struct Lane {
        typename OA::Lane a;
        typename OB::Lane b;
    };

    static __device__ __forceinline__ int lda(const GemmParams& p) { return TA ? p.M : p.K; }
    static __device__ __forceinline__ int ldb(const GemmParams& p) { return TB ? p.K : p.N; }

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn)
    {
        OA::setup(L.a, m0, p.M, lda(p), w, lane, wm * WTM, 0, p.A, p.K);
        OB::setup(L.b, n0, p.N, ldb(p), w, lane, wn * WTN, A_REGION, p.B, p.K);
    }

    // Where the copies of one strip read (per operand, DmaOperand::Strip).
    struct StripRes {
        typename OA::Strip a;
        typename OB::Strip b;
        int krem;  // valid k within the strip: [0, krem)
    };

    // BAND: both operands read through their per-tile bands (decided per
    // workgroup at setup; the loop is compiled for either case so that no
    // strip branches on it).
    template <bool BAND>
    static __device__ __forceinline__ StripRes strip_res(const GemmParams& p, int m0, int n0,
                                                         int strip, const Lane& L)
    {
        const int k0 = strip * BK;
        StripRes r;
        r.a = OA::template strip<BAND>(L.a, p.A, m0, p.M, lda(p), p.K, k0);
        r.b = OB::template strip<BAND>(L.b, p.B, n0, p.N, ldb(p), p.K, k0);
        r.krem = p.K - k0;
        return r;
    }
    static __device__ __forceinline__ bool use_band(const Lane& L)
    {
        return L.a.use_band && L.b.use_band;
    }
    static __device__ __forceinline__ StripRes strip_res_any(const GemmParams& p, int m0, int n0,
                                                             int strip, const Lane& L)
    {
        return use_band(L) ? strip_res<true>(p, m0, n0, strip, L)
                           : strip_res<false>(p, m0, n0, strip, L);
    }

    // Copy d (0 .. NCOPY-1) of a strip into LDS stage ST: A's copies first.
    template <int ST>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const StripRes& r, int d,
                                                      int w, u32 smem0)
    {
        if (d < OA::J)
            OA::template copy<ST>(L.a, r.a, r.krem, d, w, smem0);
        else
            OB::template copy<ST>(L.b, r.b, r.krem, d - OA::J, w, smem0 + A_REGION);
    }

    template <int ST>
    static __device__ __forceinline__ void issue_copies(const Lane& L, const GemmParams& p,
                                                        int m0, int n0, int strip, int w,
                                                        u32 smem0)
    {
        const StripRes r = strip_res_any(p, m0, n0, strip, L);
#pragma unroll
        for (int d = 0; d < NCOPY; ++d)
            issue_copy<ST>(L, r, d, w, smem0);
    }

    // Fragment read i (0 .. NREAD-1) of slab S of stage ST: A's reads first.
    template <int ST, int S>
    static __device__ __forceinline__ void read_one(Frag& F, const Lane& L, lds_char* sm, int i)
    {
        if (i < OA::NRD)
            OA::template read<ST, S>(F.a, L.a, sm, i);
        else
            OB::template read<ST, S>(F.b, L.b, sm, i - OA::NRD);
    }

    static __device__ __forceinline__ void mfma_one(f32x16 (&acc)[FM][FN], const Frag& F, int i)
    {
        const int fm = i / FN, fn = i % FN;
        const s16x8 a8 = OA::frag(F.a, fm);
        const s16x8 b8 = OB::frag(F.b, fn);
        if constexpr (DT == DT_BF16)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, b8), __builtin_bit_cast(bf16x8, a8), acc[fm][fn], 0, 0,
                0);
        else
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, b8), __builtin_bit_cast(f16x8, a8), acc[fm][fn], 0, 0,
                0);
    }

    // Reads of slab S + PFD of stage ST (past the strip's last slab: of the
    // next stage NXT, which the barrier in slot 0 has published) into the
    // ring set that slab uses.  Slab S of stage ST uses set (ST SL + S) % RF;
    // NS SL is a multiple of RF, so the ring continues across strips.
    template <int ST, int NXT, int S>
    static __device__ __forceinline__ void read_next(Frag (&F)[RF], const Lane& L, lds_char* sm,
                                                     int i)
    {
        constexpr int T = S + PFD;
        constexpr int SET = (ST * SL + T) % RF;
        if constexpr (T < SL)
            read_one<ST, T>(F[SET], L, sm, i);
        else
            read_one<NXT, T - SL>(F[SET], L, sm, i);
    }

    // Step i of slab S: its MFMA, then (NS == 2, last slab, first step) the
    // barrier, then its read of the next slab's fragments.
    template <int ST, int NXT, int S, int I>
    static __device__ __forceinline__ void slab_step(f32x16 (&acc)[FM][FN], Frag (&F)[RF],
                                                     const Lane& L, lds_char* sm)
    {
        constexpr int NM = FM * FN;
        if constexpr (I < NM) {
            mfma_one(acc, F[(ST * SL + S) % RF], I);
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (NS == 2 && S == SL - 1 && I == 0) {
            wait_all_barrier();
            __builtin_amdgcn_sched_barrier(0);
        }
        if constexpr (I < NREAD) {
            read_next<ST, NXT, S>(F, L, sm, I);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    static constexpr int NM_ = FM * FN;
    static constexpr int STEPS = NM_ > NREAD ? NM_ : NREAD;  // slots per slab
    static constexpr int SLOTS = SL * STEPS;                 // slots per strip
    // NS >= 3: the copies of a strip use every slot of the strip.  NS == 2:
    // the copies of strip t + 2 are spread over CSPREAD slabs that start
    // with the last slab of strip t (after the barrier that frees strip t's
    // stage) and go on into the first CSPREAD - 1 slabs of strip t + 1.
#ifndef TG_CSPREAD
#define TG_CSPREAD 2
#endif
    static constexpr int CSPREAD = TG_CSPREAD < SL ? TG_CSPREAD : SL;
    static constexpr int CSLOTS = NS == 2 ? CSPREAD * STEPS : SLOTS;
    // position of copy d of wave W in the copy window (slot index)
    static constexpr int cpos(int d, int W) { return ((d * NW + W) * CSLOTS) / (NCOPY * NW); }

    // Slot SLOT of a strip (stage ST) of wave W, then the following slots: the
    // recursion unrolls the strip at compile time whatever its length.
    template <int ST, int W, int SLOT, bool BAND>
    static __device__ __forceinline__ void slots(f32x16 (&acc)[FM][FN], Frag (&F)[RF],
                                                 const Lane& L, lds_char* sm, const GemmParams& p,
                                                 int m0, int n0, int t, u32 smem0, StripRes& r,
                                                 const StripRes& r1)
    {
        constexpr int NXT = (ST + 1) % NS;
        slab_step<ST, NXT, SLOT / STEPS, SLOT % STEPS>(acc, F, L, sm);
        if constexpr (NS >= 3) {
            if constexpr (SLOT == 0) {
                wait_copies_barrier<VM_AHEAD>();
                __builtin_amdgcn_sched_barrier(0);
                r = strip_res<BAND>(p, m0, n0, t + NS - 1, L);
            }
            // strip t + NS - 1 into the stage strip t - 1 used: copy d of wave
            // W at slot cpos(d, W)
            constexpr int CPY = (ST + NS - 1) % NS;
#pragma unroll
            for (int d = 0; d < NCOPY; ++d) {
                if (cpos(d, W) == SLOT) {
                    issue_copy<CPY>(L, r, d, W, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        } else {
            // window positions q < STEPS: strip t + 2 into this strip's own
            // stage, in the last slab (after the barrier); q >= STEPS: the
            // rest of strip t + 1 into the other stage, in the first slabs
#pragma unroll
            for (int d = 0; d < NCOPY; ++d) {
                constexpr int LAST = (SL - 1) * STEPS;
                if (cpos(d, W) < STEPS && LAST + cpos(d, W) == SLOT) {
                    issue_copy<ST>(L, r, d, W, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                } else if (cpos(d, W) >= STEPS && cpos(d, W) - STEPS == SLOT) {
                    issue_copy<NXT>(L, r1, d, W, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        if constexpr (SLOT + 1 < SLOTS)
            slots<ST, W, SLOT + 1, BAND>(acc, F, L, sm, p, m0, n0, t, smem0, r, r1);
    }

    // One strip: SL slabs of FM x FN MFMAs; slab s uses one fragment set of
    // the ring while its reads fill the set of slab s + PFD (past the last
    // slab, the first slabs of strip t + 1).  Copies of strip t + NS - 1 go to
    // the stage strip t - 1 used.
    //   NS >= 3: the barrier sits in slot 0 (after its MFMA and read): before
    //     it, strip t + 1's copies are waited for (at most the NCOPY x (NS - 3)
    //     younger ones stay in flight); after it, strip t + 1 is visible and the
    //     stage of strip t - 1 is free, and the copies are spread over the
    //     whole strip, staggered across the waves.
    //   NS == 2: the barrier sits at the start of the last slab, before the
    //     reads of strip t + 1: each wave first waits for all its copies (those
    //     of strip t + 1) and LDS reads (those of strip t, whose last slab is
    //     in registers by then), so after the barrier strip t + 1 is visible
    //     and no wave reads strip t's stage again.  The copies of strip t + 2
    //     go into that stage right away, spread over the last slab: they have
    //     a whole strip to land before the barrier of strip t + 1 waits for
    //     them.  `carry` holds strip t + 1's resources, computed by the strip
    //     before as its t + 2; this strip computes t + 2's and leaves them
    //     there for the next.
    template <int ST, int W, bool BAND>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Frag (&F)[RF],
                                                 const Lane& L, lds_char* sm, const GemmParams& p,
                                                 int m0, int n0, int t, u32 smem0, StripRes& carry)
    {
        StripRes r;
        if constexpr (NS == 2)
            r = strip_res<BAND>(p, m0, n0, t + 2, L);
        slots<ST, W, 0, BAND>(acc, F, L, sm, p, m0, n0, t, smem0, r, carry);
        if constexpr (NS == 2)
            carry = r;
    }

    // The strip loop of wave W (the copy slots differ per wave).  The strip
    // count is rounded up to a multiple of NS: strips at or past KT copy only
    // out-of-range zeros, which add exactly nothing.
    template <int W, bool BAND>
    static __device__ __forceinline__ void main_loop(f32x16 (&acc)[FM][FN], Frag (&F)[RF],
                                                     const Lane& L, lds_char* sm,
                                                     const GemmParams& p, int m0, int n0, int KT,
                                                     u32 smem0)
    {
        StripRes carry;
        if constexpr (NS == 2)
            carry = strip_res<BAND>(p, m0, n0, 1, L);
        for (int t = 0; t < KT; t += NS) {
            strip<0, W, BAND>(acc, F, L, sm, p, m0, n0, t, smem0, carry);
            strip<1, W, BAND>(acc, F, L, sm, p, m0, n0, t + 1, smem0, carry);
            if constexpr (NS > 2)
                strip<2 % NS, W, BAND>(acc, F, L, sm, p, m0, n0, t + 2, smem0, carry);
            if constexpr (NS > 3)
                strip<3 % NS, W, BAND>(acc, F, L, sm, p, m0, n0, t + 3, smem0, carry);
            if constexpr (NS > 4)
                strip<4 % NS, W, BAND>(acc, F, L, sm, p, m0, n0, t + 4, smem0, carry);
        }
    }

    template <int W>
    static __device__ __forceinline__ void loop_for(f32x16 (&acc)[FM][FN], Frag (&F)[RF],
                                                    const Lane& L, lds_char* sm,
                                                    const GemmParams& p, int m0, int n0, int KT,
                                                    u32 smem0)
    {
        if (use_band(L))
            main_loop<W, true>(acc, F, L, sm, p, m0, n0, KT, smem0);
        else
            main_loop<W, false>(acc, F, L, sm, p, m0, n0, KT, smem0);
    }

    static __device__ __forceinline__ void epilogue(const f32x16 (&acc)[FM][FN],
                                                    const GemmParams& p, int m0, int n0, int wm,
                                                    int wn, int lane)
    {
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
                        *(u32x2*)(C + idx) = u32x2{pack2(v[0], v[1], DT), pack2(v[2], v[3], DT)};
                    } else {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            if (n + e < p.N)
                                C[idx + e] = cvt1(v[e], DT);
                    }
                }
            }
        }
    }

    static __device__ __forceinline__ void run(const GemmParams& p)
    {
        __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];
        lds_char* sm = (lds_char*)smem;
        const u32 smem0 = lds_offset(smem);
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
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

        // prologue: strips 0 .. NS-2 into stages 0 .. NS-2 (NS == 2: strip 0
        // and the part of strip 1 that the main loop issues in the last slab
        // of strip -1; strip 0 issues the rest)
        issue_copies<0>(L, p, m0, n0, 0, w, smem0);
        if constexpr (NS == 2) {
            const StripRes r1 = strip_res_any(p, m0, n0, 1, L);
#pragma unroll
            for (int d = 0; d < NCOPY; ++d)
                if (((d * NW + w) * CSLOTS) / (NCOPY * NW) < STEPS)
                    issue_copy<1>(L, r1, d, w, smem0);
        }
        if constexpr (NS > 2)
            issue_copies<1>(L, p, m0, n0, 1, w, smem0);
        if constexpr (NS > 3)
            issue_copies<2 % NS>(L, p, m0, n0, 2, w, smem0);
        if constexpr (NS > 4)
            issue_copies<3 % NS>(L, p, m0, n0, 3, w, smem0);
        // strip 0 must be complete and visible before its first fragments are
        // read (NS == 2: wait for all)
        wait_copies_barrier<(NS == 2 ? 0 : NS - 2) * NCOPY>();
        Frag F[RF];
#pragma unroll
        for (int i = 0; i < NREAD; ++i)
            read_one<0, 0>(F[0], L, sm, i);
        if constexpr (PFD > 1) {
#pragma unroll
            for (int i = 0; i < NREAD; ++i)
                read_one<0, 1 % SL>(F[1], L, sm, i);
#pragma unroll
            for (int i = 0; i < NREAD; ++i)
                read_one<0, 2 % SL>(F[2], L, sm, i);
        }

        switch (w) {
        case 0:
            loop_for<0>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        case 1:
            loop_for<1 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        case 2:
            loop_for<2 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        case 3:
            loop_for<3 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        case 4:
            loop_for<4 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        case 5:
            loop_for<5 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        case 6:
            loop_for<6 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        default:
            loop_for<7 % NW>(acc, F, L, sm, p, m0, n0, KT, smem0);
            break;
        }
        // drain the copies of the strips past the end (all out of range)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if ((p.N & 7) == 0 && ((uintptr_t)p.C & 15) == 0 &&
            NW * WTM * WTN * 2 <= LDS_BYTES) {
            wait_all_barrier();  // every wave's copies landed and reads done
            store_tile_staged<DT, WTM, WTN, FM, FN>(acc, p, m0 + wm * WTM, n0 + wn * WTN, lane,
                                                   sm + w * (WTM * WTN * 2));
        } else {
            epilogue(acc, p, m0, n0, wm, wn, lane);
        }
    }
};

// Waves per SIMD the kernel is compiled for: one on four waves for the
// largest tiles (all 512 registers of a lane available, 256 of them
// accumulators) and for rings of more than half the LDS (no second workgroup
// fits beside them), else two.
template <int BM, int BN, int NW, int LDS>
struct DmaOcc {
    static constexpr int value =
        (NW <= 4 && (BM * BN >= 256 * 128 || 2 * LDS > 160 * 1024)) ? 1 : 2;
};

template <int BM, int BN, int WGM, int WGN, int NS, int BK>
using DmaOccOf = DmaOcc<BM, BN, WGM * WGN, NS * (BM + BN) * BK * 2>;

template <int DT, bool TA, bool TB, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M,
          int BK>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * 64, WGM * WGN * 64),
                          amdgpu_waves_per_eu(DmaOccOf<BM, BN, WGM, WGN, NS, BK>::value,
                                              DmaOccOf<BM, BN, WGM, WGN, NS, BK>::value))) void
gemm_dma_kernel(GemmParams p)
{
    const ClockStamp clk = stamp_begin(p);
    DmaGemm<DT, TA, TB, BM, BN, WGM, WGN, NS, GROUP_M, BK>::run(p);
    stamp_end(p, clk);
}

}  // namespace tg

#pragma clang diagnostic pop
