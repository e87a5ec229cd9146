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

// Wait until at most N copies of this wave are in flight, then barrier.
template <int N>
__device__ __forceinline__ void wait_copies_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Chunk swizzles.  A rows are 64 bytes (4 chunks): rows r, r+2, r+4, r+6 and
// rows r, r+4, r+8, r+12 each get four different chunk positions.  B rows are
// at least 256 bytes: the four k-rows one transposing read touches get chunk
// masks 0, 6, 10, 12, distinct in bits 1-2 and in bits 2-3.
__device__ __forceinline__ int swz_a(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1); }
__device__ __forceinline__ int swz_b(int k) { return ((k & 1) * 6) ^ ((k & 2) * 5); }

template <int DT, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M>
struct DmaGemm {
    static_assert(DT == DT_BF16 || DT == DT_F16, "16-bit operands only");
    static constexpr int BK = 32;
    static constexpr int NW = WGM * WGN;
    static constexpr int NT = NW * 64;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr int A_STAGE = BM * BK * 2;  // bytes
    static constexpr int B_STAGE = BK * BN * 2;
    static constexpr int A_REGION = NS * A_STAGE;
    static constexpr int LDS_BYTES = NS * (A_STAGE + B_STAGE);
    static constexpr int JA = A_STAGE / 1024 / NW;  // copies per wave per strip
    static constexpr int JB = B_STAGE / 1024 / NW;
    static constexpr int LPR = BN / 8;               // lanes (16-byte chunks) per B row
    static constexpr int RPB = 64 / LPR;             // B rows per 1 KiB block
    static constexpr int VM_AHEAD = (NS - 3) * (JA + JB);  // copies allowed in flight at the barrier
    static constexpr int NREAD = FM + 2 * FN;        // LDS reads per slab
    static constexpr int NCOPY = JA + JB;            // copies per wave per strip

    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tiles of whole 32x32 blocks");
    static_assert(JA >= 1 && JB >= 1 && A_STAGE % (1024 * NW) == 0 && B_STAGE % (1024 * NW) == 0,
                  "strips split into whole 1 KiB copies per wave");
    static_assert(LPR >= 16 && LPR <= 64, "B rows of 256 to 1024 bytes");
    static_assert(NS >= 3, "the barrier publishes strip t + 1 while t - 1 is free");
    static_assert(NW <= 4, "the main loop is instantiated for up to four waves");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

    struct Frag {
        u32x4 a[FM];
        s16x4 b[FN][2];
    };

    struct Lane {
        // copy offsets within a strip (already out of range for rows past M / cols past N)
        u32 a_off[JA];
        int a_k[JA];  // first k of the chunk this lane copies
        u32 b_off[JB];
        int b_k[JB];  // k row this lane copies
        // LDS read offsets from the start of the LDS buffer (stage 0)
        u32 a_rd[2];
        u32 b_rd[FN];
    };

    static __device__ __forceinline__ void setup(Lane& L, const GemmParams& p, int m0, int n0,
                                                 int w, int lane, int wm, int wn)
    {
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int blk = w * JA + j;
            const int row = blk * 16 + (lane >> 2);
            const int c = (lane & 3) ^ swz_a(row);
            L.a_k[j] = c * 8;
            L.a_off[j] = (m0 + row < p.M) ? (u32)(row * p.K + c * 8) * 2u : kOob;
        }
#pragma unroll
        for (int j = 0; j < JB; ++j) {
            const int blk = w * JB + j;
            const int row = blk * RPB + lane / LPR;
            const int c = (lane % LPR) ^ swz_b(row);
            L.b_k[j] = row;
            L.b_off[j] = (n0 + c * 8 < p.N) ? (u32)(row * p.N + c * 8) * 2u : kOob;
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = wm * WTM + (lane & 31);
            const int c = 2 * s + (lane >> 5);
            L.a_rd[s] = row * (BK * 2) + ((c ^ swz_a(row)) << 4);
        }
        const int g = lane >> 4, t = lane & 15;
        const int k = 8 * (g >> 1) + (t >> 2);
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int n = wn * WTN + fn * 32 + 16 * (g & 1) + 4 * (t & 3);
            L.b_rd[fn] = A_REGION + k * (BN * 2) + (((n >> 3) ^ swz_b(k)) << 4) + (n & 7) * 2;
        }
    }

    // Buffer descriptors of one strip, rebased to the strip's first element so
    // that every offset stays inside 31 bits.
    struct StripRes {
        __amdgpu_buffer_rsrc_t a, b;
        int krem;  // valid k within the strip: [0, krem)
    };

    static __device__ __forceinline__ StripRes strip_res(const GemmParams& p, int m0, int n0,
                                                         int strip)
    {
        const int k0 = strip * BK;
        const char* abase = (const char*)p.A + ((int64_t)m0 * p.K + k0) * 2;
        const int64_t abytes = ((int64_t)(p.M - m0 - 1) * p.K + (p.K - k0)) * 2;
        const char* bbase = (const char*)p.B + ((int64_t)k0 * p.N + n0) * 2;
        const int64_t bbytes = ((int64_t)(p.K - k0 - 1) * p.N + (p.N - n0)) * 2;
        StripRes r;
        r.a = make_rsrc(abase, clamp_bytes(abytes));
        r.b = make_rsrc(bbase, clamp_bytes(bbytes));
        r.krem = p.K - k0;
        return r;
    }

    // Copy d (0 .. NCOPY-1) of a strip into LDS stage ST: the JA copies of A
    // first, then the JB copies of B.
    template <int ST>
    static __device__ __forceinline__ void issue_copy(const Lane& L, const StripRes& r, int d,
                                                      int w, u32 smem0)
    {
        if (d < JA)
            dma16(smem0 + ST * A_STAGE + (w * JA + d) * 1024,
                  L.a_k[d] < r.krem ? L.a_off[d] : kOob, r.a);
        else
            dma16(smem0 + A_REGION + ST * B_STAGE + (w * JB + d - JA) * 1024,
                  L.b_k[d - JA] < r.krem ? L.b_off[d - JA] : kOob, r.b);
    }

    template <int ST>
    static __device__ __forceinline__ void issue_copies(const Lane& L, const GemmParams& p,
                                                        int m0, int n0, int strip, int w,
                                                        u32 smem0)
    {
        const StripRes r = strip_res(p, m0, n0, strip);
#pragma unroll
        for (int d = 0; d < NCOPY; ++d)
            issue_copy<ST>(L, r, d, w, smem0);
    }

    // Fragment read i (0 .. NREAD-1) of slab s of stage ST.
    template <int ST, int S>
    static __device__ __forceinline__ void read_one(Frag& F, const Lane& L, lds_char* sm, int i)
    {
        if (i < FM) {
            const u32 off = L.a_rd[S] + ST * A_STAGE + i * 32 * (BK * 2);
            F.a[i] = *(const lds_u32x4*)(sm + off);
        } else {
            const int fn = (i - FM) >> 1, h = (i - FM) & 1;
            const u32 off = L.b_rd[fn] + ST * B_STAGE + (16 * S + 4 * h) * (BN * 2);
            F.b[fn][h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(sm + off));
        }
    }

    static __device__ __forceinline__ void mfma_one(f32x16 (&acc)[FM][FN], const Frag& F, int i)
    {
        const int fm = i / FN, fn = i % FN;
        const s16x8 b8 = __builtin_shufflevector(F.b[fn][0], F.b[fn][1], 0, 1, 2, 3, 4, 5, 6, 7);
        if constexpr (DT == DT_BF16)
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, b8), __builtin_bit_cast(bf16x8, F.a[fm]), acc[fm][fn], 0,
                0, 0);
        else
            acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                __builtin_bit_cast(f16x8, b8), __builtin_bit_cast(f16x8, F.a[fm]), acc[fm][fn], 0,
                0, 0);
    }

    // One strip: MFMAs on slab 0 (fragments F0) then slab 1 (F1), SLOTS MFMA
    // slots in all.
    //   slot 0, after its MFMA and read: wait for strip t + 1's copies and
    //           barrier; strip t + 1 is then visible and the stage of strip
    //           t - 1 is free;
    //   the NCOPY x NW copies of strip t + NS - 1 (NCOPY per wave) are spread
    //           evenly over the strip and staggered across the waves, so the
    //           address unit sees a steady stream instead of bursts that back
    //           up into the MFMA issue;
    //   slab 0 slots: reads of slab 1 into F1; slab 1 slots: reads of strip
    //           t + 1's slab 0 into F0.
    template <int ST, int W>
    static __device__ __forceinline__ void strip(f32x16 (&acc)[FM][FN], Frag& F0, Frag& F1,
                                                 const Lane& L, lds_char* sm, const GemmParams& p,
                                                 int m0, int n0, int t, u32 smem0)
    {
        constexpr int NXT = (ST + 1) % NS;
        constexpr int CPY = (ST + NS - 1) % NS;
        constexpr int NM = FM * FN;
        constexpr int STEPS = NM > NREAD ? NM : NREAD;
        constexpr int SLOTS = 2 * STEPS;
        StripRes r;
#pragma unroll
        for (int slot = 0; slot < SLOTS; ++slot) {
            const int i = slot % STEPS;
            if (slot < STEPS) {
                if (i < NM) {
                    mfma_one(acc, F0, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (i < NREAD) {
                    read_one<ST, 1>(F1, L, sm, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            } else {
                if (i < NM) {
                    mfma_one(acc, F1, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if (i < NREAD) {
                    read_one<NXT, 0>(F0, L, sm, i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            if (slot == 0) {
                wait_copies_barrier<VM_AHEAD>();
                __builtin_amdgcn_sched_barrier(0);
                r = strip_res(p, m0, n0, t + NS - 1);
            }
            // copy d of wave W goes to slot ((d * NW + W) * SLOTS) / (NCOPY * NW)
#pragma unroll
            for (int d = 0; d < NCOPY; ++d) {
                if (((d * NW + W) * SLOTS) / (NCOPY * NW) == slot) {
                    issue_copy<CPY>(L, r, d, W, smem0);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
    }

    // The strip loop of wave W (the copy slots differ per wave).  The strip
    // count is rounded up to a multiple of NS: strips at or past KT copy only
    // out-of-range zeros, which add exactly nothing.
    template <int W>
    static __device__ __forceinline__ void main_loop(f32x16 (&acc)[FM][FN], Frag& F0, Frag& F1,
                                                     const Lane& L, lds_char* sm,
                                                     const GemmParams& p, int m0, int n0, int KT,
                                                     u32 smem0)
    {
        for (int t = 0; t < KT; t += NS) {
            strip<0, W>(acc, F0, F1, L, sm, p, m0, n0, t, smem0);
            strip<1, W>(acc, F0, F1, L, sm, p, m0, n0, t + 1, smem0);
            strip<2, W>(acc, F0, F1, L, sm, p, m0, n0, t + 2, smem0);
            if constexpr (NS > 3)
                strip<3 % NS, W>(acc, F0, F1, L, sm, p, m0, n0, t + 3, smem0);
            if constexpr (NS > 4)
                strip<4 % NS, W>(acc, F0, F1, L, sm, p, m0, n0, t + 4, smem0);
        }
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
        const TileCoord tc = tile_of(blockIdx.x, p.tiles_m, p.tiles_n, GROUP_M);
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

        // prologue: strips 0 .. NS-2 into stages 0 .. NS-2
        issue_copies<0>(L, p, m0, n0, 0, w, smem0);
        issue_copies<1>(L, p, m0, n0, 1, w, smem0);
        if constexpr (NS > 3)
            issue_copies<2 % NS>(L, p, m0, n0, 2, w, smem0);
        if constexpr (NS > 4)
            issue_copies<3 % NS>(L, p, m0, n0, 3, w, smem0);
        static_assert(NS <= 5, "prologue written for up to 5 stages");
        // strip 0 must be complete and visible before its first fragments are read
        wait_copies_barrier<(NS - 2) * (JA + JB)>();
        Frag F0, F1;
#pragma unroll
        for (int i = 0; i < NREAD; ++i)
            read_one<0, 0>(F0, L, sm, i);

        switch (w) {
        case 0:
            main_loop<0>(acc, F0, F1, L, sm, p, m0, n0, KT, smem0);
            break;
        case 1:
            main_loop<1 % NW>(acc, F0, F1, L, sm, p, m0, n0, KT, smem0);
            break;
        case 2:
            main_loop<2 % NW>(acc, F0, F1, L, sm, p, m0, n0, KT, smem0);
            break;
        default:
            main_loop<3 % NW>(acc, F0, F1, L, sm, p, m0, n0, KT, smem0);
            break;
        }
        // drain the copies of the strips past the end (all out of range)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        epilogue(acc, p, m0, n0, wm, wn, lane);
    }
};

// Waves per SIMD the kernel is compiled for: one for the largest tiles (all
// 512 registers of a lane available, 256 of them accumulators), else two.
template <int BM, int BN>
struct DmaOcc {
    static constexpr int value = BM * BN >= 256 * 128 ? 1 : 2;
};

template <int DT, int BM, int BN, int WGM, int WGN, int NS, int GROUP_M>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * 64, WGM * WGN * 64),
                          amdgpu_waves_per_eu(DmaOcc<BM, BN>::value, DmaOcc<BM, BN>::value))) void
gemm_dma_kernel(GemmParams p)
{
    DmaGemm<DT, BM, BN, WGM, WGN, NS, GROUP_M>::run(p);
}

}  // namespace tg

#pragma clang diagnostic pop
