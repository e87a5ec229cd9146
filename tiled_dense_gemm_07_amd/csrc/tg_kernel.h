// Tiled GEMM kernel template for CDNA4 (gfx950).
//
// One workgroup owns a BM x BN tile of C and walks K in BK-deep strips, as in
// the mhpq.cn page's GEMM ("TileLang ... 一个高效 GEMM 内核", sections 2.1, 2.3,
// 3.2): the A strip (BM x BK) and the B strip (BK x BN) are staged in on-chip
// memory (LDS), an fp32 accumulator lives in registers (here the AccVGPRs fed
// by MFMA), and copies of the next strips overlap the math on the current one
// (section 3.3; the blog.hotdry.top page's num_stages = 3, 2-4 to start).
//
// MI355X-specific choices (not from the pages):
//  * LDS holds both operands "K-contiguous": A as [BM][BK], B as [BN][BK]
//    (row-major B is transposed in registers on its way into LDS; the 4-bit
//    weights [N][K] are K-contiguous already and are expanded to bf16 there).
//    Every MFMA operand fragment is then one 16-byte ds_read_b128 per lane.
//  * 16-byte chunks of each LDS row are XOR-swizzled by the row index, so the
//    global->LDS writes and the MFMA fragment reads are both free of bank
//    conflicts without padding (the pages pad a column instead, mhpq.cn 4.2).
//  * The MFMA is issued with the B fragment as its first operand, so each lane
//    ends up owning 4 consecutive columns of one row of C: the epilogue
//    (ReLU, one rounding to the output type, edge mask) stores 8 or 16 bytes.
//  * Global reads go through buffer instructions whose range check returns 0
//    past the end of the tile band, plus explicit masks for the ragged K and N
//    edges, so partial tiles need no second code path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tg_sched.h"

namespace tg {

typedef uint32_t u32;
typedef __attribute__((ext_vector_type(2))) u32 u32x2;
typedef __attribute__((ext_vector_type(4))) u32 u32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;

enum Dtype { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };
enum BMode { B_KN = 0, B_W4 = 1 };

template <int DT>
struct DtTraits;
template <>
struct DtTraits<DT_F32> {
    static constexpr int ES = 4;   // bytes per element
    static constexpr int VEC = 4;  // elements per 16-byte chunk
};
template <>
struct DtTraits<DT_F16> {
    static constexpr int ES = 2;
    static constexpr int VEC = 8;
};
template <>
struct DtTraits<DT_BF16> {
    static constexpr int ES = 2;
    static constexpr int VEC = 8;
};

struct GemmParams {
    const void* A;   // [M][K] row-major (MX: element codes, [M][K] or [M][K/2] bytes)
    const void* B;   // B_KN: [K][N] row-major; B_W4 and MX: packed codes [N][K/2]
    const void* Bs;  // B_W4 and MX: scale bytes [N][K/32]; unused otherwise
    const void* As;  // MX: scale bytes of A [M][K/32]; unused otherwise
    void* C;         // [M][N] row-major
    int M, N, K;
    int tiles_m, tiles_n;
    int relu;
    int c_vec;  // 1 if C rows allow 4-element vector stores
    // split K (register-staged kernel with k-slice groups only): splits > 1
    // workgroups per output tile, each over kc consecutive k (a multiple of
    // the strip depth); each writes its fp32 partial tile to ws, and the last
    // to arrive at the tile's counter sums the partials in split order and
    // runs the epilogue.  splits <= 1: no split, ws and counters unused.
    int splits;
    int kc;
    float* ws;      // [tiles][splits][BM * BN] fp32 partial tiles
    int* counters;  // [tiles] arrival counts, zero before and after each call
    // Optional clock record (a measurement aid, normally NULL): wave 0 of
    // workgroups 0..7 (one per XCD under round-robin dispatch) writes the
    // shader clock counter (s_memtime) and the 100 MHz reference counter
    // (s_memrealtime) at its start and end: stamps[4 b + 0..3] = t0, r0, t1, r1.
    unsigned long long* stamps;
    // Swizzle group (tile rows per group of the block-swizzled tile order);
    // 0: the configuration's compiled default.
    int group_m;
};

// The swizzle group a launch uses: its override, else the compiled default.
__device__ __forceinline__ int group_of(const GemmParams& p, int dflt)
{
    return p.group_m > 0 ? p.group_m : dflt;
}

struct ClockStamp {
    unsigned long long t, r;
    bool on;
};

__device__ __forceinline__ ClockStamp stamp_begin(const GemmParams& p)
{
    ClockStamp s{0, 0, false};
    if (p.stamps != nullptr && blockIdx.x < 8 &&
        __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) == 0) {
        s.t = __builtin_amdgcn_s_memtime();
        s.r = __builtin_amdgcn_s_memrealtime();
        s.on = true;
    }
    return s;
}

__device__ __forceinline__ void stamp_end(const GemmParams& p, const ClockStamp& s)
{
    if (s.on) {
        const unsigned long long t = __builtin_amdgcn_s_memtime();
        const unsigned long long r = __builtin_amdgcn_s_memrealtime();
        if (threadIdx.x == 0) {
            unsigned long long* o = p.stamps + 4 * blockIdx.x;
            o[0] = s.t;
            o[1] = s.r;
            o[2] = t;
            o[3] = r;
        }
    }
}

// --------------------------------------------------------------------------
// Buffer resources (range-checked global access).
// --------------------------------------------------------------------------
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, u32 bytes)
{
    // 4th dword 0x00020000: raw (untyped) 32-bit data format on gfx9-family parts
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}

constexpr u32 kOob = 0x80000000u;  // any offset >= num_records reads as 0

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, u32 off)
{
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32 buf_load4(__amdgpu_buffer_rsrc_t r, u32 off)
{
    return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32 buf_load2(__amdgpu_buffer_rsrc_t r, u32 off)
{
    return (u32)__builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32 buf_load1(__amdgpu_buffer_rsrc_t r, u32 off)
{
    return (u32)__builtin_amdgcn_raw_buffer_load_b8(r, (int)off, 0, 0);
}

__device__ __forceinline__ u32 clamp_bytes(int64_t b)
{
    return b <= 0 ? 0u : (b >= 0x7FFFFFFF ? 0x7FFFFFFFu : (u32)b);
}

// XOR swizzle of the 16-byte chunk index within an LDS row.  Rows are at
// least 128 bytes (8 chunks), so a group of 8 lanes that reads 8 consecutive
// rows at one logical chunk, or writes rows 8c + j for c = 0..7, touches 8
// different 16-byte bank groups.
__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

// --------------------------------------------------------------------------
// Output conversion (one rounding, nearest-even).
// --------------------------------------------------------------------------
__device__ __forceinline__ u32 pack2(float a, float b, int dt)
{
    if (dt == DT_BF16) {
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(u32, v);
    }
    _Float16 ha = (_Float16)a, hb = (_Float16)b;
    return (u32)__builtin_bit_cast(uint16_t, ha) | ((u32)__builtin_bit_cast(uint16_t, hb) << 16);
}
__device__ __forceinline__ uint16_t cvt1(float a, int dt)
{
    if (dt == DT_BF16)
        return __builtin_bit_cast(uint16_t, (__bf16)a);
    return __builtin_bit_cast(uint16_t, (_Float16)a);
}

// Write-back of a staged result tile from LDS (rows of CH 16-byte chunks,
// chunk c of row r at c ^ (r % CH)) to C (element size ES), RPI rows per
// store instruction.  The stores use the system-coherent write-through
// policy (SC0 SC1): the results stream to memory as they are stored instead
// of sitting dirty in L2 for the end-of-kernel write-back, which all tiles
// reach at once.  Measured on the 4096^3 bf16 kernel: 108.3 -> 104.2 us.
// Each group of RPI rows gets its own buffer base (uniform), so offsets stay
// below RPI rows.
constexpr int kStoreThrough = 17;  // SC0 | SC1

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

template <int WTM, int RPI, int CH, int ES>
__device__ __forceinline__ void store_rows_through(const lds_char* st, const GemmParams& p,
                                                   int mw0, int nw0, int lane)
{
    constexpr int ROWB = CH * 16;
    constexpr int EPC = 16 / ES;  // elements per 16-byte chunk
    const int c = lane % CH;
    const int rl = lane / CH;  // row within a store instruction
    const int n = nw0 + EPC * c;
    const u32 off = (u32)(rl * p.N + EPC * c) * (u32)ES;
    char* C = (char*)p.C;
#pragma unroll 4
    for (int r0 = 0; r0 < WTM; r0 += RPI) {
        const int r = r0 + rl;
        const u32x4 v = *(const lds_u32x4*)(st + r * ROWB + ((c ^ (r & (CH - 1))) << 4));
        const auto rs = make_rsrc(C + ((int64_t)(mw0 + r0) * p.N + nw0) * ES, 0x7FFFFFFFu);
        if (mw0 + r < p.M && n < p.N)
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, (int)off, 0, kStoreThrough);
    }
}

// Coalesced store of one wave's WTM x WTN result tile (FM x FN blocks of
// 32 x 32 fp32, the MFMA layout where lane l holds row l % 32 and, for
// element 4 q + e, column 8 q + 4 (l / 32) + e of its block).  The tile is
// rounded (after ReLU) into the wave's own LDS region `st` as rows of
// WTN * ES bytes with 16-byte chunk c of row r at position c ^ (r % CH) (CH
// chunks per row; writes then spread over the banks), and written back to C
// as 16-byte pieces, CH lanes per row: whole row runs instead of 8- or
// 16-byte pieces of 32 rows.  Needs N a multiple of 16 / ES and a 16-byte
// aligned C (else the caller stores directly); the caller has synchronised
// so that no wave still reads or copies into the wave's region.
template <int DT, int WTM, int WTN, int FM, int FN>
__device__ __forceinline__ void store_tile_staged(const f32x16 (&acc)[FM][FN],
                                                  const GemmParams& p, int mw0, int nw0,
                                                  int lane, lds_char* st)
{
    constexpr int ES = DT == DT_F32 ? 4 : 2;
    constexpr int ROWB = WTN * ES;
    constexpr int CH = ROWB / 16;
    static_assert(CH >= 4 && CH <= 64 && (CH & (CH - 1)) == 0, "rows of 64 to 1024 bytes");
    const int lr = lane & 31;
    const int g = lane >> 5;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
        const int r = fm * 32 + lr;
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float x = acc[fm][fn][4 * q + e];
                    v[e] = (p.relu && !(x > 0.0f)) ? 0.0f : x;
                }
                if constexpr (DT == DT_F32) {
                    const int c = 8 * fn + 2 * q + g;  // 4 floats: one whole chunk
                    *(lds_u32x4*)(st + r * ROWB + ((c ^ (r & (CH - 1))) << 4)) =
                        __builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]});
                } else {
                    const int c = 4 * fn + q;  // 4 halves: one half chunk
                    *(lds_u32x2*)(st + r * ROWB + ((c ^ (r & (CH - 1))) << 4) + 8 * g) =
                        u32x2{pack2(v[0], v[1], DT), pack2(v[2], v[3], DT)};
                }
            }
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // own region: no barrier needed
    constexpr int RPI = 64 / CH;  // rows per store instruction
    store_rows_through<WTM, RPI, CH, ES>(st, p, mw0, nw0, lane);
}


// Scale operand of the v_cvt_scalef32_pk_*_fp4 conversions for E8M0 byte e
// (0 .. 255, the scale 2^(e - 127), 255 NaN).  Those instructions take the
// scale from the exponent field of the fp32 they are given, so the byte
// moved into that field serves as is: for every scale byte and every pair of
// codes the results equal those for the decoded value (2^-127 as the fp32
// subnormal for e = 0, a NaN for 255), bit for bit on the GPU, without the
// two compares and selects the decoding takes.
__device__ __forceinline__ float e8m0_cvt_scale(u32 e)
{
    return __builtin_bit_cast(float, e << 23);
}

// --------------------------------------------------------------------------
// The kernel.
// --------------------------------------------------------------------------
// KS > 1 slices each strip's k range over KS groups of WGM x WGN waves: every
// group multiplies the whole tile over its share of the strip's slabs, and the
// groups' partial accumulators are summed through LDS before the epilogue.
// This puts KS times more waves on a tile, for shapes whose tile grid alone
// cannot occupy the compute units.
template <int DT, int BMODE, int BM, int BN, int BK, int WGM, int WGN, int STAGES, int GROUP_M,
          bool WIDE, int PIPE, bool TA = false, bool TB = false, int KS = 1>
struct GemmKernel {
    using TR = DtTraits<DT>;
    static constexpr int ES = TR::ES;
    static constexpr int VEC = TR::VEC;
    static constexpr int NT = WGM * WGN * KS * 64;
    static constexpr int WTM = BM / WGM;
    static constexpr int WTN = BN / WGN;
    static constexpr int FM = WTM / 32;
    static constexpr int FN = WTN / 32;
    static constexpr int CPR = BK / VEC;         // 16-byte chunks per LDS row
    static constexpr int NSLAB = BK / (2 * VEC);  // MFMA k-slabs per strip
    static constexpr int ROWB = BK * ES;          // bytes per LDS row
    static constexpr int A_STAGE = BM * ROWB;
    static constexpr int B_STAGE = BN * ROWB;
    static constexpr int STAGE_BYTES = A_STAGE + B_STAGE;
    static constexpr int RING_BYTES = STAGES * STAGE_BYTES;
    static constexpr int NSL = NSLAB / KS;  // slabs per wave group per strip
    // partial accumulators of wave groups 1 .. KS-1 (fp32 tile each)
    static constexpr int RED_BYTES = (KS - 1) * BM * BN * 4;
    static constexpr int LDS_BYTES = RING_BYTES > RED_BYTES ? RING_BYTES : RED_BYTES;

    // Chunk swizzle of LDS row `row`.  Rows of 128 bytes take swz.  Rows of
    // 16 or more chunks all start on the same bank: a b128 read pass (16
    // lanes, 256 bytes: 16 consecutive rows at one logical chunk) needs 16
    // different positions, and a b128 write pass (8 lanes, 128 bytes: the
    // transposing stores put rows UW = 1, 2, 4 or 8 apart at one chunk) 8
    // different positions mod 8.  swz keeps the latter and row bit 3 adds
    // the fourth bit for the former.
    static __device__ __forceinline__ int sw(int row)
    {
        if constexpr (CPR >= 16)
            return swz(row) | (row & 8);
        else
            return swz(row);
    }

    // Both operands sit in LDS k-contiguous ([rows][BK], 16-byte chunk
    // swizzle).  In global memory an operand is either k-contiguous (KOp: X
    // rows of K consecutive elements: A as [M][K], B stored [N][K]) or
    // x-contiguous (XOp: K rows of X consecutive elements: B as [K][N], A
    // stored [K][M]), which is transposed in registers on its way to LDS.
    template <int X>
    struct KOp {
        static constexpr int NCH = X * CPR / NT;  // 16-byte chunks per thread
        static_assert(X * CPR % NT == 0 && NCH >= 1, "strip must split evenly over threads");
        static constexpr int NREG = NCH;

        // rows x0 .. of an operand with xtot rows of ld = K elements; k at or
        // past kend reads as zero
        static __device__ __forceinline__ void load(u32x4 (&dst)[NREG], const void* ptr, int x0,
                                                    int xtot, int K, int k0, int kend, int tid)
        {
            const char* base = (const char*)ptr + ((int64_t)x0 * K + k0) * ES;
            const int rows_valid = xtot - x0;
            const int64_t bytes = ((int64_t)(rows_valid - 1) * K + (K - k0)) * ES;
            const auto rs = make_rsrc(base, clamp_bytes(bytes));
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int q = tid + NT * i;
                const int row = q / CPR;
                const int c = q % CPR;
                const int kk = c * VEC;  // k offset within the strip
                const bool rv = row < rows_valid;
                const u32 off = (u32)(row * K + kk) * ES;
                if (WIDE) {
                    const bool v = rv && (k0 + kk < kend);
                    dst[i] = buf_load16(rs, v ? off : kOob);
                } else {
                    u32 w[4] = {0, 0, 0, 0};
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        const bool v = rv && (k0 + kk + e < kend);
                        const u32 o = v ? off + e * ES : kOob;
                        if (ES == 4)
                            w[e] = buf_load4(rs, o);
                        else
                            w[e / 2] |= buf_load2(rs, o) << (16 * (e & 1));
                    }
                    dst[i] = u32x4{w[0], w[1], w[2], w[3]};
                }
            }
        }

        static __device__ __forceinline__ void store(const u32x4 (&src)[NREG], char* S, int tid)
        {
#pragma unroll
            for (int i = 0; i < NCH; ++i) {
                const int q = tid + NT * i;
                const int row = q / CPR;
                const int c = q % CPR;
                *(u32x4*)(S + row * ROWB + ((c ^ sw(row)) << 4)) = src[i];
            }
        }
    };

    // Units of VEC k-rows by UW x-columns (UW <= VEC), so that every thread
    // owns a whole number of units; a unit is UW*ES-byte loads of VEC rows,
    // transposed into UW LDS rows of one 16-byte chunk.
    template <int X>
    struct XOp {
        static constexpr int UW_RAW = (BK / VEC) * X / NT;
        static constexpr int UW = UW_RAW >= VEC ? VEC : UW_RAW;
        static constexpr int NU = (BK / VEC) * (X / (UW > 0 ? UW : 1)) / NT;
        static_assert(UW >= 1 && (UW & (UW - 1)) == 0 && ((BK / VEC) * (X / UW)) % NT == 0 &&
                          NU >= 1,
                      "units must split evenly");
        static_assert(UW * ES >= 4, "loads of at least 4 bytes");
        static constexpr int NREG = NU * VEC;

        // columns x0 .. of an operand stored as K rows of ld = xtot elements;
        // rows at or past kend read as zero
        static __device__ __forceinline__ void load(u32x4 (&dst)[NREG], const void* ptr, int x0,
                                                    int xtot, int K, int k0, int kend, int tid)
        {
            const int ld = xtot;
            const char* base = (const char*)ptr + ((int64_t)k0 * ld + x0) * ES;
            const int64_t bytes = ((int64_t)(K - k0 - 1) * ld + (xtot - x0)) * ES;
            const auto rs = make_rsrc(base, clamp_bytes(bytes));
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                const int u = tid + NT * i;
                const int nc = u % (X / UW);
                const int kg = u / (X / UW);
                const int nn = nc * UW;
#pragma unroll
                for (int r = 0; r < VEC; ++r) {
                    const int kr = kg * VEC + r;  // k row within the strip
                    const bool kv = k0 + kr < kend;
                    const u32 off = (u32)(kr * ld + nn) * ES;
                    u32x4 w = {0, 0, 0, 0};
                    if (WIDE) {
                        const u32 o = (kv && x0 + nn < xtot) ? off : kOob;
                        if constexpr (UW * ES == 16) {
                            w = buf_load16(rs, o);
                        } else if constexpr (UW * ES == 8) {
                            const u32x2 h = __builtin_bit_cast(
                                u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)o, 0, 0));
                            w[0] = h[0];
                            w[1] = h[1];
                        } else {
                            w[0] = buf_load4(rs, o);
                        }
                    } else {
#pragma unroll
                        for (int e = 0; e < UW; ++e) {
                            const bool v = kv && (x0 + nn + e < xtot);
                            const u32 o = v ? off + e * ES : kOob;
                            if (ES == 4)
                                w[e] = buf_load4(rs, o);
                            else
                                w[e / 2] |= buf_load2(rs, o) << (16 * (e & 1));
                        }
                    }
                    dst[i * VEC + r] = w;
                }
            }
        }

        static __device__ __forceinline__ void store(const u32x4 (&src)[NREG], char* S, int tid)
        {
#pragma unroll
            for (int i = 0; i < NU; ++i) {
                const int u = tid + NT * i;
                const int nc = u % (X / UW);
                const int kg = u / (X / UW);
                const u32x4* L = &src[i * VEC];
#pragma unroll
                for (int j = 0; j < UW; ++j) {
                    u32x4 o;
                    if (ES == 4) {
                        // 4 k-rows of fp32: column j
                        o = u32x4{L[0][j], L[1][j], L[2][j], L[3][j]};
                    } else {
                        // 8 k-rows of 16-bit values: column j, k pairs packed low-to-high
                        const u32 sel = (j & 1) ? 0x07060302u : 0x05040100u;
                        const int d = j >> 1;
                        o = u32x4{__builtin_amdgcn_perm(L[1][d], L[0][d], sel),
                                  __builtin_amdgcn_perm(L[3][d], L[2][d], sel),
                                  __builtin_amdgcn_perm(L[5][d], L[4][d], sel),
                                  __builtin_amdgcn_perm(L[7][d], L[6][d], sel)};
                    }
                    const int n = nc * UW + j;
                    *(u32x4*)(S + n * ROWB + ((kg ^ sw(n)) << 4)) = o;
                }
            }
        }
    };

    using OpA = typename std::conditional<TA, XOp<BM>, KOp<BM>>::type;
    using OpB = typename std::conditional<TB, KOp<BN>, XOp<BN>>::type;

    // B (4-bit weights): units of CU codes (CU/2 bytes) of one weight row,
    // CU in {8, 16, 32}, all under one scale byte
    static constexpr int CU_RAW = BN * BK / NT;
    static constexpr int CU = CU_RAW >= 32 ? 32 : CU_RAW;
    static constexpr int BU_W4 = BN * BK / (CU > 0 ? CU : 1) / NT;

    static_assert(DT != DT_F32 || BMODE == B_KN, "4-bit weights feed the bf16 path only");
    static_assert(BMODE == B_KN || DT == DT_BF16, "4-bit weights feed the bf16 path only");
    static_assert(BMODE == B_KN || (!TA && !TB), "4-bit weights: row-major activations only");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be 32x32 blocks");
    static_assert(CPR >= 8 && (CPR & (CPR - 1)) == 0, "LDS rows must be >= 128 B, power of 2");
    static_assert(BK % (2 * VEC) == 0, "BK must hold whole MFMA k-slabs");
    static_assert(BMODE != B_W4 || (CU >= 8 && (CU & (CU - 1)) == 0 && BU_W4 >= 1 &&
                                    (BN * BK / CU) % NT == 0),
                  "W4 units must split evenly");
    static_assert(BMODE != B_W4 || BK % 32 == 0, "W4 strips hold whole scale groups");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
    static_assert(STAGES >= 2, "at least double buffering");
    static_assert(KS >= 1 && NSLAB % KS == 0, "k slices split each strip's slabs evenly");
    static_assert(KS == 1 || BMODE == B_KN, "k slices: plain operands only");

    struct Regs {
        u32x4 a[OpA::NREG];
        u32x4 b[BMODE == B_KN ? OpB::NREG : BU_W4];
        u32 s[BMODE == B_W4 ? BU_W4 : 1];
    };

    // ---- global -> registers --------------------------------------------
    // strip k0 .. k0 + BK; k at or past kend reads as zero
    static __device__ __forceinline__ void load_a(Regs& R, const GemmParams& p, int m0, int k0,
                                                  int kend, int tid)
    {
        OpA::load(R.a, p.A, m0, p.M, p.K, k0, kend, tid);
    }

    static __device__ __forceinline__ void load_b(Regs& R, const GemmParams& p, int n0, int k0,
                                                  int kend, int tid)
    {
        if constexpr (BMODE == B_KN) {
            OpB::load(R.b, p.B, n0, p.N, p.K, k0, kend, tid);
        } else {
            // packed codes: row n has K/2 bytes; this strip covers bytes k0/2 .. (k0+BK)/2
            const int rows_valid = p.N - n0;
            const int rowb = p.K / 2;
            const char* base = (const char*)p.B + (int64_t)n0 * rowb + k0 / 2;
            const int64_t bytes = (int64_t)(rows_valid - 1) * rowb + (rowb - k0 / 2);
            const auto rs = make_rsrc(base, clamp_bytes(bytes));
            const int srow = p.K / 32;
            const char* sbase = (const char*)p.Bs + (int64_t)n0 * srow + k0 / 32;
            const int64_t sbytes = (int64_t)(rows_valid - 1) * srow + (srow - k0 / 32);
            const auto ss = make_rsrc(sbase, clamp_bytes(sbytes));
            constexpr int UPR = BK / CU;  // units per row
#pragma unroll
            for (int i = 0; i < BU_W4; ++i) {
                const int u = tid + NT * i;
                const int row = u / UPR;
                const int g = u % UPR;
                const int kk = g * CU;  // first code of this unit within the strip
                const bool v = row < rows_valid && (k0 + kk < p.K);
                const u32 off = (u32)(row * rowb + kk / 2);
                u32x4 w = {0, 0, 0, 0};
                if (WIDE) {
                    const u32 o = v ? off : kOob;
                    if constexpr (CU == 32) {
                        w = buf_load16(rs, o);
                    } else if constexpr (CU == 16) {
                        const u32x2 h = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rs, (int)o, 0, 0));
                        w[0] = h[0];
                        w[1] = h[1];
                    } else {
                        w[0] = buf_load4(rs, o);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < CU / 2; ++e)
                        w[e / 4] |= buf_load1(rs, v ? off + e : kOob) << (8 * (e & 3));
                }
                R.b[i] = w;
                R.s[i] = buf_load1(ss, v ? (u32)(row * srow + kk / 32) : kOob);
            }
        }
    }

    // ---- registers -> LDS ---------------------------------------------------
    static __device__ __forceinline__ void store_lds(const Regs& R, char* stage, int tid)
    {
        char* As = stage;
        char* Bs = stage + A_STAGE;
        OpA::store(R.a, As, tid);
        if constexpr (BMODE == B_KN) {
            OpB::store(R.b, Bs, tid);
        } else {
            constexpr int UPR = BK / CU;
#pragma unroll
            for (int i = 0; i < BU_W4; ++i) {
                const int u = tid + NT * i;
                const int row = u / UPR;
                const int g = u % UPR;
                const float sc = e8m0_cvt_scale(R.s[i]);
#pragma unroll
                for (int cc = 0; cc < CU / 8; ++cc) {
                    const u32 packed = R.b[i][cc];  // 8 codes: k = 8cc .. 8cc+7 of this unit
                    u32x4 o;
                    o[0] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 0));
                    o[1] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 1));
                    o[2] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 2));
                    o[3] = __builtin_bit_cast(u32, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(packed, sc, 3));
                    const int chunk = g * (CU / 8) + cc;
                    *(u32x4*)(Bs + row * ROWB + ((chunk ^ sw(row)) << 4)) = o;
                }
            }
        }
    }

    // ---- LDS -> MFMA ---------------------------------------------------------
    // Fragments of one k-slab (two 16-byte chunks deep): lane l reads chunk
    // 2s + l/32 of LDS row (fragment base + l%32), for FM A-blocks and FN B-blocks.
    struct Frags {
        u32x4 a[FM];
        u32x4 b[FN];
    };

    static __device__ __forceinline__ void read_frags(Frags& F, const char* stage, int s, int wm,
                                                      int wn, int lane)
    {
        const char* As = stage;
        const char* Bs = stage + A_STAGE;
        const int lr = lane & 31;
        const int chunk = 2 * s + (lane >> 5);
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
            const int row = wm * WTM + fm * 32 + lr;
            F.a[fm] = *(const u32x4*)(As + row * ROWB + ((chunk ^ sw(row)) << 4));
        }
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int row = wn * WTN + fn * 32 + lr;
            F.b[fn] = *(const u32x4*)(Bs + row * ROWB + ((chunk ^ sw(row)) << 4));
        }
    }

    static __device__ __forceinline__ void mfma_slab(f32x16 (&acc)[FM][FN], const Frags& F)
    {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                if constexpr (DT == DT_F32) {
                    // cast whole vectors: clang reads element 0 when
                    // __builtin_bit_cast is applied to a vector element
                    const f32x4 bv = __builtin_bit_cast(f32x4, F.b[fn]);
                    const f32x4 av = __builtin_bit_cast(f32x4, F.a[fm]);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(bv[e], av[e],
                                                                           acc[fm][fn], 0, 0, 0);
                } else if constexpr (DT == DT_F16) {
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                        __builtin_bit_cast(f16x8, F.b[fn]), __builtin_bit_cast(f16x8, F.a[fm]),
                        acc[fm][fn], 0, 0, 0);
                } else {
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, F.b[fn]), __builtin_bit_cast(bf16x8, F.a[fm]),
                        acc[fm][fn], 0, 0, 0);
                }
            }
        }
    }

    static __device__ __forceinline__ void compute(f32x16 (&acc)[FM][FN], const char* stage,
                                                   int s0, int wm, int wn, int lane)
    {
#pragma unroll
        for (int s = 0; s < NSL; ++s) {
            Frags F;
            read_frags(F, stage, s0 + s, wm, wn, lane);
            mfma_slab(acc, F);
        }
    }

    // Sum the k-slice groups' accumulators into group 0's (KS > 1).  Entered
    // by all waves after the last use of the LDS ring; group 0 holds the
    // tile's sums on return.
    static __device__ __forceinline__ void reduce_slices(f32x16 (&acc)[FM][FN], char* smem,
                                                         int ks, int w2, int lane)
    {
        if constexpr (KS > 1) {
            constexpr int WB = FM * FN * 64 * 64;  // bytes of one wave's accumulators
            __syncthreads();
            if (ks > 0) {
                char* dst = smem + ((ks - 1) * WGM * WGN + w2) * WB;
#pragma unroll
                for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int q = 0; q < 4; ++q)
                            *(f32x4*)(dst + (((fm * FN + fn) * 4 + q) * 64 + lane) * 16) =
                                f32x4{acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1],
                                      acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
            }
            __syncthreads();
            if (ks == 0) {
#pragma unroll
                for (int g = 1; g < KS; ++g) {
                    const char* src = smem + ((g - 1) * WGM * WGN + w2) * WB;
#pragma unroll
                    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const f32x4 v = *(const f32x4*)(
                                    src + (((fm * FN + fn) * 4 + q) * 64 + lane) * 16);
#pragma unroll
                                for (int e = 0; e < 4; ++e)
                                    acc[fm][fn][4 * q + e] += v[e];
                            }
                }
            }
        }
    }

    // ---- result store ------------------------------------------------------------
    // Staged through LDS (store_tile_staged: whole row runs, write-through)
    // when C is 16-byte aligned with rows of whole 16-byte chunks and the
    // wave tiles fit the LDS; else direct per-lane stores (epilogue below).
    static constexpr int SROW = WTN * ES / 16;  // 16-byte chunks per staged row
    static constexpr bool STAGED =
        SROW >= 4 && SROW <= 64 && (SROW & (SROW - 1)) == 0 && WGM * WGN * WTM * WTN * ES <= LDS_BYTES;

    static __device__ __forceinline__ void finish(const f32x16 (&acc)[FM][FN], char* smem,
                                                  const GemmParams& p, int m0, int n0, int ks,
                                                  int w2, int wm, int wn, int lane)
    {
        if constexpr (STAGED) {
            if (p.N % (16 / ES) == 0 && ((uintptr_t)p.C & 15) == 0) {
                __syncthreads();  // no wave still reads the ring or the slice partials
                if (ks == 0)
                    store_tile_staged<DT, WTM, WTN, FM, FN>(
                        acc, p, m0 + wm * WTM, n0 + wn * WTN, lane,
                        (lds_char*)smem + w2 * (WTM * WTN * ES));
                return;
            }
        }
        if (ks == 0)
            epilogue(acc, p, m0, n0, wm, wn, lane);
    }

    // ---- epilogue: ReLU, one rounding, edge-masked stores -----------------------
    static __device__ __forceinline__ void epilogue(const f32x16 (&acc)[FM][FN],
                                                    const GemmParams& p, int m0, int n0, int wm,
                                                    int wn, int lane)
    {
        const int lr = lane & 31;
        const int g = lane >> 5;
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
                        float x = acc[fm][fn][4 * q + e];
                        v[e] = (p.relu && !(x > 0.0f)) ? 0.0f : x;
                    }
                    const int64_t idx = (int64_t)m * p.N + n;
                    if (DT == DT_F32) {
                        float* C = (float*)p.C;
                        if (p.c_vec && n + 3 < p.N) {
                            *(f32x4*)(C + idx) = f32x4{v[0], v[1], v[2], v[3]};
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e)
                                if (n + e < p.N)
                                    C[idx + e] = v[e];
                        }
                    } else {
                        uint16_t* C = (uint16_t*)p.C;
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
    }

    static __device__ __forceinline__ void run(const GemmParams& p)
    {
        __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int ks = wave / (WGM * WGN);  // k-slice group
        const int w2 = wave % (WGM * WGN);
        const int wm = w2 / WGN;
        const int wn = w2 % WGN;
        const TileCoord t = tile_of(blockIdx.x, p.tiles_m, p.tiles_n, group_of(p, GROUP_M));
        const int m0 = t.m * BM;
        const int n0 = t.n * BN;
        const int KT = (p.K + BK - 1) / BK;

        f32x16 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[fm][fn][r] = 0.0f;

        Regs R;
        // prologue: fill STAGES-1 strips
#pragma unroll
        for (int s = 0; s < STAGES - 1; ++s) {
            if (s < KT) {
                load_a(R, p, m0, s * BK, p.K, tid);
                load_b(R, p, n0, s * BK, p.K, tid);
                store_lds(R, smem + s * STAGE_BYTES, tid);
            }
        }
        __syncthreads();

        for (int it = 0; it < KT; ++it) {
            const int nxt = it + STAGES - 1;
            if (nxt < KT) {
                load_a(R, p, m0, nxt * BK, p.K, tid);
                load_b(R, p, n0, nxt * BK, p.K, tid);
            }
            compute(acc, smem + (it % STAGES) * STAGE_BYTES, ks * NSL, wm, wn, lane);
            if (nxt < KT)
                store_lds(R, smem + (nxt % STAGES) * STAGE_BYTES, tid);
            __syncthreads();
        }

        reduce_slices(acc, smem, ks, w2, lane);
        finish(acc, smem, p, m0, n0, ks, w2, wm, wn, lane);
    }

    // Deep pipeline (two LDS stages, two register staging sets): the global
    // loads for strip t+3 are issued while strip t is multiplied, so each load
    // has about two strips of MFMA work to land; strip t+1 is written from
    // registers into the free LDS stage two slabs before the end of strip t;
    // and the fragments of slab s+1 are read while slab s is multiplied, the
    // first slab of the next strip right after the one barrier per strip.
    static __device__ __forceinline__ void strip_deep(f32x16 (&acc)[FM][FN], Regs& R,
                                                      Frags& Fa, Frags& Fb, char* smem,
                                                      const GemmParams& p, int it, int kbeg,
                                                      int kend, int m0, int n0, int s0, int wm,
                                                      int wn, int tid, int lane)
    {
        static_assert(NSL % 2 == 0 && NSL >= 2, "slab fragments alternate in pairs");
        char* cur = smem + (it & 1) * STAGE_BYTES;
        char* nxt = smem + ((it + 1) & 1) * STAGE_BYTES;
#pragma unroll
        for (int s = 0; s < NSL; ++s) {
            Frags& F = (s & 1) ? Fb : Fa;    // slab s
            Frags& G = (s & 1) ? Fa : Fb;    // slab s + 1 (or the first slab of the next strip)
            if (s + 1 < NSL)
                read_frags(G, cur, s0 + s + 1, wm, wn, lane);
            // No branches in the steady state: a strip past the end of K loads as
            // out-of-range zeros and is written to (or read from) an LDS stage
            // nothing uses, which keeps the wait counters exact.
            if (s == NSL - 2) {
                store_lds(R, nxt, tid);
                load_a(R, p, m0, kbeg + (it + 3) * BK, kend, tid);
                load_b(R, p, n0, kbeg + (it + 3) * BK, kend, tid);
            }
            if (s == NSL - 1) {
                __syncthreads();
                read_frags(G, nxt, s0, wm, wn, lane);
            }
            mfma_slab(acc, F);
        }
    }

    static __device__ __forceinline__ void run_deep(const GemmParams& p)
    {
        static_assert(STAGES == 2, "the deep pipeline uses two LDS stages");
        __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];
        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = tid >> 6;
        const int ks = wave / (WGM * WGN);  // k-slice group
        const int w2 = wave % (WGM * WGN);
        const int wm = w2 / WGN;
        const int wn = w2 % WGN;
        const int s0 = ks * NSL;
        // split K: the workgroups of one tile are consecutive ids
        const int S = (KS > 1 && p.splits > 1) ? p.splits : 1;
        const int tile = S > 1 ? (int)blockIdx.x / S : (int)blockIdx.x;
        const int sp = (int)blockIdx.x - tile * S;
        const int kbeg = S > 1 ? sp * p.kc : 0;
        const int kend = S > 1 ? min(p.K, kbeg + p.kc) : p.K;
        const TileCoord t = tile_of(tile, p.tiles_m, p.tiles_n, group_of(p, GROUP_M));
        const int m0 = t.m * BM;
        const int n0 = t.n * BN;
        const int KT = (kend - kbeg + BK - 1) / BK;

        f32x16 acc[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    acc[fm][fn][r] = 0.0f;

        Regs X, Y;
        Frags Fa, Fb;
        // strips at or past kend load as zeros (all offsets out of range)
        load_a(X, p, m0, kbeg, kend, tid);
        load_b(X, p, n0, kbeg, kend, tid);
        store_lds(X, smem, tid);
        load_a(X, p, m0, kbeg + BK, kend, tid);
        load_b(X, p, n0, kbeg + BK, kend, tid);
        load_a(Y, p, m0, kbeg + 2 * BK, kend, tid);
        load_b(Y, p, n0, kbeg + 2 * BK, kend, tid);
        __syncthreads();
        read_frags(Fa, smem, s0, wm, wn, lane);
        // an even number of strips: a trailing all-zero strip adds nothing
        for (int it = 0; it < KT; it += 2) {
            strip_deep(acc, X, Fa, Fb, smem, p, it, kbeg, kend, m0, n0, s0, wm, wn, tid, lane);
            strip_deep(acc, Y, Fa, Fb, smem, p, it + 1, kbeg, kend, m0, n0, s0, wm, wn, tid,
                       lane);
        }
        reduce_slices(acc, smem, ks, w2, lane);
        if constexpr (KS > 1) {
            if (S > 1) {
                split_fixup(acc, smem, p, tile, sp, S, m0, n0, ks, w2, wm, wn, tid, lane);
                return;
            }
        }
        finish(acc, smem, p, m0, n0, ks, w2, wm, wn, lane);
    }

    // Split K: every workgroup of the tile stores its partial tile (k-slice
    // group 0's sums) and counts itself in at the tile's counter; the last to
    // arrive resets the counter, sums all partials in split order 0 .. S-1
    // (its own from registers), so the result does not depend on arrival
    // order, and runs the epilogue.  No workgroup waits for another.
    //
    // The partial tiles are written and read with device-scope cache policy
    // (the write goes through this XCD's L2 to memory, the read does not take
    // a stale line from another XCD's L2), so the hand-off needs no L2
    // write-back or invalidate: the stores are complete (vmcnt drained at the
    // barrier) before thread 0's device-scope atomic counts the workgroup in.
    static constexpr int kDeviceScope = 16;  // SC1: coherent across the device's L2s

    static __device__ __forceinline__ void split_fixup(const f32x16 (&acc)[FM][FN], char* smem,
                                                       const GemmParams& p, int tile, int sp,
                                                       int S, int m0, int n0, int ks, int w2,
                                                       int wm, int wn, int tid, int lane)
    {
        constexpr int WB = FM * FN * 64 * 64;  // bytes of one wave's accumulators
        const auto rs = make_rsrc(p.ws + (int64_t)tile * S * (BM * BN), (u32)(S * BM * BN * 4));
        if (ks == 0) {
            const u32 dst = (u32)(sp * (BM * BN * 4) + w2 * WB);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        // whole-vector cast: clang reads element 0 when
                        // __builtin_bit_cast is applied to a vector element
                        __builtin_amdgcn_raw_buffer_store_b128(
                            __builtin_bit_cast(u32x4, f32x4{acc[fm][fn][4 * q],
                                                            acc[fm][fn][4 * q + 1],
                                                            acc[fm][fn][4 * q + 2],
                                                            acc[fm][fn][4 * q + 3]}),
                            rs, (int)(dst + (((fm * FN + fn) * 4 + q) * 64 + lane) * 16), 0,
                            kDeviceScope);
        }
        __builtin_amdgcn_s_waitcnt(0);  // this wave's partial stores are complete
        __syncthreads();
        int* flag = (int*)smem;
        if (tid == 0) {
            const int old = atomicAdd(p.counters + tile, 1);
            const int last = old == S - 1;
            if (last)
                atomicExch(p.counters + tile, 0);
            *flag = last;
        }
        __syncthreads();
        if (!*flag || ks != 0)
            return;
        f32x16 sum[FM][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    sum[fm][fn][r] = 0.0f;
        for (int g = 0; g < S; ++g) {
            const u32 src = (u32)(g * (BM * BN * 4) + w2 * WB);
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        f32x4 v;
                        if (g == sp)
                            v = f32x4{acc[fm][fn][4 * q], acc[fm][fn][4 * q + 1],
                                      acc[fm][fn][4 * q + 2], acc[fm][fn][4 * q + 3]};
                        else
                            v = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           rs, (int)(src + (((fm * FN + fn) * 4 + q) * 64 + lane) * 16),
                                           0, kDeviceScope));
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sum[fm][fn][4 * q + e] += v[e];
                    }
        }
        epilogue(sum, p, m0, n0, wm, wn, lane);
    }
};

// PIPE 0: one register staging set, STAGES-deep LDS ring.
// PIPE 1: the deep pipeline above (two register sets, two LDS stages).
template <int DT, int BMODE, int BM, int BN, int BK, int WGM, int WGN, int STAGES, int GROUP_M,
          bool WIDE, int PIPE, bool TA = false, bool TB = false, int KS = 1>
__global__ __attribute__((amdgpu_flat_work_group_size(WGM * WGN * KS * 64,
                                                       WGM * WGN * KS * 64))) void
gemm_kernel(GemmParams p)
{
    using Kern =
        GemmKernel<DT, BMODE, BM, BN, BK, WGM, WGN, STAGES, GROUP_M, WIDE, PIPE, TA, TB, KS>;
    const ClockStamp clk = stamp_begin(p);
    if constexpr (PIPE == 1)
        Kern::run_deep(p);
    else
        Kern::run(p);
    stamp_end(p, clk);
}

}  // namespace tg
