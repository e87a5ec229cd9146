/*
 * tilegemm — tiled dense GEMM, weight-only 4-bit dequant GEMM, MX-format GEMM
 * and 2:4 structured-sparse GEMM for one AMD Instinct MI355X (gfx950), as
 * hand-written HIP kernels behind a C ABI.
 *
 * The operation follows the pages' problem statement:
 *   - "TileLang ... 一个高效 GEMM 内核" (mhpq.cn), section 3.2: the caller
 *     allocates A (M x K), B (K x N) and C (M x N) on the device and launches
 *     kernel(A, B, C); the result is C = A x B.  Section 3.4 checks that the
 *     inner dimensions agree before launching.
 *   - "TileLang：用Python DSL简化GPU算子开发" (gtnt.cn), section 4.3: operands
 *     are row-major unless stated otherwise; mixed precision needs an explicit
 *     cast.
 *   - "使用 Tilelang DSL 开发 GPU/CPU/加速器高性能内核" (blog.hotdry.top): an
 *     elementwise post-processing loop (ReLU) on the output tile, and the
 *     weight-only low-bit "Dequant GEMM" as a target workload.
 *
 * Conventions shared by every entry point:
 *   - All matrix pointers are DEVICE pointers owned by the caller.  The library
 *     never allocates, frees or synchronises, and keeps no per-call state.
 *   - Dense row-major storage with implied leading dimensions
 *     (lda = K, ldb = N, ldc = N; packed weights: K/2 bytes per row).
 *   - Calls are asynchronous on `stream` (NULL = the null stream): they return
 *     once the kernel is enqueued.  Thread-safe.
 *   - Arguments are validated before any HIP call; on a non-OK status nothing
 *     has been launched and C is untouched.
 *   - M == 0 or N == 0: TG_OK, nothing launched (all pointers may be NULL).
 *     K == 0: C = epilogue(0) = 0; the operand pointers may be NULL then.
 *   - Accumulation is always fp32; the output is rounded to its type once,
 *     round-to-nearest-even (fp32 -> fp16 overflow gives +-inf).
 *   - Each operand must fit a 31-bit byte offset per tile row band (up to 256
 *     rows of a k-contiguous operand, up to 128 k-rows of an n-contiguous one):
 *     the library returns TG_ERR_BAD_SHAPE when 256 * K * element_size or
 *     128 * N * element_size exceeds 2^31 - 1 (and for M, N, K above 2^31 - 1).
 */
#ifndef TILEGEMM_H
#define TILEGEMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* tg_stream_t; /* same object as hipStream_t */

typedef enum {
    TG_OK = 0,
    TG_ERR_NULL_POINTER = 1, /* a required pointer is NULL                        */
    TG_ERR_BAD_SHAPE = 2,    /* negative / too large size, dequant K % 32 != 0,   */
                             /* or MX K % 128 != 0                                */
    TG_ERR_BAD_DTYPE = 3,    /* dtype not one of tg_dtype (MX: tg_mx_format)      */
    TG_ERR_BAD_EPILOGUE = 4, /* epilogue not one of tg_epilogue                   */
    TG_ERR_ALIAS = 5,        /* C overlaps an input                               */
    TG_ERR_NO_CONFIG = 6,    /* forced config index out of range / wrong op       */
    TG_ERR_HIP = 7,          /* the HIP runtime reported an error at launch       */
    TG_ERR_BAD_LAYOUT = 8,   /* trans_a / trans_b not 0 or 1                      */
    TG_ERR_WORKSPACE = 9,    /* split-K workspace NULL, too small or misaligned    */
    TG_ERR_SCRATCH = 10      /* split-K partials exceed TG_SPLITK_SCRATCH_BYTES    */
} tg_status;

typedef enum { TG_F32 = 0, TG_F16 = 1, TG_BF16 = 2 } tg_dtype;

typedef enum { TG_EPI_NONE = 0, TG_EPI_RELU = 1 } tg_epilogue;

typedef enum { TG_OP_GEMM = 0, TG_OP_DEQUANT_W4 = 1, TG_OP_MX = 2, TG_OP_SP24 = 3 } tg_op;

/* Element format of the activations of tg_gemm_mx. */
typedef enum { TG_MX_E2M1 = 0, TG_MX_E4M3 = 1 } tg_mx_format;

/*
 * C = epilogue(A x B).
 *   A: [M][K] row-major, B: [K][N] row-major, C: [M][N] row-major, all of
 *   `dtype` (fp32, fp16 or bf16); products accumulate in fp32 on the matrix
 *   cores; TG_EPI_RELU maps every accumulated value v to (v > 0 ? v : +0)
 *   before the single rounding to `dtype`.
 *   Non-multiple-of-tile shapes are handled inside the kernel (out-of-range
 *   rows and columns are never read into the sum nor written).
 * Errors: TG_ERR_NULL_POINTER (C NULL with M, N > 0, or A or B NULL with
 *   M, N, K > 0), TG_ERR_BAD_SHAPE,
 *   TG_ERR_BAD_DTYPE, TG_ERR_BAD_EPILOGUE, TG_ERR_ALIAS (C's bytes overlap A's
 *   or B's), TG_ERR_HIP.
 */
tg_status tg_gemm(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* A, const void* B,
                  void* C, tg_epilogue epi, tg_stream_t stream);

/*
 * C = epilogue(op(A) x op(B)) with either operand stored transposed: the
 * operand layouts of the backward products of the mhpq.cn page's autograd
 * wrapper (section 3.4: dA = dC x B^T, dB = A^T x dC) and the column-major
 * option the gtnt.cn page names (section 4.3).
 *   trans_a = 0: A is [M][K] row-major (as tg_gemm); 1: A is stored [K][M]
 *                row-major, i.e. op(A) = (stored A)^T, M x K.
 *   trans_b = 0: B is [K][N] row-major (as tg_gemm); 1: B is stored [N][K]
 *                row-major, i.e. op(B) = (stored B)^T, K x N.
 *   C: [M][N] row-major.  Same arithmetic, epilogue and rounding as tg_gemm;
 *   tg_gemm_ex(..., A, 0, B, 0, ...) is tg_gemm.
 * Every layout runs every dtype and alignment: 16-byte aligned operands whose
 * stored rows are whole 16-byte chunks take 16-byte loads (16-bit types: the
 * LDS-DMA kernel; fp32: the register-staged kernel), any other call takes
 * element loads.
 * Errors: as tg_gemm; TG_ERR_BAD_LAYOUT (trans_a or trans_b not 0 or 1),
 *   TG_ERR_BAD_SHAPE also when trans_a and 128 * M * element_size exceeds
 *   2^31 - 1.
 */
tg_status tg_gemm_ex(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* A, int trans_a,
                     const void* B, int trans_b, void* C, tg_epilogue epi, tg_stream_t stream);

/*
 * Split-K GEMM: C = epilogue(A x B) as tg_gemm, with each output tile's K range
 * split over several workgroups, for shapes whose tile grid alone leaves most
 * compute units idle (few output tiles, long K).  The mhpq.cn page names the
 * tail effect of small problems (section 4.3); split K is the standard remedy
 * for it and, unlike tg_gemm, needs memory for partial sums: the caller brings
 * it as `workspace`.
 *   A, B, C, dtype, epi: as tg_gemm (row-major, fp32 / fp16 / bf16).
 *   splits: 0 = chosen by the library (about one workgroup per compute unit,
 *     at least two k strips per split); n >= 1 = at most n splits (fewer when
 *     K holds fewer strips); 1 = no split, identical to tg_gemm.
 *   workspace: device memory, 16-byte aligned, of at least the size
 *     tg_gemm_splitk_workspace_size reports for the same M, N, K, dtype and
 *     splits.  It holds per-tile arrival counters and fp32 partial tiles.  It
 *     must be zero-filled before its first use; every call leaves the counters
 *     zero again, so it is reused without clearing.  Calls that share a
 *     workspace must not run concurrently (issue them on one stream).
 *   Numerics: each split sums its k range in fp32 on the matrix cores; the
 *     split sums are added in fp32 in split order 0, 1, ... by whichever
 *     workgroup of the tile finishes last, so the result does not depend on
 *     the order in which workgroups run; then the ReLU and the single rounding
 *     of tg_gemm.  Integer-valued inputs give tg_gemm's result bit for bit
 *     (every partial sum is exact in fp32).
 *   When no split pays off (or the operands are not 16-byte aligned with rows
 *   of whole 16-byte chunks) the call runs tg_gemm's kernel and does not touch
 *   the workspace, which may then be NULL.
 * Errors: as tg_gemm; TG_ERR_BAD_SHAPE also for splits < 0; TG_ERR_ALIAS also
 *   when the workspace overlaps A, B or C; TG_ERR_WORKSPACE when a split is
 *   launched and the workspace is NULL, smaller than needed or not 16-byte
 *   aligned.
 */
tg_status tg_gemm_splitk(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* A,
                         const void* B, void* C, tg_epilogue epi, int splits, void* workspace,
                         size_t workspace_bytes, tg_stream_t stream);

/*
 * Workspace bytes tg_gemm_splitk (and tg_gemm_splitk_config with any
 * configuration) needs for this call: written to *bytes, 0 when no split
 * would be launched.  Pure host function.
 * Errors: TG_ERR_NULL_POINTER (bytes NULL), TG_ERR_BAD_DTYPE,
 *   TG_ERR_BAD_SHAPE (as tg_gemm, or splits < 0).
 */
tg_status tg_gemm_splitk_workspace_size(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                        int splits, size_t* bytes);

/*
 * Split-K GEMM that allocates nothing, for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  Same arguments, numerics and
 * results as tg_gemm_splitk, without the workspace: the arrival counters and
 * fp32 partial tiles live in a fixed static device array of
 * TG_SPLITK_SCRATCH_BYTES, one per GPU, held from the library's first use on
 * that GPU until the process ends.  The array's device address is looked up
 * once per device (the calling thread's current device, which must be the
 * stream's).  Each call that splits first zeroes the counters it uses with a
 * small fill kernel on `stream` (no memset node, so it can be captured), then
 * launches the GEMM; nothing is allocated or freed.
 * Every call on one GPU shares the array: calls that overlap in time on one
 * GPU (other streams, other threads) race and give wrong results; issue them
 * on one stream.
 * Errors: as tg_gemm_splitk (never TG_ERR_WORKSPACE); TG_ERR_SCRATCH when the
 *   split launched would need more than TG_SPLITK_SCRATCH_BYTES
 *   (tg_gemm_splitk_workspace_size gives the bytes; lower `splits` or use
 *   tg_gemm_splitk); TG_ERR_HIP also when the array's address lookup fails.
 */
#define TG_SPLITK_SCRATCH_BYTES (16 * 1024 * 1024)
tg_status tg_gemm_splitk_noalloc(int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                 const void* A, const void* B, void* C, tg_epilogue epi,
                                 int splits, tg_stream_t stream);

/*
 * Weight-only 4-bit dequant GEMM: C = epilogue(A x W^T).
 *   A : bf16 [M][K] row-major activations.
 *   Wq: uint8 [N][K/2]: weight row n holds its K E2M1 codes (OCP MX v1.0 FP4:
 *       sign, 2-bit exponent with bias 1, 1-bit mantissa) two per byte, even k
 *       in bits 3:0 and odd k in bits 7:4.
 *   Ws: uint8 [N][K/32]: one E8M0 scale byte E per 32 consecutive k of a row,
 *       scale 2^(E - 127).
 *   W[n][k] = e2m1(code(n, k)) * 2^(Ws[n][k/32] - 127); C[m][n] = sum_k A[m][k] * W[n][k].
 *   C : bf16 [M][N].  The weights are expanded to bf16 on chip (exact for
 *       E in [2, 252]; other scale bytes follow the hardware conversion) and
 *       multiplied on the bf16 matrix cores with fp32 accumulation.
 *   The pages name this workload ("WFP4" GEMM, "Dequant GEMM") but not its
 *   format; the format above is the workload statement's.
 * Errors: as tg_gemm; TG_ERR_BAD_SHAPE also when K % 32 != 0.
 */
tg_status tg_dequant_gemm_w4(int64_t M, int64_t N, int64_t K, const void* A, const uint8_t* Wq,
                             const uint8_t* Ws, void* C, tg_epilogue epi, tg_stream_t stream);

/*
 * MX-format GEMM: C = epilogue(A x W^T) with the activations, too, in OCP
 * microscaling blocks (the pages' "WFP4" GEMM of "TileLang架构深度剖析", the
 * performance section, run natively in the block formats instead of
 * dequantised: the matrix cores of gfx950 multiply E2M1 / E4M3 elements and
 * apply the E8M0 block scales themselves).
 *   Aq: activation element codes, format a_fmt:
 *       TG_MX_E2M1: uint8 [M][K/2], two E2M1 codes per byte as in Wq below;
 *       TG_MX_E4M3: uint8 [M][K], one OCP E4M3 code per byte (sign, 4-bit
 *                   exponent with bias 7, 3-bit mantissa; no infinities;
 *                   S.1111.111 is NaN; largest finite value 448).
 *   As: uint8 [M][K/32]: one E8M0 scale byte per 32 consecutive k of a row.
 *   Wq: uint8 [N][K/2] E2M1 weight codes, Ws: uint8 [N][K/32] E8M0 scales,
 *       laid out as for tg_dequant_gemm_w4.
 *   a(m, k) = elem(Aq, m, k) * 2^(As[m][k/32] - 127),
 *   w(n, k) = e2m1(Wq, n, k) * 2^(Ws[n][k/32] - 127),
 *   C[m][n] = sum_k a(m, k) * w(n, k), rounded once to bf16; C: bf16 [M][N].
 *   Scale byte 255 is NaN: every result that takes a product of that block is
 *   NaN (as is every one that takes an E4M3 NaN).
 *   Arithmetic: the gfx950 scaled matrix instruction adds each group of 8
 *   consecutive products (within one 32-k block) in fixed point whose last
 *   bit is 2^(e - 13), e being the group's largest exponent sum E(a) + E(w)
 *   of the unscaled elements (subnormal and zero elements count with their
 *   format's smallest normal exponent), each product truncated toward zero;
 *   group sums are scaled and accumulated in fp32.  E2M1 x E2M1 products
 *   never reach that window (exact up to the fp32 accumulation); E4M3
 *   products more than 2^13 below their group's largest lose their low bits.
 *   (Measured on MI355X with in-bounds probes; the reference is the exact
 *   sum.)
 *   The pages give no format for this workload; the one above is the OCP MX
 *   v1.0 definition.
 * Requirements: K % 128 == 0 (else TG_ERR_BAD_SHAPE); Aq and Wq 16-byte
 *   aligned, As and Ws 4-byte aligned (else TG_ERR_NO_CONFIG).  (Forced
 *   configurations whose name ends in _sc8 also need K % 512 == 0 and 16-byte
 *   aligned As and Ws.)
 * Errors: as tg_gemm; TG_ERR_BAD_DTYPE when a_fmt is not a tg_mx_format.
 */
tg_status tg_gemm_mx(int64_t M, int64_t N, int64_t K, tg_mx_format a_fmt, const uint8_t* Aq,
                     const uint8_t* As, const uint8_t* Wq, const uint8_t* Ws, void* C,
                     tg_epilogue epi, tg_stream_t stream);

/*
 * 2:4 structured-sparse GEMM: C = epilogue(A x B) with A [M][K] keeping at
 * most two values in every group of four consecutive k, given compressed
 * (the 2:4 sparse GEMM of "使用 Tilelang DSL 开发 GPU/CPU/加速器高性能内核",
 * its monitoring-and-debugging paragraph, which skips the dense work):
 *   Ac: [M][K/2] of `dtype`: group j (k = 4j .. 4j + 3) of row m keeps
 *       Ac[m][2j] and Ac[m][2j + 1];
 *   Ai: uint8 [M][K/8]: group j's positions as the nibble
 *       (Ai[m][j/2] >> (4 * (j % 2))) & 0xF = p0 | p1 << 2 (p0, p1 in 0..3;
 *       a repeated position adds both values);
 *   B : [K][N] row-major of `dtype`; C: [M][N] of `dtype`.
 *   C[m][n] = sum_j (Ac[m][2j] * B[4j + p0][n] + Ac[m][2j + 1] * B[4j + p1][n]),
 *   fp32 accumulation on the sparse matrix instruction, one RNE rounding;
 *   TG_EPI_RELU as for tg_gemm.  The pages give no storage format; this one
 *   is the library's (two values per group in k order, 4-bit position pairs).
 * Requirements: dtype TG_F16 or TG_BF16 (else TG_ERR_BAD_DTYPE); K % 32 == 0
 *   (else TG_ERR_BAD_SHAPE); Ac and B 16-byte aligned, N % 8 == 0, Ai 4-byte
 *   aligned (else TG_ERR_NO_CONFIG).
 * Errors: as tg_gemm.
 */
tg_status tg_gemm_sp24(int64_t M, int64_t N, int64_t K, tg_dtype dtype, const void* Ac,
                       const uint8_t* Ai, const void* B, void* C, tg_epilogue epi,
                       tg_stream_t stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* tg_status_str(tg_status s);

/*
 * Which compiled kernel configuration the library would launch for this call.
 * Writes a NUL-terminated description (tile sizes, waves, stages, swizzle
 * group, launch grid) into buf[0 .. len-1], truncating if needed.
 * op: TG_OP_GEMM, TG_OP_DEQUANT_W4 (dtype ignored), TG_OP_MX (dtype
 * carries the tg_mx_format of the activations) or TG_OP_SP24.
 * Errors: TG_ERR_NULL_POINTER (buf NULL or len 0), TG_ERR_BAD_SHAPE,
 *   TG_ERR_BAD_DTYPE, TG_ERR_NO_CONFIG (op unknown).
 */
tg_status tg_query_config(int op, int64_t M, int64_t N, int64_t K, tg_dtype dtype, char* buf,
                          size_t len);

/* As tg_query_config, for the operand layouts of tg_gemm_ex (dequant, MX and
 * sparse: 0, 0; TG_ERR_BAD_LAYOUT otherwise). */
tg_status tg_query_config_ex(int op, int64_t M, int64_t N, int64_t K, tg_dtype dtype, int trans_a,
                             int trans_b, char* buf, size_t len);

/*
 * Offline sweep support: the compiled configurations, listed per (op, dtype),
 * can be launched by index instead of by the built-in selection table.  The
 * dequant list ignores dtype; the MX list holds both activation formats and
 * ignores dtype too (a configuration runs calls of its own format only).
 *   tg_config_count: number of configurations for (op, dtype); 0 if none.
 *   tg_config_name : description of configuration `index` (as tg_query_config).
 *   tg_gemm_config / tg_gemm_ex_config / tg_dequant_gemm_w4_config /
 *     tg_gemm_mx_config / tg_gemm_sp24_config / tg_gemm_splitk_config: same
 *     contract as tg_gemm / tg_gemm_ex / tg_dequant_gemm_w4 / tg_gemm_mx /
 *     tg_gemm_sp24 / tg_gemm_splitk, launching configuration `index`;
 *     TG_ERR_NO_CONFIG if `index` is out of range or the configuration cannot
 *     run the call (operand layout, alignment, a K multiple it needs, another
 *     activation format, or, for split K, a configuration without k-slice
 *     wave groups: names with three wave counts, "_w1x1x4_").
 */
int tg_config_count(int op, tg_dtype dtype);
tg_status tg_config_name(int op, tg_dtype dtype, int index, char* buf, size_t len);
tg_status tg_gemm_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                         const void* A, const void* B, void* C, tg_epilogue epi,
                         tg_stream_t stream);
tg_status tg_gemm_ex_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                            const void* A, int trans_a, const void* B, int trans_b, void* C,
                            tg_epilogue epi, tg_stream_t stream);
tg_status tg_dequant_gemm_w4_config(int index, int64_t M, int64_t N, int64_t K, const void* A,
                                    const uint8_t* Wq, const uint8_t* Ws, void* C,
                                    tg_epilogue epi, tg_stream_t stream);
tg_status tg_gemm_mx_config(int index, int64_t M, int64_t N, int64_t K, tg_mx_format a_fmt,
                            const uint8_t* Aq, const uint8_t* As, const uint8_t* Wq,
                            const uint8_t* Ws, void* C, tg_epilogue epi, tg_stream_t stream);
tg_status tg_gemm_sp24_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                              const void* Ac, const uint8_t* Ai, const void* B, void* C,
                              tg_epilogue epi, tg_stream_t stream);
tg_status tg_gemm_splitk_config(int index, int64_t M, int64_t N, int64_t K, tg_dtype dtype,
                                const void* A, const void* B, void* C, tg_epilogue epi,
                                int splits, void* workspace, size_t workspace_bytes,
                                tg_stream_t stream);

/*
 * The block-swizzled tile order, for host-side checking.  For a grid of
 * tiles_m x tiles_n output tiles and a swizzle group of `group_m` tile rows,
 * writes for every workgroup id w in [0, tiles_m * tiles_n) the tile it
 * computes: out_m[w], out_n[w].  Workgroup ids are first regrouped so that
 * the ids the hardware dispatches to one XCD (w mod 8) form a contiguous run,
 * then walked in groups of `group_m` tile rows, column by column.
 * Pure host function; touches no device.  Errors: TG_ERR_NULL_POINTER,
 * TG_ERR_BAD_SHAPE (tiles_m, tiles_n < 1, product above 2^31 - 1, group_m < 1).
 */
tg_status tg_tile_map(int64_t tiles_m, int64_t tiles_n, int group_m, int32_t* out_m,
                      int32_t* out_n);

/*
 * Clock record, a measurement aid.  The mhpq.cn page (section 4.2) reads a
 * GEMM's speed against the theoretical ceiling first; on a power-limited card
 * that ceiling moves with the shader clock, so a benchmark needs the clock the
 * kernel actually ran at.  With `stamps` set (a DEVICE pointer to 32 uint64,
 * caller-owned, NULL to switch off), every kernel launched afterwards by any
 * entry point has wave 0 of its workgroups 0..7 (one per XCD) write
 * stamps[4 b + 0..3] = shader-clock counter and 100 MHz reference counter at
 * its start, then the same at its end (workgroups b < 8 only; a grid of fewer
 * workgroups leaves the rest untouched).  Each launch overwrites the previous
 * one's record, so read it after synchronising.  Clock of workgroup b:
 * (t1 - t0) / ((r1 - r0) / 100 MHz).  Process-wide setting for benchmarks;
 * calls on several threads or streams while it is set write the same buffer.
 */
void tg_set_clock_stamps(uint64_t* stamps);

/*
 * Tuning aids for the offline sweep (tiled_dense_gemm_07_amd/sweep.py), which
 * follows the mhpq.cn page's tuning advice (sections 4.2 and 4.3: measure
 * candidate tilings on the target GPU, check occupancy, keep the best).
 *   tg_set_swizzle_override: every launch afterwards, by any entry point, uses
 *     swizzle group `group_m` (tile rows per group of the block-swizzled tile
 *     order, a pure reordering: results are unchanged); 0 restores the
 *     selection's own group.  Process-wide, for timing runs.
 *   tg_config_occupancy: workgroups of compiled configuration `index` of
 *     (op, dtype) that one compute unit holds at once (registers, LDS and
 *     waves), from the HIP occupancy query on the current device.
 *     Errors: TG_ERR_NULL_POINTER, TG_ERR_NO_CONFIG (index out of range),
 *     TG_ERR_HIP (no device or the query failed).
 */
void tg_set_swizzle_override(int group_m);
tg_status tg_config_occupancy(int op, tg_dtype dtype, int index, int* workgroups_per_cu);

#ifdef __cplusplus
}
#endif

#endif /* TILEGEMM_H */
