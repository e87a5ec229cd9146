/*
 * Oracle for the tiled dense GEMM, the weight-only 4-bit dequant GEMM, the
 * MX-format GEMM and the 2:4 structured-sparse GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the library calls, links or includes
 * this file; only the tests, the smoke check and the CPU-baseline leg of the
 * benchmark load it.  It shares no code, header or table with the HIP path.
 *
 * What it computes is the plain definition, not the tiled algorithm:
 *   - "TileLang: 用Python DSL简化GPU算子开发" (gtnt.cn), section 2.2, writes the
 *     GEMM as C[i, j] = sum over k of A[i, k] * B[k, j] on row-major operands;
 *   - "TileLang ... 一个高效 GEMM 内核" (mhpq.cn), sections 2.1 and 3.2, state the
 *     same product C = A x B for an M x K and a K x N matrix, and section 4.3
 *     says tiling only changes the fp32 summation order.
 * So every result here is the exact sum in fp64 (exact for the integer and
 * dyadic test inputs; within K * 2^-52 * sum|a||b| otherwise), followed by an
 * optional ReLU (the blog.hotdry.top page's post-processing loop) and, for
 * bitwise checks, ONE round-to-nearest-even from fp64 to the output type.
 *
 * Number formats are decoded and encoded from their field definitions
 * (sign / biased exponent / fraction), never through a hardware cast:
 *   IEEE-754 binary32 and binary16, bfloat16 (binary32 with a 7-bit fraction),
 *   and the OCP Microscaling (MX) v1.0 element types E2M1 and E4M3 and scale
 *   type E8M0.
 * The 4-bit weight format is not on the pages; it follows the workload text:
 * two E2M1 codes per byte (even k in bits 3:0, odd k in bits 7:4), one E8M0
 * scale per 32 consecutive k of a weight row, C = A * W^T with W stored [N][K].
 *
 * dtype codes: 0 = fp32, 1 = fp16, 2 = bf16 (operands and output share it).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_F16 1
#define ORC_BF16 2

/* ---------------------------------------------------------------------- */
/* Field-level decoding.                                                   */
/* ---------------------------------------------------------------------- */

/* Decode a binary floating-point code with `ebits` exponent bits and `fbits`
 * fraction bits.  has_special: top exponent encodes Inf/NaN (IEEE); E2M1 has
 * no special values, so its top exponent is an ordinary binade. */
static double decode_bits(uint64_t bits, int ebits, int fbits, int has_special)
{
    const uint64_t fmask = (1ull << fbits) - 1ull;
    const uint64_t emask = (1ull << ebits) - 1ull;
    const int bias = (1 << (ebits - 1)) - 1;
    const int sign = (int)((bits >> (ebits + fbits)) & 1ull);
    const uint64_t e = (bits >> fbits) & emask;
    const uint64_t f = bits & fmask;
    double v;
    if (has_special && e == emask) {
        v = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        /* subnormal: f * 2^(1 - bias - fbits) */
        v = ldexp((double)f, 1 - bias - fbits);
    } else {
        /* normal: (2^fbits + f) * 2^(e - bias - fbits) */
        v = ldexp((double)((1ull << fbits) + f), (int)e - bias - fbits);
    }
    return sign ? -v : v;
}

double orc_decode_f32(uint32_t b) { return decode_bits(b, 8, 23, 1); }
double orc_decode_f16(uint16_t b) { return decode_bits(b, 5, 10, 1); }
double orc_decode_bf16(uint16_t b) { return decode_bits(b, 8, 7, 1); }

/* OCP MX E2M1: bit 3 sign, bits 2:1 exponent (bias 1), bit 0 fraction. */
double orc_decode_e2m1(uint8_t code) { return decode_bits(code & 0xFu, 2, 1, 0); }

/* OCP MX E8M0: 2^(E - 127); E = 255 is NaN. */
double orc_decode_e8m0(uint8_t e) { return e == 255 ? NAN : ldexp(1.0, (int)e - 127); }

/* OCP MX E4M3: bit 7 sign, bits 6:3 exponent (bias 7), bits 2:0 fraction.
 * No infinities: exponent 15 is an ordinary binade, except that S.1111.111
 * is NaN (so the largest finite magnitude is 1.75 * 2^8 = 448). */
double orc_decode_e4m3(uint8_t code)
{
    if ((code & 0x7Fu) == 0x7Fu)
        return NAN;
    return decode_bits(code, 4, 3, 0);
}

/* ---------------------------------------------------------------------- */
/* Field-level encoding: one round-to-nearest-even from a double.          */
/* ---------------------------------------------------------------------- */

static uint64_t encode_rne(double x, int ebits, int fbits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const uint64_t emax_field = (1ull << ebits) - 1ull;
    const uint64_t sign = signbit(x) ? 1ull : 0ull;
    const uint64_t sbit = sign << (ebits + fbits);
    if (isnan(x))
        return sbit | (emax_field << fbits) | (1ull << (fbits - 1)); /* quiet NaN */
    double a = fabs(x);
    if (isinf(a))
        return sbit | (emax_field << fbits);
    if (a == 0.0)
        return sbit;

    /* a = m * 2^(ex - 53), m a 53-bit integer (exact). */
    int ex;
    double fr = frexp(a, &ex);            /* a = fr * 2^ex, fr in [0.5, 1) */
    uint64_t m = (uint64_t)ldexp(fr, 53); /* exact */
    int ue = ex - 1;                      /* a in [2^ue, 2^(ue+1)) */
    int emin = 1 - bias;                  /* smallest normal exponent */
    /* quantum of the target grid around a: 2^q */
    int q = (ue > emin ? ue : emin) - fbits;
    int s = q - (ex - 53); /* right shift applied to m; always > 0 here */
    uint64_t n;
    if (s >= 64) {
        n = 0; /* a < 2^(q-11): rounds to zero */
    } else {
        n = m >> s;
        uint64_t rem = m & ((1ull << s) - 1ull);
        uint64_t half = 1ull << (s - 1);
        if (rem > half || (rem == half && (n & 1ull)))
            n += 1;
    }
    /* value = n * 2^q.  n < 2^fbits only in the subnormal binade. */
    uint64_t efield, ffield;
    if (n < (1ull << fbits)) {
        efield = 0; /* subnormal (q == emin - fbits) or zero */
        ffield = n;
    } else {
        if (n == (2ull << fbits)) { /* carry into the next binade */
            n >>= 1;
            q += 1;
        }
        efield = (uint64_t)(q + fbits + bias);
        ffield = n - (1ull << fbits);
    }
    if (efield >= emax_field) /* overflow: RNE rounds to infinity */
        return sbit | (emax_field << fbits);
    return sbit | (efield << fbits) | ffield;
}

uint32_t orc_encode_f32(double x) { return (uint32_t)encode_rne(x, 8, 23); }
uint16_t orc_encode_f16(double x) { return (uint16_t)encode_rne(x, 5, 10); }
uint16_t orc_encode_bf16(double x) { return (uint16_t)encode_rne(x, 8, 7); }

/* Bulk helpers used by the Python side. */
void orc_decode_array(int dtype, int64_t n, const void* src, double* dst)
{
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == ORC_F32)
            dst[i] = orc_decode_f32(((const uint32_t*)src)[i]);
        else if (dtype == ORC_F16)
            dst[i] = orc_decode_f16(((const uint16_t*)src)[i]);
        else
            dst[i] = orc_decode_bf16(((const uint16_t*)src)[i]);
    }
}

void orc_encode_array(int dtype, int64_t n, const double* src, void* dst)
{
    for (int64_t i = 0; i < n; ++i) {
        if (dtype == ORC_F32)
            ((uint32_t*)dst)[i] = orc_encode_f32(src[i]);
        else if (dtype == ORC_F16)
            ((uint16_t*)dst)[i] = orc_encode_f16(src[i]);
        else
            ((uint16_t*)dst)[i] = orc_encode_bf16(src[i]);
    }
}

/* ---------------------------------------------------------------------- */
/* GEMM: Y = epi(A * B), A [M][K], B [K][N] row-major, Y [M][N] fp64.      */
/* ---------------------------------------------------------------------- */

static double relu_f64(double y) { return y > 0.0 ? y : 0.0; /* x <= 0 -> +0 */ }

/* Returns 0 on success, -1 on allocation failure. */
int orc_gemm_f64(int64_t M, int64_t N, int64_t K, int dtype, const void* A, const void* B,
                 int relu, double* Y)
{
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -1;
    }
    orc_decode_array(dtype, M * K, A, Ad);
    orc_decode_array(dtype, K * N, B, Bd);

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* yi = Y + i * N;
        for (int64_t j = 0; j < N; ++j)
            yi[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = Ad[i * K + k];
            const double* bk = Bd + k * N;
            for (int64_t j = 0; j < N; ++j)
                yi[j] += a * bk[j];
        }
        if (relu)
            for (int64_t j = 0; j < N; ++j)
                yi[j] = relu_f64(yi[j]);
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* Selected entries only: out[t] = epi(sum_k A[rows[t]][k] * B[k][cols[t]]).
 * For checking large outputs one element at a time. */
void orc_gemm_entries_f64(int64_t M, int64_t N, int64_t K, int dtype, const void* A,
                          const void* B, int relu, int64_t count, const int64_t* rows,
                          const int64_t* cols, double* out)
{
    (void)M;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a, b;
            if (dtype == ORC_F32) {
                a = orc_decode_f32(((const uint32_t*)A)[i * K + k]);
                b = orc_decode_f32(((const uint32_t*)B)[k * N + j]);
            } else if (dtype == ORC_F16) {
                a = orc_decode_f16(((const uint16_t*)A)[i * K + k]);
                b = orc_decode_f16(((const uint16_t*)B)[k * N + j]);
            } else {
                a = orc_decode_bf16(((const uint16_t*)A)[i * K + k]);
                b = orc_decode_bf16(((const uint16_t*)B)[k * N + j]);
            }
            s += a * b;
        }
        out[t] = relu ? relu_f64(s) : s;
    }
}

/* ---------------------------------------------------------------------- */
/* Operands stored transposed.                                             */
/*   Y[i][j] = epi(sum_k opA[i][k] * opB[k][j]) with                       */
/*   opA[i][k] = A[i][k] (A stored [M][K]) or A[k][i] (A stored [K][M]),   */
/*   opB[k][j] = B[k][j] (B stored [K][N]) or B[j][k] (B stored [N][K]).   */
/* The same plain sum; only the element each (i, k) / (k, j) names moves.  */
/* ---------------------------------------------------------------------- */

static double op_a(const double* Ad, int trans_a, int64_t M, int64_t K, int64_t i, int64_t k)
{
    return trans_a ? Ad[k * M + i] : Ad[i * K + k];
}

static double op_b(const double* Bd, int trans_b, int64_t N, int64_t K, int64_t k, int64_t j)
{
    return trans_b ? Bd[j * K + k] : Bd[k * N + j];
}

int orc_gemm_layout_f64(int64_t M, int64_t N, int64_t K, int dtype, const void* A, int trans_a,
                        const void* B, int trans_b, int relu, double* Y)
{
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -1;
    }
    orc_decode_array(dtype, M * K, A, Ad);
    orc_decode_array(dtype, K * N, B, Bd);

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            double s = 0.0;
            for (int64_t k = 0; k < K; ++k)
                s += op_a(Ad, trans_a, M, K, i, k) * op_b(Bd, trans_b, N, K, k, j);
            Y[i * N + j] = relu ? relu_f64(s) : s;
        }
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* Selected entries of the above, one element at a time. */
void orc_gemm_layout_entries_f64(int64_t M, int64_t N, int64_t K, int dtype, const void* A,
                                 int trans_a, const void* B, int trans_b, int relu, int64_t count,
                                 const int64_t* rows, const int64_t* cols, double* out)
{
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const int64_t ia = trans_a ? k * M + i : i * K + k;
            const int64_t ib = trans_b ? j * K + k : k * N + j;
            double a, b;
            if (dtype == ORC_F32) {
                a = orc_decode_f32(((const uint32_t*)A)[ia]);
                b = orc_decode_f32(((const uint32_t*)B)[ib]);
            } else if (dtype == ORC_F16) {
                a = orc_decode_f16(((const uint16_t*)A)[ia]);
                b = orc_decode_f16(((const uint16_t*)B)[ib]);
            } else {
                a = orc_decode_bf16(((const uint16_t*)A)[ia]);
                b = orc_decode_bf16(((const uint16_t*)B)[ib]);
            }
            s += a * b;
        }
        out[t] = relu ? relu_f64(s) : s;
    }
}

/* ---------------------------------------------------------------------- */
/* Weight-only 4-bit dequant GEMM.                                         */
/*   W[n][k] = E2M1(code(n, k)) * E8M0(Ws[n][k / 32])                      */
/*   code(n, k) = (Wq[n][k / 2] >> (4 * (k % 2))) & 0xF                    */
/*   Y[m][n] = epi(sum_k A[m][k] * W[n][k]),  A bf16 [M][K]                */
/* K must be a multiple of 32 (one scale per 32 consecutive k).            */
/* ---------------------------------------------------------------------- */

static double w4_value(const uint8_t* Wq, const uint8_t* Ws, int64_t K, int64_t n, int64_t k)
{
    const uint8_t byte = Wq[n * (K / 2) + k / 2];
    const uint8_t code = (uint8_t)((byte >> (4 * (k % 2))) & 0xF);
    return orc_decode_e2m1(code) * orc_decode_e8m0(Ws[n * (K / 32) + k / 32]);
}

/* Decode the whole weight matrix to fp64 [N][K]. */
void orc_w4_decode(int64_t N, int64_t K, const uint8_t* Wq, const uint8_t* Ws, double* W)
{
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            W[n * K + k] = w4_value(Wq, Ws, K, n, k);
}

int orc_dequant_w4_f64(int64_t M, int64_t N, int64_t K, const uint16_t* A, const uint8_t* Wq,
                       const uint8_t* Ws, int relu, double* Y)
{
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -1;
    }
    orc_decode_array(ORC_BF16, M * K, A, Ad);
    /* B[k][n] := W[n][k] */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Bd[k * N + n] = w4_value(Wq, Ws, K, n, k);

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* yi = Y + i * N;
        for (int64_t j = 0; j < N; ++j)
            yi[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = Ad[i * K + k];
            const double* bk = Bd + k * N;
            for (int64_t j = 0; j < N; ++j)
                yi[j] += a * bk[j];
        }
        if (relu)
            for (int64_t j = 0; j < N; ++j)
                yi[j] = relu_f64(yi[j]);
    }
    free(Ad);
    free(Bd);
    return 0;
}

void orc_dequant_w4_entries_f64(int64_t M, int64_t N, int64_t K, const uint16_t* A,
                                const uint8_t* Wq, const uint8_t* Ws, int relu, int64_t count,
                                const int64_t* rows, const int64_t* cols, double* out)
{
    (void)M;
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += orc_decode_bf16(A[i * K + k]) * w4_value(Wq, Ws, K, j, k);
        out[t] = relu ? relu_f64(s) : s;
    }
}

/* ---------------------------------------------------------------------- */
/* MX-format GEMM: both operands in OCP MX v1.0 blocks of 32 along k (the  */
/* "WFP4" GEMM of the TileLang architecture page, performance section,     */
/* with block-format activations as well).                                 */
/*   a(m, k) = ELEM(codeA(m, k)) * E8M0(As[m][k / 32])                     */
/*     E2M1 activations (fmt 0): codeA = nibble k % 2 of Aq[m][k / 2]      */
/*     E4M3 activations (fmt 1): codeA = Aq[m][k]                          */
/*   w(n, k) = E2M1(code(n, k)) * E8M0(Ws[n][k / 32])  (as the dequant)    */
/*   Y[m][n] = epi(sum_k a(m, k) * w(n, k))                                */
/* The plain sum in fp64: every product is exact (at most 3 + 1 significant */
/* bits times powers of two), so Y is exact while K * 2^-52 * sum|a w| is   */
/* below half an ulp of the output, and NaN scales / codes give NaN.        */
/* ---------------------------------------------------------------------- */

static double mx_a_value(int fmt, const uint8_t* Aq, const uint8_t* As, int64_t K, int64_t m,
                         int64_t k)
{
    double e;
    if (fmt == 0) {
        const uint8_t byte = Aq[m * (K / 2) + k / 2];
        e = orc_decode_e2m1((uint8_t)((byte >> (4 * (k % 2))) & 0xF));
    } else {
        e = orc_decode_e4m3(Aq[m * K + k]);
    }
    return e * orc_decode_e8m0(As[m * (K / 32) + k / 32]);
}

/* Decode the activations to fp64 [M][K]. */
void orc_mx_decode_a(int64_t M, int64_t K, int fmt, const uint8_t* Aq, const uint8_t* As,
                     double* A)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k)
            A[m * K + k] = mx_a_value(fmt, Aq, As, K, m, k);
}

int orc_mx_gemm_f64(int64_t M, int64_t N, int64_t K, int fmt, const uint8_t* Aq,
                    const uint8_t* As, const uint8_t* Wq, const uint8_t* Ws, int relu, double* Y)
{
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -1;
    }
    orc_mx_decode_a(M, K, fmt, Aq, As, Ad);
    /* B[k][n] := w(n, k) */
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n)
            Bd[k * N + n] = w4_value(Wq, Ws, K, n, k);

#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* yi = Y + i * N;
        for (int64_t j = 0; j < N; ++j)
            yi[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = Ad[i * K + k];
            const double* bk = Bd + k * N;
            for (int64_t j = 0; j < N; ++j)
                yi[j] += a * bk[j];
        }
        if (relu)
            for (int64_t j = 0; j < N; ++j)
                yi[j] = relu_f64(yi[j]);
    }
    free(Ad);
    free(Bd);
    return 0;
}

void orc_mx_gemm_entries_f64(int64_t M, int64_t N, int64_t K, int fmt, const uint8_t* Aq,
                             const uint8_t* As, const uint8_t* Wq, const uint8_t* Ws, int relu,
                             int64_t count, const int64_t* rows, const int64_t* cols, double* out)
{
    (void)M;
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows[t], j = cols[t];
        double s = 0.0;
        for (int64_t k = 0; k < K; ++k)
            s += mx_a_value(fmt, Aq, As, K, i, k) * w4_value(Wq, Ws, K, j, k);
        out[t] = relu ? relu_f64(s) : s;
    }
}

/* ---------------------------------------------------------------------- */
/* 2:4 structured-sparse GEMM (the sparse GEMM the blog.hotdry.top page    */
/* names for 2:4 sparsity, its monitoring-and-debugging paragraph).        */
/*   A [M][K] is given compressed: group j of a row (k = 4j .. 4j + 3)     */
/*   keeps two values, Ac[m][2j] at position p0 and Ac[m][2j + 1] at p1,   */
/*   nib = (Ai[m][j / 2] >> (4 * (j % 2))) & 0xF, p0 = nib & 3,            */
/*   p1 = nib >> 2; the other positions are zero (a repeated position      */
/*   holds the sum of both values).                                        */
/*   Y[m][n] = epi(sum_j sum_t Ac[m][2j + t] * B[4j + p_t][n]).            */
/* K must be a multiple of 8 (whole metadata bytes).                       */
/* ---------------------------------------------------------------------- */

static int sp24_pos(const uint8_t* Ai, int64_t K, int64_t m, int64_t j, int t)
{
    const int nib = (Ai[m * (K / 8) + j / 2] >> (4 * (j % 2))) & 0xF;
    return t == 0 ? (nib & 3) : (nib >> 2);
}

static double decode_one(int dtype, const void* X, int64_t i)
{
    if (dtype == ORC_F32)
        return orc_decode_f32(((const uint32_t*)X)[i]);
    if (dtype == ORC_F16)
        return orc_decode_f16(((const uint16_t*)X)[i]);
    return orc_decode_bf16(((const uint16_t*)X)[i]);
}

/* The dense A [M][K] in fp64 that the compressed form stands for. */
void orc_sp24_densify(int64_t M, int64_t K, int dtype, const void* Ac, const uint8_t* Ai,
                      double* A)
{
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t k = 0; k < K; ++k)
            A[m * K + k] = 0.0;
        for (int64_t j = 0; j < K / 4; ++j)
            for (int t = 0; t < 2; ++t)
                A[m * K + 4 * j + sp24_pos(Ai, K, m, j, t)] +=
                    decode_one(dtype, Ac, m * (K / 2) + 2 * j + t);
    }
}

int orc_gemm_sp24_f64(int64_t M, int64_t N, int64_t K, int dtype, const void* Ac,
                      const uint8_t* Ai, const void* B, int relu, double* Y)
{
    double* Ad = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* Bd = (double*)malloc(sizeof(double) * (size_t)(K * N > 0 ? K * N : 1));
    if (!Ad || !Bd) {
        free(Ad);
        free(Bd);
        return -1;
    }
    orc_sp24_densify(M, K, dtype, Ac, Ai, Ad);
    orc_decode_array(dtype, K * N, B, Bd);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < M; ++i) {
        double* yi = Y + i * N;
        for (int64_t j = 0; j < N; ++j)
            yi[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double a = Ad[i * K + k];
            const double* bk = Bd + k * N;
            for (int64_t j = 0; j < N; ++j)
                yi[j] += a * bk[j];
        }
        if (relu)
            for (int64_t j = 0; j < N; ++j)
                yi[j] = relu_f64(yi[j]);
    }
    free(Ad);
    free(Bd);
    return 0;
}

/* Selected entries, straight from the compressed form (no densified A). */
void orc_gemm_sp24_entries_f64(int64_t M, int64_t N, int64_t K, int dtype, const void* Ac,
                               const uint8_t* Ai, const void* B, int relu, int64_t count,
                               const int64_t* rows, const int64_t* cols, double* out)
{
    (void)M;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t c = 0; c < count; ++c) {
        const int64_t i = rows[c], n = cols[c];
        double s = 0.0;
        for (int64_t j = 0; j < K / 4; ++j)
            for (int t = 0; t < 2; ++t) {
                const int64_t k = 4 * j + sp24_pos(Ai, K, i, j, t);
                s += decode_one(dtype, Ac, i * (K / 2) + 2 * j + t) * decode_one(dtype, B, k * N + n);
            }
        out[c] = relu ? relu_f64(s) : s;
    }
}

/* Number of OpenMP threads the oracle runs with (for reporting). */
#ifdef _OPENMP
#include <omp.h>
int orc_num_threads(void) { return omp_get_max_threads(); }
#else
int orc_num_threads(void) { return 1; }
#endif
