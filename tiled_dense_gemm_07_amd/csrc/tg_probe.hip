// Power / clock ceiling probes for the rooflines (measurement only; not part
// of the GEMM path and not exported by libtilegemm).
//
// One workgroup of 4 waves per tile of the 4096^3 bf16 GEMM's 256-tile grid,
// each wave issuing exactly the MFMA work of the GEMM kernel (128 strips x 32
// v_mfma_f32_32x32x16_bf16 into 16 accumulators of 32x32), but on register
// operands loaded once: no LDS, no global traffic in the loop.  The operands
// come from the caller's buffer (random or zero bit patterns), so the run shows
// how the sustained clock depends on the data the matrix cores multiply.
// Workgroup 0 reads the shader clock counter (s_memtime) and the fixed
// 100 MHz counter (s_memrealtime) around its loop: their ratio is the average
// shader clock during the kernel.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kFrag = 8;  // operand fragments per wave (16 bytes per lane each)

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
mfma_ceiling(const u32x4* __restrict__ src, float* __restrict__ out, uint64_t* __restrict__ clk,
             int strips)
{
    const int tid = threadIdx.x;
    uint64_t c0 = 0, r0 = 0;
    if (blockIdx.x == 0 && tid == 0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    const u32x4* s = src + (size_t)(blockIdx.x * 256 + tid) * 2 * kFrag;
    u32x4 a[kFrag], b[kFrag];
#pragma unroll
    for (int i = 0; i < kFrag; ++i) {
        a[i] = s[i];
        b[i] = s[kFrag + i];
    }
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
    for (int t = 0; t < strips; ++t) {
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, b[(j + 4 * sl) % kFrag]),
                        __builtin_bit_cast(bf16x8, a[(i + 4 * sl + t) % kFrag]), acc[i][j], 0, 0,
                        0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sum += acc[i][j][r];
    out[blockIdx.x * 256 + tid] = sum;
    if (blockIdx.x == 0 && tid == 0) {
        clk[0] = __builtin_amdgcn_s_memtime() - c0;
        clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

// The same MFMA work as mfma_ceiling with the 16 x 16 x 32 bf16 instruction:
// twice the instructions of half the size (8 x 8 blocks of 16 x 16 per wave,
// 64 v_mfma_f32_16x16x32_bf16 per strip), same accumulator registers.
typedef __attribute__((ext_vector_type(4))) float f32x4;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
mfma16_ceiling(const u32x4* __restrict__ src, float* __restrict__ out, uint64_t* __restrict__ clk,
               int strips)
{
    const int tid = threadIdx.x;
    uint64_t c0 = 0, r0 = 0;
    if (blockIdx.x == 0 && tid == 0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    const u32x4* s = src + (size_t)(blockIdx.x * 256 + tid) * 2 * kFrag;
    u32x4 a[kFrag], b[kFrag];
#pragma unroll
    for (int i = 0; i < kFrag; ++i) {
        a[i] = s[i];
        b[i] = s[kFrag + i];
    }
    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
            acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int t = 0; t < strips; ++t) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    __builtin_bit_cast(bf16x8, b[j]), __builtin_bit_cast(bf16x8, a[(i + t) % kFrag]),
                    acc[i][j], 0, 0, 0);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                sum += acc[i][j][r];
    out[blockIdx.x * 256 + tid] = sum;
    if (blockIdx.x == 0 && tid == 0) {
        clk[0] = __builtin_amdgcn_s_memtime() - c0;
        clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

// The same for the MX-format GEMM at 8192^3: one workgroup of 4 waves per
// tile of its grid, each wave issuing the scaled MFMAs of the kernel (64
// strips x 2 k-steps x FM x FN v_mfma_scale_f32_32x32x64_f8f6f4 on register
// operands; first operand E2M1, second E2M1 (AFMT 4) or E4M3 (AFMT 0); all
// scale bytes 127).
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kFragMx = 4;  // operand fragments per wave (32 bytes per lane each)

template <int AFMT, int FM, int FN>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void
mx_ceiling(const i32x8* __restrict__ src, float* __restrict__ out, uint64_t* __restrict__ clk,
           int strips)
{
    const int tid = threadIdx.x;
    uint64_t c0 = 0, r0 = 0;
    if (blockIdx.x == 0 && tid == 0) {
        c0 = __builtin_amdgcn_s_memtime();
        r0 = __builtin_amdgcn_s_memrealtime();
    }
    const i32x8* s = src + (size_t)(blockIdx.x * 256 + tid) * 2 * kFragMx;
    i32x8 a[kFragMx], b[kFragMx];
#pragma unroll
    for (int i = 0; i < kFragMx; ++i) {
        a[i] = s[i];
        b[i] = s[kFragMx + i];
        if (AFMT == 4)  // E2M1 uses the first four dwords only
            a[i][4] = a[i][5] = a[i][6] = a[i][7] = 0;
        b[i][4] = b[i][5] = b[i][6] = b[i][7] = 0;
    }
    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                acc[i][j][r] = 0.0f;
    for (int t = 0; t < strips; ++t) {
#pragma unroll
        for (int q = 0; q < 2; ++q)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        b[(j + FN * q) % kFragMx], a[(i + FM * q + t) % kFragMx], acc[i][j], 4, AFMT,
                        0, 127, 0, 127);
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                sum += acc[i][j][r];
    out[blockIdx.x * 256 + tid] = sum;
    if (blockIdx.x == 0 && tid == 0) {
        clk[0] = __builtin_amdgcn_s_memtime() - c0;
        clk[1] = __builtin_amdgcn_s_memrealtime() - r0;
    }
}

}  // namespace

extern "C" {

// Operand buffer: grid * 256 * 2 * kFrag 16-byte words.  out: grid * 256
// floats.  clk: 2 words (shader-clock ticks, 100 MHz ticks).  Returns 0 on a
// successful launch.
int tgp_operand_words(int grid) { return grid * 256 * 2 * kFrag; }

int tgp_mfma_ceiling(const void* src, void* out, void* clk, int grid, int strips,
                     hipStream_t stream)
{
    if (!src || !out || !clk || grid < 1 || strips < 1)
        return 1;
    hipLaunchKernelGGL(mfma_ceiling, dim3(grid), dim3(256), 0, stream, (const u32x4*)src,
                       (float*)out, (uint64_t*)clk, strips);
    return hipPeekAtLastError() == hipSuccess ? 0 : 2;
}

// As tgp_mfma_ceiling, with the 16 x 16 x 32 instruction (same operand buffer).
int tgp_mfma16_ceiling(const void* src, void* out, void* clk, int grid, int strips,
                       hipStream_t stream)
{
    if (!src || !out || !clk || grid < 1 || strips < 1)
        return 1;
    hipLaunchKernelGGL(mfma16_ceiling, dim3(grid), dim3(256), 0, stream, (const u32x4*)src,
                       (float*)out, (uint64_t*)clk, strips);
    return hipPeekAtLastError() == hipSuccess ? 0 : 2;
}

// MX probe: fmt 0 = E2M1 activations (256 x 256 tiles: FM = FN = 4), 1 = E4M3
// (128 x 256 tiles: FM = 2, FN = 4).  Operand buffer: grid * 256 * 2 * kFragMx
// 32-byte words (tgp_mx_operand_words).
int tgp_mx_operand_words(int grid) { return grid * 256 * 2 * kFragMx; }

int tgp_mx_ceiling(int fmt, const void* src, void* out, void* clk, int grid, int strips,
                   hipStream_t stream)
{
    if (!src || !out || !clk || grid < 1 || strips < 1 || (fmt != 0 && fmt != 1))
        return 1;
    if (fmt == 0)
        hipLaunchKernelGGL((mx_ceiling<4, 4, 4>), dim3(grid), dim3(256), 0, stream,
                           (const i32x8*)src, (float*)out, (uint64_t*)clk, strips);
    else
        hipLaunchKernelGGL((mx_ceiling<0, 2, 4>), dim3(grid), dim3(256), 0, stream,
                           (const i32x8*)src, (float*)out, (uint64_t*)clk, strips);
    return hipPeekAtLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
