// Plain streaming kernels: the HBM rates this library's own code reaches
// for a read+write stream (copy) and a write-only stream (fill), the
// attainable reference the bench puts beside the HBM-bound steps (im2col,
// col2im, transposes, split-K reductions); and the MFMA rate the GPU
// sustains with no data movement at all, the reference beside the GEMMs.
// Not steps of the method.
#include "internal.hpp"

namespace d4r {

namespace {

constexpr int NT = 256;
typedef uint32_t u32x4_s __attribute__((ext_vector_type(4)));

// One 16-byte vector per thread over a grid that covers the buffer: on
// MI355X many short-lived wavefronts stream faster than a grid-stride loop
// over a few thousand workgroups (1 GiB fill 6.9 against 4.0-5.1 TB/s; copy
// 6.25 against 4.4 TB/s; hipMemcpyAsync 4.9 TB/s).
__global__ __launch_bounds__(NT) void stream_copy_kernel(const u32x4_s *__restrict__ src,
                                                         u32x4_s *__restrict__ dst, long long n)
{
    const long long i = (long long)blockIdx.x * NT + threadIdx.x;
    if (i < n)
        dst[i] = src[i];
}

__global__ __launch_bounds__(NT) void stream_fill_kernel(u32x4_s *__restrict__ dst, uint32_t value, long long n)
{
    const long long i = (long long)blockIdx.x * NT + threadIdx.x;
    if (i < n)
        dst[i] = u32x4_s{value, value, value, value};
}

dim3 stream_grid(long long n) { return dim3((unsigned)((n + NT - 1) / NT)); }

typedef float f32x16_m __attribute__((ext_vector_type(16)));
typedef __fp16 f16x8_m __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_m __attribute__((ext_vector_type(8)));

// Eight wavefronts per workgroup, each holding a 4 x 2 grid of 32 x 32
// accumulators (the per-wavefront tile of the 256 x 256 GEMM) and issuing,
// per iteration, one MFMA per accumulator on operand fragments read once
// from src: 16 bytes per lane and fragment for 16-bit operands (8 k values,
// v_mfma_f32_32x32x16), one float per lane and fragment for f32 (2 k
// values, v_mfma_f32_32x32x2).  Lane 0 of each wavefront writes the sum of
// its accumulators, so no MFMA can be dropped.
template <int DTID>
__global__ __launch_bounds__(512) void mfma_ceiling_kernel(const uint32_t *__restrict__ src,
                                                           float *__restrict__ out, int iters)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    f32x16_m acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;
    if constexpr (DTID == DT_F32) {
        float a[4], b[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = __uint_as_float(src[i * 64 + lane]);
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j] = __uint_as_float(src[(4 + j) * 64 + lane]);
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i], b[j], acc[i][j], 0, 0, 0);
    } else {
        u32x4_s a[4], b[2];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = ((const u32x4_s *)src)[i * 64 + lane];
#pragma unroll
        for (int j = 0; j < 2; ++j)
            b[j] = ((const u32x4_s *)src)[(4 + j) * 64 + lane];
        for (int it = 0; it < iters; ++it)
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    if constexpr (DTID == DT_F16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_m, a[i]),
                                                                           __builtin_bit_cast(f16x8_m, b[j]),
                                                                           acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_m, a[i]),
                                                                            __builtin_bit_cast(bf16x8_m, b[j]),
                                                                            acc[i][j], 0, 0, 0);
                }
    }
    float t = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                t += acc[i][j][e];
    if (lane == 0)
        out[blockIdx.x * 8 + wave] = t;
}

}  // namespace

hipError_t launch_mfma_ceiling(int dt, const void *src, float *out, int blocks, int iters, hipStream_t s)
{
    const dim3 grid((unsigned)blocks), block(512);
    if (dt == DT_F32)
        hipLaunchKernelGGL(mfma_ceiling_kernel<DT_F32>, grid, block, 0, s, (const uint32_t *)src, out, iters);
    else if (dt == DT_F16)
        hipLaunchKernelGGL(mfma_ceiling_kernel<DT_F16>, grid, block, 0, s, (const uint32_t *)src, out, iters);
    else
        hipLaunchKernelGGL(mfma_ceiling_kernel<DT_BF16>, grid, block, 0, s, (const uint32_t *)src, out, iters);
    return hipGetLastError();
}

hipError_t launch_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t s)
{
    const long long n = (long long)(bytes / 16);
    hipLaunchKernelGGL(stream_copy_kernel, stream_grid(n), dim3(NT), 0, s, (const u32x4_s *)src,
                       (u32x4_s *)dst, n);
    return hipGetLastError();
}

hipError_t launch_stream_fill(void *dst, uint32_t value, size_t bytes, hipStream_t s)
{
    const long long n = (long long)(bytes / 16);
    hipLaunchKernelGGL(stream_fill_kernel, stream_grid(n), dim3(NT), 0, s, (u32x4_s *)dst, value, n);
    return hipGetLastError();
}

}  // namespace d4r
