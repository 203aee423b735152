// Plain streaming kernels: the HBM rates this library's own code reaches
// for a read+write stream (copy) and a write-only stream (fill), the
// attainable reference the bench puts beside the HBM-bound steps (im2col,
// col2im, transposes, split-K reductions).  Not a step of the method.
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

}  // namespace

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
