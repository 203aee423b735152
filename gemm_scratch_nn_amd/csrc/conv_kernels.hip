// HBM-bound steps of convolution lowered to GEMM, for gfx950.
//
// Steps (directcompute-nn page, "Convolution: The im2col Approach" and the
// "Convolution Shaders" table): im2col (patches -> column matrix), col2im
// (column matrix -> image, the adjoint of im2col), conv_grad_reshape
// ((batch, C, H, W) gradient -> matrix form), and the bias gradient (a
// per-channel sum of the reshaped gradient).
//
// All of these move data and do at most a few adds per element, so they are
// written for coalesced HBM access: consecutive lanes touch consecutive
// addresses of the larger side, stores are 16-byte vectors where the row
// length allows, and nothing uses atomics (col2im is a gather with a fixed
// summation order; reductions go through per-block partials).
#include "internal.hpp"

namespace d4r {

namespace {

constexpr int NT = 256;

template <typename T>
struct Vec16;
template <>
struct Vec16<uint32_t> { typedef uint32_t type __attribute__((ext_vector_type(4))); static constexpr int N = 4; };
template <>
struct Vec16<uint16_t> { typedef uint16_t type __attribute__((ext_vector_type(8))); static constexpr int N = 8; };

__device__ __forceinline__ float to_f32(uint32_t v, int) { return __uint_as_float(v); }
__device__ __forceinline__ float to_f32(uint16_t v, int dt)
{
    if (dt == DT_BF16)
        return __uint_as_float(((uint32_t)v) << 16);
    return (float)__builtin_bit_cast(_Float16, v);
}

// ---------------------------------------------------------------------------
// im2col: col[r][n] = xt(b, c, i*s - p + u, j*s - p + v) with r = (c*kH+u)*kW+v
// and n = (b*OH + i)*OW + j.  A thread owns VW consecutive n (one 16-byte
// store per row) and one (c, u) pair, and walks the kW rows v = 0..kW-1 of
// that pair: the x row segment it gathers from is the same for every v up
// to a shift, so after the first v it is served from L1 / L2 instead of
// HBM.  Raw bit copy: T is the storage word of the dtype.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void im2col_kernel(const T *__restrict__ x, T *__restrict__ col,
                                                    ConvGeom g, int vec_store)
{
    constexpr int VW = Vec16<T>::N;
    const int n0 = (blockIdx.x * NT + threadIdx.x) * VW;
    if (n0 >= g.N)
        return;
    // per element: image plane offset (b*C*H*W) and the window origin
    int base[VW], h0[VW], w0[VW];
    {
        int b = n0 / g.P;
        int rem = n0 - b * g.P;
        int i = rem / g.OW;
        int j = rem - i * g.OW;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            base[e] = b < g.B ? b * g.C * g.H * g.W : -1;
            h0[e] = i * g.s - g.p;
            w0[e] = j * g.s - g.p;
            if (++j == g.OW) {
                j = 0;
                if (++i == g.OH) {
                    i = 0;
                    ++b;
                }
            }
        }
    }
    const int CU = g.C * g.kH;
    for (int cu = blockIdx.y; cu < CU; cu += gridDim.y) {
        const int c = cu / g.kH;
        const int u = cu - c * g.kH;
        const int plane = c * g.H * g.W;
        for (int v = 0; v < g.kW; ++v) {
            typename Vec16<T>::type out;
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                const int hh = h0[e] + u;
                const int ww = w0[e] + v;
                T val = 0;
                if (base[e] >= 0 && hh >= 0 && hh < g.H && ww >= 0 && ww < g.W)
                    val = x[base[e] + plane + hh * g.W + ww];
                out[e] = val;
            }
            T *dst = col + (long long)(cu * g.kW + v) * g.N + n0;
            if (vec_store) {
                *(typename Vec16<T>::type *)dst = out;
            } else {
#pragma unroll
                for (int e = 0; e < VW; ++e)
                    if (n0 + e < g.N)
                        dst[e] = out[e];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// col2im as a gather: one thread per dx element (b, c, h, w) sums the dcol
// entries that im2col copied from (b, c, h, w).  Tap u contributes when
// h + p - u >= 0, divisible by s and (h + p - u)/s < OH, i.e. u runs over one
// residue class mod s between u_lo and u_hi; same for v.  Order: u
// ascending, then v ascending.  TU / TV > 0 fix the number of candidate taps
// per axis (ceil(k / s)) at compile time so every load of a thread is issued
// before the adds; TU = TV = 0 is the general loop.
// ---------------------------------------------------------------------------
template <int TU, int TV>
__global__ __launch_bounds__(NT) void col2im_kernel(const float *__restrict__ dcol,
                                                    float *__restrict__ dx, ConvGeom g, int total)
{
    const int idx = blockIdx.x * NT + threadIdx.x;
    if (idx >= total)
        return;
    const int w = idx % g.W;
    int t = idx / g.W;
    const int h = t % g.H;
    t /= g.H;
    const int c = t % g.C;
    const int b = t / g.C;

    const int hp = h + g.p, wp = w + g.p;
    // smallest u >= max(0, hp - s*(OH-1)) with u = hp (mod s); largest u <= min(kH-1, hp)
    int u_lo = hp - g.s * (g.OH - 1);
    if (u_lo < 0)
        u_lo = 0;
    u_lo += ((hp - u_lo) % g.s);
    const int u_hi = min(g.kH - 1, hp);
    int v_lo = wp - g.s * (g.OW - 1);
    if (v_lo < 0)
        v_lo = 0;
    v_lo += ((wp - v_lo) % g.s);
    const int v_hi = min(g.kW - 1, wp);

    const long long Nl = g.N;
    const int nb = b * g.P;
    float acc = 0.0f;
    if constexpr (TU > 0) {
        float vals[TU][TV];
#pragma unroll
        for (int a = 0; a < TU; ++a) {
            const int u = u_lo + a * g.s;
            const int i = (hp - u) / g.s;
#pragma unroll
            for (int q = 0; q < TV; ++q) {
                const int v = v_lo + q * g.s;
                const int j = (wp - v) / g.s;
                const bool ok = (u <= u_hi) && (v <= v_hi);
                vals[a][q] = ok ? dcol[(long long)((c * g.kH + u) * g.kW + v) * Nl + nb + i * g.OW + j]
                                : 0.0f;
            }
        }
#pragma unroll
        for (int a = 0; a < TU; ++a)
#pragma unroll
            for (int q = 0; q < TV; ++q)
                acc += vals[a][q];
    } else {
        for (int u = u_lo; u <= u_hi; u += g.s) {
            const int i = (hp - u) / g.s;
            const int rbase = (c * g.kH + u) * g.kW;
            for (int v = v_lo; v <= v_hi; v += g.s) {
                const int j = (wp - v) / g.s;
                acc += dcol[(long long)(rbase + v) * Nl + nb + i * g.OW + j];
            }
        }
    }
    dx[idx] = acc;
}

// ---------------------------------------------------------------------------
// conv_grad_reshape: G[o][n] = dy[b][o][pix], n = b*P + pix.  Thread per VW
// consecutive n of one row o: consecutive lanes read consecutive pixels of
// an image plane and write consecutive columns of G.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void grad_reshape_kernel(const T *__restrict__ dy, T *__restrict__ G,
                                                          ConvGeom g, int vec_store)
{
    constexpr int VW = Vec16<T>::N;
    const int n0 = (blockIdx.x * NT + threadIdx.x) * VW;
    if (n0 >= g.N)
        return;
    for (int o = blockIdx.y; o < g.O; o += gridDim.y) {
        int b = n0 / g.P;
        int pix = n0 - b * g.P;
        typename Vec16<T>::type out;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            out[e] = (b < g.B) ? dy[((long long)b * g.O + o) * g.P + pix] : (T)0;
            if (++pix == g.P) {
                pix = 0;
                ++b;
            }
        }
        T *dst = G + (long long)o * g.N + n0;
        if (vec_store) {
            *(typename Vec16<T>::type *)dst = out;
        } else {
#pragma unroll
            for (int e = 0; e < VW; ++e)
                if (n0 + e < g.N)
                    dst[e] = out[e];
        }
    }
}

// ---------------------------------------------------------------------------
// Batched transpose out[b][c][r] = in[b][r][c] through a 64x64 LDS tile
// (one extra column of padding so the column reads hit distinct banks).
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void transpose_kernel(const T *__restrict__ in, T *__restrict__ out,
                                                       int R, int Cc)
{
    __shared__ T tile[64][65];
    const long long base = (long long)blockIdx.z * R * Cc;
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    for (int rr = ty; rr < 64; rr += 4) {
        int r = r0 + rr, c = c0 + tx;
        if (r < R && c < Cc)
            tile[rr][tx] = in[base + (long long)r * Cc + c];
    }
    __syncthreads();
    for (int cc = ty; cc < 64; cc += 4) {
        int c = c0 + cc, r = r0 + tx;
        if (r < R && c < Cc)
            out[base + (long long)c * R + r] = tile[tx][cc];
    }
}

// ---------------------------------------------------------------------------
// Bias gradient.  Pass 1: block (s, o) sums images [s*per, (s+1)*per) of
// channel o; the block reduces through a fixed wave-shuffle tree and LDS.
// Pass 2: one thread per channel adds the partials in split order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

template <typename T>
__global__ __launch_bounds__(NT) void bias_partial_kernel(const T *__restrict__ dy,
                                                          float *__restrict__ partial, ConvGeom g,
                                                          int splits, int per, int dt)
{
    __shared__ float red[NT / 64];
    const int s = blockIdx.x, o = blockIdx.y;
    const int b0 = s * per, b1 = min(g.B, b0 + per);
    float acc = 0.0f;
    for (int b = b0; b < b1; ++b) {
        const T *plane = dy + ((long long)b * g.O + o) * g.P;
        for (int t = threadIdx.x; t < g.P; t += NT)
            acc += to_f32(plane[t], dt);
    }
    acc = wave_sum(acc);
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        float tot = 0.0f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w)
            tot += red[w];
        partial[o * splits + s] = tot;
    }
}

__global__ __launch_bounds__(NT) void bias_final_kernel(const float *__restrict__ partial,
                                                        float *__restrict__ db, int O, int splits)
{
    const int o = blockIdx.x * NT + threadIdx.x;
    if (o >= O)
        return;
    float tot = 0.0f;
    for (int s = 0; s < splits; ++s)
        tot += partial[o * splits + s];
    db[o] = tot;
}

// ---------------------------------------------------------------------------
// Split-K reduction: C = sum_{s} part[s] in split order, then the GEMM
// epilogue (row-major store, or NCHW store with bias).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(NT) void splitk_reduce_kernel(const float *__restrict__ part, int splits,
                                                           int M, int N, long long stride, int epi,
                                                           float *__restrict__ C, int ldc,
                                                           const float *__restrict__ bias, int P)
{
    const long long idx = (long long)blockIdx.x * NT + threadIdx.x;
    if (idx >= (long long)M * N)
        return;
    const int m = (int)(idx / N);
    const int n = (int)(idx - (long long)m * N);
    float acc = 0.0f;
    for (int s = 0; s < splits; ++s)
        acc += part[s * stride + idx];
    if (epi == EPI_NCHW) {
        if (bias)
            acc += bias[m];
        const int b = n / P, pix = n - b * P;
        C[((long long)b * M + m) * P + pix] = acc;
    } else {
        C[(long long)m * ldc + n] = acc;
    }
}

inline dim3 grid2(long long x, long long y)
{
    return dim3((unsigned)x, (unsigned)(y < 65535 ? y : 65535), 1);
}

}  // namespace

hipError_t launch_im2col(int dt, const ConvGeom &g, const void *x, void *col, hipStream_t s)
{
    const int VW = dt == DT_F32 ? 4 : 8;
    const long long threads = (g.N + VW - 1) / VW;
    dim3 grid = grid2((threads + NT - 1) / NT, (long long)g.C * g.kH);
    const int vec = (g.N % VW) == 0;
    if (dt == DT_F32)
        hipLaunchKernelGGL(im2col_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)x,
                           (uint32_t *)col, g, vec);
    else
        hipLaunchKernelGGL(im2col_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)x,
                           (uint16_t *)col, g, vec);
    return hipGetLastError();
}

hipError_t launch_col2im(const ConvGeom &g, const float *dcol, float *dx, hipStream_t s)
{
    const int total = g.B * g.C * g.H * g.W;
    const dim3 grid((total + NT - 1) / NT), block(NT);
    const int tu = (g.kH + g.s - 1) / g.s, tv = (g.kW + g.s - 1) / g.s;
    if (tu == 1 && tv == 1)
        hipLaunchKernelGGL((col2im_kernel<1, 1>), grid, block, 0, s, dcol, dx, g, total);
    else if (tu == 2 && tv == 2)
        hipLaunchKernelGGL((col2im_kernel<2, 2>), grid, block, 0, s, dcol, dx, g, total);
    else if (tu == 3 && tv == 3)
        hipLaunchKernelGGL((col2im_kernel<3, 3>), grid, block, 0, s, dcol, dx, g, total);
    else if (tu == 5 && tv == 5)
        hipLaunchKernelGGL((col2im_kernel<5, 5>), grid, block, 0, s, dcol, dx, g, total);
    else
        hipLaunchKernelGGL((col2im_kernel<0, 0>), grid, block, 0, s, dcol, dx, g, total);
    return hipGetLastError();
}

hipError_t launch_grad_reshape(int dt, const ConvGeom &g, const void *dy, void *G, hipStream_t s)
{
    const int VW = dt == DT_F32 ? 4 : 8;
    const long long threads = (g.N + VW - 1) / VW;
    dim3 grid = grid2((threads + NT - 1) / NT, g.O);
    const int vec = (g.N % VW) == 0;
    if (dt == DT_F32)
        hipLaunchKernelGGL(grad_reshape_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)dy,
                           (uint32_t *)G, g, vec);
    else
        hipLaunchKernelGGL(grad_reshape_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)dy,
                           (uint16_t *)G, g, vec);
    return hipGetLastError();
}

hipError_t launch_transpose(int dt, int batch, int R, int Cc, const void *in, void *out, hipStream_t s)
{
    dim3 grid((Cc + 63) / 64, (R + 63) / 64, batch);
    if (dt == DT_F32)
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)in,
                           (uint32_t *)out, R, Cc);
    else
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)in,
                           (uint16_t *)out, R, Cc);
    return hipGetLastError();
}

int bias_grad_splits(const ConvGeom &g)
{
    // enough blocks to cover the chip (>= ~2048), at most one image per block
    int want = (2048 + g.O - 1) / g.O;
    if (want > g.B)
        want = g.B;
    if (want < 1)
        want = 1;
    int per = (g.B + want - 1) / want;
    return (g.B + per - 1) / per;
}

hipError_t launch_bias_grad(int dt, const ConvGeom &g, const void *dy, float *db, float *partial,
                            int splits, hipStream_t s)
{
    const int per = (g.B + splits - 1) / splits;
    dim3 grid(splits, g.O);
    if (dt == DT_F32)
        hipLaunchKernelGGL(bias_partial_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)dy,
                           partial, g, splits, per, dt);
    else
        hipLaunchKernelGGL(bias_partial_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)dy,
                           partial, g, splits, per, dt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(bias_final_kernel, dim3((g.O + NT - 1) / NT), dim3(NT), 0, s, partial, db, g.O,
                       splits);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N, long long split_stride,
                                int epi, float *C, int ldc, const float *bias, int P, hipStream_t s)
{
    const long long total = (long long)M * N;
    hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((total + NT - 1) / NT)), dim3(NT), 0, s,
                       part, splits, M, N, split_stride, epi, C, ldc, bias, P);
    return hipGetLastError();
}

}  // namespace d4r
