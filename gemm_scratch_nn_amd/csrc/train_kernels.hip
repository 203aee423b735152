// The rest of a training step around the convolutions, for gfx950, f32:
// ReLU and its gradient, max pooling with argmax and its backward, the row
// bias of a linear layer and its gradient, the softmax-cross-entropy
// gradient with the mean loss, SGD with gradient clipping, and gradient
// accumulation (directcompute-nn page, "HLSL Shader Reference":
// "Activation / Loss Shaders", "Pooling Shaders", "Utility Shaders").
//
// Everything here is HBM- or latency-bound elementwise / small-reduction
// work: grid-stride loops with 16-byte accesses where the data allows, and
// no atomics.  The max-pool backward is a gather (each input element sums
// the windows whose saved argmax is itself, windows in row-major order), so
// overlapping windows need no scatter conflicts; reductions use fixed
// per-thread orders and fixed trees, so every result is run-to-run
// deterministic.
#include <algorithm>

#include "internal.hpp"

namespace d4r {

namespace {

constexpr int NT = 256;

inline unsigned blocks_for(long long n, int per_thread)
{
    long long b = (n + (long long)NT * per_thread - 1) / ((long long)NT * per_thread);
    if (b < 1)
        b = 1;
    return (unsigned)(b < 65536 * 16 ? b : 65536 * 16);
}

// y = max(x, 0); dx = dy where x > 0 (strictly), else 0.  Each element is
// read and written by one thread at one index, so y may be x and dx may be
// dy (in place).  Pointers are 16-byte aligned (checked by the caller).
__global__ __launch_bounds__(NT) void relu_fwd_kernel(const float *x, float *y, long long n)
{
    const long long n4 = n / 4;
    const long long stride = (long long)gridDim.x * NT;
    for (long long i = (long long)blockIdx.x * NT + threadIdx.x; i < n4; i += stride) {
        float4 v = ((const float4 *)x)[i];
        v.x = v.x > 0.0f ? v.x : 0.0f;
        v.y = v.y > 0.0f ? v.y : 0.0f;
        v.z = v.z > 0.0f ? v.z : 0.0f;
        v.w = v.w > 0.0f ? v.w : 0.0f;
        ((float4 *)y)[i] = v;
    }
    for (long long i = n4 * 4 + (long long)blockIdx.x * NT + threadIdx.x; i < n; i += stride)
        y[i] = x[i] > 0.0f ? x[i] : 0.0f;
}

__global__ __launch_bounds__(NT) void relu_bwd_kernel(const float *__restrict__ x, const float *dy, float *dx,
                                                      long long n)
{
    const long long n4 = n / 4;
    const long long stride = (long long)gridDim.x * NT;
    for (long long i = (long long)blockIdx.x * NT + threadIdx.x; i < n4; i += stride) {
        const float4 v = ((const float4 *)x)[i];
        const float4 g = ((const float4 *)dy)[i];
        float4 r;
        r.x = v.x > 0.0f ? g.x : 0.0f;
        r.y = v.y > 0.0f ? g.y : 0.0f;
        r.z = v.z > 0.0f ? g.z : 0.0f;
        r.w = v.w > 0.0f ? g.w : 0.0f;
        ((float4 *)dx)[i] = r;
    }
    for (long long i = n4 * 4 + (long long)blockIdx.x * NT + threadIdx.x; i < n; i += stride)
        dx[i] = x[i] > 0.0f ? dy[i] : 0.0f;
}

// One thread per output: scan the k x k window row-major, the first strict
// maximum wins; idx = its offset h*W + w inside the (b, c) plane.
__global__ __launch_bounds__(NT) void maxpool_fwd_kernel(const float *__restrict__ x, float *__restrict__ y,
                                                         int32_t *__restrict__ idx, long long planes, int H,
                                                         int W, int OH, int OW, int k, int s)
{
    const long long total = planes * OH * OW;
    const long long stride = (long long)gridDim.x * NT;
    for (long long o = (long long)blockIdx.x * NT + threadIdx.x; o < total; o += stride) {
        const long long pl = o / ((long long)OH * OW);
        const int r = (int)(o - pl * OH * OW);
        const int i = r / OW, j = r - (r / OW) * OW;
        const float *xp = x + pl * H * W;
        int best = (i * s) * W + j * s;
        float bv = xp[best];
        for (int u = 0; u < k; ++u)
            for (int v = 0; v < k; ++v) {
                const int at = (i * s + u) * W + (j * s + v);
                const float xv = xp[at];
                if (xv > bv) {
                    bv = xv;
                    best = at;
                }
            }
        y[o] = bv;
        idx[o] = best;
    }
}

// The same scan with the window size K fixed at compile time: blockIdx.y is
// the plane, blockIdx.x * NT + thread the output position (the host checks
// OH*OW < 2^20, OW <= 1024 for small_div, planes <= 65535).  The K*K loads
// are issued before the scan, which keeps the first strict maximum in
// row-major order as above.
template <int K>
__global__ __launch_bounds__(NT) void maxpool_fwd_fixed_kernel(const float *__restrict__ x, float *__restrict__ y,
                                                               int32_t *__restrict__ idx, int H, int W, int OH,
                                                               int OW, int s)
{
    const int r = blockIdx.x * NT + threadIdx.x;
    if (r >= OH * OW)
        return;
    const int i = small_div(r, OW), j = r - i * OW;
    const float *xp = x + (long long)blockIdx.y * H * W;
    float v[K][K];
#pragma unroll
    for (int u = 0; u < K; ++u)
#pragma unroll
        for (int q = 0; q < K; ++q)
            v[u][q] = xp[(i * s + u) * W + (j * s + q)];
    int best = (i * s) * W + j * s;
    float bv = v[0][0];
#pragma unroll
    for (int u = 0; u < K; ++u)
#pragma unroll
        for (int q = 0; q < K; ++q)
            if (v[u][q] > bv) {
                bv = v[u][q];
                best = (i * s + u) * W + (j * s + q);
            }
    const long long o = (long long)blockIdx.y * OH * OW + r;
    y[o] = bv;
    idx[o] = best;
}

// One thread per input element: add dy of every window that covers it and
// saved it as the maximum, windows i ascending then j ascending.  A gather,
// so overlapping windows (stride < k) need no atomics and every dx element
// is written (0 where no window chose it).
__global__ __launch_bounds__(NT) void maxpool_bwd_kernel(const float *__restrict__ dy,
                                                         const int32_t *__restrict__ idx,
                                                         float *__restrict__ dx, long long planes, int H,
                                                         int W, int OH, int OW, int k, int s)
{
    const long long total = planes * H * W;
    const long long stride = (long long)gridDim.x * NT;
    for (long long e = (long long)blockIdx.x * NT + threadIdx.x; e < total; e += stride) {
        const long long pl = e / ((long long)H * W);
        const int at = (int)(e - pl * H * W);
        const int h = at / W, w = at - (at / W) * W;
        // windows i with i*s <= h < i*s + k, clipped to the output extent
        const int i0 = h >= k ? (h - k) / s + 1 : 0, i1 = min(h / s, OH - 1);
        const int j0 = w >= k ? (w - k) / s + 1 : 0, j1 = min(w / s, OW - 1);
        float acc = 0.0f;
        const long long base = pl * OH * OW;
        for (int i = i0; i <= i1; ++i)
            for (int j = j0; j <= j1; ++j) {
                const long long o = base + (long long)i * OW + j;
                if (idx[o] == at)
                    acc += dy[o];
            }
        dx[e] = acc;
    }
}

// The same gather with T = ceil(k/s) candidate windows per axis fixed at
// compile time: blockIdx.y is the plane and blockIdx.x * NT + thread the
// position in it (the host checks H*W < 2^20, W <= 1024 for small_div, and
// planes <= 65535).  Every candidate's argmax and dy are loaded
// unconditionally (a candidate outside the window range reads window 0 of
// the plane and is dropped), so all loads of an element are in flight
// together; they are added in the same order as above (i, then j
// ascending), so the sums are identical.
template <int T>
__global__ __launch_bounds__(NT) void maxpool_bwd_fixed_kernel(const float *__restrict__ dy,
                                                               const int32_t *__restrict__ idx,
                                                               float *__restrict__ dx, int H, int W, int OH,
                                                               int OW, int k, int s)
{
    const int at = blockIdx.x * NT + threadIdx.x;
    if (at >= H * W)
        return;
    const int h = small_div(at, W), w = at - h * W;
    const int i0 = h >= k ? (h - k) / s + 1 : 0, i1 = min(h / s, OH - 1);
    const int j0 = w >= k ? (w - k) / s + 1 : 0, j1 = min(w / s, OW - 1);
    const long long base = (long long)blockIdx.y * OH * OW;
    int id[T][T];
    float v[T][T];
#pragma unroll
    for (int a = 0; a < T; ++a)
#pragma unroll
        for (int b = 0; b < T; ++b) {
            const bool ok = i0 + a <= i1 && j0 + b <= j1;
            const long long o = base + (ok ? (i0 + a) * OW + j0 + b : 0);
            const int32_t io = idx[o];
            id[a][b] = ok ? io : -1;
            v[a][b] = dy[o];
        }
    float acc = 0.0f;
#pragma unroll
    for (int a = 0; a < T; ++a)
#pragma unroll
        for (int b = 0; b < T; ++b)
            if (id[a][b] == at)
                acc += v[a][b];
    dx[(long long)blockIdx.y * H * W + at] = acc;
}

// y[i][j] = x[i][j] + bias[j]; y may be x (one thread per element)
__global__ __launch_bounds__(NT) void add_bias_rows_kernel(const float *x, const float *__restrict__ bias,
                                                           float *y, long long rows, int cols)
{
    const long long total = rows * cols;
    const long long stride = (long long)gridDim.x * NT;
    for (long long e = (long long)blockIdx.x * NT + threadIdx.x; e < total; e += stride)
        y[e] = x[e] + bias[e % cols];
}

// db[j] = sum over rows of dy[i][j].  A block of kBgWaves wavefronts owns
// 64 columns; wave w sums the rows [w*rows/kBgWaves, (w+1)*rows/kBgWaves)
// ascending with lane = column (one 256-byte row segment per load, eight
// loads in flight), then the partial sums are added in wave order.
constexpr int kBgWaves = 16;

__global__ __launch_bounds__(kBgWaves * 64) void bias_grad_rows_kernel(const float *__restrict__ dy,
                                                                       float *__restrict__ db, long long rows,
                                                                       int cols)
{
    __shared__ float part[kBgWaves][64];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int j = blockIdx.x * 64 + lane;
    const long long r0 = rows * wv / kBgWaves, r1 = rows * (wv + 1) / kBgWaves;
    float acc = 0.0f;
    if (j < cols) {
        const float *col = dy + j;
        long long i = r0;
        for (; i + 8 <= r1; i += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                v[u] = col[(i + u) * cols];
#pragma unroll
            for (int u = 0; u < 8; ++u)
                acc += v[u];
        }
        for (; i < r1; ++i)
            acc += col[i * cols];
    }
    part[wv][lane] = acc;
    __syncthreads();
    if (wv == 0 && j < cols) {
        float t = part[0][lane];
#pragma unroll
        for (int w = 1; w < kBgWaves; ++w)
            t += part[w][lane];
        db[j] = t;
    }
}

// Butterfly sum / max over aligned groups of G lanes (G a power of two <= 64)
template <int G>
__device__ __forceinline__ float group_sum(float v)
{
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

template <int G>
__device__ __forceinline__ float group_max(float v)
{
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1)
        v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

constexpr int kSmWaves = 16;  // waves per softmax block

// Row softmax by groups of G lanes (G = the class count rounded up to a
// power of two, at most 64; lanes stride over the classes), 64/G rows per
// wavefront at a time; max and sum by fixed butterfly trees, the row
// maximum subtracted before exp.
//   label == NULL: out = softmax(z)
//   label != NULL: out = softmax(z) - one_hot(label), and when loss != NULL
//                  *loss = mean over rows of log(sum) + max - z[label]
// With a loss the launch is one block: the first lane of each group adds its
// rows' losses in row order, the groups of a wave are added by a fixed
// tree, then thread 0 adds the waves' sums in wave order, so the loss is
// run-to-run deterministic.  A label outside [0, classes) makes that row of
// out and the loss NaN.  out must not overlap z.
template <int G>
__global__ __launch_bounds__(kSmWaves * 64) void softmax_rows_kernel(const float *__restrict__ z,
                                                                     const int32_t *__restrict__ label,
                                                                     float *__restrict__ out,
                                                                     float *__restrict__ loss, int rows,
                                                                     int classes)
{
    constexpr int RPW = 64 / G;  // rows per wavefront pass
    __shared__ float red[kSmWaves];
    const int lane = threadIdx.x & 63;
    const int gl = lane % G;  // lane within the group
    const int wave = blockIdx.x * kSmWaves + (threadIdx.x >> 6);
    const int nrows = gridDim.x * kSmWaves * RPW;
    float lsum = 0.0f;
    for (int r0 = wave * RPW; r0 < rows; r0 += nrows) {
        const int r = r0 + lane / G;
        const bool live = r < rows;  // uniform within a group
        const int rr = live ? r : r0;
        const float *zr = z + (long long)rr * classes;
        float *orow = out + (long long)rr * classes;
        float m = -__builtin_inff();
        for (int j = gl; j < classes; j += G)
            m = fmaxf(m, zr[j]);
        m = group_max<G>(m);
        float sum = 0.0f;
        for (int j = gl; j < classes; j += G)
            sum += expf(zr[j] - m);
        sum = group_sum<G>(sum);
        if (!live)
            continue;
        const float inv = 1.0f / sum;
        if (!label) {
            for (int j = gl; j < classes; j += G)
                orow[j] = expf(zr[j] - m) * inv;
            continue;
        }
        const int lab = label[r];
        const bool ok = lab >= 0 && lab < classes;
        for (int j = gl; j < classes; j += G)
            orow[j] = ok ? expf(zr[j] - m) * inv - (j == lab ? 1.0f : 0.0f) : __builtin_nanf("");
        const float zl = zr[ok ? lab : 0];  // never read outside the row
        lsum += ok ? logf(sum) + m - zl : __builtin_nanf("");
    }
    if (!loss)
        return;
    // the group leaders hold the row sums; add the wave's groups in order
    float w = 0.0f;
#pragma unroll
    for (int g = 0; g < RPW; ++g)
        w += __shfl(lsum, g * G, 64);
    if (lane == 0)
        red[threadIdx.x >> 6] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = red[0];
#pragma unroll
        for (int v = 1; v < kSmWaves; ++v)
            t += red[v];
        *loss = t / (float)rows;
    }
}

// param -= lr * clamp(grad, -clip, clip); 16-byte accesses plus a tail
__device__ __forceinline__ float sgd_one(float p, float g, float lr, float clip)
{
    return p - lr * fminf(fmaxf(g, -clip), clip);
}

__global__ __launch_bounds__(NT) void sgd_kernel(float *__restrict__ p, const float *__restrict__ g, long long n,
                                                 float lr, float clip)
{
    const long long n4 = n / 4;
    const long long stride = (long long)gridDim.x * NT;
    for (long long i = (long long)blockIdx.x * NT + threadIdx.x; i < n4; i += stride) {
        float4 v = ((float4 *)p)[i];
        const float4 d = ((const float4 *)g)[i];
        v.x = sgd_one(v.x, d.x, lr, clip);
        v.y = sgd_one(v.y, d.y, lr, clip);
        v.z = sgd_one(v.z, d.z, lr, clip);
        v.w = sgd_one(v.w, d.w, lr, clip);
        ((float4 *)p)[i] = v;
    }
    for (long long i = n4 * 4 + (long long)blockIdx.x * NT + threadIdx.x; i < n; i += stride)
        p[i] = sgd_one(p[i], g[i], lr, clip);
}

// acc += g; 16-byte accesses plus a tail
__global__ __launch_bounds__(NT) void grad_accum_kernel(float *__restrict__ acc, const float *__restrict__ g,
                                                        long long n)
{
    const long long n4 = n / 4;
    const long long stride = (long long)gridDim.x * NT;
    for (long long i = (long long)blockIdx.x * NT + threadIdx.x; i < n4; i += stride) {
        float4 a = ((float4 *)acc)[i];
        const float4 d = ((const float4 *)g)[i];
        a.x += d.x;
        a.y += d.y;
        a.z += d.z;
        a.w += d.w;
        ((float4 *)acc)[i] = a;
    }
    for (long long i = n4 * 4 + (long long)blockIdx.x * NT + threadIdx.x; i < n; i += stride)
        acc[i] = acc[i] + g[i];
}

}  // namespace

hipError_t launch_relu_forward(const float *x, float *y, long long n, hipStream_t s)
{
    hipLaunchKernelGGL(relu_fwd_kernel, dim3(blocks_for(n, 4)), dim3(NT), 0, s, x, y, n);
    return hipGetLastError();
}

hipError_t launch_relu_backward(const float *x, const float *dy, float *dx, long long n, hipStream_t s)
{
    hipLaunchKernelGGL(relu_bwd_kernel, dim3(blocks_for(n, 4)), dim3(NT), 0, s, x, dy, dx, n);
    return hipGetLastError();
}

hipError_t launch_maxpool_forward(const float *x, float *y, int32_t *idx, long long planes, int H, int W,
                                  int OH, int OW, int k, int st, hipStream_t s)
{
    if (planes <= 65535 && (long long)OH * OW < (1 << 20) && OW <= 1024 && (k == 2 || k == 3)) {
        const dim3 grid((unsigned)((OH * OW + NT - 1) / NT), (unsigned)planes);
        if (k == 2)
            hipLaunchKernelGGL(maxpool_fwd_fixed_kernel<2>, grid, dim3(NT), 0, s, x, y, idx, H, W, OH, OW, st);
        else
            hipLaunchKernelGGL(maxpool_fwd_fixed_kernel<3>, grid, dim3(NT), 0, s, x, y, idx, H, W, OH, OW, st);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(maxpool_fwd_kernel, dim3(blocks_for(planes * OH * OW, 1)), dim3(NT), 0, s, x, y, idx,
                       planes, H, W, OH, OW, k, st);
    return hipGetLastError();
}

hipError_t launch_maxpool_backward(const float *dy, const int32_t *idx, float *dx, long long planes, int H,
                                   int W, int OH, int OW, int k, int st, hipStream_t s)
{
    const long long total = planes * H * W;
    const int t = (k + st - 1) / st;  // candidate windows per axis
    if (planes <= 65535 && (long long)H * W < (1 << 20) && W <= 1024 && t <= 3) {
        const dim3 grid((unsigned)((H * W + NT - 1) / NT), (unsigned)planes);
        if (t == 1)
            hipLaunchKernelGGL(maxpool_bwd_fixed_kernel<1>, grid, dim3(NT), 0, s, dy, idx, dx, H, W, OH, OW, k, st);
        else if (t == 2)
            hipLaunchKernelGGL(maxpool_bwd_fixed_kernel<2>, grid, dim3(NT), 0, s, dy, idx, dx, H, W, OH, OW, k, st);
        else
            hipLaunchKernelGGL(maxpool_bwd_fixed_kernel<3>, grid, dim3(NT), 0, s, dy, idx, dx, H, W, OH, OW, k, st);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(maxpool_bwd_kernel, dim3(blocks_for(total, 1)), dim3(NT), 0, s, dy, idx, dx, planes, H, W,
                       OH, OW, k, st);
    return hipGetLastError();
}

hipError_t launch_add_bias_rows(const float *x, const float *bias, float *y, long long rows, int cols,
                                hipStream_t s)
{
    hipLaunchKernelGGL(add_bias_rows_kernel, dim3(blocks_for(rows * cols, 1)), dim3(NT), 0, s, x, bias, y,
                       rows, cols);
    return hipGetLastError();
}

hipError_t launch_bias_grad_rows(const float *dy, float *db, long long rows, int cols, hipStream_t s)
{
    hipLaunchKernelGGL(bias_grad_rows_kernel, dim3((cols + 63) / 64), dim3(kBgWaves * 64), 0, s, dy, db, rows,
                       cols);
    return hipGetLastError();
}

template <int G>
static hipError_t softmax_launch(const float *z, const int32_t *label, float *out, float *loss, int rows,
                                 int classes, hipStream_t s)
{
    // with a loss: one block (fixed-order mean); else enough blocks for one
    // pass over the rows
    const int per_block = kSmWaves * (64 / G);
    const int blocks = loss ? 1 : std::min((rows + per_block - 1) / per_block, 65535);
    hipLaunchKernelGGL(softmax_rows_kernel<G>, dim3(blocks), dim3(kSmWaves * 64), 0, s, z, label, out, loss,
                       rows, classes);
    return hipGetLastError();
}

hipError_t launch_softmax_rows(const float *z, const int32_t *label, float *out, float *loss, int rows,
                               int classes, hipStream_t s)
{
    if (classes <= 1)
        return softmax_launch<1>(z, label, out, loss, rows, classes, s);
    if (classes <= 2)
        return softmax_launch<2>(z, label, out, loss, rows, classes, s);
    if (classes <= 4)
        return softmax_launch<4>(z, label, out, loss, rows, classes, s);
    if (classes <= 8)
        return softmax_launch<8>(z, label, out, loss, rows, classes, s);
    if (classes <= 16)
        return softmax_launch<16>(z, label, out, loss, rows, classes, s);
    if (classes <= 32)
        return softmax_launch<32>(z, label, out, loss, rows, classes, s);
    return softmax_launch<64>(z, label, out, loss, rows, classes, s);
}

hipError_t launch_sgd(float *p, const float *g, long long n, float lr, float clip, hipStream_t s)
{
    hipLaunchKernelGGL(sgd_kernel, dim3(blocks_for(n, 4)), dim3(NT), 0, s, p, g, n, lr, clip);
    return hipGetLastError();
}

hipError_t launch_grad_accum(float *acc, const float *g, long long n, hipStream_t s)
{
    hipLaunchKernelGGL(grad_accum_kernel, dim3(blocks_for(n, 4)), dim3(NT), 0, s, acc, g, n);
    return hipGetLastError();
}

}  // namespace d4r
