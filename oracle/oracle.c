/*
 * CPU oracle for convolution lowered to matrix multiplication.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  The product path (the HIP library
 * and its Python binding) never calls it, links it or shares code with it.
 *
 * Everything here is the plain definition of what the method computes,
 * written as direct loop nests in double precision.  The convolution routines
 * do NOT lower to im2col: they sum over the kernel window directly, so they
 * check the im2col -> GEMM -> reshape pipeline against the definition it is
 * meant to reach (up to floating-point summation order).
 *
 * Source passages (directcompute-nn 0.1.0 page):
 *   - "Convolution: The im2col Approach", Forward: the col matrix is
 *     (inC*kH*kW) x (batch*outH*outW); filters are outC x (inC*kH*kW);
 *     conv_reshape adds bias and gives (batch, outC, outH, outW).
 *   - same section, Backward: filter grad = grad_reshaped x col^T, input grad
 *     = filters^T x grad_reshaped then col2im, bias grad = per-channel sum.
 *   - "Transpose via Flags": the two operand index formulas of the matmul.
 *   - "Constant Buffer Convention": the im2col parameter list
 *     (batch, inC, inH, inW, kH, stride, padding, outH, outW).
 *
 * Readings where the page is silent: zero padding on all four sides by the
 * one padding value; the same stride on both axes; output extent
 * floor((in + 2p - k)/s) + 1; tensors NCHW, filters OIHW, col rows ordered
 * (c, u, v) with v fastest and columns (b, i, j) with j fastest.
 *
 * Error behaviour: every routine returns 0 on success and -1 on an invalid
 * size (non-positive extent, stride < 1, padding < 0, output extent < 1 or a
 * flags value above 3); outputs are then left untouched.
 *
 * Parallelism: OpenMP over independent outer loops only, each output element
 * written by one thread with a fixed summation order, so results do not
 * depend on the thread count.
 */
#include <stddef.h>
#include <stdint.h>
#include <math.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef long long i64;

static i64 extent(i64 in, i64 k, i64 s, i64 p)
{
    i64 span = in + 2 * p - k;
    if (span < 0)
        return 0;
    return span / s + 1;
}

static int bad_shape(i64 B, i64 C, i64 H, i64 W, i64 O, i64 kH, i64 kW,
                     i64 s, i64 p, i64 *OH, i64 *OW)
{
    if (B < 1 || C < 1 || H < 1 || W < 1 || O < 1 || kH < 1 || kW < 1 ||
        s < 1 || p < 0)
        return 1;
    *OH = extent(H, kH, s, p);
    *OW = extent(W, kW, s, p);
    return (*OH < 1 || *OW < 1);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_out_dims(i64 H, i64 W, i64 kH, i64 kW, i64 s, i64 p,
                    i64 *OH, i64 *OW)
{
    if (H < 1 || W < 1 || kH < 1 || kW < 1 || s < 1 || p < 0)
        return -1;
    *OH = extent(H, kH, s, p);
    *OW = extent(W, kW, s, p);
    return 0;
}

/*
 * Forward:  y[b,o,i,j] = bias[o] + sum_{c,u,v} w[o,c,u,v] * xt(b,c,i*s-p+u, j*s-p+v)
 * where xt is x inside the image and 0 outside.  bias may be NULL (= 0).
 */
int oracle_conv_forward(const double *x, const double *w, const double *bias,
                        double *y, i64 B, i64 C, i64 H, i64 W, i64 O,
                        i64 kH, i64 kW, i64 s, i64 p)
{
    i64 OH, OW;
    if (bad_shape(B, C, H, W, O, kH, kW, s, p, &OH, &OW))
        return -1;
    i64 BO = B * O;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 bo = 0; bo < BO; ++bo) {
        i64 b = bo / O, o = bo % O;
        double *yp = y + bo * OH * OW;
        for (i64 t = 0; t < OH * OW; ++t)
            yp[t] = 0.0;
        for (i64 c = 0; c < C; ++c) {
            const double *xp = x + (b * C + c) * H * W;
            for (i64 u = 0; u < kH; ++u) {
                for (i64 v = 0; v < kW; ++v) {
                    double wv = w[((o * C + c) * kH + u) * kW + v];
                    for (i64 i = 0; i < OH; ++i) {
                        i64 h = i * s - p + u;
                        if (h < 0 || h >= H)
                            continue;
                        for (i64 j = 0; j < OW; ++j) {
                            i64 ww = j * s - p + v;
                            if (ww < 0 || ww >= W)
                                continue;
                            yp[i * OW + j] += wv * xp[h * W + ww];
                        }
                    }
                }
            }
        }
        double bv = bias ? bias[o] : 0.0;
        for (i64 t = 0; t < OH * OW; ++t)
            yp[t] += bv;
    }
    return 0;
}

/*
 * Filter gradient: dw[o,c,u,v] = sum_{b,i,j} g[b,o,i,j] * xt(b,c,i*s-p+u, j*s-p+v).
 */
int oracle_conv_backward_filter(const double *x, const double *g, double *dw,
                                i64 B, i64 C, i64 H, i64 W, i64 O,
                                i64 kH, i64 kW, i64 s, i64 p)
{
    i64 OH, OW;
    if (bad_shape(B, C, H, W, O, kH, kW, s, p, &OH, &OW))
        return -1;
    i64 OC = O * C;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 oc = 0; oc < OC; ++oc) {
        i64 o = oc / C, c = oc % C;
        for (i64 u = 0; u < kH; ++u) {
            for (i64 v = 0; v < kW; ++v) {
                double acc = 0.0;
                for (i64 b = 0; b < B; ++b) {
                    const double *gp = g + (b * O + o) * OH * OW;
                    const double *xp = x + (b * C + c) * H * W;
                    for (i64 i = 0; i < OH; ++i) {
                        i64 h = i * s - p + u;
                        if (h < 0 || h >= H)
                            continue;
                        for (i64 j = 0; j < OW; ++j) {
                            i64 ww = j * s - p + v;
                            if (ww < 0 || ww >= W)
                                continue;
                            acc += gp[i * OW + j] * xp[h * W + ww];
                        }
                    }
                }
                dw[((o * C + c) * kH + u) * kW + v] = acc;
            }
        }
    }
    return 0;
}

/*
 * Bias gradient: db[o] = sum_{b,i,j} g[b,o,i,j]  (a per-channel sum over the
 * batch and both spatial axes).
 */
int oracle_conv_backward_bias(const double *g, double *db, i64 B, i64 O, i64 P)
{
    if (B < 1 || O < 1 || P < 1)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 o = 0; o < O; ++o) {
        double acc = 0.0;
        for (i64 b = 0; b < B; ++b) {
            const double *gp = g + (b * O + o) * P;
            for (i64 t = 0; t < P; ++t)
                acc += gp[t];
        }
        db[o] = acc;
    }
    return 0;
}

/*
 * Data gradient: dx[b,c,h,w] = sum over (o,u,v,i,j) with i*s-p+u = h and
 * j*s-p+v = w of g[b,o,i,j] * w[o,c,u,v].  Each (b,c) plane is owned by one
 * thread, which adds every contribution into it in a fixed order.
 */
int oracle_conv_backward_data(const double *g, const double *w, double *dx,
                              i64 B, i64 C, i64 H, i64 W, i64 O,
                              i64 kH, i64 kW, i64 s, i64 p)
{
    i64 OH, OW;
    if (bad_shape(B, C, H, W, O, kH, kW, s, p, &OH, &OW))
        return -1;
    i64 BC = B * C;
#pragma omp parallel for schedule(dynamic, 1)
    for (i64 bc = 0; bc < BC; ++bc) {
        i64 b = bc / C, c = bc % C;
        double *dp = dx + bc * H * W;
        for (i64 t = 0; t < H * W; ++t)
            dp[t] = 0.0;
        for (i64 o = 0; o < O; ++o) {
            const double *gp = g + (b * O + o) * OH * OW;
            for (i64 u = 0; u < kH; ++u) {
                for (i64 v = 0; v < kW; ++v) {
                    double wv = w[((o * C + c) * kH + u) * kW + v];
                    for (i64 i = 0; i < OH; ++i) {
                        i64 h = i * s - p + u;
                        if (h < 0 || h >= H)
                            continue;
                        for (i64 j = 0; j < OW; ++j) {
                            i64 ww = j * s - p + v;
                            if (ww < 0 || ww >= W)
                                continue;
                            dp[h * W + ww] += gp[i * OW + j] * wv;
                        }
                    }
                }
            }
        }
    }
    return 0;
}

/*
 * GEMM with transpose flags: C[m,n] = sum_k A'(m,k) * B'(k,n), C overwritten,
 * where A'(m,k) = A[m*K+k], or A[k*M+m] when flags&1 (A stored transposed);
 * B'(k,n) = B[k*N+n], or B[n*K+k] when flags&2 (B stored transposed).
 * Operands are packed with no leading dimension, as the two index formulas
 * on the page assume.
 */
int oracle_gemm(const double *A, const double *Bm, double *Cm, i64 M, i64 K,
                i64 N, int flags)
{
    if (M < 1 || K < 1 || N < 1 || flags < 0 || flags > 3)
        return -1;
    int ta = flags & 1, tb = (flags >> 1) & 1;
#pragma omp parallel for schedule(static)
    for (i64 m = 0; m < M; ++m) {
        for (i64 n = 0; n < N; ++n) {
            double acc = 0.0;
            for (i64 k = 0; k < K; ++k) {
                double a = ta ? A[k * M + m] : A[m * K + k];
                double b = tb ? Bm[n * K + k] : Bm[k * N + n];
                acc += a * b;
            }
            Cm[m * N + n] = acc;
        }
    }
    return 0;
}

/*
 * Index-map specifications (used by tests to check the GPU's col matrix and
 * col2im result element by element; the convolution routines above do not
 * use them).
 *
 * im2col: col[(c*kH+u)*kW+v, (b*OH+i)*OW+j] = xt(b,c,i*s-p+u, j*s-p+v),
 * a (C*kH*kW) x (B*OH*OW) row-major matrix.
 */
int oracle_im2col_spec(const double *x, double *col, i64 B, i64 C, i64 H,
                       i64 W, i64 kH, i64 kW, i64 s, i64 p)
{
    i64 OH, OW;
    if (bad_shape(B, C, H, W, 1, kH, kW, s, p, &OH, &OW))
        return -1;
    i64 N = B * OH * OW;
    i64 R = C * kH * kW;
#pragma omp parallel for schedule(static)
    for (i64 r = 0; r < R; ++r) {
        i64 c = r / (kH * kW), u = (r / kW) % kH, v = r % kW;
        for (i64 b = 0; b < B; ++b) {
            for (i64 i = 0; i < OH; ++i) {
                for (i64 j = 0; j < OW; ++j) {
                    i64 h = i * s - p + u, ww = j * s - p + v;
                    double val = 0.0;
                    if (h >= 0 && h < H && ww >= 0 && ww < W)
                        val = x[((b * C + c) * H + h) * W + ww];
                    col[r * N + (b * OH + i) * OW + j] = val;
                }
            }
        }
    }
    return 0;
}

/*
 * col2im: the adjoint of im2col.  dx[b,c,h,w] is the sum of every col entry
 * whose im2col source is (b,c,h,w), taken in the order u ascending, then v
 * ascending.  Entries that im2col fills with padding zeros contribute
 * nowhere.
 */
int oracle_col2im_spec(const double *col, double *dx, i64 B, i64 C, i64 H,
                       i64 W, i64 kH, i64 kW, i64 s, i64 p)
{
    i64 OH, OW;
    if (bad_shape(B, C, H, W, 1, kH, kW, s, p, &OH, &OW))
        return -1;
    i64 N = B * OH * OW;
    i64 BC = B * C;
#pragma omp parallel for schedule(static)
    for (i64 bc = 0; bc < BC; ++bc) {
        i64 b = bc / C, c = bc % C;
        for (i64 h = 0; h < H; ++h) {
            for (i64 ww = 0; ww < W; ++ww) {
                double acc = 0.0;
                for (i64 u = 0; u < kH; ++u) {
                    i64 ti = h + p - u;
                    if (ti < 0 || ti % s != 0 || ti / s >= OH)
                        continue;
                    for (i64 v = 0; v < kW; ++v) {
                        i64 tj = ww + p - v;
                        if (tj < 0 || tj % s != 0 || tj / s >= OW)
                            continue;
                        i64 r = (c * kH + u) * kW + v;
                        acc += col[r * N + (b * OH + ti / s) * OW + tj / s];
                    }
                }
                dx[(bc * H + h) * W + ww] = acc;
            }
        }
    }
    return 0;
}

/*
 * ---------------------------------------------------------------------------
 * The rest of a training step (directcompute-nn page, "HLSL Shader
 * Reference": "Activation / Loss Shaders", "Pooling Shaders", "Utility
 * Shaders"), as plain double-precision definitions.
 *
 * Readings where the page is silent:
 *   - ReLU gradient passes dy where x > 0 (strictly) and 0 elsewhere.
 *   - Max pooling has no padding, one window size k and one stride s for
 *     both axes, output extent floor((in - k)/s) + 1.  The saved argmax is
 *     the offset h*W + w inside the (b, c) plane of the first maximum met in
 *     the scan order u ascending, then v ascending (strictly greater wins).
 *     Its backward adds each dy element to dx at the saved position, scanning
 *     outputs i ascending, then j ascending (overlapping windows add up).
 *   - Bias add for row-major rows x cols: y[i][j] = x[i][j] + bias[j]; its
 *     gradient sums over the rows.
 *   - Softmax-cross-entropy gradient: softmax(z) - one_hot(label) per row,
 *     as the page states it (no 1/rows factor); the loss is the mean over the
 *     rows of -log softmax(z)[label].  Softmax subtracts the row maximum.
 *   - SGD: param -= lr * clamp(grad, -clip, clip).
 * ---------------------------------------------------------------------------
 */
int oracle_relu(const double *x, double *y, i64 n)
{
    if (n < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i)
        y[i] = x[i] > 0.0 ? x[i] : 0.0;
    return 0;
}

int oracle_relu_grad(const double *x, const double *dy, double *dx, i64 n)
{
    if (n < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i)
        dx[i] = x[i] > 0.0 ? dy[i] : 0.0;
    return 0;
}

static int bad_pool(i64 B, i64 C, i64 H, i64 W, i64 k, i64 s, i64 *OH, i64 *OW)
{
    if (B < 1 || C < 1 || H < 1 || W < 1 || k < 1 || s < 1 || k > H || k > W)
        return 1;
    *OH = (H - k) / s + 1;
    *OW = (W - k) / s + 1;
    return 0;
}

int oracle_maxpool_forward(const double *x, double *y, int32_t *idx, i64 B, i64 C,
                           i64 H, i64 W, i64 k, i64 s)
{
    i64 OH, OW;
    if (bad_pool(B, C, H, W, k, s, &OH, &OW))
        return -1;
    i64 BC = B * C;
#pragma omp parallel for schedule(static)
    for (i64 bc = 0; bc < BC; ++bc) {
        const double *xp = x + bc * H * W;
        for (i64 i = 0; i < OH; ++i)
            for (i64 j = 0; j < OW; ++j) {
                i64 best = (i * s) * W + j * s;
                for (i64 u = 0; u < k; ++u)
                    for (i64 v = 0; v < k; ++v) {
                        i64 at = (i * s + u) * W + (j * s + v);
                        if (xp[at] > xp[best])
                            best = at;
                    }
                y[(bc * OH + i) * OW + j] = xp[best];
                idx[(bc * OH + i) * OW + j] = (int32_t)best;
            }
    }
    return 0;
}

int oracle_maxpool_backward(const double *dy, const int32_t *idx, double *dx, i64 B,
                            i64 C, i64 H, i64 W, i64 k, i64 s)
{
    i64 OH, OW;
    if (bad_pool(B, C, H, W, k, s, &OH, &OW))
        return -1;
    i64 BC = B * C;
#pragma omp parallel for schedule(static)
    for (i64 bc = 0; bc < BC; ++bc) {
        double *dp = dx + bc * H * W;
        for (i64 t = 0; t < H * W; ++t)
            dp[t] = 0.0;
        for (i64 i = 0; i < OH; ++i)
            for (i64 j = 0; j < OW; ++j) {
                i64 o = (bc * OH + i) * OW + j;
                dp[idx[o]] += dy[o];
            }
    }
    return 0;
}

int oracle_add_bias_rows(const double *x, const double *bias, double *y, i64 rows, i64 cols)
{
    if (rows < 1 || cols < 1)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < rows; ++i)
        for (i64 j = 0; j < cols; ++j)
            y[i * cols + j] = x[i * cols + j] + bias[j];
    return 0;
}

int oracle_bias_grad_rows(const double *dy, double *db, i64 rows, i64 cols)
{
    if (rows < 1 || cols < 1)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 j = 0; j < cols; ++j) {
        double acc = 0.0;
        for (i64 i = 0; i < rows; ++i)
            acc += dy[i * cols + j];
        db[j] = acc;
    }
    return 0;
}

int oracle_softmax(const double *z, double *prob, i64 rows, i64 classes)
{
    if (rows < 1 || classes < 1)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < rows; ++i) {
        const double *zr = z + i * classes;
        double m = zr[0];
        for (i64 j = 1; j < classes; ++j)
            if (zr[j] > m)
                m = zr[j];
        double sum = 0.0;
        for (i64 j = 0; j < classes; ++j)
            sum += exp(zr[j] - m);
        for (i64 j = 0; j < classes; ++j)
            prob[i * classes + j] = exp(zr[j] - m) / sum;
    }
    return 0;
}

int oracle_softmax_ce_grad(const double *z, const int32_t *label, double *dz, i64 rows,
                           i64 classes)
{
    if (oracle_softmax(z, dz, rows, classes))
        return -1;
    for (i64 i = 0; i < rows; ++i) {
        if (label[i] < 0 || label[i] >= classes)
            return -1;
        dz[i * classes + label[i]] -= 1.0;
    }
    return 0;
}

/* mean over the rows of -log softmax(z)[label] */
int oracle_ce_loss(const double *z, const int32_t *label, double *loss, i64 rows, i64 classes)
{
    if (rows < 1 || classes < 1)
        return -1;
    double total = 0.0;
    for (i64 i = 0; i < rows; ++i) {
        const double *zr = z + i * classes;
        if (label[i] < 0 || label[i] >= classes)
            return -1;
        double m = zr[0];
        for (i64 j = 1; j < classes; ++j)
            if (zr[j] > m)
                m = zr[j];
        double sum = 0.0;
        for (i64 j = 0; j < classes; ++j)
            sum += exp(zr[j] - m);
        total += log(sum) + m - zr[label[i]];
    }
    *loss = total / (double)rows;
    return 0;
}

int oracle_sgd(double *param, const double *grad, i64 n, double lr, double clip)
{
    if (n < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i) {
        double g = grad[i];
        if (g > clip)
            g = clip;
        if (g < -clip)
            g = -clip;
        param[i] -= lr * g;
    }
    return 0;
}

int oracle_grad_accum(double *acc, const double *grad, i64 n)
{
    if (n < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (i64 i = 0; i < n; ++i)
        acc[i] += grad[i];
    return 0;
}
