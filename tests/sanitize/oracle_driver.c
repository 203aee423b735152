/*
 * Test driver for the CPU oracle under AddressSanitizer and
 * UndefinedBehaviorSanitizer (built and run by tests/test_sanitizers.py).
 * Every oracle routine runs on small shapes -- ragged, strided, padded,
 * kernels larger than the input -- with each buffer allocated at exactly
 * the size the routine may touch, so any read or write past it is
 * reported; invalid sizes must return -1; two identities that tie the
 * routines together (the im2col / col2im adjoint and the 1x1 convolution as
 * a GEMM) are checked on the way.  Exit status 0 on success.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

typedef long long i64;

int oracle_out_dims(i64 H, i64 W, i64 kH, i64 kW, i64 s, i64 p, i64 *OH, i64 *OW);
int oracle_conv_forward(const double *x, const double *w, const double *bias, double *y, i64 B, i64 C, i64 H,
                        i64 W, i64 O, i64 kH, i64 kW, i64 s, i64 p);
int oracle_conv_backward_filter(const double *x, const double *g, double *dw, i64 B, i64 C, i64 H, i64 W, i64 O,
                                i64 kH, i64 kW, i64 s, i64 p);
int oracle_conv_backward_bias(const double *g, double *db, i64 B, i64 O, i64 P);
int oracle_conv_backward_data(const double *g, const double *w, double *dx, i64 B, i64 C, i64 H, i64 W, i64 O,
                              i64 kH, i64 kW, i64 s, i64 p);
int oracle_gemm(const double *A, const double *Bm, double *Cm, i64 M, i64 K, i64 N, int flags);
int oracle_im2col_spec(const double *x, double *col, i64 B, i64 C, i64 H, i64 W, i64 kH, i64 kW, i64 s, i64 p);
int oracle_col2im_spec(const double *col, double *dx, i64 B, i64 C, i64 H, i64 W, i64 kH, i64 kW, i64 s, i64 p);
int oracle_relu(const double *x, double *y, i64 n);
int oracle_relu_grad(const double *x, const double *dy, double *dx, i64 n);
int oracle_maxpool_forward(const double *x, double *y, int32_t *idx, i64 B, i64 C, i64 H, i64 W, i64 k, i64 s);
int oracle_maxpool_backward(const double *dy, const int32_t *idx, double *dx, i64 B, i64 C, i64 H, i64 W, i64 k,
                            i64 s);
int oracle_add_bias_rows(const double *x, const double *bias, double *y, i64 rows, i64 cols);
int oracle_bias_grad_rows(const double *dy, double *db, i64 rows, i64 cols);
int oracle_softmax(const double *z, double *prob, i64 rows, i64 classes);
int oracle_softmax_ce_grad(const double *z, const int32_t *label, double *dz, i64 rows, i64 classes);
int oracle_ce_loss(const double *z, const int32_t *label, double *loss, i64 rows, i64 classes);
int oracle_sgd(double *param, const double *grad, i64 n, double lr, double clip);
int oracle_grad_accum(double *acc, const double *grad, i64 n);

static int failures = 0;
#define CHECK(cond, ...)                                  \
    do {                                                  \
        if (!(cond)) {                                    \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
            fprintf(stderr, __VA_ARGS__);                 \
            fputc('\n', stderr);                          \
            ++failures;                                   \
        }                                                 \
    } while (0)

static unsigned long long rng = 88172645463325252ULL;
static double rnd(void)
{
    rng ^= rng << 13;
    rng ^= rng >> 7;
    rng ^= rng << 17;
    return (double)(rng >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double *buf(i64 n)
{
    double *p = (double *)malloc((size_t)(n > 0 ? n : 1) * sizeof(double));
    for (i64 i = 0; i < n; ++i)
        p[i] = rnd();
    return p;
}

static void conv_case(i64 B, i64 C, i64 H, i64 W, i64 O, i64 kH, i64 kW, i64 s, i64 p)
{
    i64 OH, OW;
    CHECK(oracle_out_dims(H, W, kH, kW, s, p, &OH, &OW) == 0, "dims");
    const i64 P = OH * OW, Kc = C * kH * kW, N = B * P;
    double *x = buf(B * C * H * W), *w = buf(O * Kc), *bias = buf(O), *y = buf(B * O * P);
    double *g = buf(B * O * P), *dw = buf(O * Kc), *db = buf(O), *dx = buf(B * C * H * W);
    double *col = buf(Kc * N), *dx2 = buf(B * C * H * W);
    CHECK(oracle_conv_forward(x, w, bias, y, B, C, H, W, O, kH, kW, s, p) == 0, "forward");
    CHECK(oracle_conv_forward(x, w, NULL, y, B, C, H, W, O, kH, kW, s, p) == 0, "forward, no bias");
    CHECK(oracle_conv_backward_filter(x, g, dw, B, C, H, W, O, kH, kW, s, p) == 0, "filter gradient");
    CHECK(oracle_conv_backward_bias(g, db, B, O, P) == 0, "bias gradient");
    CHECK(oracle_conv_backward_data(g, w, dx, B, C, H, W, O, kH, kW, s, p) == 0, "data gradient");
    CHECK(oracle_im2col_spec(x, col, B, C, H, W, kH, kW, s, p) == 0, "im2col");
    /* adjoint: <im2col(x), c> = <x, col2im(c)> */
    double *c = buf(Kc * N);
    CHECK(oracle_col2im_spec(c, dx2, B, C, H, W, kH, kW, s, p) == 0, "col2im");
    double lhs = 0.0, rhs = 0.0, mag = 0.0;
    for (i64 i = 0; i < Kc * N; ++i) {
        lhs += col[i] * c[i];
        mag += fabs(col[i] * c[i]);
    }
    for (i64 i = 0; i < B * C * H * W; ++i)
        rhs += x[i] * dx2[i];
    CHECK(fabs(lhs - rhs) <= 1e-12 * (mag + 1.0), "adjoint %g vs %g", lhs, rhs);
    /* invalid sizes leave outputs alone and return -1 */
    CHECK(oracle_conv_forward(x, w, bias, y, B, C, H, W, O, kH, kW, 0, p) == -1, "stride 0");
    CHECK(oracle_conv_forward(x, w, bias, y, B, C, H, W, O, kH, kW, s, -1) == -1, "padding -1");
    CHECK(oracle_im2col_spec(x, col, B, C, H, W, H + 2 * p + 1, kW, s, p) == -1, "kernel too large");
    free(x); free(w); free(bias); free(y); free(g); free(dw); free(db); free(dx); free(col); free(dx2); free(c);
}

int main(void)
{
    /* (B, C, H, W, O, kH, kW, s, p): ragged, strided, padded, kernel wider
       than the unpadded input, 1x1, AlexNet conv1's 11x11 stride 4 at a
       small size */
    conv_case(2, 3, 7, 9, 4, 3, 3, 1, 1);
    conv_case(1, 2, 8, 5, 3, 3, 2, 2, 0);
    conv_case(2, 1, 4, 4, 2, 5, 5, 1, 2);
    conv_case(3, 4, 6, 6, 5, 1, 1, 1, 0);
    conv_case(1, 3, 23, 19, 2, 11, 11, 4, 2);
    conv_case(1, 2, 5, 7, 2, 2, 3, 3, 3);

    /* 1x1 stride-1 convolution of one image == W (O x C) * x (C x H*W) */
    {
        const i64 C = 5, H = 3, W = 4, O = 6, P = H * W;
        double *x = buf(C * P), *w = buf(O * C), *y = buf(O * P), *ref = buf(O * P);
        CHECK(oracle_conv_forward(x, w, NULL, y, 1, C, H, W, O, 1, 1, 1, 0) == 0, "1x1");
        CHECK(oracle_gemm(w, x, ref, O, C, P, 0) == 0, "gemm");
        for (i64 i = 0; i < O * P; ++i)
            CHECK(fabs(y[i] - ref[i]) <= 1e-12, "1x1 vs gemm at %lld", i);
        free(x); free(w); free(y); free(ref);
    }
    /* GEMM with every flag on odd sizes */
    for (int flags = 0; flags < 4; ++flags) {
        const i64 M = 7, K = 5, N = 3;
        double *A = buf(M * K), *Bm = buf(K * N), *Cm = buf(M * N);
        CHECK(oracle_gemm(A, Bm, Cm, M, K, N, flags) == 0, "gemm flags %d", flags);
        CHECK(oracle_gemm(A, Bm, Cm, M, K, N, 4) == -1, "gemm flags 4");
        free(A); free(Bm); free(Cm);
    }
    /* the rest of a training step */
    {
        const i64 B = 2, C = 3, H = 7, W = 6, k = 2, s = 2, OH = (H - k) / s + 1, OW = (W - k) / s + 1;
        double *x = buf(B * C * H * W), *y = buf(B * C * OH * OW), *dy = buf(B * C * OH * OW);
        double *dx = buf(B * C * H * W);
        int32_t *idx = (int32_t *)malloc((size_t)(B * C * OH * OW) * sizeof(int32_t));
        CHECK(oracle_maxpool_forward(x, y, idx, B, C, H, W, k, s) == 0, "maxpool");
        CHECK(oracle_maxpool_backward(dy, idx, dx, B, C, H, W, k, s) == 0, "maxpool backward");
        CHECK(oracle_maxpool_forward(x, y, idx, B, C, H, W, H + 1, s) == -1, "pool window too large");
        free(x); free(y); free(dy); free(dx); free(idx);
    }
    {
        const i64 rows = 5, cols = 7, n = rows * cols;
        double *x = buf(n), *y = buf(n), *dy = buf(n), *dx = buf(n), *bias = buf(cols), *db = buf(cols);
        double *prob = buf(n), *dz = buf(n), *loss = buf(1), *acc = buf(n);
        int32_t *label = (int32_t *)malloc((size_t)rows * sizeof(int32_t));
        for (i64 i = 0; i < rows; ++i)
            label[i] = (int32_t)(i % cols);
        CHECK(oracle_relu(x, y, n) == 0, "relu");
        CHECK(oracle_relu_grad(x, dy, dx, n) == 0, "relu gradient");
        CHECK(oracle_add_bias_rows(x, bias, y, rows, cols) == 0, "row bias");
        CHECK(oracle_bias_grad_rows(dy, db, rows, cols) == 0, "row bias gradient");
        CHECK(oracle_softmax(x, prob, rows, cols) == 0, "softmax");
        CHECK(oracle_softmax_ce_grad(x, label, dz, rows, cols) == 0, "softmax-CE gradient");
        CHECK(oracle_ce_loss(x, label, loss, rows, cols) == 0 && *loss > 0.0, "CE loss");
        label[2] = (int32_t)cols;
        CHECK(oracle_ce_loss(x, label, loss, rows, cols) == -1, "label out of range");
        CHECK(oracle_sgd(x, dy, n, 0.1, 0.5) == 0, "sgd");
        CHECK(oracle_grad_accum(acc, dy, n) == 0, "accumulation");
        free(x); free(y); free(dy); free(dx); free(bias); free(db); free(prob); free(dz); free(loss);
        free(acc); free(label);
    }
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("oracle driver: all checks passed\n");
    return 0;
}
