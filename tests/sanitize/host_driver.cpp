// Test driver for the library's host code (handle creation, launch planning,
// plan description, workspace sizing and every argument check) under
// AddressSanitizer and UndefinedBehaviorSanitizer, built and run by
// tests/test_sanitizers.py with api.hip compiled for a sanitized host.  No
// call here reaches a kernel launch: every error path returns before one,
// and the valid calls only create, describe, size and destroy handles, so
// the driver runs without a GPU.  Exit status 0 on success.
#include <initializer_list>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "d4r_conv.h"

static int failures = 0;
#define CHECK(cond, ...)                                             \
    do {                                                             \
        if (!(cond)) {                                               \
            fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__);      \
            fprintf(stderr, __VA_ARGS__);                            \
            fputc('\n', stderr);                                     \
            ++failures;                                              \
        }                                                            \
    } while (0)

// fake device addresses, 16 GiB apart so no two operands overlap: the
// checks look at them, nothing dereferences them
static void *fake(int i) { return (void *)(uintptr_t)((unsigned long long)(i + 1) << 34); }
static void *const FAKE = fake(0);
static void *const MISALIGNED = (void *)((char *)fake(0) + 4);
static void *const FAR = fake(9);

struct Shape {
    int b, c, h, w, kh, kw, s, p, o;
};

static void plan_shape(const Shape &sh, d4r_dtype dt)
{
    d4r_conv_t h = nullptr;
    d4r_status st = d4r_conv_create(&h, sh.b, sh.c, sh.h, sh.w, sh.kh, sh.kw, sh.s, sh.p, sh.o, dt);
    CHECK(st == D4R_OK && h, "create %d %d %d %d %d %d %d %d %d: %s", sh.b, sh.c, sh.h, sh.w, sh.kh, sh.kw, sh.s,
          sh.p, sh.o, d4r_last_error());
    if (st != D4R_OK)
        return;
    int oh = 0, ow = 0;
    CHECK(d4r_conv_output_dims(h, &oh, &ow) == D4R_OK && oh == (sh.h + 2 * sh.p - sh.kh) / sh.s + 1 &&
              ow == (sh.w + 2 * sh.p - sh.kw) / sh.s + 1,
          "dims");
    size_t ws = 0, packed = 0;
    CHECK(d4r_conv_workspace_size(h, &ws) == D4R_OK && ws > 0, "workspace");
    CHECK(d4r_conv_packed_filter_size(h, &packed) == D4R_OK && packed > 0, "packed size");
    // describe: query the length, then into an exact buffer, then one short
    size_t need = 0;
    CHECK(d4r_conv_describe(h, nullptr, 0, &need) == D4R_OK && need > 1, "describe length");
    char *text = (char *)malloc(need);
    CHECK(d4r_conv_describe(h, text, need, nullptr) == D4R_OK && strlen(text) + 1 == need, "describe");
    CHECK(strstr(text, "workspace=") != nullptr, "describe keys");
    CHECK(d4r_conv_describe(h, text, need - 1, nullptr) == D4R_ERR_INVALID_ARG, "describe short buffer");
    free(text);
    // argument checks of every conv call: NULL / misaligned operands, short
    // or missing workspace
    void *x = fake(0), *w = fake(1), *dy = fake(2);
    float *y = (float *)fake(3), *dx = (float *)fake(4), *dw = (float *)fake(5);
    CHECK(d4r_conv_forward(h, nullptr, w, nullptr, y, FAR, ws, nullptr) == D4R_ERR_INVALID_ARG, "forward x NULL");
    CHECK(d4r_conv_forward(h, MISALIGNED, w, nullptr, y, FAR, ws, nullptr) == D4R_ERR_INVALID_ARG,
          "forward x misaligned");
    CHECK(d4r_conv_forward(h, x, w, nullptr, y, FAR, ws - 1, nullptr) == D4R_ERR_WORKSPACE,
          "forward short workspace: %s", d4r_last_error());
    CHECK(d4r_conv_forward(h, x, w, nullptr, y, nullptr, ws, nullptr) == D4R_ERR_WORKSPACE, "forward no workspace");
    CHECK(d4r_conv_backward_data(h, w, nullptr, dx, FAR, ws, nullptr) == D4R_ERR_INVALID_ARG,
          "backward_data dy NULL");
    CHECK(d4r_conv_backward_data_implicit(h, w, dy, (float *)((char *)dx + 4), FAR, ws, nullptr) ==
              D4R_ERR_INVALID_ARG,
          "backward_data_implicit dx misaligned");
    CHECK(d4r_conv_backward_filter(h, nullptr, dy, dw, nullptr, 0, FAR, ws, nullptr) == D4R_ERR_INVALID_ARG,
          "backward_filter x NULL without reuse_col");
    CHECK(d4r_conv_backward(h, x, w, dy, dx, dw, nullptr, 0, FAR, ws - 1, nullptr) == D4R_ERR_WORKSPACE,
          "backward short workspace: %s", d4r_last_error());
    CHECK(d4r_conv_im2col(h, nullptr, fake(6), nullptr) == D4R_ERR_INVALID_ARG, "im2col x NULL");
    CHECK(d4r_conv_col2im(h, (const float *)fake(6), nullptr, nullptr) == D4R_ERR_INVALID_ARG, "col2im dx NULL");
    CHECK(d4r_conv_bias_grad(h, dy, nullptr, FAR, ws, nullptr) == D4R_ERR_INVALID_ARG, "bias_grad db NULL");
    CHECK(d4r_conv_pack_filter(h, w, nullptr, nullptr) == D4R_ERR_INVALID_ARG, "pack_filter wp NULL");
    CHECK(d4r_conv_destroy(h) == D4R_OK, "destroy");
}

int main()
{
    // invalid handles
    d4r_conv_t h = nullptr;
    CHECK(d4r_conv_create(nullptr, 1, 1, 4, 4, 3, 3, 1, 0, 1, D4R_F32) == D4R_ERR_INVALID_ARG, "out NULL");
    const int bad[][9] = {{0, 1, 4, 4, 3, 3, 1, 0, 1}, {1, 0, 4, 4, 3, 3, 1, 0, 1}, {1, 1, 0, 4, 3, 3, 1, 0, 1},
                          {1, 1, 4, 4, 0, 3, 1, 0, 1}, {1, 1, 4, 4, 3, 3, 0, 0, 1}, {1, 1, 4, 4, 3, 3, 1, -1, 1},
                          {1, 1, 4, 4, 3, 3, 1, 0, 0}, {1, 1, 2, 2, 5, 5, 1, 1, 1}};
    for (const auto &a : bad) {
        h = (d4r_conv_t)FAKE;
        CHECK(d4r_conv_create(&h, a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], D4R_F32) ==
                      D4R_ERR_INVALID_ARG &&
                  h == nullptr,
              "bad shape");
        CHECK(strlen(d4r_last_error()) > 0, "error text");
    }
    CHECK(d4r_conv_create(&h, 1, 1, 4, 4, 3, 3, 1, 0, 1, (d4r_dtype)9) == D4R_ERR_INVALID_ARG, "dtype");
    CHECK(d4r_conv_create(&h, 4096, 1024, 224, 224, 3, 3, 1, 1, 64, D4R_F32) == D4R_ERR_UNSUPPORTED,
          "2^31 elements");
    CHECK(d4r_conv_destroy(nullptr) == D4R_OK, "destroy NULL");
    CHECK(d4r_conv_describe(nullptr, nullptr, 0, nullptr) == D4R_ERR_INVALID_ARG, "describe NULL");

    // every workload layer in every dtype, and shapes that take the other
    // planning branches: stride 2 to 4, padding past the kernel, 1x1,
    // non-square kernels, ragged channel counts, batch 1
    const Shape shapes[] = {
        {8, 1, 28, 28, 5, 5, 1, 0, 6},    {64, 6, 12, 12, 5, 5, 1, 0, 16},   {32, 3, 224, 224, 11, 11, 4, 2, 96},
        {64, 256, 13, 13, 3, 3, 1, 1, 384}, {64, 384, 13, 13, 3, 3, 1, 1, 384}, {64, 384, 13, 13, 3, 3, 1, 1, 256},
        {4, 256, 46, 80, 3, 3, 1, 1, 256}, {4, 256, 46, 80, 1, 1, 1, 0, 128}, {4, 256, 46, 80, 3, 3, 2, 1, 128},
        {2, 64, 9, 11, 3, 3, 2, 1, 64},    {1, 64, 12, 12, 11, 11, 4, 2, 64}, {2, 130, 7, 8, 3, 2, 2, 0, 64},
        {2, 32, 6, 6, 2, 2, 1, 3, 64},     {1, 2, 6, 6, 2, 2, 1, 3, 3},       {3, 5, 7, 7, 1, 1, 1, 0, 6},
        {1, 3, 23, 21, 5, 5, 2, 1, 32},    {2, 3, 8, 7, 3, 3, 1, 2, 4},       {1, 1, 1, 1, 1, 1, 1, 0, 1},
    };
    const d4r_dtype dts[] = {D4R_F32, D4R_F16, D4R_BF16};
    for (const Shape &sh : shapes)
        for (d4r_dtype dt : dts)
            plan_shape(sh, dt);

    // GEMM sizing and argument checks
    for (int flags = 0; flags < 4; ++flags)
        for (d4r_dtype dt : dts)
            for (int m : {1, 7, 64, 129, 4096})
                for (int k : {1, 17, 363, 4096})
                    for (int n : {1, 65, 4096}) {
                        size_t bytes = 1;
                        CHECK(d4r_gemm_workspace_size(m, k, n, flags, dt, &bytes) == D4R_OK, "gemm ws");
                    }
    size_t bytes = 0;
    CHECK(d4r_gemm_workspace_size(0, 1, 1, 0, D4R_F32, &bytes) == D4R_ERR_INVALID_ARG, "gemm M 0");
    CHECK(d4r_gemm_workspace_size(1, 1, 1, 4, D4R_F32, &bytes) == D4R_ERR_INVALID_ARG, "gemm flags 4");
    CHECK(d4r_gemm(4, 4, 4, 0, D4R_F32, nullptr, fake(1), (float *)fake(2), nullptr, 0, nullptr) ==
              D4R_ERR_INVALID_ARG,
          "gemm A NULL");
    CHECK(d4r_gemm(4, 4, 4, 0, D4R_F32, fake(0), MISALIGNED, (float *)fake(2), nullptr, 0, nullptr) ==
              D4R_ERR_INVALID_ARG,
          "gemm B misaligned");
    CHECK(d4r_gemm_noalloc(4, 4, 4, 7, D4R_F32, fake(0), fake(1), (float *)FAR, nullptr) == D4R_ERR_INVALID_ARG,
          "noalloc flags");
    CHECK(d4r_stream_copy(FAKE, FAR, 100, nullptr) == D4R_ERR_INVALID_ARG, "stream copy size");
    CHECK(d4r_mfma_ceiling((d4r_dtype)5, FAKE, (float *)FAR, 1, 1, nullptr) == D4R_ERR_INVALID_ARG, "ceiling dtype");
    for (int bad : {-1, 3, 5, 2147483647, -2147483647 - 1}) {
        size_t ws = 0;
        CHECK(d4r_conv_create(&h, 1, 1, 4, 4, 3, 3, 1, 0, 1, (d4r_dtype)bad) == D4R_ERR_INVALID_ARG,
              "create dtype %d", bad);
        CHECK(d4r_gemm_workspace_size(8, 8, 8, 0, (d4r_dtype)bad, &ws) == D4R_ERR_INVALID_ARG,
              "gemm workspace dtype %d", bad);
        CHECK(d4r_gemm(8, 8, 8, 0, (d4r_dtype)bad, FAKE, fake(1), (float *)fake(2), nullptr, 0, nullptr) ==
                  D4R_ERR_INVALID_ARG,
              "gemm dtype %d", bad);
        CHECK(d4r_mfma_ceiling((d4r_dtype)bad, FAKE, (float *)FAR, 1, 1, nullptr) == D4R_ERR_INVALID_ARG,
              "ceiling dtype %d", bad);
    }
    CHECK(d4r_relu_forward(nullptr, (float *)FAKE, 16, nullptr) == D4R_ERR_INVALID_ARG, "relu x NULL");
    CHECK(d4r_softmax((const float *)FAKE, (float *)FAR, 0, 10, nullptr) == D4R_ERR_INVALID_ARG, "softmax rows 0");

    // status strings, the unknown code included
    for (int s = 0; s <= 6; ++s)
        CHECK(d4r_status_string((d4r_status)s) != nullptr, "status string %d", s);
    if (failures) {
        fprintf(stderr, "%d checks failed\n", failures);
        return 1;
    }
    printf("host driver: all checks passed\n");
    return 0;
}
