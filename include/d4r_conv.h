/*
 * d4r_conv.h -- C ABI of libd4r_conv.so: convolution lowered to matrix
 * multiplication on AMD Instinct MI355X (gfx950).
 *
 * The method (directcompute-nn 0.1.0 page, "Convolution: The im2col
 * Approach"):
 *   forward   x --im2col--> col (C*kH*kW x B*OH*OW)
 *             Cmat = Wmat (O x C*kH*kW) * col
 *             y = conv_reshape(Cmat) + bias       -> (B, O, OH, OW)
 *   backward  G = conv_grad_reshape(dy)           (O x B*OH*OW)
 *             dW = G * col^T                      (matmul flags = 2)
 *             dcol = Wmat^T * G                   (matmul flags = 1)
 *             dx = col2im(dcol)
 *             db[o] = sum of row o of G
 * Transposes are expressed by the matmul flags ("Transpose via Flags"):
 * flags & 1 reads A as stored transposed, flags & 2 reads B as stored
 * transposed.  (For the data gradient this library reshapes dy straight
 * into G^T and keeps a transposed copy of the small filter matrix, so both
 * MFMA operands stream with k contiguous; the product is the same.)
 *
 * Conventions shared by every call
 * --------------------------------
 * Geometry.  Square stride and symmetric zero padding (one value each, as
 * the page's im2col parameter list has); kH and kW may differ.  Output
 * extent OH = floor((inH + 2*padding - kH) / stride) + 1, likewise OW.  No
 * dilation, no groups.
 *
 * Layouts (all packed, row-major, no leading dimensions):
 *   x, dx       (batch, inC, inH, inW)        NCHW
 *   w, dw       (outC, inC, kH, kW)           OIHW, i.e. Wmat O x Kc
 *   y, dy       (batch, outC, OH, OW)         NCHW
 *   bias, db    (outC)
 *   col         Kc x N row-major, Kc = inC*kH*kW rows ordered (c, u, v) with
 *               v fastest, N = batch*OH*OW columns ordered (b, i, j) with j
 *               fastest; col[(c*kH+u)*kW+v][(b*OH+i)*OW+j] =
 *               x[b][c][i*stride-padding+u][j*stride-padding+v], or 0 when
 *               that position falls in the padding.
 *
 * Types.  x, w, dy and GEMM operands A, B are in the handle's / call's
 * d4r_dtype (float32, IEEE binary16 or bfloat16).  bias, y, dx, dw, db and
 * GEMM C are always float32.  Half-precision products accumulate in float32.
 *
 * Memory ownership.  Every pointer argument is a caller-owned device
 * pointer (e.g. a torch tensor's data_ptr()).  The library never allocates,
 * frees or keeps device memory of the caller's; its only device memory is
 * the static 64 MiB split-K array of d4r_gemm_noalloc, which each GPU holds
 * from when the library's code is loaded on it until the process ends.
 * Pointers to tensors must be 16-byte aligned, bias and db 4-byte aligned,
 * ws 256-byte aligned.
 *
 * Workspace.  Scratch memory (the col matrix, the reshaped gradient, the
 * float32 dcol, split-K partial sums) lives in a caller buffer ws of at least
 * d4r_conv_workspace_size() bytes.  d4r_conv_forward leaves the col matrix
 * of x at the start of ws; d4r_conv_backward_data does not touch that
 * region, so a following d4r_conv_backward_filter (or d4r_conv_backward)
 * with reuse_col = 1 and the same ws reuses it (the page saves the im2col
 * buffer in forward for the filter gradient, "Memory Management").
 *
 * Streams.  hip_stream is a hipStream_t (NULL = the null stream).  Calls
 * only enqueue kernels on it: no host synchronisation, no allocation.
 * Results are deterministic: no atomics, fixed summation orders.  Calls
 * that may run at the same time on different streams must not share a
 * workspace: e.g. a layer's data gradient may overlap its filter gradient
 * (both only read w and dy) when given a workspace of its own.
 *
 * Errors.  Every call returns a d4r_status.  All argument validation runs
 * before any HIP call, so an invalid call enqueues nothing.  A kernel launch
 * error is returned as D4R_ERR_LAUNCH; faults inside kernels surface at the
 * caller's next synchronisation.  d4r_last_error() gives a thread-local
 * message for the last failing call on the calling thread.
 *
 * Sizes.  Every tensor, col and dcol must hold fewer than 2^31 elements.
 */
#ifndef D4R_CONV_H
#define D4R_CONV_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    D4R_F32 = 0,  /* IEEE binary32 */
    D4R_F16 = 1,  /* IEEE binary16, float32 accumulation */
    D4R_BF16 = 2, /* bfloat16, float32 accumulation */
    /* Not a dtype.  It widens the type's range of values to every int, so
     * that an unknown value passed in is a defined value the argument
     * checks report (D4R_ERR_INVALID_ARG) rather than undefined behaviour
     * in the library's C++. */
    D4R_DTYPE_INT_RANGE = -2147483647 - 1
} d4r_dtype;

typedef enum {
    D4R_OK = 0,
    D4R_ERR_INVALID_ARG = 1, /* bad size, NULL/misaligned pointer, bad flag or dtype */
    D4R_ERR_UNSUPPORTED = 2, /* valid request this build cannot run (e.g. > 2^31 elements) */
    D4R_ERR_WORKSPACE = 3,   /* ws NULL or smaller than the size query returned */
    D4R_ERR_LAUNCH = 4,      /* a HIP launch failed */
    D4R_ERR_INTERNAL = 5
} d4r_status;

typedef struct d4r_conv *d4r_conv_t;

/*
 * Create a host-side handle for one convolution shape.  Argument order is
 * the problem statement's (batch, inC, inH, inW, kH, kW, stride, padding,
 * outC); the page's im2col parameter block ("Constant Buffer Convention")
 * carries the same fields.  Validates the geometry, computes OH/OW and
 * chooses the GEMM tilings and split-K factors of the three passes.  The
 * handle is immutable and may be shared between threads; free it with
 * d4r_conv_destroy.  Errors: D4R_ERR_INVALID_ARG (out NULL, a size < 1,
 * stride < 1, padding < 0, OH or OW < 1, unknown dtype),
 * D4R_ERR_UNSUPPORTED (a tensor reaches 2^31 elements).
 */
d4r_status d4r_conv_create(d4r_conv_t *out, int batch, int inC, int inH, int inW,
                           int kH, int kW, int stride, int padding, int outC,
                           d4r_dtype dtype);

/* Free a handle.  NULL is accepted and ignored. */
d4r_status d4r_conv_destroy(d4r_conv_t h);

/* Output extent of the handle's convolution. */
d4r_status d4r_conv_output_dims(d4r_conv_t h, int *outH, int *outW);

/*
 * Bytes of workspace every pass of this handle needs (the maximum over
 * forward, backward_data and backward_filter); at least the size of col.
 */
d4r_status d4r_conv_workspace_size(d4r_conv_t h, size_t *bytes);

/*
 * The launch plan of a handle, as text: space-separated key=value pairs
 * naming the kernel each step runs and its shape (im2col / col2im kernel
 * and images per block, GEMM tile and split-K count of every pass, how the
 * gradient GEMMs take dy, the workspace size).  Host only, no HIP call;
 * the plan reflects the D4R_* experiment switches set at the time of the
 * call, as a launch made then would.  *needed (if not NULL) receives the
 * length including the terminating NUL; buf may be NULL to query it.
 * Errors: D4R_ERR_INVALID_ARG for a NULL handle or when buf is not NULL and
 * cap is below *needed (nothing is written then).  (Not a step of the
 * pages' method: it lets tests confirm which kernel configuration ran.)
 */
d4r_status d4r_conv_describe(d4r_conv_t h, char *buf, size_t cap, size_t *needed);

/*
 * 1x1 convolutions.  When kH = kW = 1, stride = 1 and padding = 0, col is x
 * itself with the batch folded into its columns, so three calls read x and
 * dy in place instead of going through col (the mlvc.cpp design page runs
 * dense pointwise convolution as a direct matrix-core GEMM, "Driver-only
 * AOT cubin direction"):
 *   d4r_conv_forward_implicit          y[b] = Wmat * x[b] + bias
 *   d4r_conv_backward_data(_implicit)  dx[b] = Wmat^T * dy[b], stored NCHW
 *                                      by the GEMM (no dcol, no col2im)
 *   d4r_conv_backward_filter, reuse_col = 0
 *                                      dw = sum_b dy[b] * x[b]^T (no im2col;
 *                                      the col region of ws is untouched)
 * d4r_conv_forward still writes col (for reuse_col = 1).  Results equal the
 * general path up to summation order.
 */

/*
 * Forward (page: im2col -> matmul flags 0 -> conv_reshape with bias):
 * y = conv(x; w) + bias.  x, w in the handle's dtype; bias float32 or NULL
 * (no bias); y float32.  Leaves col at the start of ws.
 */
d4r_status d4r_conv_forward(d4r_conv_t h, const void *x, const void *w,
                            const float *bias, float *y, void *ws,
                            size_t ws_bytes, void *hip_stream);

/*
 * Forward as an implicit GEMM (same result as d4r_conv_forward up to
 * summation order; the mlvc.cpp design page runs dense spatial convolution
 * as an implicit GEMM, "Driver-only AOT cubin direction").  The GEMM gathers
 * each col tile from x into on-chip memory, so the col matrix is never
 * written: ws is used only for split-K partial sums and does NOT hold col
 * afterwards (a following d4r_conv_backward_filter must pass reuse_col = 0).
 */
d4r_status d4r_conv_forward_implicit(d4r_conv_t h, const void *x, const void *w,
                                     const float *bias, float *y, void *ws,
                                     size_t ws_bytes, void *hip_stream);

/*
 * Forward with the layer's activation fused (the directcompute-nn page
 * trains LeNet-5 and AlexNet, "File Structure", whose hidden convolutions
 * are followed by ReLU, the page's relu shader, "Activation / Loss
 * Shaders"):
 * y = relu(conv(x; w) + bias) when flags has D4R_FWD_RELU, where relu(v) =
 * v if v > 0 else 0 (NaN gives 0, as d4r_relu_forward).  The GEMM's
 * epilogue (or the split-K reduction) applies it before the only store of
 * y, so y equals d4r_conv_forward followed by d4r_relu_forward bit for bit
 * without a second pass over y.  D4R_FWD_IMPLICIT selects the implicit
 * GEMM of d4r_conv_forward_implicit (ws then does not hold col); without it
 * col is left at the start of ws as by d4r_conv_forward.  flags = 0 is
 * d4r_conv_forward.  The ReLU backward needs the stored y (dx = dy where
 * y > 0), so y is what d4r_relu_backward takes as x.
 * Errors: those of d4r_conv_forward, and D4R_ERR_INVALID_ARG for other
 * flag bits.
 */
#define D4R_FWD_RELU 1
#define D4R_FWD_IMPLICIT 2
d4r_status d4r_conv_forward_ex(d4r_conv_t h, const void *x, const void *w,
                               const float *bias, float *y, int flags, void *ws,
                               size_t ws_bytes, void *hip_stream);

/*
 * Data gradient (page: Input gradients = filters^T x grad_reshaped, then
 * col2im): dx = col2im(Wmat^T * G).  w, dy in the handle's dtype; dx
 * float32, fully overwritten.  dcol is float32 in ws, after the col region.
 */
d4r_status d4r_conv_backward_data(d4r_conv_t h, const void *w, const void *dy,
                                  float *dx, void *ws, size_t ws_bytes,
                                  void *hip_stream);

/*
 * Data gradient without the dcol matrix.  The directcompute-nn page lists a
 * fused direct input-gradient kernel among the shaders the im2col path
 * replaced ("HLSL Shader Reference", "Legacy / Unused Shaders"); the
 * mlvc.cpp design page runs dense spatial convolution as an implicit GEMM
 * ("Driver-only AOT cubin direction").  For stride 1 and a square kernel,
 * dx is the stride-1 convolution of dy (padding kH-1-p) with the filter
 * Wf[c][o][u][v] = w[o][c][kH-1-u][kW-1-v]; it runs as an implicit GEMM on
 * that geometry: no dcol, no col2im.  When outC is a multiple of 32 (f32)
 * or 64 (f16, bf16), dy is first transposed to NHWC and the filter flipped
 * with k ordered by blocks of 32 / 64 output channels, then tap (u, v),
 * then channel, so that every GEMM stage reads contiguous channel runs of
 * dy (16-byte loads straight into LDS) and the taps of one block reread
 * the same channels while they are cached;
 * otherwise the GEMM gathers im2col(dy) element by element.  For stride
 * s >= 2 (s <= kH, kW, inH, inW; s*s <= 16; outC a multiple of 32 f32 / 64
 * 16-bit; inC >= 64) dx splits into s*s output phases, the rows and columns
 * with (h + p) mod s and (w + p) mod s fixed; each phase is a stride-1
 * convolution of dy (read as NHWC) with a sub-filter of ceil(kH/s) x
 * ceil(kW/s) taps of w, and all phases run in one GEMM launch.  With fewer
 * input channels (AlexNet conv1's 3) the explicit path runs instead: its
 * GEMM rows are inC*kH*kW, where the phases' would be inC (the environment
 * switch D4R_DGRAD_PHASED=force takes the phased form there too; =0 never).
 * 1x1 stride-1 unpadded convolutions take their direct path, other shapes
 * the explicit path of d4r_conv_backward_data.  Same arguments, result
 * equal up to summation order; ws holds dy^T, the flipped (or phase)
 * filters and split-K partials, and the col region is left untouched
 * (reuse_col stays valid).
 */
d4r_status d4r_conv_backward_data_implicit(d4r_conv_t h, const void *w,
                                           const void *dy, float *dx, void *ws,
                                           size_t ws_bytes, void *hip_stream);

/*
 * Pre-packed filter for the data gradient.  The data-gradient GEMM reads
 * Wmat^T; d4r_conv_pack_filter writes it once as wp[kc][o] = w[o][kc] (Kc x
 * O, row-major, the handle's dtype, d4r_conv_packed_filter_size() bytes), and
 * d4r_conv_backward_data_packed then reads wp k-contiguous instead of
 * transposing or striding through w on every call -- for callers that run
 * several data gradients per weight update (gradient accumulation over
 * micro-batches).  Same result as d4r_conv_backward_data up to summation
 * order.  (The d4r engine page packs its weights once as [K/16][N/16]
 * [N16][K16] tiles so that its matrix-core loads become plain row loads,
 * "The network on the native HIP layers".  Here the forward already reads
 * w's rows as contiguous 16-byte runs, so only the transposed copy for the
 * data gradient is worth keeping.)  wp must not overlap w; it stays valid
 * while w is unchanged.
 */
d4r_status d4r_conv_packed_filter_size(d4r_conv_t h, size_t *bytes);
d4r_status d4r_conv_pack_filter(d4r_conv_t h, const void *w, void *wp, void *hip_stream);
d4r_status d4r_conv_backward_data_packed(d4r_conv_t h, const void *wp, const void *dy,
                                         float *dx, void *ws, size_t ws_bytes,
                                         void *hip_stream);

/*
 * Filter and bias gradients (page: Filter gradients = grad_reshaped x
 * im2col_matrix^T, reusing the saved im2col; Bias gradients = per-channel
 * sum of grad_reshaped): dw = G * col^T (float32, OIHW), db[o] = sum over
 * batch and both spatial axes of dy[:, o] (float32; db NULL skips it).
 * reuse_col = 0: x must be given and col is rebuilt in ws.  reuse_col = 1:
 * x must be NULL and ws must still hold the col of the same x written by
 * d4r_conv_forward (or d4r_conv_im2col) with this handle.
 */
d4r_status d4r_conv_backward_filter(d4r_conv_t h, const void *x, const void *dy,
                                    float *dw, float *db, int reuse_col,
                                    void *ws, size_t ws_bytes, void *hip_stream);

/*
 * The whole backward pass of one layer in one call (the page's backward,
 * "Convolution: The im2col Approach": data, filter and bias gradients from
 * one upstream gradient dy): dx as d4r_conv_backward_data_implicit, dw and
 * db as d4r_conv_backward_filter with the same x / reuse_col rules, all
 * arguments as in those two calls (db NULL skips the bias).  When the
 * implicit data gradient reads dy as NHWC and the filter gradient copies dy
 * (16-bit, or float32 with C*kH*kW >= 1024), one pass over dy writes both
 * gradients' operands and the bias partial sums (the reshape the page runs
 * as conv_grad_reshape, and the NHWC transpose) and the filter flip rides
 * in the same launch; dx and dw then equal the two separate calls bit for
 * bit, db agrees up to summation order.  Otherwise it is those two calls in
 * sequence.  col in ws is left intact with reuse_col = 1 and rebuilt from x
 * with reuse_col = 0.
 */
d4r_status d4r_conv_backward(d4r_conv_t h, const void *x, const void *w, const void *dy,
                             float *dx, float *dw, float *db, int reuse_col, void *ws,
                             size_t ws_bytes, void *hip_stream);

/*
 * Single steps of the path, for measurement and for checking the index
 * maps bit for bit.
 *
 * d4r_conv_im2col: col (Kc x N, handle dtype) = im2col(x), the layout given
 * above; a raw bit copy (no arithmetic).  col needs Kc*N elements.
 *
 * d4r_conv_col2im: dx (float32 NCHW) = col2im(dcol) for a float32 Kc x N
 * dcol: a gather (no atomics); each dx element sums its in-image dcol
 * entries in the order u ascending, then v ascending.
 *
 * d4r_conv_bias_grad: db[o] = sum_{b,i,j} dy[b][o][i][j] (float32).  Needs
 * d4r_conv_workspace_size() bytes of ws for per-block partial sums.
 */
d4r_status d4r_conv_im2col(d4r_conv_t h, const void *x, void *col, void *hip_stream);
d4r_status d4r_conv_col2im(d4r_conv_t h, const float *dcol, float *dx, void *hip_stream);
d4r_status d4r_conv_bias_grad(d4r_conv_t h, const void *dy, float *db, void *ws,
                              size_t ws_bytes, void *hip_stream);

/*
 * Workspace bytes d4r_gemm needs for these arguments (0 when it runs
 * without split-K).  Same validation as d4r_gemm.
 */
d4r_status d4r_gemm_workspace_size(int M, int K, int N, int flags, d4r_dtype dtype,
                                   size_t *bytes);

/*
 * C = op(A) * op(B), C float32 M x N row-major, overwritten (no alpha/beta).
 * The parameter block {M, K, N, flags} and the operand index formulas are
 * the page's ("Matmul Shaders", "Transpose via Flags"):
 *   op(A)[m][k] = A[m*K + k], or A[k*M + m] when flags & 1;
 *   op(B)[k][n] = B[k*N + n], or B[n*K + k] when flags & 2.
 * flags 0 = NN, 1 = TN, 2 = NT, 3 = TT.  A, B in dtype.
 * Errors: D4R_ERR_INVALID_ARG for M, K or N < 1, flags outside 0..3, NULL or
 * misaligned pointers; D4R_ERR_WORKSPACE when ws is short.
 */
d4r_status d4r_gemm(int M, int K, int N, int flags, d4r_dtype dtype, const void *A,
                    const void *B, float *C, void *ws, size_t ws_bytes,
                    void *hip_stream);

/*
 * d4r_gemm for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same product,
 * plan and kernels as d4r_gemm, so C equals d4r_gemm's bit for bit, but
 * the split-K partial sums go to a device array the library owns
 * (d4r_gemm_noalloc_scratch_bytes() = 64 MiB per GPU, held from when the
 * library is loaded on that GPU until the process ends) instead of a
 * workspace argument.  No hipMalloc, hipFree or allocating library call is
 * made; the array's address on the current device is looked up on the
 * first call there.  Every call on one GPU shares that GPU's array, so
 * calls that may overlap on one GPU (different streams, or host threads)
 * race and give wrong results: serialise them.  The array keeps the last
 * call's partial sums; each call overwrites what it reads.
 * Errors: those of d4r_gemm; D4R_ERR_UNSUPPORTED when the plan needs more
 * split-K scratch than the array holds (d4r_gemm_workspace_size() bytes >
 * d4r_gemm_noalloc_scratch_bytes(): call d4r_gemm with a workspace).
 */
d4r_status d4r_gemm_noalloc(int M, int K, int N, int flags, d4r_dtype dtype, const void *A,
                            const void *B, float *C, void *hip_stream);
size_t d4r_gemm_noalloc_scratch_bytes(void);

/*
 * A linear layer's forward in one call: C = op(A) * op(B) + bias, then
 * ReLU when relu != 0 (the directcompute-nn page's fully connected layer is
 * matmul then add_bias, x * W^T being flags 2, "Matmul Shaders" and
 * "Utility Shaders"; hidden layers of its LeNet-5 and AlexNet apply ReLU
 * next, "File Structure").
 * bias has N float32 entries, added per column: C[m][n] = sum + bias[n];
 * NULL adds nothing.  The epilogue applies both before the one store of C
 * (the split-K reduction does when the GEMM splits K), so C equals d4r_gemm,
 * then d4r_add_bias_rows, then d4r_relu_forward, bit for bit.  Workspace
 * as d4r_gemm_workspace_size gives for the same M, K, N, flags, dtype.
 * Errors: those of d4r_gemm; bias misaligned (4 bytes).
 */
d4r_status d4r_gemm_bias_act(int M, int K, int N, int flags, d4r_dtype dtype,
                             const void *A, const void *B, const float *bias,
                             int relu, float *C, void *ws, size_t ws_bytes,
                             void *hip_stream);

/*
 * The rest of a training step around the convolutions (directcompute-nn
 * page, "HLSL Shader Reference": "Activation / Loss Shaders", "Pooling
 * Shaders", "Utility Shaders"; the page's framework composes them with the
 * convolutions and matmuls into LeNet and AlexNet training, "Layer Stack"
 * and "File Structure").  All float32 (labels and argmax indices int32), all device
 * pointers owned by the caller, 16-byte aligned except bias, db, labels and
 * loss (4-byte).  Counts n, batch*channels and rows may be 0: nothing is
 * enqueued and the pointers are not examined (except d4r_bias_grad_rows,
 * which still writes db = 0 when rows is 0).  Every result is
 * run-to-run deterministic (fixed summation orders, no atomics).
 *
 * d4r_relu_forward: y = max(x, 0) elementwise; y may be x.
 * d4r_relu_backward: dx = dy where x > 0 (strictly), else 0; dx may be dy,
 *   not x.
 */
d4r_status d4r_relu_forward(const float *x, float *y, long long n, void *hip_stream);
d4r_status d4r_relu_backward(const float *x, const float *dy, float *dx, long long n,
                             void *hip_stream);

/*
 * Max pooling with argmax, window k x k, stride `stride` on both axes, no
 * padding: x (batch, channels, H, W) -> y (batch, channels, OH, OW), OH =
 * (H - k)/stride + 1, OW likewise (H, W >= k).  idx[b][c][i][j] = h*W + w,
 * the position of the maximum inside its (b, c) plane: the first strictly
 * greater value met scanning the window row by row.  The backward writes
 * every dx element: the sum of the dy entries whose saved index is that
 * element (overlapping windows add up, windows in row-major order), 0 where
 * none chose it (a gather, so dx needs no clearing first, unlike the page's
 * scatter after a buffer clear, "How the Engine Works").  idx must come from
 * the forward with the same geometry.
 * y, idx and dx must not overlap the other arguments.
 */
d4r_status d4r_maxpool_forward(const float *x, float *y, int *idx, int batch, int channels,
                               int H, int W, int k, int stride, void *hip_stream);
d4r_status d4r_maxpool_backward(const float *dy, const int *idx, float *dx, int batch,
                                int channels, int H, int W, int k, int stride,
                                void *hip_stream);

/*
 * Linear-layer bias on row-major rows x cols (the page's add_bias:
 * out[i] = A[i] + B[i mod cols]): y[r][c] = x[r][c] + bias[c]; y may be x.
 * d4r_bias_grad_rows: db[c] = sum over r of dy[r][c].  Use d4r_gemm for the layer's matmuls (x * W^T is flags 2, the data
 * gradient dy * W flags 0, the weight gradient dy^T * x flags 1).
 */
d4r_status d4r_add_bias_rows(const float *x, const float *bias, float *y, int rows, int cols,
                             void *hip_stream);
d4r_status d4r_bias_grad_rows(const float *dy, float *db, int rows, int cols, void *hip_stream);

/*
 * Row softmax of z (rows x classes, row-major), the row maximum subtracted
 * before exponentiation: p = softmax(z).  p must not overlap z.
 *
 * d4r_softmax_ce_grad: dz = softmax(z) - one_hot(labels) per row (no 1/rows
 * factor), and, when loss is not NULL, *loss = the mean over rows of
 * -log softmax(z)[label] (one float).  A label outside [0, classes) cannot be
 * rejected without a host synchronisation: that row of dz and the loss
 * become NaN.  With a loss the kernel runs as one workgroup (a fixed-order
 * mean); without, one wavefront per row.  dz and loss must not overlap z.
 */
d4r_status d4r_softmax(const float *z, float *p, int rows, int classes, void *hip_stream);
d4r_status d4r_softmax_ce_grad(const float *z, const int *labels, float *dz, float *loss,
                               int rows, int classes, void *hip_stream);

/*
 * d4r_sgd_update: param -= lr * clamp(grad, -clip, clip), elementwise, in
 * place (clip >= 0; +infinity disables clipping).
 * d4r_grad_accum: acc += grad, in place (a tensor that receives gradients
 * along several paths).  grad must not overlap param / acc.
 */
d4r_status d4r_sgd_update(float *param, const float *grad, long long n, float lr, float clip,
                          void *hip_stream);
d4r_status d4r_grad_accum(float *acc, const float *grad, long long n, void *hip_stream);

/*
 * Kernel timing (measurement aid).  While enabled, every kernel launch made
 * by the calls above is bracketed by a pair of HIP events recorded on the
 * call's stream, and tagged with the launch's algorithmic work: flops for
 * the GEMMs (2*M*N*K, padding zeros included), bytes for the data-movement
 * kernels (bytes the step must read plus bytes it must write).  Disabled by
 * default; when disabled it costs one branch per launch.
 *
 * d4r_profile_read synchronises on the recorded events and returns one
 * entry per kernel class, named "<kernel>:<pass>", e.g.
 * "gemm_f32_128x128_kk:wgrad" or "im2col_f32:fwd".  Names stay valid for the
 * life of the process.  *count receives the number of classes (entries
 * beyond max are dropped).  d4r_profile_reset forgets all records.  The
 * recorder is process-wide and guarded by a mutex.
 */
typedef struct {
    const char *name;
    int launches;
    double ms;     /* summed event-to-event time of all launches */
    double flops;  /* summed algorithmic flops (0 for data movement) */
    double bytes;  /* summed algorithmic bytes */
} d4r_kernel_stat;

d4r_status d4r_profile_enable(int on);
d4r_status d4r_profile_reset(void);
d4r_status d4r_profile_read(d4r_kernel_stat *out, int max, int *count);

/*
 * Measurement aids (not steps of the method): plain streaming kernels whose
 * rates are the attainable HBM reference the bench reports beside the
 * HBM-bound steps.  d4r_stream_copy: dst[i] = src[i] over `bytes` (read +
 * write stream); d4r_stream_fill: every 32-bit word of dst = value (write
 * stream).  16-byte aligned device pointers, bytes a multiple of 16 (0 does
 * nothing), dst and src must not overlap.  Errors: D4R_ERR_INVALID_ARG.
 */
d4r_status d4r_stream_copy(void *dst, const void *src, size_t bytes, void *hip_stream);
d4r_status d4r_stream_fill(void *dst, unsigned int value, size_t bytes, void *hip_stream);

/*
 * Measurement aid (not a step of the method): the MFMA rate this GPU
 * sustains with no data movement, the reference the bench reports beside
 * the GEMMs (the published dense peak assumes a clock the chip does not
 * hold under a full MFMA load).  blocks workgroups of eight wavefronts each
 * run iters iterations of eight MFMAs -- the dtype's GEMM instruction,
 * v_mfma_f32_32x32x16_{f16,bf16} or v_mfma_f32_32x32x2_f32 -- on operand
 * fragments read once from src (6 x 64 x 16 bytes for f16/bf16, 6 x 64
 * floats for f32, lane-major), for 2*32*32*k*64*iters*blocks flops (k = 16,
 * or 2 for f32).  Lane 0 of each wavefront writes the sum of its 8 x 16
 * accumulator elements to out (blocks * 8 floats): with every operand 1.0
 * that is 128 * k * iters.  16-byte aligned device pointers that do not
 * overlap.  Errors: D4R_ERR_INVALID_ARG (dtype, blocks outside [1, 2^20],
 * iters < 1, pointers).
 */
d4r_status d4r_mfma_ceiling(d4r_dtype dtype, const void *src, float *out, int blocks, int iters,
                            void *hip_stream);

/* Static string naming a status code. */
const char *d4r_status_string(d4r_status s);

/* Thread-local message describing the last failing call ("" if none). */
const char *d4r_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* D4R_CONV_H */
