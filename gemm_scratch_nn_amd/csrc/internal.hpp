// Internal declarations shared by the C-ABI layer and the gfx950 kernels of
// libd4r_conv.  Nothing here is part of the public ABI.
#pragma once

#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace d4r {

enum Dt : int { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

inline int dt_size(int dt) { return dt == DT_F32 ? 4 : 2; }

// GEMM tile shapes: a workgroup is NWM x NWN wavefronts (64 lanes each); a
// wavefront owns TM x TN blocks of 32x32 outputs.
enum TileCfg : int {
    TILE_128x128 = 0,  // 2x2 waves, 2x2 blocks
    TILE_64x64 = 1,    // 2x2 waves, 1x1 block
    TILE_32x128 = 2,   // 1x4 waves, 1x1 block (M <= 32)
    TILE_96x128 = 3,   // 1x4 waves, 3x1 blocks (M = 96)
    TILE_128x256 = 4,  // 2x4 waves, 2x2 blocks (16-bit operands only)
    TILE_256x128 = 5,  // 4x2 waves, 2x2 blocks (16-bit operands only)
    TILE_128x64 = 6,   // 2x2 waves, 2x1 blocks (f32 operands only)
    TILE_256x256 = 7,  // 2x4 waves, 4x2 blocks (16-bit, direct-to-LDS kernel only)
    TILE_COUNT = 8
};

struct TileShape { int bm, bn; };
inline TileShape tile_shape(int cfg)
{
    switch (cfg) {
    case TILE_128x128: return {128, 128};
    case TILE_64x64: return {64, 64};
    case TILE_32x128: return {32, 128};
    case TILE_96x128: return {96, 128};
    case TILE_128x256: return {128, 256};
    case TILE_128x64: return {128, 64};
    case TILE_256x256: return {256, 256};
    default: return {256, 128};
    }
}

// Bijective renumbering of workgroup ids so that the ids the dispatcher
// deals to one XCD (round-robin over the 8 XCDs of MI355X, each with its own
// L2) form one contiguous range of tiles.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_tile(int pid, int n)
{
    const int per = (n + kXcds - 1) / kXcds;
    int tall = n % kXcds;
    if (tall == 0)
        tall = kXcds;
    const int xcd = pid % kXcds, local = pid / kXcds;
    if (xcd < tall)
        return xcd * per + local;
    return tall * per + (xcd - tall) * (per - 1) + local;
}

// floor(n / d) for 0 <= n < 2^20 and 1 <= d <= 1024, from the hardware
// reciprocal (v_rcp_f32, within 1 ulp) instead of an integer division
// sequence: (n + 0.5) / d lies at least 0.5 / d from an integer, more than
// the float error over that range (checked exhaustively on the host with
// the reciprocal rounded either way).  Callers guarantee the ranges.
__device__ __forceinline__ int small_div(int n, int d)
{
    return (int)(((float)n + 0.5f) * __builtin_amdgcn_rcpf((float)d));
}

// 128x128 tiles of two k-contiguous 16-bit operands run on the direct-to-LDS
// kernel (the planner then rates them like the larger direct tiles);
// D4R_DL128=0 keeps them on the register-staged kernel (experiments).
inline bool dl128_enabled()
{
    const char *e = getenv("D4R_DL128");
    return !(e && e[0] == '0');
}

// The 16-bit direct-to-LDS 128x128 tile: eight wavefronts of 64x32 with a
// ring of four 32 KB stages (one workgroup per CU), the default, or the
// other forms measured against it (D4R_DL128_FORM = w4n2 | w8n2 | w8n3 |
// w8n4; experiments): four wavefronts of 64x64, rings of two or three.
// On the AlexNet conv3-5 bf16 step the default plans take 4 split-K
// reductions instead of 9 (0.543 -> 0.516 ms against w4n2).
struct Dl128Form {
    int waves, nbuf, wg_per_cu;
};
inline Dl128Form dl128_form()
{
    const char *e = getenv("D4R_DL128_FORM");
    if (e && !strcmp(e, "w4n2"))
        return {4, 2, 2};
    if (e && !strcmp(e, "w8n2"))
        return {8, 2, 2};
    if (e && !strcmp(e, "w8n3"))
        return {8, 3, 1};
    return {8, 4, 1};
}

// Work item of workgroup `pid` in a GEMM's 1-D grid of tiles x splits.  The
// XCD renumbering runs over all work items with the split outermost, so the
// contiguous range one XCD receives covers one or two K ranges (split-K
// slices) of the operands instead of a share of every slice: each XCD's L2
// then fetches the operand rows of its own K ranges only.
struct WorkItem {
    int tile, split;
};
__device__ __forceinline__ WorkItem xcd_work(int pid, int tiles, int splits)
{
    const int w = xcd_tile(pid, tiles * splits);
    return {w % tiles, w / tiles};
}

// Store of a GEMM result v = acc (+ bias) (then max(v, 0) with p.relu):
enum Epilogue : int {
    EPI_ROWMAJOR = 0,  // C[m*ldc + n] (+ blockIdx.z * c_split_stride); bias per column n
    EPI_NCHW = 1,      // y[((n/P)*M + m)*P + n%P]; bias per row m (the output channel)
    EPI_PHASE = 2      // one phase of a strided data gradient: column n = (b, i, j) of a
                       // g.OH x g.OW sub-grid lands at dx[b][m][ph_h0 + ph_s*i][ph_w0 + ph_s*j]
                       // of a ph_H x ph_W map (no bias)
};

// The epilogue's value: bias (per row for EPI_NCHW, per column otherwise)
// and ReLU (x > 0 ? x : 0, so NaN gives 0 like the ReLU kernel).
__device__ __forceinline__ float epi_value(float v, const float *bias, int relu, int epi, int m, int n)
{
    if (bias)
        v += bias[epi == EPI_NCHW ? m : n];
    if (relu)
        v = v > 0.0f ? v : 0.0f;
    return v;
}

struct ConvGeom {
    int B, C, H, W, O, kH, kW, s, p, OH, OW;
    int P;    // OH*OW
    int Kc;   // C*kH*kW
    int N;    // B*P
    int pw;   // padding along the width for the NHWC loaders (OP_IMPL_T); equals
              // p except in the sub-convolutions of a strided data gradient
};

// How a GEMM operand is laid out in memory.  Operand "rows" are m for A and
// n for B.
enum OperandMode : int {
    OP_ROWS = 0,  // row index contiguous: A[k*lda + m], B[k*ldb + n]
    OP_KC = 1,    // k contiguous: A[m*lda + k], B[n*ldb + k]
    OP_IMPL = 2,  // B only: op(B) = im2col(x), gathered from x (geometry p.g)
    OP_NCHW = 3,  // an NCHW tensor t[b][c][pix] with ch channels (p.a_ch /
                  // p.b_ch) and P = p.g.P pixels, whose (image, pixel) pair
                  // n = b*P + pix is the k index of A (A[c][n]) or the
                  // column index of B (B[c][n]); c is the row of A or the k
                  // of B.  Element address b*ch*P + c*P + pix.  (dy read in
                  // place; x or dy of a 1x1 stride-1 unpadded convolution.)
    OP_NCHW_K = 4,// B only: an NCHW tensor whose channel c is the row n of
                  // B and whose (image, pixel) pair is the k index:
                  // op(B)[k][c] = t[k / P][c][k % P] (x in the filter
                  // gradient of a 1x1 stride-1 unpadded convolution)
    OP_IMPL_T = 5 // B only: the im2col of an NHWC tensor t[b][h][w][c]
                  // (geometry p.g, stride 1) with k ordered by channel block,
                  // then tap, then channel inside the block: k = (cb*kH*kW +
                  // u*kW + v)*BK + ci for c = cb*BK + ci, BK the GEMM stage
                  // depth (32 f32, 64 16-bit); op(B)[k][n] =
                  // t[b][i-p+u][j-p+v][c] for n = (b, i, j), or 0 in the
                  // padding (read from p.zero).  Needs p.g.C % BK == 0.  The
                  // kH*kW stages of one channel block read overlapping
                  // windows of the same BK channels back to back.
};

// C = op(A) * op(B) over k in [z*k_per_split, min(K, (z+1)*k_per_split)).
struct GemmParams {
    const void *A;
    const void *B;
    float *C;
    const float *bias;
    int M, N, K;
    int lda, ldb, ldc;
    int P;              // EPI_NCHW: pixels per image
    int epi;
    int relu;           // apply ReLU after the bias
    int k_per_split;    // multiple of the tile's K depth
    int splits;
    long long c_split_stride;
    int a_vec, b_vec;   // 16-byte vector loads allowed (ld and base aligned;
                        // NCHW operands: P a multiple of the vector width)
    int a_ch, b_ch;     // channel counts of OP_NCHW / OP_NCHW_K operands
    const void *zero;   // OP_IMPL_T: 256 zero bytes, 16-byte aligned
    ConvGeom g;         // OP_IMPL and OP_NCHW operands
    int ph_s, ph_h0, ph_w0, ph_H, ph_W;  // EPI_PHASE: stride, first row / column, full map
    int group_m;        // direct-to-LDS kernel: tiles ordered in groups of group_m M tiles
                        // (0 or 1: M tiles fastest)
};

// Tile (m, n) of tile index t in an mt x nt grid.  With group > 1 the tiles
// run in bands of `group` M tiles, N fastest within a band, so the
// contiguous range of tiles an XCD receives is a near-square block (fewer
// distinct operand panels per L2) instead of whole columns of M tiles.
__device__ __forceinline__ void tile_mn(int t, int mt, int nt, int group, int &tm, int &tn)
{
    if (group <= 1) {
        tm = t % mt;
        tn = t / mt;
        return;
    }
    const int per = group * nt;
    const int first = (t / per) * group;
    const int size = min(mt - first, group);
    const int r = t - (t / per) * per;
    tm = first + r % size;
    tn = r / size;
}

// The data gradient of a stride-s convolution as s*s stride-1 sub-
// convolutions of dy, one per output phase (rh, rw): dx rows h with
// (h + p) mod s = rh take the taps u = rh + s*t, and
//   dx[b][c][h0 + s*i][w0 + s*j] = sum_{u', v', o} Wph[c][u'][v'][o] *
//       dy[b][o][i - ph + u'][j - pw + v'],
//   Wph[c][u'][v'][o] = W[o][c][rh + s*(Tu-1-u')][rw + s*(Tv-1-v')]
// with Tu = ceil((kH - rh)/s) taps, ph = Tu - 1 - (h0 + p - rh)/s (likewise
// for the width).  Each phase is one GEMM (M = C, K = Tu*Tv*O, N = B * its
// pixels) over dy read as NHWC; all phases run in one launch.
constexpr int kMaxPhases = 16;
struct PhaseItem {
    long long a_off;  // element offset of the phase filter Wph (C x K) in A
    int K;            // Tu*Tv*O
    int tile0;        // the phase's first work item
    int h0, w0;       // its first dx row and column
    ConvGeom g;       // the stride-1 sub-convolution over dy (C = O, O = dx channels)
};
struct PhaseArgs {
    int n, tiles;     // phases, work items of all phases
    PhaseItem ph[kMaxPhases];
};
// one launch over every phase of pa (tile 128x128, direct-to-LDS kernel,
// K of each phase a whole number of stages); p carries M, A (the phase
// filters, concatenated), B (dy as NHWC), C (dx) and the EPI_PHASE fields
hipError_t launch_gemm_phased(int dt, const GemmParams &p, const PhaseArgs &pa, hipStream_t s);
// Wph of every phase (offsets and tap counts in pa), from W (O x C x kH x kW)
hipError_t launch_phase_filter(int dt, const ConvGeom &g, const PhaseArgs &pa, const void *w, void *wph,
                               hipStream_t s);

// Supported (A, B) modes: every pair of OP_ROWS / OP_KC, (OP_KC, OP_IMPL),
// (OP_KC, OP_NCHW), (OP_ROWS, OP_NCHW), (OP_NCHW, OP_NCHW_K), and for f32
// also (OP_NCHW, OP_KC).  Others return
// hipErrorInvalidValue.
hipError_t launch_gemm(int dt, int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s);
int gemm_bk(int dt);  // K depth of one LDS stage, in elements



// The kernel an im2col / col2im launch runs and its block shape (host only;
// launch_im2col / launch_col2im follow exactly this plan).  RB output rows
// and BB images of one channel per block; Rl x Wl window; shm LDS bytes.
enum Im2colKind : int { IM2COL_GATHER = 0, IM2COL_LDS = 1, IM2COL_SHIFT = 2 };
struct Im2colPlan {
    int kind, RB, BB, Rl, Wl;
    size_t shm;
};
Im2colPlan plan_im2col(int dt, const ConvGeom &g);
enum Col2imKind : int { COL2IM_GATHER = 0, COL2IM_LDS = 1 };
struct Col2imPlan {
    int kind, BB, Rl, Wl;
    size_t shm;
};
Col2imPlan plan_col2im(const ConvGeom &g);

hipError_t launch_im2col(int dt, const ConvGeom &g, const void *x, void *col, hipStream_t s);
hipError_t launch_col2im(const ConvGeom &g, const float *dcol, float *dx, hipStream_t s);
// G[o][n] = dy[b][o][pix], n = b*P + pix  (O x N row-major); with bias_part
// set, also the bias gradient's per-block partial sums, O x
// grad_reshape_blocks() floats (finish with launch_bias_final)
hipError_t launch_grad_reshape(int dt, const ConvGeom &g, const void *dy, void *G, float *bias_part,
                               hipStream_t s);
int grad_reshape_blocks(int dt, const ConvGeom &g);
// db[o] = sum over s < splits of partial[o*splits + s], in order
hipError_t launch_bias_final(const float *partial, float *db, int O, int splits, hipStream_t s);
// out[b][c][r] = in[b][r][c] for a batch of R x Cc matrices of dt elements
hipError_t launch_transpose(int dt, int batch, int R, int Cc, const void *in, void *out,
                            hipStream_t s);
// db[o] = sum_{b,pix} dy[b][o][pix]; partial holds O*splits floats
// pass 1 of launch_bias_grad alone: partial[o*splits + k] (the per-channel
// sums then come from a BiasSum)
hipError_t launch_bias_partials(int dt, const ConvGeom &g, const void *dy, float *partial, int splits,
                                hipStream_t s);
hipError_t launch_bias_grad(int dt, const ConvGeom &g, const void *dy, float *db,
                            float *partial, int splits, hipStream_t s);
int bias_grad_splits(const ConvGeom &g);
// wf[c][o][u][v] = w[o][c][kH-1-u][kW-1-v] (the implicit data gradient's filter)
hipError_t launch_flip_filter(int dt, const ConvGeom &g, const void *w, void *wf, hipStream_t s);
// A per-channel sum db[o] = sum over k < parts of partial[o*parts + k] (in k
// order) that a split-K reduction can run in extra blocks; db NULL: none.
struct BiasSum {
    const float *partial;
    float *db;
    int O, parts;
};

// One batched transpose out[z][c][r] = in[z][r][c] (batch z, R x Cc); zero,
// when set, gets 256 bytes cleared.  `blocks` is filled in by the launcher.
struct TransposeJob {
    const void *in;
    void *out;
    int R, Cc, batch;
    uint32_t *zero;
    int blocks;
};

// The filter w (O x C x taps, taps = kH*kW) written in the NHWC loader's k
// order, blocks of kb channels outermost, then tap, then the channel inside
// the block: flip = 0 (forward) out[o][cb][tap][ci] = w[o][cb*kb+ci][tap];
// flip = 1 (data gradient, taps reversed) out[c][ob][t][oi] =
// w[ob*kb+oi][c][taps-1-t].  Needs C (flip 0) or O (flip 1) a multiple of
// kb, kb a multiple of the 16-byte vector.  zero, when set, gets 256 bytes
// cleared.  `blocks` is filled in by the launcher.
struct FilterJob {
    const void *in;
    void *out;
    int O, C, taps, kb, flip;
    uint32_t *zero;
    int blocks;
};

// a data transpose and a filter job in one launch (either may be empty: no
// rows; they must not overlap in memory)
hipError_t launch_transpose_filter(int dt, TransposeJob a, FilterJob f, hipStream_t s);

// dy (B x O x P) read once, written as G[o][b*P + pix] and Gt[b][pix][o],
// with the bias gradient's partial sums (dy_prep_bias_parts(g) per channel)
// when bias_part is set; the filter job w rides in the same launch.  dt and
// blocks are filled in by launch_dy_prep.
struct DyPrep {
    const void *dy;
    void *gt, *g;
    float *bias_part;
    int B, O, P, dt, blocks;
};
int dy_prep_bias_parts(const ConvGeom &g);
hipError_t launch_dy_prep(int dt, DyPrep a, FilterJob w, hipStream_t s);

// the BiasSum on its own (wavefront per channel), and the block count it
// takes as extra blocks of a reduction
int bias_sum_blocks(const BiasSum &bs);
hipError_t launch_bias_sum(const BiasSum &bs, hipStream_t s);

// out = sum over s of part[s] (fixed order) with the GEMM epilogue, plus the
// bias sum bs when bs.db is set
hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N,
                                long long split_stride, int epi, float *C, int ldc,
                                const float *bias, int P, int relu, const BiasSum &bs, hipStream_t s);

// Streaming reference kernels (stream_kernels.hip): bytes a multiple of 16,
// 16-byte aligned pointers.
hipError_t launch_stream_copy(void *dst, const void *src, size_t bytes, hipStream_t s);
hipError_t launch_stream_fill(void *dst, uint32_t value, size_t bytes, hipStream_t s);
// MFMA ceiling (stream_kernels.hip): blocks x 8 wavefronts, iters x 8 MFMAs
// each; src holds 6 x 64 16-byte fragments (16-bit) or 6 x 64 floats (f32);
// out gets blocks * 8 floats
hipError_t launch_mfma_ceiling(int dt, const void *src, float *out, int blocks, int iters, hipStream_t s);

// The rest of a training step (f32; train_kernels.hip).  Elementwise
// kernels take 16-byte aligned pointers; n may be 0.
hipError_t launch_relu_forward(const float *x, float *y, long long n, hipStream_t s);
hipError_t launch_relu_backward(const float *x, const float *dy, float *dx, long long n, hipStream_t s);
// planes = batch * channels of H x W; output OH x OW; idx = plane offsets
hipError_t launch_maxpool_forward(const float *x, float *y, int32_t *idx, long long planes, int H, int W,
                                  int OH, int OW, int k, int st, hipStream_t s);
hipError_t launch_maxpool_backward(const float *dy, const int32_t *idx, float *dx, long long planes, int H,
                                   int W, int OH, int OW, int k, int st, hipStream_t s);
hipError_t launch_add_bias_rows(const float *x, const float *bias, float *y, long long rows, int cols,
                                hipStream_t s);
hipError_t launch_bias_grad_rows(const float *dy, float *db, long long rows, int cols, hipStream_t s);
// label NULL: out = softmax(z); else out = softmax(z) - one_hot(label) and
// *loss (if loss != NULL) = mean cross-entropy
hipError_t launch_softmax_rows(const float *z, const int32_t *label, float *out, float *loss, int rows,
                               int classes, hipStream_t s);
hipError_t launch_sgd(float *p, const float *g, long long n, float lr, float clip, hipStream_t s);
hipError_t launch_grad_accum(float *acc, const float *g, long long n, hipStream_t s);

}  // namespace d4r
