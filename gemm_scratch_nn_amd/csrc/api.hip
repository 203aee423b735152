// C ABI of libd4r_conv (declared in include/d4r_conv.h): argument
// validation, output extents, workspace layout, GEMM tile / split-K choice
// and the launch sequence of each pass.  Everything is validated before the
// first HIP call, so an invalid call enqueues nothing.
//
// Pass sequences (directcompute-nn page, "Convolution: The im2col
// Approach"):
//   forward          im2col(x) -> col;  GEMM NN  Wmat[O x Kc] * col[Kc x N]
//                    with the conv_reshape + bias store fused in its epilogue
//   backward_data    GEMM dcol[Kc x N] = Wmat^T * G, then col2im(dcol) -> dx.
//                    G is dy read in place (f32, small Kc) or copied as
//                    Gt[N x O] with W copied as Wt[Kc x O], so both operands
//                    stream k-contiguous
//   backward_filter  [im2col(x) -> col]; GEMM NT dW[O x Kc] = G * col^T,
//                    split over k with partial sums reduced in a fixed order;
//                    G is dy read in place or reshaped to G[O x N] (that pass
//                    also yields the bias partial sums); db by reduction
//   backward_data_implicit  (stride 1, square kernel) the implicit-GEMM
//                    forward of dy with the flipped filter; no dcol
#include <mutex>
#include <new>
#include <algorithm>
#include <string>
#include <unordered_map>
#include <vector>
#include <stdio.h>
#include <stdlib.h>
#include <stdarg.h>
#include <string.h>

#include "../../include/d4r_conv.h"
#include "internal.hpp"

using namespace d4r;

namespace {

thread_local char g_err[512];

d4r_status fail(d4r_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

d4r_status ok()
{
    g_err[0] = 0;
    return D4R_OK;
}

constexpr long long kMaxElems = 0x7fffffffLL;  // every tensor < 2^31 elements
constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

struct GemmPlan {
    int cfg;
    int splits;
    int k_per_split;
};

// Tile and split-K choice.  A tile config keeps wg_per_cu workgroups
// resident per compute unit (from its LDS and register use), so a launch
// runs in ceil(workgroups / slots) waves.  Splitting K into s slices
// multiplies the workgroups by s and divides each one's work by s, at the
// price of writing and re-reading s partial M x N slabs.  The split count
// minimises a small cost model of those two terms.
//
// Compute units of the current device (256 on MI355X), read once per
// process; 256 when no device answers (the host-only tests).
int compute_units()
{
    static int cus = [] {
        int dev = 0, n = 0;
        if (hipGetDevice(&dev) == hipSuccess &&
            hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
            return n;
        (void)hipGetLastError();
        return 256;
    }();
    return cus;
}

// Workgroups resident per CU for each tile config (LDS and register use of
// the compiled kernels), f32 and 16-bit builds; dl: the 16-bit product runs
// on the direct-to-LDS kernel (whose 128x128 form sets its own count).
int wg_per_cu(int cfg, int dt, bool dl)
{
    const bool h = dt != DT_F32;
    switch (cfg) {
    case TILE_128x128: return h && dl && dl128_enabled() ? dl128_form().wg_per_cu : 2;
    case TILE_64x64: return h ? 3 : 4;
    case TILE_32x128: return 3;
    case TILE_96x128: return 2;
    case TILE_128x64: return 2;  // f32 only
    default: return 1;  // 128x256, 256x128 (16-bit only, 8 waves)
    }
}

struct TileCand {
    int cfg;
    double eff;  // relative sustained MFMA rate per CU (L2 traffic per flop)
};

int tile_from_env(int dt)
{
    // experiment override, e.g. D4R_GEMM_TILE=128x256
    const char *e = getenv("D4R_GEMM_TILE");
    if (!e)
        return -1;
    for (int c = 0; c < TILE_COUNT; ++c) {
        if (dt == DT_F32 && (c == TILE_128x256 || c == TILE_256x128 || c == TILE_256x256))
            continue;
        if (dt != DT_F32 && c == TILE_128x64)
            continue;
        TileShape ts = tile_shape(c);
        char buf[32];
        snprintf(buf, sizeof buf, "%dx%d", ts.bm, ts.bn);
        if (strcmp(buf, e) == 0)
            return c;
    }
    return -1;
}

// dl16: only the tiles of the 16-bit direct-to-LDS kernel (OP_IMPL_T).
GemmPlan plan_gemm(int M, int N, int K, int dt, bool dl16 = false, bool kk16 = false)
{
    TileCand cands[8];
    int nc = 0;
    // 256x256 (direct-to-LDS only, one workgroup per CU): a third less
    // operand traffic per flop than 128x256; measured 1.25x its rate on
    // square products (4096^3 bf16 977 against 780 TFLOP/s)
    const double e256 = 1.25;
    if (dl16) {
        cands[nc++] = {TILE_128x256, 1.0};
        cands[nc++] = {TILE_256x128, 1.0};
        cands[nc++] = {TILE_256x256, e256};
        // a shade below the larger direct tiles: preferred only where it
        // saves whole waves (the 129-tile data gradients of conv4/conv5)
        if (dl128_enabled())
            cands[nc++] = {TILE_128x128, 0.95};
    } else if (M <= 32) {
        cands[nc++] = {TILE_32x128, 1.0};
    } else if (M <= 64 || N <= 64) {
        cands[nc++] = {TILE_64x64, 1.0};
    } else if (dt == DT_F32) {
        if (M % 128 != 0 && M % 96 == 0 && M <= 192) {
            cands[nc++] = {TILE_96x128, 1.0};
        } else {
            // 128x64 fills the chip without split-K where 128x128 tiles
            // would not make one full wave; elsewhere it measured 4-8%
            // slower per flop, more than the model's wave rounding shows
            cands[nc++] = {TILE_128x128, 1.0};
            const long long t128 = (long long)((M + 127) / 128) * ((N + 127) / 128);
            if (t128 < (long long)compute_units() * wg_per_cu(TILE_128x128, dt, false))
                cands[nc++] = {TILE_128x64, 0.92};
        }
    } else {
        // kk16: both operands k-contiguous, 16-byte rows, whole 64-deep
        // stages, so 128x128 runs on the direct-to-LDS kernel too
        cands[nc++] = {TILE_128x128, kk16 && dl128_enabled() ? 0.95 : 0.85};
        cands[nc++] = {TILE_128x256, 1.0};
        cands[nc++] = {TILE_256x128, 1.0};
        if (kk16)
            cands[nc++] = {TILE_256x256, e256};
        // small products (a 1x1 layer on the 46x80 map): when the large
        // tiles leave most CUs idle, 64x64 tiles at three per CU hide the
        // load latency better than split-K (measured 12 against 22 us)
        const long long tbig = (long long)((M + 127) / 128) * ((N + 255) / 256);
        if (tbig < compute_units())
            cands[nc++] = {TILE_64x64, 0.5};
        if (M % 128 != 0 && M % 96 == 0 && M <= 192)
            cands[nc++] = {TILE_96x128, 0.8};
    }
    const int forced = tile_from_env(dt);
    if (forced >= 0) {
        nc = 1;
        cands[0] = {forced, 1.0};
    }
    const int bk = gemm_bk(dt);
    const long long ktiles = (K + bk - 1) / bk;
    const double peak = dt == DT_F32 ? 157.3e12 * 0.6 : 2516.6e12 * 0.3;
    const double bw = 3.0e12;       // bytes/s for the partial-sum round trip
    const double t_launch = 3e-6;   // one extra kernel
    double best = 1e30;
    GemmPlan pl{cands[0].cfg, 1, (int)(ktiles * bk)};
    for (int ci = 0; ci < nc; ++ci) {
        const TileShape ts = tile_shape(cands[ci].cfg);
        const long long tiles = (long long)((M + ts.bm - 1) / ts.bm) * ((N + ts.bn - 1) / ts.bn);
        const long long slots = (long long)compute_units() * wg_per_cu(cands[ci].cfg, dt, dl16 || kk16);
        // seconds per K stage of one workgroup when every slot is busy
        const double t_stage = 2.0 * ts.bm * ts.bn * bk / (peak * cands[ci].eff / (double)slots);
        long long smax = ktiles < 256 ? ktiles : 256;
    if (const char *e = getenv("D4R_GEMM_MAX_SPLITS"))  // experiments: cap split-K
        smax = std::max(1LL, std::min(smax, atoll(e)));
        for (long long sp = 1; sp <= smax; ++sp) {
            const long long per = (ktiles + sp - 1) / sp;
            const long long se = (ktiles + per - 1) / per;
            if (se != sp)
                continue;
            const long long waves = (tiles * se + slots - 1) / slots;
            double t = (double)waves * per * t_stage;
            if (se > 1)
                t += (double)(se + 1) * M * N * 4.0 / bw + t_launch;
            if (t < best * 0.999) {
                best = t;
                pl.cfg = cands[ci].cfg;
                pl.splits = (int)se;
                pl.k_per_split = (int)(per * bk);
            }
        }
    }
    return pl;
}

// d4r_gemm with both operands k-contiguous (flags 2), 16-bit, whole 64-deep
// stages and 16-byte aligned rows: the direct-to-LDS kernel applies
bool gemm_kk16(int K, int flags, int dt) { return dt != DT_F32 && flags == 2 && K % 64 == 0; }

size_t plan_partial_bytes(const GemmPlan &pl, int M, int N)
{
    return pl.splits > 1 ? (size_t)pl.splits * M * N * sizeof(float) : 0;
}

const char *dt_name(int dt) { return dt == DT_F32 ? "f32" : (dt == DT_F16 ? "f16" : "bf16"); }

// ---------------------------------------------------------------------------
// Kernel timing: HIP event pairs around each launch, on the launch stream.
// ---------------------------------------------------------------------------
struct ProfRec {
    hipEvent_t a, b;
    int key;
    double flops, bytes;
};

struct Profiler {
    std::mutex mu;
    bool on = false;
    std::vector<ProfRec> recs;       // pool; the first `used` are live
    size_t used = 0;
    std::vector<std::string> names;  // key -> name (never shrinks)
    std::unordered_map<std::string, int> ids;
};

Profiler &prof()
{
    static Profiler *p = new Profiler;  // never destroyed: names stay valid
    return *p;
}

// Brackets one launch.  Constructed before the launch, finished after it.
struct ProfScope {
    long long idx = -1;  // index into recs (the vector may grow under another thread)
    hipStream_t s;
    ProfScope(hipStream_t st, const std::string &name, double flops, double bytes) : s(st)
    {
        Profiler &P = prof();
        std::lock_guard<std::mutex> lk(P.mu);
        if (!P.on)
            return;
        auto it = P.ids.find(name);
        int key;
        if (it == P.ids.end()) {
            key = (int)P.names.size();
            P.names.push_back(name);
            P.ids[name] = key;
        } else {
            key = it->second;
        }
        if (P.used == P.recs.size()) {
            ProfRec r{};
            // no system-scope fence on record: the events only time kernels
            // on this device, and a fenced record stalls the queue between
            // launches
            if (hipEventCreateWithFlags(&r.a, hipEventDisableSystemFence) != hipSuccess ||
                hipEventCreateWithFlags(&r.b, hipEventDisableSystemFence) != hipSuccess)
                return;
            P.recs.push_back(r);
        }
        idx = (long long)P.used++;
        ProfRec &rec = P.recs[idx];
        rec.key = key;
        rec.flops = flops;
        rec.bytes = bytes;
        (void)hipEventRecord(rec.a, s);
    }
    void done()
    {
        if (idx < 0)
            return;
        Profiler &P = prof();
        std::lock_guard<std::mutex> lk(P.mu);
        (void)hipEventRecord(P.recs[idx].b, s);
    }
};

// Kernel names: gemm_<dtype>_<tile>_<A><B>, one letter per operand form:
// k = k-contiguous, m / n = row-contiguous A / B, g = NCHW gradient read in
// place; the implicit forward adds "_implicit".
std::string gemm_kernel_name(int dt, int cfg, int amode, int bmode)
{
    TileShape ts = tile_shape(cfg);
    const char a = amode == OP_KC ? 'k' : (amode == OP_NCHW ? 'g' : 'm');
    const char b = (bmode == OP_KC) ? 'k' : (bmode == OP_NCHW ? 'g' : (bmode == OP_NCHW_K ? 'c' : 'n'));
    return std::string("gemm_") + dt_name(dt) + "_" + std::to_string(ts.bm) + "x" + std::to_string(ts.bn) +
           "_" + a + b + (bmode == OP_IMPL ? "_implicit" : (bmode == OP_IMPL_T ? "_nhwc" : ""));
}


// Runs one planned GEMM (split-K partials + reduction when the plan splits).
// Operand forms follow OperandMode; OP_IMPL (B = x, op(B) = im2col(x)) and
// the NCHW forms take their geometry from `geom`; a_ch / b_ch are the channel
// counts of NCHW operands (default: geom->O, the gradient dy).  The epilogue
// adds bias (per row m for EPI_NCHW, per column n for EPI_ROWMAJOR) and then
// applies ReLU when relu is set; with split K both happen in the reduction.
hipError_t run_gemm(int dt, const GemmPlan &pl, int amode, int bmode, const void *A, int lda,
                    const void *B, int ldb, int M, int N, int K, int epi, float *C, int ldc,
                    const float *bias, int P, float *partial, hipStream_t s, const char *pass,
                    const ConvGeom *geom = nullptr, int a_ch = 0, int b_ch = 0, const void *zero = nullptr,
                    int relu = 0, const BiasSum *bsum = nullptr)
{
    const bool implicit = bmode == OP_IMPL;
    const int vw = dt == DT_F32 ? 4 : 8;
    GemmParams p;
    memset(&p, 0, sizeof p);
    p.A = A;
    p.B = B;
    p.bias = bias;
    p.M = M;
    p.N = N;
    p.K = K;
    p.lda = lda;
    p.ldb = ldb;
    p.P = P;
    p.k_per_split = pl.k_per_split;
    p.splits = pl.splits;
    {
        // large grids run in bands of 8 M tiles: each XCD's range of tiles is
        // a near-square block (8192^3 bf16 953 -> 1027 TFLOP/s on 256x256
        // tiles; conv shapes, with a few M tiles, are unaffected)
        const TileShape ts = tile_shape(pl.cfg);
        const int mt = (M + ts.bm - 1) / ts.bm, nt = (N + ts.bn - 1) / ts.bn;
        p.group_m = (mt >= 16 && nt >= 16) ? 8 : 0;
    }
    // vector loads need every 16-byte vector wholly inside or outside the
    // operand: leading dimension and the contiguous extent multiples of vw
    p.a_vec = (lda % vw) == 0 && ((amode == OP_KC ? K : M) % vw) == 0;
    p.b_vec = (ldb % vw) == 0 && ((bmode == OP_KC ? K : N) % vw) == 0;
    if (geom)
        p.g = *geom;
    else
        memset(&p.g, 0, sizeof p.g);
    p.zero = zero;
    p.a_ch = a_ch ? a_ch : p.g.O;
    p.b_ch = b_ch ? b_ch : p.g.O;
    // an NCHW operand takes whole vectors when they cannot straddle images
    if (amode == OP_NCHW)
        p.a_vec = geom && geom->P % vw == 0;
    if (bmode == OP_NCHW || bmode == OP_NCHW_K)
        p.b_vec = geom && geom->P % vw == 0;
    if (pl.splits > 1) {
        // raw partial sums: bias and ReLU wait for the reduction
        p.C = partial;
        p.ldc = N;
        p.epi = EPI_ROWMAJOR;
        p.c_split_stride = (long long)M * N;
        p.bias = nullptr;
        p.relu = 0;
    } else {
        p.C = C;
        p.ldc = ldc;
        p.epi = epi;
        p.c_split_stride = 0;
        p.relu = relu;
    }
    const int es = dt_size(dt);
    const double b_bytes = (implicit || bmode == OP_IMPL_T) ? (double)geom->B * geom->C * geom->H * geom->W
                                                             : (double)K * N;
    ProfScope ps(s, gemm_kernel_name(dt, pl.cfg, amode, bmode) + ":" + pass, 2.0 * M * N * K,
                 (double)es * ((double)M * K + b_bytes) + 4.0 * M * N);
    hipError_t e = launch_gemm(dt, pl.cfg, amode, bmode, p, s);
    ps.done();
    if (e != hipSuccess)
        return e;
    const BiasSum none{nullptr, nullptr, 0, 0};
    const BiasSum &bs = bsum ? *bsum : none;
    if (pl.splits == 1) {
        if (!bs.db)
            return hipSuccess;
        ProfScope pb(s, std::string("bias_final:") + pass, 0.0, 4.0 * bs.O * (bs.parts + 1.0));
        e = launch_bias_sum(bs, s);
        pb.done();
        return e;
    }
    // the reduction's extra blocks finish the bias sum, if any
    ProfScope pr(s, std::string("splitk_reduce:") + pass, 0.0,
                 4.0 * (double)M * N * (pl.splits + 1) + (bs.db ? 4.0 * bs.O * (bs.parts + 1.0) : 0.0));
    e = launch_splitk_reduce(partial, pl.splits, M, N, (long long)M * N, epi, C, ldc, bias, P, relu, bs, s);
    pr.done();
    return e;
}

bool valid_dtype(int dt) { return dt == D4R_F32 || dt == D4R_F16 || dt == D4R_BF16; }

}  // namespace

// How the gradient GEMMs take dy.  GP_INPLACE reads it where it lies (NCHW
// operand loaders, f32 only): no copy, but single-element loads inside the
// GEMM.  GP_COPY first copies it into the workspace with 16-byte-friendly
// rows: transposed (N x O) for the data gradient, reshaped (O x N) for the
// filter gradient.
enum GradPath : int { GP_INPLACE = 0, GP_COPY = 1 };

struct d4r_conv {
    ConvGeom g;
    int dt;
    int es;
    GemmPlan fwd, bwd_data, bwd_filter;
    int bias_splits;
    size_t off_g, off_wt, off_wflip, off_bias, off_big, ws_bytes;
    GradPath dgrad, wgrad;  // how the gradient GEMMs take dy
    bool dgrad_wt;          // data gradient reads a k-contiguous copy of W^T
    // implicit data gradient (stride 1, square kernel): dx is the forward
    // convolution of dy with the flipped filter, geometry gd
    bool dgrad_impl;
    ConvGeom gd;
    GemmPlan bwd_data_impl;
    // 1x1 kernel, stride 1, no padding: col is x with the batch folded into
    // its columns, so the GEMMs can read x and dy in place (no im2col, no
    // dcol, no col2im)
    bool pointwise;
    // implicit data gradient from dy read as NHWC (its transpose Gt): filter
    // wd[c][ob][u][v][oi] (o = ob*BK + oi, the loader's k order), a zero
    // page (direct-to-LDS loads of padding)
    bool dgrad_nhwc;
    GemmPlan bwd_data_nhwc;
    size_t off_zero;
    size_t off_gt;  // Gt (NHWC dy), a region of its own next to G
    // d4r_conv_backward prepares dy for both gradient GEMMs in one pass
    // (NHWC data gradient and a copied G for the filter gradient)
    bool fused_bwd;
    // f32 layers whose data gradient is explicit (dcol + col2im): the
    // combined backward reshapes dy once into G (with the bias partials),
    // which the data-gradient GEMM reads row-contiguous and the filter
    // gradient k-contiguous; fx_wt: the data gradient reads a transposed
    // copy of W (k-contiguous) instead of W row-contiguous
    bool fused_explicit, fx_wt;
    // implicit forward from x read as NHWC (stride 1, whole GEMM stages of
    // input channels): x transposed to xt[b][h][w][c], the filter reordered
    // to wr[o][cb][u][v][ci] (c = cb*BK + ci); the loader of the NHWC data
    // gradient
    bool fwd_nhwc;
    GemmPlan fwd_nhwc_plan;
    size_t off_xt, off_wr;
    // data gradient of a strided layer as stride^2 stride-1 sub-convolutions
    // of dy read as NHWC (one per output phase), in one launch
    bool dgrad_phased;
    PhaseArgs phases;
    size_t col_bytes;
    double in_image_col;  // col entries copied from inside the image
};

namespace d4r {

int gemm_bk(int dt) { return dt == DT_F32 ? 32 : 64; }

hipError_t launch_gemm_f32(int, int, int, const GemmParams &, hipStream_t);
hipError_t launch_gemm_f16(int, int, int, const GemmParams &, hipStream_t);
hipError_t launch_gemm_bf16(int, int, int, const GemmParams &, hipStream_t);

hipError_t launch_gemm(int dt, int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    switch (dt) {
    case DT_F32: return launch_gemm_f32(cfg, amode, bmode, p, s);
    case DT_F16: return launch_gemm_f16(cfg, amode, bmode, p, s);
    default: return launch_gemm_bf16(cfg, amode, bmode, p, s);
    }
}

hipError_t launch_gemm_phased_f32(const GemmParams &, const PhaseArgs &, hipStream_t);
hipError_t launch_gemm_phased_f16(const GemmParams &, const PhaseArgs &, hipStream_t);
hipError_t launch_gemm_phased_bf16(const GemmParams &, const PhaseArgs &, hipStream_t);

hipError_t launch_gemm_phased(int dt, const GemmParams &p, const PhaseArgs &pa, hipStream_t s)
{
    switch (dt) {
    case DT_F32: return launch_gemm_phased_f32(p, pa, s);
    case DT_F16: return launch_gemm_phased_f16(p, pa, s);
    default: return launch_gemm_phased_bf16(p, pa, s);
    }
}

}  // namespace d4r

namespace {

// Launch wrappers that tag each step with its algorithmic bytes.
hipError_t step_im2col(const d4r_conv *h, const void *x, void *col, hipStream_t s, const char *pass)
{
    const ConvGeom &g = h->g;
    double bytes = (double)h->es * ((double)g.B * g.C * g.H * g.W + (double)g.Kc * g.N);
    ProfScope ps(s, std::string("im2col_") + dt_name(h->dt) + ":" + pass, 0.0, bytes);
    hipError_t e = launch_im2col(h->dt, g, x, col, s);
    ps.done();
    return e;
}

hipError_t step_col2im(const d4r_conv *h, const float *dcol, float *dx, hipStream_t s, const char *pass)
{
    const ConvGeom &g = h->g;
    double bytes = 4.0 * h->in_image_col + 4.0 * ((double)g.B * g.C * g.H * g.W);
    ProfScope ps(s, std::string("col2im_f32:") + pass, 0.0, bytes);
    hipError_t e = launch_col2im(g, dcol, dx, s);
    ps.done();
    return e;
}

hipError_t step_transpose(const d4r_conv *h, int batch, int R, int C, const void *in, void *out,
                          hipStream_t s, const char *what)
{
    double bytes = 2.0 * h->es * (double)batch * R * C;
    ProfScope ps(s, std::string("transpose_") + dt_name(h->dt) + ":" + what, 0.0, bytes);
    hipError_t e = launch_transpose(h->dt, batch, R, C, in, out, s);
    ps.done();
    return e;
}

// With bias_part set, the reshape also produces the bias gradient's partial
// sums (one per reshape block and channel), which a BiasSum adds up.
hipError_t step_grad_reshape(const d4r_conv *h, const void *dy, void *G, float *bias_part, hipStream_t s)
{
    const ConvGeom &g = h->g;
    ProfScope ps(s, std::string(bias_part ? "grad_reshape_bias_" : "grad_reshape_") + dt_name(h->dt) + ":wgrad",
                 0.0, 2.0 * h->es * (double)g.O * g.N);
    hipError_t e = launch_grad_reshape(h->dt, g, dy, G, bias_part, s);
    ps.done();
    return e;
}

// The bias gradient's partial sums only; their per-channel sums ride on the
// filter-gradient GEMM (a BiasSum with h->bias_splits parts).
hipError_t step_bias_partials(const d4r_conv *h, const void *dy, float *partial, hipStream_t s)
{
    const ConvGeom &g = h->g;
    ProfScope ps(s, std::string("bias_partial_") + dt_name(h->dt) + ":wgrad", 0.0,
                 (double)h->es * g.O * g.N + 4.0 * g.O * h->bias_splits);
    hipError_t e = launch_bias_partials(h->dt, g, dy, partial, h->bias_splits, s);
    ps.done();
    return e;
}

hipError_t step_bias(const d4r_conv *h, const void *dy, float *db, float *partial, hipStream_t s)
{
    const ConvGeom &g = h->g;
    ProfScope ps(s, std::string("bias_grad_") + dt_name(h->dt) + ":wgrad", 0.0,
                 (double)h->es * g.O * g.N + 4.0 * g.O);
    hipError_t e = launch_bias_grad(h->dt, g, dy, db, partial, h->bias_splits, s);
    ps.done();
    return e;
}

}  // namespace

extern "C" {

const char *d4r_status_string(d4r_status s)
{
    switch (s) {
    case D4R_OK: return "D4R_OK";
    case D4R_ERR_INVALID_ARG: return "D4R_ERR_INVALID_ARG";
    case D4R_ERR_UNSUPPORTED: return "D4R_ERR_UNSUPPORTED";
    case D4R_ERR_WORKSPACE: return "D4R_ERR_WORKSPACE";
    case D4R_ERR_LAUNCH: return "D4R_ERR_LAUNCH";
    case D4R_ERR_INTERNAL: return "D4R_ERR_INTERNAL";
    }
    return "unknown d4r_status";
}

const char *d4r_last_error(void) { return g_err; }

namespace {

// Experiment / test override: D4R_GRAD_PATH=inplace|copy (f32 only).
GradPath grad_path_env(GradPath dflt)
{
    const char *e = getenv("D4R_GRAD_PATH");
    if (!e)
        return dflt;
    if (!strcmp(e, "inplace"))
        return GP_INPLACE;
    if (!strcmp(e, "copy"))
        return GP_COPY;
    return dflt;
}

// The in-place loaders issue single-element loads where a copied operand
// takes 16-byte vectors, which costs a roughly fixed fraction of every GEMM
// stage; the copy costs one pass over dy.  The GEMM work per dy element is
// Kc multiply-adds, so the copy pays off for large Kc.  Measured on the
// full step: in place is 4% faster at Kc = 363 (AlexNet conv1), the copy 5%
// faster at Kc = 2304-3456 (conv3-5); the switch sits at Kc = 1024.
constexpr int kInplaceMaxKc = 1024;

void choose_grad_paths(d4r_conv *h)
{
    GradPath gp = GP_COPY;
    if (h->dt == D4R_F32) {
        gp = h->g.Kc < kInplaceMaxKc ? GP_INPLACE : GP_COPY;
        gp = grad_path_env(gp);
    }
    h->dgrad = gp;
    h->wgrad = gp;
    // With dy copied, a transposed copy of W (small next to dy) lets the
    // data-gradient GEMM read both operands k-contiguous: 1% faster per
    // step on AlexNet conv3-5 (f32 and bf16) than reading W row-contiguous.
    // D4R_DGRAD_WT=0|1 overrides (experiments, tests).
    h->dgrad_wt = h->dgrad == GP_COPY;
    if (const char *e = getenv("D4R_DGRAD_WT"))
        h->dgrad_wt = h->dgrad == GP_COPY && e[0] == '1';
}

}  // namespace

namespace {

// The output phases of a strided layer's data gradient (see PhaseArgs).  The
// phased form applies when every phase has taps and outputs (stride at most
// the kernel and the input extents), dy's channels fill whole GEMM stages,
// the NHWC loader's divisions stay in range, and (unless any_rows) the GEMM
// rows (the input channels) fill at least half a 128-row tile: with fewer
// (AlexNet conv1's 3) the explicit GEMM, whose rows are C*kH*kW, keeps the
// matrix cores busy, so the phased form runs there only when forced.
bool plan_phases(const ConvGeom &g, int dt, PhaseArgs *pa, bool any_rows)
{
    memset(pa, 0, sizeof *pa);
    const int s = g.s, bk = gemm_bk(dt);
    if (s < 2 || s * s > kMaxPhases || s > g.kH || s > g.kW || g.H < s || g.W < s || g.O % bk != 0 ||
        (g.C < 64 && !any_rows))
        return false;
    long long a_off = 0;
    int tiles = 0;
    for (int rh = 0; rh < s; ++rh)
        for (int rw = 0; rw < s; ++rw) {
            // per axis: taps t = ceil((k - r) / s), first output x0 with
            // (x0 + p) mod s = r, outputs m, offset q0 = (x0 + p - r) / s of
            // dy's window, padding t - 1 - q0 of the sub-convolution
            auto axis = [&](int r, int n, int k, int *t, int *x0, int *m, int *pad) {
                *t = (k - r + s - 1) / s;
                *x0 = ((r - g.p) % s + s) % s;
                *m = (n - *x0 + s - 1) / s;
                *pad = *t - 1 - (*x0 + g.p - r) / s;
            };
            int tu, h0, hm, ph, tv, w0, wm, pw;
            axis(rh, g.H, g.kH, &tu, &h0, &hm, &ph);
            axis(rw, g.W, g.kW, &tv, &w0, &wm, &pw);
            if (tu < 1 || tv < 1 || hm < 1 || wm < 1 || tu * tv > 1024)
                return false;
            PhaseItem &it = pa->ph[pa->n++];
            ConvGeom &q = it.g;
            q.B = g.B; q.C = g.O; q.H = g.OH; q.W = g.OW; q.O = g.C; q.kH = tu; q.kW = tv;
            q.s = 1; q.p = ph; q.pw = pw; q.OH = hm; q.OW = wm;
            q.P = hm * wm; q.Kc = g.O * tu * tv; q.N = g.B * q.P;
            if ((long long)q.Kc / bk >= (1 << 20) || (long long)q.N > 0x7fffffffLL)
                return false;
            it.a_off = a_off;
            it.K = q.Kc;
            it.tile0 = tiles;
            it.h0 = h0;
            it.w0 = w0;
            a_off += (long long)g.C * q.Kc;
            tiles += ((g.C + 127) / 128) * ((q.N + 127) / 128);
        }
    pa->tiles = tiles;
    return a_off == (long long)g.O * g.C * g.kH * g.kW;
}

}  // namespace

d4r_status d4r_conv_create(d4r_conv_t *out, int batch, int inC, int inH, int inW, int kH, int kW,
                           int stride, int padding, int outC, d4r_dtype dtype)
{
    if (!out)
        return fail(D4R_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (batch < 1 || inC < 1 || inH < 1 || inW < 1 || kH < 1 || kW < 1 || outC < 1)
        return fail(D4R_ERR_INVALID_ARG, "every size must be >= 1");
    if (stride < 1)
        return fail(D4R_ERR_INVALID_ARG, "stride must be >= 1");
    if (padding < 0)
        return fail(D4R_ERR_INVALID_ARG, "padding must be >= 0");
    if (!valid_dtype(dtype))
        return fail(D4R_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    long long span_h = (long long)inH + 2LL * padding - kH;
    long long span_w = (long long)inW + 2LL * padding - kW;
    if (span_h < 0 || span_w < 0)
        return fail(D4R_ERR_INVALID_ARG, "kernel larger than the padded input");
    long long OH = span_h / stride + 1, OW = span_w / stride + 1;
    long long P = OH * OW, Kc = (long long)inC * kH * kW, N = (long long)batch * P;
    long long x_el = (long long)batch * inC * inH * inW;
    long long y_el = (long long)outC * N;
    long long w_el = (long long)outC * Kc;
    long long col_el = Kc * N;
    if (x_el > kMaxElems || y_el > kMaxElems || w_el > kMaxElems || col_el > kMaxElems)
        return fail(D4R_ERR_UNSUPPORTED, "a tensor or the col matrix reaches 2^31 elements");

    d4r_conv *h = new (std::nothrow) d4r_conv;
    if (!h)
        return fail(D4R_ERR_INTERNAL, "host allocation failed");
    ConvGeom &g = h->g;
    g.B = batch; g.C = inC; g.H = inH; g.W = inW; g.O = outC; g.kH = kH; g.kW = kW;
    g.s = stride; g.p = padding; g.OH = (int)OH; g.OW = (int)OW;
    g.P = (int)P; g.Kc = (int)Kc; g.N = (int)N; g.pw = padding;
    h->dt = dtype;
    h->es = dt_size(dtype);
    h->fwd = plan_gemm(g.O, g.N, g.Kc, dtype);
    h->bwd_data = plan_gemm(g.Kc, g.N, g.O, dtype);
    // 16-bit filter gradient on the copied dy: two k-contiguous operands
    h->bwd_filter = plan_gemm(g.O, g.Kc, g.N, dtype, false,
                              dtype != D4R_F32 && g.N % 64 == 0 && g.Kc % 8 == 0);
    // For stride 1, dx[b,c,h,w] = sum_{o,u,v} W[o,c,u,v] dy[b,o,h+p-u,w+p-v]
    // is a stride-1 convolution of dy (O channels, OH x OW, padding kH-1-p)
    // with Wf[c,o,u,v] = W[o,c,kH-1-u,kW-1-v], whose output is exactly H x W.
    // One padding value serves both axes, so the kernel must be square.
    h->dgrad_impl = stride == 1 && kH == kW;
    if (h->dgrad_impl) {
        ConvGeom &d = h->gd;
        d.B = batch; d.C = outC; d.H = g.OH; d.W = g.OW; d.O = inC; d.kH = kH; d.kW = kW;
        d.s = 1; d.p = kH - 1 - padding; d.OH = inH; d.OW = inW;
        d.P = inH * inW; d.Kc = outC * kH * kW; d.N = batch * d.P; d.pw = d.p;
        h->bwd_data_impl = plan_gemm(d.O, d.N, d.Kc, dtype);
    }
    // the NHWC form needs whole GEMM stages of dy (32 f32 / 64 16-bit
    // channels) within one tap; the direct-to-LDS loader decodes a stage's
    // channel block and tap with small_div, exact for stage indices below
    // 2^20 and divisors (kH*kW, kW) <= 1024
    h->dgrad_nhwc = h->dgrad_impl && outC % gemm_bk(dtype) == 0 &&
                    (long long)h->gd.Kc / gemm_bk(dtype) < (1 << 20) && (long long)kH * kW <= 1024;
    if (const char *e = getenv("D4R_DGRAD_NHWC"))  // experiments, tests: 0 = gathered path
        h->dgrad_nhwc = h->dgrad_nhwc && e[0] != '0';
    if (h->dgrad_nhwc)
        h->bwd_data_nhwc = plan_gemm(h->gd.O, h->gd.N, h->gd.Kc, dtype, dtype != D4R_F32);
    {
        // experiments, tests: D4R_DGRAD_PHASED=0 keeps the explicit data
        // gradient; =force takes the phased one wherever it is correct,
        // whatever the input channel count
        const char *e = getenv("D4R_DGRAD_PHASED");
        const bool force = e && !strcmp(e, "force");
        h->dgrad_phased = plan_phases(g, dtype, &h->phases, force);
        if (e && e[0] == '0')
            h->dgrad_phased = false;
    }
    h->pointwise = kH == 1 && kW == 1 && stride == 1 && padding == 0;
    if (const char *e = getenv("D4R_POINTWISE"))  // experiments, tests: 0 = im2col path
        h->pointwise = h->pointwise && e[0] != '0';
    // the forward's NHWC form: the same loader conditions on x (inC channels)
    h->fwd_nhwc = stride == 1 && !h->pointwise && inC % gemm_bk(dtype) == 0 &&
                  (long long)g.Kc / gemm_bk(dtype) < (1 << 20) && (long long)kH * kW <= 1024;
    if (const char *e = getenv("D4R_FWD_NHWC"))  // experiments, tests: 0 = gathered implicit forward
        h->fwd_nhwc = h->fwd_nhwc && e[0] != '0';
    if (h->fwd_nhwc)
        h->fwd_nhwc_plan = plan_gemm(g.O, g.N, g.Kc, dtype, dtype != D4R_F32);
    h->bias_splits = bias_grad_splits(g);
    // bias partials: the bias kernel's splits, or the fused reshape's blocks
    const int bias_part_cols = std::max(h->bias_splits, grad_reshape_blocks(dtype, g));
    {
        // sum over output rows i of the taps u that land inside the image
        long long rows = 0, cols = 0;
        for (int i = 0; i < g.OH; ++i)
            for (int u = 0; u < kH; ++u) {
                int hh = i * stride - padding + u;
                rows += (hh >= 0 && hh < inH);
            }
        for (int j = 0; j < g.OW; ++j)
            for (int v = 0; v < kW; ++v) {
                int ww = j * stride - padding + v;
                cols += (ww >= 0 && ww < inW);
            }
        h->in_image_col = (double)batch * inC * (double)rows * (double)cols;
    }

    choose_grad_paths(h);
    h->fused_bwd = h->dgrad_nhwc && h->wgrad == GP_COPY && !h->pointwise;
    // One reshape pass over dy in place of the in-place loaders' single-
    // element gathers (or of two copies, transposed for the data gradient
    // and reshaped for the filter gradient).  Measured on AlexNet conv1 f32
    // (O = 96, batch 32): data-gradient GEMM 111 -> 88 us (W read through a
    // 5 us transposed copy; 97 us reading W row-contiguous), filter gradient
    // 80 -> 72 us, no separate 11 us bias pass, for one 19 us reshape: step
    // 0.416 -> 0.399 ms.  Layers with few output
    // channels (LeNet's 6 and 16) keep the in-place loaders: their GEMMs are
    // short and the step is launch-bound.  The 16-bit data gradient keeps its
    // transposed copy: with both operands k-contiguous it runs on the
    // direct-to-LDS kernel.  D4R_FUSED_EXPLICIT=0|1 overrides (experiments,
    // tests; 1 still needs an explicit f32 data gradient).
    {
        const bool fits = dtype == D4R_F32 && !h->dgrad_phased && !h->dgrad_impl && !h->pointwise;
        h->fused_explicit = fits && outC >= 32;
        if (const char *e = getenv("D4R_FUSED_EXPLICIT"))
            h->fused_explicit = fits && e[0] == '1';
        h->fx_wt = true;
        if (const char *e = getenv("D4R_FX_WT"))  // experiments, tests: 0 = W row-contiguous
            h->fx_wt = e[0] != '0';
    }
    h->col_bytes = (size_t)col_el * h->es;
    size_t off = align_up(h->col_bytes);
    h->off_g = off;
    if (h->dgrad != GP_INPLACE || h->wgrad != GP_INPLACE || h->fused_explicit)
        off += align_up((size_t)y_el * h->es);
    h->off_gt = off;
    if (h->dgrad_nhwc || h->dgrad_phased)
        off += align_up((size_t)y_el * h->es);
    h->off_wt = off;
    if (h->dgrad_wt || (h->fused_explicit && h->fx_wt))
        off += align_up((size_t)w_el * h->es);
    h->off_wflip = off;
    if (h->dgrad_impl || h->dgrad_phased)
        off += align_up((size_t)w_el * h->es);
    h->off_zero = off;
    if (h->dgrad_nhwc || h->fwd_nhwc || h->dgrad_phased)
        off += align_up(256);
    h->off_xt = off;
    h->off_wr = off;
    if (h->fwd_nhwc) {
        off += align_up((size_t)x_el * h->es);
        h->off_wr = off;
        off += align_up((size_t)w_el * h->es);
    }
    h->off_bias = off;
    off += align_up((size_t)outC * std::max(bias_part_cols, h->fused_bwd ? dy_prep_bias_parts(g) : 0) *
                    sizeof(float));
    h->off_big = off;
    size_t big = plan_partial_bytes(h->fwd, g.O, g.N);
    size_t dd = align_up((size_t)col_el * sizeof(float)) + plan_partial_bytes(h->bwd_data, g.Kc, g.N);
    if (dd > big)
        big = dd;
    size_t wf = plan_partial_bytes(h->bwd_filter, g.O, g.Kc);
    if (wf > big)
        big = wf;
    if (h->dgrad_impl) {
        size_t di = plan_partial_bytes(h->bwd_data_impl, h->gd.O, h->gd.N);
        if (di > big)
            big = di;
    }
    if (h->dgrad_nhwc) {
        size_t dn = plan_partial_bytes(h->bwd_data_nhwc, h->gd.O, h->gd.N);
        if (dn > big)
            big = dn;
    }
    if (h->fwd_nhwc) {
        size_t fn = plan_partial_bytes(h->fwd_nhwc_plan, g.O, g.N);
        if (fn > big)
            big = fn;
    }
    h->ws_bytes = off + align_up(big);
    *out = h;
    return ok();
}

d4r_status d4r_conv_destroy(d4r_conv_t h)
{
    delete h;
    return ok();
}

d4r_status d4r_conv_output_dims(d4r_conv_t h, int *outH, int *outW)
{
    if (!h || !outH || !outW)
        return fail(D4R_ERR_INVALID_ARG, "NULL argument");
    *outH = h->g.OH;
    *outW = h->g.OW;
    return ok();
}

d4r_status d4r_conv_workspace_size(d4r_conv_t h, size_t *bytes)
{
    if (!h || !bytes)
        return fail(D4R_ERR_INVALID_ARG, "NULL argument");
    *bytes = h->ws_bytes;
    return ok();
}

namespace {

std::string plan_text(const GemmPlan &pl)
{
    const TileShape ts = tile_shape(pl.cfg);
    return std::to_string(ts.bm) + "x" + std::to_string(ts.bn) + "/s" + std::to_string(pl.splits);
}

}  // namespace

d4r_status d4r_conv_describe(d4r_conv_t h, char *buf, size_t cap, size_t *needed)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    const ConvGeom &g = h->g;
    static const char *const im2col_kinds[] = {"gather", "lds", "shift"};
    static const char *const col2im_kinds[] = {"gather", "lds"};
    const Im2colPlan ip = plan_im2col(h->dt, g);
    const Col2imPlan cp = plan_col2im(g);
    std::string s = std::string("dtype=") + dt_name(h->dt) + " im2col=" + im2col_kinds[ip.kind] +
                    " im2col_rb=" + std::to_string(ip.RB) + " im2col_bb=" + std::to_string(ip.BB) +
                    " col2im=" + col2im_kinds[cp.kind] + " col2im_bb=" + std::to_string(cp.BB) +
                    " fwd=" + plan_text(h->fwd) + " dgrad_explicit=" + plan_text(h->bwd_data) +
                    " wgrad=" + plan_text(h->bwd_filter) +
                    " fwd_implicit=" + (h->pointwise ? "pointwise" : h->fwd_nhwc ? "nhwc" : "gathered") +
                    " dgrad_implicit=" + (h->dgrad_phased ? "phased" : h->pointwise ? "pointwise" :
                                          h->dgrad_nhwc ? "nhwc" : h->dgrad_impl ? "gathered" : "explicit");
    if (h->dgrad_phased)
        s += " dgrad_phases=" + std::to_string(h->phases.n);
    if (h->fwd_nhwc)
        s += " fwd_nhwc=" + plan_text(h->fwd_nhwc_plan);
    if (h->dgrad_nhwc)
        s += " dgrad_nhwc=" + plan_text(h->bwd_data_nhwc);
    else if (h->dgrad_impl)
        s += " dgrad_gathered=" + plan_text(h->bwd_data_impl);
    s += std::string(" dy_dgrad=") + (h->dgrad == GP_INPLACE ? "inplace" : "copy") +
         " dy_wgrad=" + (h->wgrad == GP_INPLACE ? "inplace" : "copy") + " dgrad_wt=" + (h->dgrad_wt ? "1" : "0") +
         " fused_backward=" + (h->fused_bwd ? "1" : h->fused_explicit ? "explicit" : "0") +
         (h->fused_explicit ? std::string(" fx_wt=") + (h->fx_wt ? "1" : "0") : std::string()) +
         " workspace=" + std::to_string(h->ws_bytes);
    if (needed)
        *needed = s.size() + 1;
    if (buf) {
        if (cap < s.size() + 1)
            return fail(D4R_ERR_INVALID_ARG, "buffer holds %zu bytes, the description needs %zu", cap, s.size() + 1);
        memcpy(buf, s.c_str(), s.size() + 1);
    }
    return ok();
}

namespace {

d4r_status check_tensor(const void *p, const char *name)
{
    if (!p)
        return fail(D4R_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned(p, 16))
        return fail(D4R_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
    return D4R_OK;
}

d4r_status check_vec(const void *p, const char *name)
{
    if (p && !aligned(p, 4))
        return fail(D4R_ERR_INVALID_ARG, "%s is not 4-byte aligned", name);
    return D4R_OK;
}

d4r_status check_ws(const d4r_conv *h, const void *ws, size_t ws_bytes)
{
    if (!ws)
        return fail(D4R_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", h->ws_bytes);
    if (!aligned(ws, kAlign))
        return fail(D4R_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
    if (ws_bytes < h->ws_bytes)
        return fail(D4R_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, h->ws_bytes);
    return D4R_OK;
}

d4r_status launched(hipError_t e, const char *what)
{
    if (e != hipSuccess)
        return fail(D4R_ERR_LAUNCH, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

#define D4R_TRY(x)                   \
    do {                             \
        d4r_status st_ = (x);        \
        if (st_ != D4R_OK)           \
            return st_;              \
    } while (0)

#define D4R_LAUNCH(call, what)                       \
    do {                                             \
        hipError_t e_ = (call);                      \
        if (e_ != hipSuccess)                        \
            return launched(e_, what);               \
    } while (0)

}  // namespace

namespace {

// The forward in both forms: im2col + GEMM (col left at the start of ws) or
// the implicit GEMM (1x1 convolutions read x in place); the GEMM's epilogue
// adds the bias and, with relu, applies ReLU before storing y.
d4r_status conv_forward(d4r_conv_t h, const void *x, const void *w, const float *bias, float *y,
                        void *ws, size_t ws_bytes, void *hip_stream, bool implicit, int relu)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(w, "w"));
    D4R_TRY(check_tensor(y, "y"));
    D4R_TRY(check_vec(bias, "bias"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    hipStream_t s = (hipStream_t)hip_stream;
    const ConvGeom &g = h->g;
    float *partial = (float *)((char *)ws + h->off_big);
    if (!implicit) {
        void *col = ws;
        D4R_LAUNCH(step_im2col(h, x, col, s, "fwd"), "im2col");
        D4R_LAUNCH(run_gemm(h->dt, h->fwd, OP_KC, OP_ROWS, w, g.Kc, col, g.N, g.O, g.N, g.Kc, EPI_NCHW, y,
                            0, bias, g.P, partial, s, "fwd", nullptr, 0, 0, nullptr, relu),
                   "forward GEMM");
    } else if (h->fwd_nhwc) {
        // y = Wr(O x kH*kW*C) * im2col(x as NHWC): one launch transposes x to
        // xt[b][pix][c] and reorders the filter to wr[o][cb][u][v][ci], the
        // loader's k order (clearing the zero page it reads for padding)
        char *wsb = (char *)ws;
        void *xt = wsb + h->off_xt, *wr = wsb + h->off_wr, *zero = wsb + h->off_zero;
        {
            ProfScope ps(s, std::string("transpose_") + dt_name(h->dt) + ":fwd_x_w", 0.0,
                         2.0 * h->es * ((double)g.B * g.C * g.H * g.W + (double)g.O * g.Kc));
            const TransposeJob jx{x, xt, g.C, g.H * g.W, g.B, (uint32_t *)zero, 0};
            const FilterJob jw{w, wr, g.O, g.C, g.kH * g.kW, gemm_bk(h->dt), 0, nullptr, 0};
            hipError_t e = launch_transpose_filter(h->dt, jx, jw, s);
            ps.done();
            D4R_LAUNCH(e, "input transpose and filter reorder");
        }
        D4R_LAUNCH(run_gemm(h->dt, h->fwd_nhwc_plan, OP_KC, OP_IMPL_T, wr, g.Kc, xt, 0, g.O, g.N, g.Kc, EPI_NCHW,
                            y, 0, bias, g.P, partial, s, "fwd", &g, 0, 0, zero, relu),
                   "implicit forward GEMM (NHWC)");
    } else if (h->pointwise) {
        // 1x1: y[b] = Wmat * x[b] with x read in place (C channels)
        D4R_LAUNCH(run_gemm(h->dt, h->fwd, OP_KC, OP_NCHW, w, g.Kc, x, 0, g.O, g.N, g.Kc, EPI_NCHW, y, 0,
                            bias, g.P, partial, s, "fwd", &g, 0, g.C, nullptr, relu),
                   "pointwise forward GEMM");
    } else {
        D4R_LAUNCH(run_gemm(h->dt, h->fwd, OP_KC, OP_IMPL, w, g.Kc, x, 0, g.O, g.N, g.Kc, EPI_NCHW, y, 0,
                            bias, g.P, partial, s, "fwd", &g, 0, 0, nullptr, relu),
                   "implicit forward GEMM");
    }
    return ok();
}

}  // namespace

d4r_status d4r_conv_forward(d4r_conv_t h, const void *x, const void *w, const float *bias, float *y,
                            void *ws, size_t ws_bytes, void *hip_stream)
{
    return conv_forward(h, x, w, bias, y, ws, ws_bytes, hip_stream, false, 0);
}

d4r_status d4r_conv_forward_implicit(d4r_conv_t h, const void *x, const void *w, const float *bias,
                                     float *y, void *ws, size_t ws_bytes, void *hip_stream)
{
    return conv_forward(h, x, w, bias, y, ws, ws_bytes, hip_stream, true, 0);
}

d4r_status d4r_conv_forward_ex(d4r_conv_t h, const void *x, const void *w, const float *bias, float *y,
                               int flags, void *ws, size_t ws_bytes, void *hip_stream)
{
    if (flags & ~(D4R_FWD_RELU | D4R_FWD_IMPLICIT))
        return fail(D4R_ERR_INVALID_ARG, "flags %d has bits outside D4R_FWD_RELU | D4R_FWD_IMPLICIT", flags);
    return conv_forward(h, x, w, bias, y, ws, ws_bytes, hip_stream, (flags & D4R_FWD_IMPLICIT) != 0,
                        (flags & D4R_FWD_RELU) ? 1 : 0);
}

namespace {

// dx = col2im(Wmat^T * G): the page's data gradient.  wt, when given, is
// the caller's packed filter Wt[kc][o] = W[o][kc] (d4r_conv_pack_filter),
// read k-contiguous; otherwise W is read row-contiguous or transposed here.
d4r_status dgrad_explicit(d4r_conv_t h, const void *w, const void *wt_packed, const void *dy, float *dx,
                          void *ws, hipStream_t s)
{
    const ConvGeom &g = h->g;
    char *wsb = (char *)ws;
    const void *a = wt_packed ? wt_packed : w;
    const int amode = wt_packed ? OP_KC : OP_ROWS;
    const int lda = wt_packed ? g.O : g.Kc;
    if (h->pointwise) {
        // 1x1: dx[b] = Wmat^T * dy[b], stored NCHW by the GEMM (dcol is dx)
        D4R_LAUNCH(run_gemm(h->dt, h->bwd_data, amode, OP_NCHW, a, lda, dy, 0, g.Kc, g.N, g.O, EPI_NCHW, dx, 0,
                            nullptr, g.P, (float *)(wsb + h->off_big), s, "dgrad", &g, 0, g.O),
                   "pointwise data-gradient GEMM");
        return ok();
    }
    float *dcol = (float *)(wsb + h->off_big);
    float *partial = (float *)(wsb + h->off_big + align_up((size_t)g.Kc * g.N * sizeof(float)));
    // dcol = Wmat^T * G with A = Wmat (O x Kc) read row-contiguous as
    // op(A) = Wmat^T (or its packed transpose) and B = G (O x N) read from
    // dy in place or from its transpose Gt[b*P + pix][o] = dy[b][o][pix]
    if (h->dgrad == GP_INPLACE) {
        D4R_LAUNCH(run_gemm(h->dt, h->bwd_data, amode, OP_NCHW, a, lda, dy, 0, g.Kc, g.N, g.O,
                            EPI_ROWMAJOR, dcol, g.N, nullptr, 0, partial, s, "dgrad", &g),
                   "data-gradient GEMM");
    } else {
        void *gt = wsb + h->off_g;
        D4R_LAUNCH(step_transpose(h, g.B, g.O, g.P, dy, gt, s, "dgrad_dy"), "grad transpose");
        const void *aa = a;
        int am = amode, ld = lda;
        if (!wt_packed && h->dgrad_wt) {
            // Wt[kc][o] = W[o][kc]
            void *wt = wsb + h->off_wt;
            D4R_LAUNCH(step_transpose(h, 1, g.O, g.Kc, w, wt, s, "dgrad_w"), "filter transpose");
            aa = wt;
            am = OP_KC;
            ld = g.O;
        }
        D4R_LAUNCH(run_gemm(h->dt, h->bwd_data, am, OP_KC, aa, ld, gt, g.O, g.Kc, g.N, g.O,
                            EPI_ROWMAJOR, dcol, g.N, nullptr, 0, partial, s, "dgrad"),
                   "data-gradient GEMM");
    }
    D4R_LAUNCH(step_col2im(h, dcol, dx, s, "dgrad"), "col2im");
    return ok();
}

// dx of a strided layer without dcol or col2im: dy transposed to NHWC
// (zero page cleared in the same launch), the phase filters gathered from
// W, then one GEMM launch over every output phase, each storing its rows and
// columns of dx.
d4r_status dgrad_phased(d4r_conv_t h, const void *w, const void *dy, float *dx, void *ws, hipStream_t s)
{
    const ConvGeom &g = h->g;
    char *wsb = (char *)ws;
    void *gt = wsb + h->off_gt, *wph = wsb + h->off_wflip, *zero = wsb + h->off_zero;
    {
        ProfScope ps(s, std::string("transpose_") + dt_name(h->dt) + ":dgrad_dy", 0.0,
                     2.0 * h->es * (double)g.B * g.O * g.P);
        const TransposeJob jdy{dy, gt, g.O, g.P, g.B, (uint32_t *)zero, 0};
        const FilterJob none{nullptr, nullptr, 0, 0, 0, 1, 0, nullptr, 0};
        hipError_t e = launch_transpose_filter(h->dt, jdy, none, s);
        ps.done();
        D4R_LAUNCH(e, "grad transpose");
    }
    {
        ProfScope ps(s, std::string("phase_filter_") + dt_name(h->dt) + ":dgrad", 0.0,
                     2.0 * h->es * (double)g.O * g.Kc);
        hipError_t e = launch_phase_filter(h->dt, g, h->phases, w, wph, s);
        ps.done();
        D4R_LAUNCH(e, "phase filters");
    }
    GemmParams p;
    memset(&p, 0, sizeof p);
    p.A = wph;
    p.B = gt;
    p.C = dx;
    p.M = g.C;
    p.epi = EPI_PHASE;
    p.splits = 1;
    p.a_vec = 1;
    p.b_vec = 1;
    p.zero = zero;
    p.ph_s = g.s;
    p.ph_H = g.H;
    p.ph_W = g.W;
    double flops = 0.0;
    for (int k = 0; k < h->phases.n; ++k)
        flops += 2.0 * g.C * (double)h->phases.ph[k].g.N * h->phases.ph[k].K;
    ProfScope ps(s, std::string("gemm_") + dt_name(h->dt) + "_128x128_kn_phased:dgrad", flops,
                 (double)h->es * ((double)g.O * g.Kc + (double)g.B * g.O * g.P) +
                     4.0 * (double)g.B * g.C * g.H * g.W);
    hipError_t e = launch_gemm_phased(h->dt, p, h->phases, s);
    ps.done();
    D4R_LAUNCH(e, "phased data-gradient GEMM");
    return ok();
}

}  // namespace

d4r_status d4r_conv_backward_data(d4r_conv_t h, const void *w, const void *dy, float *dx, void *ws,
                                  size_t ws_bytes, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(w, "w"));
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(dx, "dx"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    return dgrad_explicit(h, w, nullptr, dy, dx, ws, (hipStream_t)hip_stream);
}

d4r_status d4r_conv_packed_filter_size(d4r_conv_t h, size_t *bytes)
{
    if (!h || !bytes)
        return fail(D4R_ERR_INVALID_ARG, "NULL argument");
    *bytes = (size_t)h->g.O * h->g.Kc * h->es;
    return ok();
}

d4r_status d4r_conv_pack_filter(d4r_conv_t h, const void *w, void *wp, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(w, "w"));
    D4R_TRY(check_tensor(wp, "wp"));
    const size_t bytes = (size_t)h->g.O * h->g.Kc * h->es;
    const char *a = (const char *)w, *b = (const char *)wp;
    if (a < b + bytes && b < a + bytes)
        return fail(D4R_ERR_INVALID_ARG, "wp overlaps w");
    D4R_LAUNCH(step_transpose(h, 1, h->g.O, h->g.Kc, w, wp, (hipStream_t)hip_stream, "pack_w"),
               "filter pack");
    return ok();
}

d4r_status d4r_conv_backward_data_packed(d4r_conv_t h, const void *wp, const void *dy, float *dx, void *ws,
                                         size_t ws_bytes, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(wp, "wp"));
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(dx, "dx"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    return dgrad_explicit(h, nullptr, wp, dy, dx, ws, (hipStream_t)hip_stream);
}

d4r_status d4r_conv_backward_data_implicit(d4r_conv_t h, const void *w, const void *dy, float *dx,
                                           void *ws, size_t ws_bytes, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(w, "w"));
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(dx, "dx"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    hipStream_t s = (hipStream_t)hip_stream;
    if (h->dgrad_phased)
        return dgrad_phased(h, w, dy, dx, ws, s);
    if (!h->dgrad_impl || h->pointwise)
        return dgrad_explicit(h, w, nullptr, dy, dx, ws, s);
    const ConvGeom &g = h->g, &d = h->gd;
    char *wsb = (char *)ws;
    void *wf = wsb + h->off_wflip;
    float *partial = (float *)(wsb + h->off_big);
    if (h->dgrad_nhwc) {
        // dx = Wd(C x kH*kW*O) * im2col(dy as NHWC): dy transposed to
        // Gt[b][pix][o], the filter flipped with k ordered (channel block,
        // u, v, channel)
        void *gt = wsb + h->off_gt;
        void *zero = wsb + h->off_zero;
        {
            // one launch: dy -> Gt per image, and the filter (O x C*kH*kW)
            // transposed with its taps reversed, clearing the zero page
            ProfScope ps(s, std::string("transpose_") + dt_name(h->dt) + ":dgrad_dy_w", 0.0,
                         2.0 * h->es * ((double)g.B * g.O * g.P + (double)g.O * g.Kc));
            const TransposeJob jdy{dy, gt, g.O, g.P, g.B, nullptr, 0};
            const FilterJob jw{w, wf, g.O, g.C, g.kH * g.kW, gemm_bk(h->dt), 1, (uint32_t *)zero, 0};
            hipError_t e = launch_transpose_filter(h->dt, jdy, jw, s);
            ps.done();
            D4R_LAUNCH(e, "grad transpose and filter flip");
        }
        D4R_LAUNCH(run_gemm(h->dt, h->bwd_data_nhwc, OP_KC, OP_IMPL_T, wf, d.Kc, gt, 0, d.O, d.N, d.Kc,
                            EPI_NCHW, dx, 0, nullptr, d.P, partial, s, "dgrad", &d, 0, 0, zero),
                   "implicit data-gradient GEMM");
        return ok();
    }
    {
        ProfScope ps(s, std::string("flip_filter_") + dt_name(h->dt) + ":dgrad", 0.0,
                     2.0 * h->es * (double)g.O * g.Kc);
        hipError_t e = launch_flip_filter(h->dt, g, w, wf, s);
        ps.done();
        D4R_LAUNCH(e, "filter flip");
    }
    // dx = Wf(C x O*kH*kW) * im2col_d(dy), NCHW epilogue over the H x W map
    D4R_LAUNCH(run_gemm(h->dt, h->bwd_data_impl, OP_KC, OP_IMPL, wf, d.Kc, dy, 0, d.O, d.N, d.Kc, EPI_NCHW,
                        dx, 0, nullptr, d.P, partial, s, "dgrad", &d),
               "implicit data-gradient GEMM");
    return ok();
}

d4r_status d4r_conv_backward_filter(d4r_conv_t h, const void *x, const void *dy, float *dw, float *db,
                                    int reuse_col, void *ws, size_t ws_bytes, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    if (reuse_col != 0 && reuse_col != 1)
        return fail(D4R_ERR_INVALID_ARG, "reuse_col must be 0 or 1");
    if (reuse_col && x)
        return fail(D4R_ERR_INVALID_ARG, "x must be NULL when reuse_col = 1");
    if (!reuse_col)
        D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(dw, "dw"));
    D4R_TRY(check_vec(db, "db"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    hipStream_t s = (hipStream_t)hip_stream;
    const ConvGeom &g = h->g;
    char *wsb = (char *)ws;
    void *col = wsb;
    float *partial = (float *)(wsb + h->off_big);
    // dy read in place by the GEMM: the bias partials first, their sums
    // with the GEMM's split-K reduction (or right after it)
    float *bias_part = (float *)(wsb + h->off_bias);
    const BiasSum bsum{bias_part, db, g.O, h->bias_splits};
    if (h->pointwise && !reuse_col) {
        // 1x1: dW = sum_b dy[b] * x[b]^T with dy and x read in place
        if (db)
            D4R_LAUNCH(step_bias_partials(h, dy, bias_part, s), "bias gradient");
        D4R_LAUNCH(run_gemm(h->dt, h->bwd_filter, OP_NCHW, OP_NCHW_K, dy, 0, x, 0, g.O, g.Kc, g.N,
                            EPI_ROWMAJOR, dw, g.Kc, nullptr, 0, partial, s, "wgrad", &g, g.O, g.C, nullptr, 0,
                            db ? &bsum : nullptr),
                   "pointwise filter-gradient GEMM");
        return ok();
    }
    if (!reuse_col)
        D4R_LAUNCH(step_im2col(h, x, col, s, "wgrad"), "im2col");
    // dW = G * col^T: A = G (O x N), read from dy in place or reshaped;
    // B = col (Kc x N) read k-contiguous as op(B) = col^T
    if (h->wgrad == GP_INPLACE) {
        if (db)
            D4R_LAUNCH(step_bias_partials(h, dy, bias_part, s), "bias gradient");
        D4R_LAUNCH(run_gemm(h->dt, h->bwd_filter, OP_NCHW, OP_KC, dy, 0, col, g.N, g.O, g.Kc, g.N,
                            EPI_ROWMAJOR, dw, g.Kc, nullptr, 0, partial, s, "wgrad", &g, 0, 0, nullptr, 0,
                            db ? &bsum : nullptr),
                   "filter-gradient GEMM");
        return ok();
    }
    // the reshape's pass over dy also yields the bias partial sums
    void *G = wsb + h->off_g;
    D4R_LAUNCH(step_grad_reshape(h, dy, G, db ? bias_part : nullptr, s), "grad reshape");
    // the bias sum rides on the GEMM's split-K reduction (or follows it)
    const BiasSum bs{bias_part, db, g.O, grad_reshape_blocks(h->dt, g)};
    D4R_LAUNCH(run_gemm(h->dt, h->bwd_filter, OP_KC, OP_KC, G, g.N, col, g.N, g.O, g.Kc, g.N, EPI_ROWMAJOR, dw,
                        g.Kc, nullptr, 0, partial, s, "wgrad", nullptr, 0, 0, nullptr, 0, db ? &bs : nullptr),
               "filter-gradient GEMM and bias gradient");
    return ok();
}

namespace {

// The page's data gradient (dcol = Wmat^T * G, then col2im) and filter
// gradient (dW = G * col^T) of one layer from one pass over dy: the reshape
// writes G (O x N, the batch folded into the columns) and the bias partial
// sums; the data-gradient GEMM reads G row-contiguous, the filter-gradient
// GEMM k-contiguous.  Results equal the separate calls' up to the order of
// the f32 sums.
d4r_status backward_explicit_fused(d4r_conv_t h, const void *x, const void *w, const void *dy, float *dx,
                                   float *dw, float *db, int reuse_col, void *ws, hipStream_t s)
{
    const ConvGeom &g = h->g;
    char *wsb = (char *)ws;
    void *col = wsb;
    void *G = wsb + h->off_g;
    float *bias_part = db ? (float *)(wsb + h->off_bias) : nullptr;
    float *dcol = (float *)(wsb + h->off_big);
    float *partial = (float *)(wsb + h->off_big + align_up((size_t)g.Kc * g.N * sizeof(float)));
    D4R_LAUNCH(step_grad_reshape(h, dy, G, bias_part, s), "grad reshape");
    const void *a = w;
    int am = OP_ROWS, lda = g.Kc;
    if (h->fx_wt) {
        // Wt[kc][o] = W[o][kc]
        void *wt = wsb + h->off_wt;
        D4R_LAUNCH(step_transpose(h, 1, g.O, g.Kc, w, wt, s, "dgrad_w"), "filter transpose");
        a = wt;
        am = OP_KC;
        lda = g.O;
    }
    D4R_LAUNCH(run_gemm(h->dt, h->bwd_data, am, OP_ROWS, a, lda, G, g.N, g.Kc, g.N, g.O, EPI_ROWMAJOR, dcol,
                        g.N, nullptr, 0, partial, s, "dgrad"),
               "data-gradient GEMM");
    D4R_LAUNCH(step_col2im(h, dcol, dx, s, "dgrad"), "col2im");
    if (!reuse_col)
        D4R_LAUNCH(step_im2col(h, x, col, s, "wgrad"), "im2col");
    partial = (float *)(wsb + h->off_big);
    const BiasSum bs{bias_part, db, g.O, grad_reshape_blocks(h->dt, g)};
    D4R_LAUNCH(run_gemm(h->dt, h->bwd_filter, OP_KC, OP_KC, G, g.N, col, g.N, g.O, g.Kc, g.N, EPI_ROWMAJOR, dw,
                        g.Kc, nullptr, 0, partial, s, "wgrad", nullptr, 0, 0, nullptr, 0, db ? &bs : nullptr),
               "filter-gradient GEMM and bias gradient");
    return ok();
}

}  // namespace

d4r_status d4r_conv_backward(d4r_conv_t h, const void *x, const void *w, const void *dy, float *dx, float *dw,
                             float *db, int reuse_col, void *ws, size_t ws_bytes, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    if (reuse_col != 0 && reuse_col != 1)
        return fail(D4R_ERR_INVALID_ARG, "reuse_col must be 0 or 1");
    if (reuse_col && x)
        return fail(D4R_ERR_INVALID_ARG, "x must be NULL when reuse_col = 1");
    if (!reuse_col)
        D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(w, "w"));
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(dx, "dx"));
    D4R_TRY(check_tensor(dw, "dw"));
    D4R_TRY(check_vec(db, "db"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    if (h->fused_explicit)
        return backward_explicit_fused(h, x, w, dy, dx, dw, db, reuse_col, ws, (hipStream_t)hip_stream);
    if (!h->fused_bwd) {
        // the two calls in sequence (the data gradient leaves col intact)
        d4r_status st = d4r_conv_backward_data_implicit(h, w, dy, dx, ws, ws_bytes, hip_stream);
        if (st != D4R_OK)
            return st;
        return d4r_conv_backward_filter(h, x, dy, dw, db, reuse_col, ws, ws_bytes, hip_stream);
    }
    hipStream_t s = (hipStream_t)hip_stream;
    const ConvGeom &g = h->g, &d = h->gd;
    char *wsb = (char *)ws;
    void *col = wsb;
    void *G = wsb + h->off_g;
    void *gt = wsb + h->off_gt;
    void *wf = wsb + h->off_wflip;
    void *zero = wsb + h->off_zero;
    float *bias_part = db ? (float *)(wsb + h->off_bias) : nullptr;
    float *partial = (float *)(wsb + h->off_big);
    {
        // one pass over dy: G, Gt and the bias partial sums; the flipped
        // filter and the zero page in the same launch
        ProfScope ps(s, std::string("dy_prep_") + dt_name(h->dt) + ":bwd", 0.0,
                     3.0 * h->es * (double)g.B * g.O * g.P + 2.0 * h->es * (double)g.O * g.Kc);
        const DyPrep a{dy, gt, G, bias_part, g.B, g.O, g.P, 0, 0};
        const FilterJob jw{w, wf, g.O, g.C, g.kH * g.kW, gemm_bk(h->dt), 1, (uint32_t *)zero, 0};
        hipError_t e = launch_dy_prep(h->dt, a, jw, s);
        ps.done();
        D4R_LAUNCH(e, "dy preparation");
    }
    D4R_LAUNCH(run_gemm(h->dt, h->bwd_data_nhwc, OP_KC, OP_IMPL_T, wf, d.Kc, gt, 0, d.O, d.N, d.Kc, EPI_NCHW,
                        dx, 0, nullptr, d.P, partial, s, "dgrad", &d, 0, 0, zero),
               "implicit data-gradient GEMM");
    if (!reuse_col)
        D4R_LAUNCH(step_im2col(h, x, col, s, "wgrad"), "im2col");
    const BiasSum bs{bias_part, db, g.O, dy_prep_bias_parts(g)};
    D4R_LAUNCH(run_gemm(h->dt, h->bwd_filter, OP_KC, OP_KC, G, g.N, col, g.N, g.O, g.Kc, g.N, EPI_ROWMAJOR, dw,
                        g.Kc, nullptr, 0, partial, s, "wgrad", nullptr, 0, 0, nullptr, 0, db ? &bs : nullptr),
               "filter-gradient GEMM and bias gradient");
    return ok();
}

d4r_status d4r_conv_im2col(d4r_conv_t h, const void *x, void *col, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(col, "col"));
    D4R_LAUNCH(step_im2col(h, x, col, (hipStream_t)hip_stream, "step"), "im2col");
    return ok();
}

d4r_status d4r_conv_col2im(d4r_conv_t h, const float *dcol, float *dx, void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(dcol, "dcol"));
    D4R_TRY(check_tensor(dx, "dx"));
    D4R_LAUNCH(step_col2im(h, dcol, dx, (hipStream_t)hip_stream, "step"), "col2im");
    return ok();
}

d4r_status d4r_conv_bias_grad(d4r_conv_t h, const void *dy, float *db, void *ws, size_t ws_bytes,
                              void *hip_stream)
{
    if (!h)
        return fail(D4R_ERR_INVALID_ARG, "handle is NULL");
    D4R_TRY(check_tensor(dy, "dy"));
    if (!db)
        return fail(D4R_ERR_INVALID_ARG, "db is NULL");
    D4R_TRY(check_vec(db, "db"));
    D4R_TRY(check_ws(h, ws, ws_bytes));
    D4R_LAUNCH(step_bias(h, dy, db, (float *)((char *)ws + h->off_bias), (hipStream_t)hip_stream),
               "bias gradient");
    return ok();
}

namespace {

d4r_status check_gemm_args(int M, int K, int N, int flags, int dtype)
{
    if (M < 1 || K < 1 || N < 1)
        return fail(D4R_ERR_INVALID_ARG, "M, K and N must be >= 1");
    if (flags < 0 || flags > 3)
        return fail(D4R_ERR_INVALID_ARG, "flags must be 0..3");
    if (!valid_dtype(dtype))
        return fail(D4R_ERR_INVALID_ARG, "unknown dtype %d", dtype);
    if ((long long)M * K > kMaxElems || (long long)K * N > kMaxElems || (long long)M * N > kMaxElems)
        return fail(D4R_ERR_UNSUPPORTED, "an operand reaches 2^31 elements");
    return D4R_OK;
}

}  // namespace

d4r_status d4r_gemm_workspace_size(int M, int K, int N, int flags, d4r_dtype dtype, size_t *bytes)
{
    D4R_TRY(check_gemm_args(M, K, N, flags, dtype));
    if (!bytes)
        return fail(D4R_ERR_INVALID_ARG, "bytes is NULL");
    GemmPlan pl = plan_gemm(M, N, K, dtype, false, gemm_kk16(K, flags, dtype));
    *bytes = plan_partial_bytes(pl, M, N);
    return ok();
}

namespace {

d4r_status gemm_call(const char *what, int M, int K, int N, int flags, d4r_dtype dtype, const void *A,
                     const void *B, const float *bias, int relu, float *C, void *ws, size_t ws_bytes,
                     void *hip_stream)
{
    D4R_TRY(check_gemm_args(M, K, N, flags, dtype));
    D4R_TRY(check_tensor(A, "A"));
    D4R_TRY(check_tensor(B, "B"));
    D4R_TRY(check_tensor(C, "C"));
    GemmPlan pl = plan_gemm(M, N, K, dtype, false, gemm_kk16(K, flags, dtype));
    size_t need = plan_partial_bytes(pl, M, N);
    if (need) {
        if (!ws)
            return fail(D4R_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
        if (!aligned(ws, kAlign))
            return fail(D4R_ERR_INVALID_ARG, "workspace is not 256-byte aligned");
        if (ws_bytes < need)
            return fail(D4R_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
    }
    // flags bit 0: A stored K x M (op(A) = A^T, read row-contiguous);
    // bit 1: B stored N x K (op(B) = B^T, read k-contiguous)
    const int amode = (flags & 1) ? OP_ROWS : OP_KC;
    const int bmode = (flags & 2) ? OP_KC : OP_ROWS;
    const int lda = amode == OP_KC ? K : M;
    const int ldb = bmode == OP_KC ? K : N;
    D4R_LAUNCH(run_gemm(dtype, pl, amode, bmode, A, lda, B, ldb, M, N, K, EPI_ROWMAJOR, C, N, bias, 0,
                        (float *)ws, (hipStream_t)hip_stream, what, nullptr, 0, 0, nullptr, relu),
               "GEMM");
    return ok();
}

}  // namespace

d4r_status d4r_gemm(int M, int K, int N, int flags, d4r_dtype dtype, const void *A, const void *B,
                    float *C, void *ws, size_t ws_bytes, void *hip_stream)
{
    return gemm_call("gemm", M, K, N, flags, dtype, A, B, nullptr, 0, C, ws, ws_bytes, hip_stream);
}

// ---------------------------------------------------------------------------
// d4r_gemm without a workspace argument: the split-K partial sums go to a
// file-scope device array the library owns, so the call allocates nothing.
// Each device holds its own copy of the array (from when the library's code
// object is loaded on it until the process ends); host code only ever uses
// the device address hipGetSymbolAddress returns for the current device,
// never the array's name, which on the host is a stand-in symbol.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The scratch array's address on the current device, looked up once per
// device (with that device current) and cached.
d4r_status scratch_on_current_device(void **out)
{
    int devc = -1;
    hipError_t e = hipGetDevice(&devc);
    if (e != hipSuccess)
        return fail(D4R_ERR_LAUNCH, "hipGetDevice: %s", hipGetErrorString(e));
    if (devc < 0 || devc >= kMaxDevices)
        return fail(D4R_ERR_UNSUPPORTED, "device %d is beyond the %d devices the scratch table covers", devc,
                    kMaxDevices);
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[devc]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return fail(D4R_ERR_LAUNCH, "hipGetSymbolAddress(scratch) on device %d: %s", devc,
                        hipGetErrorString(e));
        g_scratch_ptr[devc] = p;
    }
    *out = g_scratch_ptr[devc];
    return D4R_OK;
}

}  // namespace

size_t d4r_gemm_noalloc_scratch_bytes(void) { return kScratchBytes; }

d4r_status d4r_gemm_noalloc(int M, int K, int N, int flags, d4r_dtype dtype, const void *A, const void *B,
                            float *C, void *hip_stream)
{
    D4R_TRY(check_gemm_args(M, K, N, flags, dtype));
    D4R_TRY(check_tensor(A, "A"));
    D4R_TRY(check_tensor(B, "B"));
    D4R_TRY(check_tensor(C, "C"));
    // the same plan as d4r_gemm, so the result is the same bit for bit
    const GemmPlan pl = plan_gemm(M, N, K, dtype, false, gemm_kk16(K, flags, dtype));
    const size_t need = plan_partial_bytes(pl, M, N);
    if (need > kScratchBytes)
        return fail(D4R_ERR_UNSUPPORTED,
                    "this GEMM needs %zu bytes of split-K scratch; d4r_gemm_noalloc holds %zu (use d4r_gemm "
                    "with a workspace)",
                    need, kScratchBytes);
    void *ws = nullptr;
    if (need)
        D4R_TRY(scratch_on_current_device(&ws));
    const int amode = (flags & 1) ? OP_ROWS : OP_KC;
    const int bmode = (flags & 2) ? OP_KC : OP_ROWS;
    const int lda = amode == OP_KC ? K : M;
    const int ldb = bmode == OP_KC ? K : N;
    D4R_LAUNCH(run_gemm(dtype, pl, amode, bmode, A, lda, B, ldb, M, N, K, EPI_ROWMAJOR, C, N, nullptr, 0,
                        (float *)ws, (hipStream_t)hip_stream, "gemm_noalloc"),
               "GEMM");
    return ok();
}

d4r_status d4r_gemm_bias_act(int M, int K, int N, int flags, d4r_dtype dtype, const void *A, const void *B,
                             const float *bias, int relu, float *C, void *ws, size_t ws_bytes,
                             void *hip_stream)
{
    D4R_TRY(check_vec(bias, "bias"));
    return gemm_call("gemm_bias", M, K, N, flags, dtype, A, B, bias, relu ? 1 : 0, C, ws, ws_bytes,
                     hip_stream);
}

/* ---- the rest of a training step (f32) ---- */

namespace {

d4r_status check_count(long long n, const char *name)
{
    if (n < 0)
        return fail(D4R_ERR_INVALID_ARG, "%s = %lld is negative", name, n);
    return D4R_OK;
}

// Profiled launch of one training-step kernel: name, algorithmic bytes
extern "C++" template <class F>
d4r_status run_step(hipStream_t s, const char *name, double bytes, const char *what, F &&launch)
{
    ProfScope ps(s, name, 0.0, bytes);
    hipError_t e = launch();
    ps.done();
    if (e != hipSuccess)
        return launched(e, what);
    return ok();
}

}  // namespace

d4r_status d4r_relu_forward(const float *x, float *y, long long n, void *hip_stream)
{
    D4R_TRY(check_count(n, "n"));
    if (n == 0)
        return ok();
    D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(y, "y"));
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "relu_fwd", 8.0 * n, "ReLU", [&] { return launch_relu_forward(x, y, n, s); });
}

d4r_status d4r_relu_backward(const float *x, const float *dy, float *dx, long long n, void *hip_stream)
{
    D4R_TRY(check_count(n, "n"));
    if (n == 0)
        return ok();
    D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(dx, "dx"));
    if (dx == x && dx != dy)
        return fail(D4R_ERR_INVALID_ARG, "dx may be dy but not x");
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "relu_bwd", 12.0 * n, "ReLU gradient",
                    [&] { return launch_relu_backward(x, dy, dx, n, s); });
}

namespace {

d4r_status check_pool(int batch, int channels, int H, int W, int k, int stride, long long *planes, int *OH,
                      int *OW)
{
    if (batch < 0 || channels < 0)
        return fail(D4R_ERR_INVALID_ARG, "batch = %d, channels = %d must be >= 0", batch, channels);
    if (k < 1 || stride < 1)
        return fail(D4R_ERR_INVALID_ARG, "k = %d, stride = %d must be >= 1", k, stride);
    if (H < k || W < k)
        return fail(D4R_ERR_INVALID_ARG, "plane %dx%d is smaller than the %dx%d window", H, W, k, k);
    *OH = (H - k) / stride + 1;
    *OW = (W - k) / stride + 1;
    *planes = (long long)batch * channels;
    if ((long long)H * W > kMaxElems)
        return fail(D4R_ERR_INVALID_ARG, "plane %dx%d has 2^31 or more elements", H, W);
    return D4R_OK;
}

}  // namespace

d4r_status d4r_maxpool_forward(const float *x, float *y, int *idx, int batch, int channels, int H, int W, int k,
                               int stride, void *hip_stream)
{
    long long planes;
    int OH, OW;
    D4R_TRY(check_pool(batch, channels, H, W, k, stride, &planes, &OH, &OW));
    if (planes == 0)
        return ok();
    D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(y, "y"));
    D4R_TRY(check_tensor(idx, "idx"));
    hipStream_t s = (hipStream_t)hip_stream;
    const double outs = (double)planes * OH * OW;
    return run_step(s, "maxpool_fwd", 4.0 * planes * H * W + 8.0 * outs, "max pooling", [&] {
        return launch_maxpool_forward(x, y, (int32_t *)idx, planes, H, W, OH, OW, k, stride, s);
    });
}

d4r_status d4r_maxpool_backward(const float *dy, const int *idx, float *dx, int batch, int channels, int H, int W,
                                int k, int stride, void *hip_stream)
{
    long long planes;
    int OH, OW;
    D4R_TRY(check_pool(batch, channels, H, W, k, stride, &planes, &OH, &OW));
    if (planes == 0)
        return ok();
    D4R_TRY(check_tensor(dy, "dy"));
    D4R_TRY(check_tensor(idx, "idx"));
    D4R_TRY(check_tensor(dx, "dx"));
    hipStream_t s = (hipStream_t)hip_stream;
    const double outs = (double)planes * OH * OW;
    return run_step(s, "maxpool_bwd", 8.0 * outs + 4.0 * planes * H * W, "max-pool gradient", [&] {
        return launch_maxpool_backward(dy, (const int32_t *)idx, dx, planes, H, W, OH, OW, k, stride, s);
    });
}

d4r_status d4r_add_bias_rows(const float *x, const float *bias, float *y, int rows, int cols, void *hip_stream)
{
    if (rows < 0 || cols < 1)
        return fail(D4R_ERR_INVALID_ARG, "rows = %d must be >= 0 and cols = %d >= 1", rows, cols);
    if ((long long)rows * cols > kMaxElems)
        return fail(D4R_ERR_INVALID_ARG, "rows * cols has 2^31 or more elements");
    if (rows == 0)
        return ok();
    D4R_TRY(check_tensor(x, "x"));
    D4R_TRY(check_tensor(y, "y"));
    if (!bias)
        return fail(D4R_ERR_INVALID_ARG, "bias is NULL");
    D4R_TRY(check_vec(bias, "bias"));
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "add_bias_rows", 8.0 * rows * cols + 4.0 * cols, "bias add",
                    [&] { return launch_add_bias_rows(x, bias, y, rows, cols, s); });
}

d4r_status d4r_bias_grad_rows(const float *dy, float *db, int rows, int cols, void *hip_stream)
{
    if (rows < 0 || cols < 1)
        return fail(D4R_ERR_INVALID_ARG, "rows = %d must be >= 0 and cols = %d >= 1", rows, cols);
    if ((long long)rows * cols > kMaxElems)
        return fail(D4R_ERR_INVALID_ARG, "rows * cols has 2^31 or more elements");
    if (rows > 0)
        D4R_TRY(check_tensor(dy, "dy"));  // rows == 0 reads no dy (db = 0)
    if (!db)
        return fail(D4R_ERR_INVALID_ARG, "db is NULL");
    D4R_TRY(check_vec(db, "db"));
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "bias_grad_rows", 4.0 * rows * cols + 4.0 * cols, "bias gradient",
                    [&] { return launch_bias_grad_rows(dy, db, rows, cols, s); });
}

namespace {

d4r_status check_rows(int rows, int classes)
{
    if (rows < 1 || classes < 1)
        return fail(D4R_ERR_INVALID_ARG, "rows = %d and classes = %d must be >= 1", rows, classes);
    if ((long long)rows * classes > kMaxElems)
        return fail(D4R_ERR_INVALID_ARG, "rows * classes has 2^31 or more elements");
    return D4R_OK;
}

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
}

}  // namespace

d4r_status d4r_softmax(const float *z, float *p, int rows, int classes, void *hip_stream)
{
    D4R_TRY(check_rows(rows, classes));
    D4R_TRY(check_tensor(z, "z"));
    D4R_TRY(check_tensor(p, "p"));
    const size_t bytes = 4ull * rows * classes;
    if (overlaps(z, bytes, p, bytes))
        return fail(D4R_ERR_INVALID_ARG, "p overlaps z");
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "softmax", 8.0 * rows * classes, "softmax",
                    [&] { return launch_softmax_rows(z, nullptr, p, nullptr, rows, classes, s); });
}

d4r_status d4r_softmax_ce_grad(const float *z, const int *labels, float *dz, float *loss, int rows, int classes,
                               void *hip_stream)
{
    D4R_TRY(check_rows(rows, classes));
    D4R_TRY(check_tensor(z, "z"));
    D4R_TRY(check_tensor(dz, "dz"));
    if (!labels)
        return fail(D4R_ERR_INVALID_ARG, "labels is NULL");
    D4R_TRY(check_vec(labels, "labels"));
    D4R_TRY(check_vec(loss, "loss"));
    const size_t bytes = 4ull * rows * classes;
    if (overlaps(z, bytes, dz, bytes))
        return fail(D4R_ERR_INVALID_ARG, "dz overlaps z");
    if (loss && (overlaps(loss, 4, z, bytes) || overlaps(loss, 4, dz, bytes)))
        return fail(D4R_ERR_INVALID_ARG, "loss overlaps z or dz");
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "softmax_ce_grad", 8.0 * rows * classes + 4.0 * rows, "softmax-CE gradient", [&] {
        return launch_softmax_rows(z, (const int32_t *)labels, dz, loss, rows, classes, s);
    });
}

d4r_status d4r_sgd_update(float *param, const float *grad, long long n, float lr, float clip, void *hip_stream)
{
    D4R_TRY(check_count(n, "n"));
    if (!(clip >= 0.0f))
        return fail(D4R_ERR_INVALID_ARG, "clip must be >= 0 (got %g)", (double)clip);
    if (n == 0)
        return ok();
    D4R_TRY(check_tensor(param, "param"));
    D4R_TRY(check_tensor(grad, "grad"));
    if (overlaps(param, 4ull * n, grad, 4ull * n))
        return fail(D4R_ERR_INVALID_ARG, "grad overlaps param");
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "sgd", 12.0 * n, "SGD update", [&] { return launch_sgd(param, grad, n, lr, clip, s); });
}

d4r_status d4r_grad_accum(float *acc, const float *grad, long long n, void *hip_stream)
{
    D4R_TRY(check_count(n, "n"));
    if (n == 0)
        return ok();
    D4R_TRY(check_tensor(acc, "acc"));
    D4R_TRY(check_tensor(grad, "grad"));
    if (overlaps(acc, 4ull * n, grad, 4ull * n))
        return fail(D4R_ERR_INVALID_ARG, "grad overlaps acc");
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "grad_accum", 12.0 * n, "gradient accumulation",
                    [&] { return launch_grad_accum(acc, grad, n, s); });
}

d4r_status d4r_stream_copy(void *dst, const void *src, size_t bytes, void *hip_stream)
{
    if (bytes % 16 != 0)
        return fail(D4R_ERR_INVALID_ARG, "bytes = %zu is not a multiple of 16", bytes);
    if (bytes == 0)
        return ok();
    D4R_TRY(check_tensor(dst, "dst"));
    D4R_TRY(check_tensor(src, "src"));
    if (overlaps(dst, bytes, src, bytes))
        return fail(D4R_ERR_INVALID_ARG, "dst overlaps src");
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "stream_copy", 2.0 * bytes, "stream copy",
                    [&] { return launch_stream_copy(dst, src, bytes, s); });
}

d4r_status d4r_stream_fill(void *dst, unsigned int value, size_t bytes, void *hip_stream)
{
    if (bytes % 16 != 0)
        return fail(D4R_ERR_INVALID_ARG, "bytes = %zu is not a multiple of 16", bytes);
    if (bytes == 0)
        return ok();
    D4R_TRY(check_tensor(dst, "dst"));
    hipStream_t s = (hipStream_t)hip_stream;
    return run_step(s, "stream_fill", 1.0 * bytes, "stream fill",
                    [&] { return launch_stream_fill(dst, value, bytes, s); });
}

d4r_status d4r_mfma_ceiling(d4r_dtype dtype, const void *src, float *out, int blocks, int iters,
                            void *hip_stream)
{
    if (!valid_dtype(dtype))
        return fail(D4R_ERR_INVALID_ARG, "unknown dtype %d", (int)dtype);
    if (blocks < 1 || blocks > (1 << 20) || iters < 1)
        return fail(D4R_ERR_INVALID_ARG, "blocks must be in [1, 2^20] and iters >= 1");
    D4R_TRY(check_tensor(src, "src"));
    D4R_TRY(check_tensor(out, "out"));
    if (overlaps(src, dtype == D4R_F32 ? 6 * 64 * 4 : 6 * 64 * 16, out, (size_t)blocks * 8 * sizeof(float)))
        return fail(D4R_ERR_INVALID_ARG, "out overlaps src");
    // 2*32*32*k flops per MFMA (k = 2 for f32, 16 for 16-bit), 8 per
    // iteration and wavefront, 8 wavefronts per workgroup
    const double k = dtype == D4R_F32 ? 2.0 : 16.0;
    const double flops = 2.0 * 32 * 32 * k * 8.0 * 8.0 * (double)iters * blocks;
    hipStream_t s = (hipStream_t)hip_stream;
    ProfScope ps(s, std::string("mfma_ceiling_") + dt_name(dtype), flops, 0.0);
    hipError_t e = launch_mfma_ceiling(dtype, src, out, blocks, iters, s);
    ps.done();
    D4R_LAUNCH(e, "MFMA ceiling");
    return ok();
}

d4r_status d4r_profile_enable(int on)
{
    Profiler &P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    P.on = on != 0;
    return ok();
}

d4r_status d4r_profile_reset(void)
{
    Profiler &P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    P.used = 0;
    return ok();
}

d4r_status d4r_profile_read(d4r_kernel_stat *out, int max, int *count)
{
    if (!count || (max > 0 && !out))
        return fail(D4R_ERR_INVALID_ARG, "NULL argument");
    Profiler &P = prof();
    std::lock_guard<std::mutex> lk(P.mu);
    std::vector<d4r_kernel_stat> agg(P.names.size());
    for (size_t k = 0; k < P.names.size(); ++k)
        agg[k] = d4r_kernel_stat{P.names[k].c_str(), 0, 0.0, 0.0, 0.0};
    for (size_t i = 0; i < P.used; ++i) {
        ProfRec &r = P.recs[i];
        hipError_t e = hipEventSynchronize(r.b);
        float ms = 0.0f;
        if (e == hipSuccess)
            e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess)
            return fail(D4R_ERR_LAUNCH, "event timing: %s", hipGetErrorString(e));
        d4r_kernel_stat &a = agg[r.key];
        a.launches += 1;
        a.ms += ms;
        a.flops += r.flops;
        a.bytes += r.bytes;
    }
    int n = 0;
    for (auto &a : agg) {
        if (a.launches == 0)
            continue;
        if (n < max)
            out[n] = a;
        ++n;
    }
    *count = n;
    return ok();
}

}  // extern "C"
