// MFMA GEMM for f32 operands on gfx950: C(f32) = op(A) * op(B) with the
// transpose flags of the directcompute-nn page ("Matmul Shaders", "Transpose
// via Flags").  (f16 / bf16 operands have their own kernel, gemm16_impl.hpp.)
//
// Design (CDNA4, 64-lane wavefronts):
//  * A workgroup of NWM x NWN wavefronts computes a BM x BN tile; each
//    wavefront owns TM x TN blocks of 32x32 outputs held in MFMA
//    accumulators (16 floats per lane per block), fed by
//    v_mfma_f32_32x32x2_f32.
//  * A K stage is 32 floats (128 bytes) of k per operand row.  Two register
//    sets alternate (loop unrolled by two so each set stays in fixed
//    registers): while stage t is computed from one LDS buffer, the global
//    loads of stages t+1 and t+2 are in flight; one barrier per stage.
//  * With VEC (leading dimension and contiguous extent multiples of 4, so
//    every 16-byte vector is wholly inside or outside the matrix) the loads
//    are issued unconditionally and the zero mask is applied when the
//    registers are written to LDS: no branches around the loads, so the
//    compiler waits only for the register set being stored.
//  * Operands come in four forms (OperandMode): row- or k-contiguous
//    matrices, the im2col of x gathered on the fly (implicit forward), and
//    an NCHW gradient dy read in place as the O x (B*P) matrix of the
//    filter- and data-gradient products, so dy is never reshaped or
//    transposed in HBM.
//  * LDS layout follows the global layout: an operand stored with k
//    contiguous is kept as [row][k] (row pitch padded by 16 bytes so the
//    16-byte fragment reads of 8 consecutive rows hit distinct banks); an
//    operand stored row-contiguous is kept as [k][row] and read one element
//    per lane per k.  (Loading row-contiguous operands one element per lane
//    into [row][k] instead measured slower: four times the load
//    instructions.)
//  * When both layouts are [row][k], scheduling-group hints read both k
//    groups' fragments up front and spread the next stage's LDS stores
//    through the MFMAs; with [k][row] layouts the compiler's own schedule
//    measured faster.
//  * Only the sum over k matters to the result, so lane-half h of a
//    fragment takes k = 8h..8h+7 of each 16-wide k group, the same mapping
//    for A and B.
//  * Out-of-range rows and k are zero-filled in LDS; the MFMAs run on whole
//    blocks and the epilogue masks the stores.
//  * Workgroups are renumbered so that consecutive tiles share an XCD (and
//    its L2).
#pragma once

#include <type_traits>
#include <utility>

#include "internal.hpp"

namespace d4r {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBK32 = 32;   // k depth of one stage (floats)
constexpr int kPad32 = 4;   // 16 bytes of row padding

// One operand's global -> register -> LDS path (f32 elements).
//   KC = true : global X[r*ld + k], LDS [r][k] with pitch BK + PAD
//   KC = false: global X[k*ld + r], LDS [k][r] with pitch BR + PAD
template <int BR, bool KC, int NT>
struct OperandTile {
    static constexpr int VW = 4, BK = kBK32, PAD = kPad32;
    static constexpr int PITCH = KC ? (BK + PAD) : (BR + PAD);
    static constexpr int LDS_BYTES = (KC ? BR : BK) * PITCH * 4;
    static constexpr int NV = BR * BK / VW;
    static constexpr int PER = (NV + NT - 1) / NT;

    u32x4 reg[PER];
    uint32_t okmask;  // bit s: reg[s] lies inside the matrix (VEC loads)

    __device__ __forceinline__ static void slot(int id, int &row, int &kk)
    {
        if (KC) {
            row = id / (BK / VW);
            kk = (id % (BK / VW)) * VW;
        } else {
            kk = id / (BR / VW);
            row = (id % (BR / VW)) * VW;
        }
    }

    template <bool VEC>
    __device__ __forceinline__ void load(const uint32_t *__restrict__ X, int ld, int R, int K, int r0,
                                         int k0, int tid)
    {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            const bool live = NV % NT == 0 || id < NV;
            int row, kk;
            slot(live ? id : 0, row, kk);
            const int r = r0 + row, k = k0 + kk;
            const long long off = KC ? (long long)r * ld + k : (long long)k * ld + r;
            if constexpr (VEC) {
                const bool ok = live && r < R && k < K;
                reg[s] = *(const u32x4 *)(X + (ok ? off : 0));
                okmask = (s == 0 ? 0u : okmask) | ((ok ? 1u : 0u) << s);
            } else {
                u32x4 v = {0u, 0u, 0u, 0u};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const bool ok = live && (KC ? (r < R && k + e < K) : (k < K && r + e < R));
                    v[e] = ok ? X[off + e] : 0u;
                }
                reg[s] = v;
            }
        }
    }

    template <bool VEC>
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
        const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            if constexpr (NV % NT != 0) {
                if (id >= NV)
                    break;
            }
            int row, kk;
            slot(id, row, kk);
            const int e = KC ? (row * PITCH + kk) : (kk * PITCH + row);
            *(u32x4 *)(lds + e * 4) = (!VEC || ((okmask >> s) & 1u)) ? reg[s] : z;
        }
    }
};

// B operand: the im2col of an NHWC tensor t[b][h][w][c] (OP_IMPL_T, stride
// 1, C % 32 == 0) with 32-deep stages ordered by channel block, then tap:
// op(B)[k][n] = t[b][i-p+u][j-p+v][c] for n = (b, i, j), k = (cb*kH*kW +
// u*kW + v)*32 + ci, c = cb*32 + ci.  A stage lies inside one tap, so every 16-byte
// slot is 4 consecutive channels of one pixel; loads are unconditional (offset
// 0 in the padding or past N) and zeroed at the LDS store, the layout [n][k]
// of a k-contiguous operand.  The slots' pixels are the same in every stage:
// decoded once into NhwcRows (shared by both register sets).
template <int BR, int NT>
struct NhwcRows {
    using T = OperandTile<BR, true, NT>;
    // per slot: window origin (h0 far negative for a slot past N, so no tap
    // is ever in range) and the element offset ((b*H + h0)*W + w0)*C + kk;
    // a stage adds its tap's uniform offset (u*W + v)*C + c0
    int h0[T::PER], w0[T::PER];
    long long base[T::PER];

    __device__ __forceinline__ void setup(const ConvGeom &g, int n0, int tid)
    {
#pragma unroll
        for (int s = 0; s < T::PER; ++s) {
            const int id = s * NT + tid;
            const bool live = T::NV % NT == 0 || id < T::NV;
            int row, kk;
            T::slot(live ? id : 0, row, kk);
            const int n = n0 + row;
            const int bb = n / g.P, r = n - (n / g.P) * g.P;
            const int i = r / g.OW;
            h0[s] = (live && n < g.N) ? i - g.p : -(1 << 30);
            w0[s] = r - i * g.OW - g.pw;
            base[s] = (((long long)bb * g.H + (i - g.p)) * g.W + w0[s]) * g.C + kk;
        }
    }
};

template <int BR, int NT>
struct ImplNhwcTileF32 : OperandTile<BR, true, NT> {
    using T = OperandTile<BR, true, NT>;

    __device__ __forceinline__ void load(const uint32_t *__restrict__ X, const ConvGeom &g,
                                         const NhwcRows<BR, NT> &rows, int K, int k0, int tid)
    {
        // stages ordered by channel block, then tap (OP_IMPL_T)
        const int ks = k0 / kBK32, taps = g.kH * g.kW;
        const int cblk = ks / taps, tap = ks - cblk * taps, c0 = cblk * kBK32;
        const int u = tap / g.kW, v = tap - (tap / g.kW) * g.kW;
        const long long toff = ((long long)u * g.W + v) * g.C + c0;
#pragma unroll
        for (int s = 0; s < T::PER; ++s) {
            const int id = s * NT + tid;
            int row, kk;
            T::slot(id, row, kk);
            const bool ok = k0 + kk < K && (unsigned)(rows.h0[s] + u) < (unsigned)g.H &&
                            (unsigned)(rows.w0[s] + v) < (unsigned)g.W;
            this->reg[s] = *(const u32x4 *)(X + (ok ? rows.base[s] + toff : 0));
            this->okmask = (s == 0 ? 0u : this->okmask) | ((ok ? 1u : 0u) << s);
        }
    }
};

// Forward-GEMM B operand gathered straight from x (the implicit GEMM):
// op(B)[kc][n] = xt(b, c, i*s - p + u, j*s - p + v), kc = (c*kH + u)*kW + v,
// n = (b*OH + i)*OW + j, stored in the same [k][n] LDS layout as a
// row-contiguous operand.  A thread's four columns n are the same in every
// K stage, so their image offsets and window origins are decoded once (in
// ImplicitColsF32, shared by both register sets); each stage decodes only
// the thread's kc rows.
template <int BR, int NT>
struct ImplicitColsF32 {
    static constexpr int VW = 4;
    int nb[VW], nh[VW], nw[VW];  // image offset (-1 past N), window origin row / column

    __device__ __forceinline__ void setup(const ConvGeom &g, int n_blk, int tid)
    {
        const int n0 = n_blk + (tid % (BR / VW)) * VW;
        int b = n0 / g.P;
        int rem = n0 - b * g.P;
        int i = rem / g.OW;
        int j = rem - i * g.OW;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            nb[e] = (n0 + e < g.N) ? b * g.C * g.H * g.W : -1;
            nh[e] = i * g.s - g.p;
            nw[e] = j * g.s - g.p;
            if (++j == g.OW) {
                j = 0;
                if (++i == g.OH) {
                    i = 0;
                    ++b;
                }
            }
        }
    }
};

template <int BR, int NT>
struct ImplicitTileF32 {
    using Base = OperandTile<BR, false, NT>;
    static constexpr int VW = 4, BK = kBK32;
    static constexpr int PITCH = Base::PITCH, LDS_BYTES = Base::LDS_BYTES;
    static constexpr int NV = Base::NV, PER = Base::PER;
    static_assert(NT % (BR / VW) == 0, "a thread's columns must not change between slots");

    u32x4 reg[PER];

    __device__ __forceinline__ void gather(const uint32_t *__restrict__ x, const ConvGeom &g,
                                           const ImplicitColsF32<BR, NT> &cols, int K, int k0, int tid)
    {
        const int khw = g.kH * g.kW;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            if (NV % NT != 0 && id >= NV)
                break;
            const int k = k0 + id / (BR / VW);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (k < K) {
                const int c = k / khw;
                const int r = k - c * khw;
                const int u = r / g.kW;
                const int vv = r - u * g.kW;
                const int plane = c * g.H * g.W;
#pragma unroll
                for (int e = 0; e < VW; ++e) {
                    const int hh = cols.nh[e] + u, ww = cols.nw[e] + vv;
                    const bool ok = cols.nb[e] >= 0 && hh >= 0 && hh < g.H && ww >= 0 && ww < g.W;
                    v[e] = ok ? x[cols.nb[e] + plane + hh * g.W + ww] : 0u;
                }
            }
            reg[s] = v;
        }
    }

    template <bool VEC>
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            if (NV % NT != 0 && id >= NV)
                break;
            const int kk = id / (BR / VW), row = (id % (BR / VW)) * VW;
            *(u32x4 *)(lds + (kk * PITCH + row) * 4) = reg[s];
        }
    }
};

// Operand read straight from an NCHW tensor t[b][c][pix] (ch channels) with
// row r = c and k = b*P + pix, so op[r][k] = t[(k / P)*ch*P + r*P + k % P]:
// A = dy of the filter gradient, or B = x of a 1x1 filter gradient.  Kept in
// LDS as [r][k] like a k-contiguous operand.  The 32 lanes of a half-wave take
// 32 consecutive k of one row (pixel runs, split at most once per image
// boundary), so each load instruction reads whole 128-byte runs; a thread
// decodes its k once per stage.  Loads are unconditional (offset 0 when
// outside) and zeroed at the LDS store.
template <int BR, int NT>
struct NchwKTile {
    static constexpr int BK = kBK32, PAD = kPad32, PITCH = BK + PAD;
    static constexpr int LDS_BYTES = BR * PITCH * 4;
    static constexpr int RSTEP = NT / BK;  // rows per pass
    static constexpr int PER = BR / RSTEP;
    static_assert(NT % BK == 0 && BR % RSTEP == 0, "whole passes");

    uint32_t reg[PER];
    uint32_t okmask;

    __device__ __forceinline__ void load(const uint32_t *__restrict__ X, const ConvGeom &g, int ch, int R,
                                         int K, int r0, int k0, int tid)
    {
        const int k = k0 + tid % BK;
        const int b = k / g.P;
        const long long base = (long long)b * ch * g.P + (k - b * g.P);
        const bool kok = k < K;
        okmask = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int r = r0 + tid / BK + j * RSTEP;
            const bool ok = kok && r < R;
            reg[j] = X[ok ? base + (long long)r * g.P : 0];
            okmask |= (ok ? 1u : 0u) << j;
        }
    }

    template <bool VEC>
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
        uint32_t *l = (uint32_t *)lds;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            l[(tid / BK + j * RSTEP) * PITCH + tid % BK] = ((okmask >> j) & 1u) ? reg[j] : 0u;
    }
};

// B operand read straight from an NCHW tensor t[b][c][pix] (ch channels):
// k = c, column n = b*P + pix, so op(B)[k][n] = t[(n / P)*ch*P + k*P + n % P]
// (dy of the data gradient, or x of a 1x1 forward).  Kept in LDS as [k][n]
// like a row-contiguous operand.  Each thread owns one
// column for the whole K loop (decoded once, in NchwCol); consecutive lanes
// take consecutive columns, so a load instruction reads pixel runs.
struct NchwCol {
    long long off;  // element offset of (b, o = 0, pix)
    bool ok;        // n < N

    __device__ __forceinline__ void setup(const ConvGeom &g, int ch, int n)
    {
        ok = n < g.N;
        const int b = n / g.P;
        off = (long long)b * ch * g.P + (n - b * g.P);
    }
};

template <int BR, int NT>
struct NchwNTile {
    static constexpr int BK = kBK32, PAD = kPad32, PITCH = BR + PAD;
    static constexpr int LDS_BYTES = BK * PITCH * 4;
    static constexpr int KSTEP = NT / BR;  // k rows per pass
    static constexpr int PER = BK / KSTEP;
    static_assert(NT % BR == 0 && BK % KSTEP == 0, "whole passes");

    uint32_t reg[PER];
    uint32_t okmask;

    __device__ __forceinline__ void load(const uint32_t *__restrict__ X, const ConvGeom &g,
                                         const NchwCol &c, int K, int k0, int tid)
    {
        okmask = 0u;
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int k = k0 + tid / BR + j * KSTEP;
            const bool ok = c.ok && k < K;
            reg[j] = X[ok ? c.off + (long long)k * g.P : 0];
            okmask |= (ok ? 1u : 0u) << j;
        }
    }

    template <bool VEC>
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
        uint32_t *l = (uint32_t *)lds;
#pragma unroll
        for (int j = 0; j < PER; ++j)
            l[(tid / BR + j * KSTEP) * PITCH + tid % BR] = ((okmask >> j) & 1u) ? reg[j] : 0u;
    }
};

// Fragment reads: 8 consecutive k (one k group of 16, lane half h) for one
// 32-row block; the 8 MFMAs of the group use element t.
template <bool KC, int PITCH>
__device__ __forceinline__ void frag_f32(const float *lds, int row, int kg, int h, float (&f)[8])
{
    if (KC) {
        const float *p = lds + row * PITCH + kg * 16 + h * 8;
        u32x4 a = *(const u32x4 *)p;
        u32x4 b = *(const u32x4 *)(p + 4);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f[t] = __uint_as_float(a[t]);
            f[t + 4] = __uint_as_float(b[t]);
        }
    } else {
#pragma unroll
        for (int t = 0; t < 8; ++t)
            f[t] = lds[(kg * 16 + h * 8 + t) * PITCH + row];
    }
}

// Scheduling hints for one stage (fragment reads, MFMAs and the LDS stores
// of the next stage): both k groups' fragments are read up front, then the
// next stage's LDS stores are spread evenly through the MFMAs.  Masks:
// 0x008 MFMA, 0x100 LDS read, 0x200 LDS write.
template <int STEP, int... W>
__device__ __forceinline__ void sched_spread_writes(std::integer_sequence<int, W...>)
{
    ((__builtin_amdgcn_sched_group_barrier(0x008, STEP + 0 * W, 0),
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0)),
     ...);
}

template <int RD_KG, int MF_KG, int WR>
__device__ __forceinline__ void sched_stage()
{
    constexpr int LEAD = 2;
    constexpr int REST = 2 * MF_KG - LEAD;
    constexpr int STEP = REST / (WR + 1);
    __builtin_amdgcn_sched_group_barrier(0x100, RD_KG, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, LEAD, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, RD_KG, 0);
    sched_spread_writes<STEP>(std::make_integer_sequence<int, WR>{});
    __builtin_amdgcn_sched_group_barrier(0x008, REST - STEP * WR, 0);
}

// VEC: bit 0 lets a plainly strided A take 16-byte vector loads, bit 1 a
// plainly strided B (the other operand forms ignore their bit).  Separate
// bits, because one misaligned operand (a filter with Kc % 4 != 0) must not
// cost the other one its vector loads.
template <int NWM, int NWN, int TM, int TN, int AMODE, int BMODE, int VEC>
__global__ __launch_bounds__(NWM *NWN * 64) void gemm_kernel(GemmParams p)
{
    constexpr bool VA = (VEC & 1) != 0, VB = (VEC & 2) != 0;
    constexpr int NT = NWM * NWN * 64;
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32;
    constexpr int BK = kBK32;
    static_assert(AMODE == OP_ROWS || AMODE == OP_KC || AMODE == OP_NCHW, "A mode");
    // LDS layouts: [m][k] unless A is row-contiguous; [n][k] only for a
    // k-contiguous B
    constexpr bool A_KC = AMODE != OP_ROWS;
    constexpr bool B_KC = BMODE == OP_KC || BMODE == OP_NCHW_K || BMODE == OP_IMPL_T;
    using TA = std::conditional_t<AMODE == OP_NCHW, NchwKTile<BM, NT>, OperandTile<BM, A_KC, NT>>;
    using TB = std::conditional_t<
        BMODE == OP_IMPL, ImplicitTileF32<BN, NT>,
        std::conditional_t<
            BMODE == OP_NCHW, NchwNTile<BN, NT>,
            std::conditional_t<BMODE == OP_NCHW_K, NchwKTile<BN, NT>,
                               std::conditional_t<BMODE == OP_IMPL_T, ImplNhwcTileF32<BN, NT>,
                                                  OperandTile<BN, B_KC, NT>>>>>;
    constexpr int STAGE = TA::LDS_BYTES + TB::LDS_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % NWM, wn = wave / NWM;
    const int h = lane >> 5, l32 = lane & 31;

    const int mt = (p.M + BM - 1) / BM;
    const WorkItem wi = xcd_work(blockIdx.x, mt * ((p.N + BN - 1) / BN), p.splits);
    const int m_blk = (wi.tile % mt) * BM;
    const int n_blk = (wi.tile / mt) * BN;

    const int kbeg = wi.split * p.k_per_split;
    const int kend = min(p.K, kbeg + p.k_per_split);
    const int nk = (kend - kbeg + BK - 1) / BK;

    f32x16 acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    const uint32_t *A = (const uint32_t *)p.A;
    const uint32_t *B = (const uint32_t *)p.B;
    TA ta0, ta1;
    TB tb0, tb1;
    ImplicitColsF32<BN, NT> cols;
    if constexpr (BMODE == OP_IMPL)
        cols.setup(p.g, n_blk, tid);
    NchwCol ncol;
    if constexpr (BMODE == OP_NCHW)
        ncol.setup(p.g, p.b_ch, n_blk + tid % BN);
    NhwcRows<BN, NT> nrows;
    if constexpr (BMODE == OP_IMPL_T)
        nrows.setup(p.g, n_blk, tid);
    // K bound for this split: the loaders zero-fill k >= kend.
    auto load = [&](TA &a, TB &b, int k0) {
        if constexpr (AMODE == OP_NCHW)
            a.load(A, p.g, p.a_ch, p.M, kend, m_blk, k0, tid);
        else
            a.template load<VA>(A, p.lda, p.M, kend, m_blk, k0, tid);
        if constexpr (BMODE == OP_IMPL)
            b.gather(B, p.g, cols, kend, k0, tid);
        else if constexpr (BMODE == OP_NCHW)
            b.load(B, p.g, ncol, kend, k0, tid);
        else if constexpr (BMODE == OP_NCHW_K)
            b.load(B, p.g, p.b_ch, p.N, kend, n_blk, k0, tid);
        else if constexpr (BMODE == OP_IMPL_T)
            b.load(B, p.g, nrows, kend, k0, tid);
        else
            b.template load<VB>(B, p.ldb, p.N, kend, n_blk, k0, tid);
    };
    auto store = [&](const TA &a, const TB &b, char *buf) {
        a.template store<VA>(buf, tid);
        b.template store<VB>(buf + TA::LDS_BYTES, tid);
    };
    auto compute = [&](const char *buf) {
        const float *fa = (const float *)buf;
        const float *fb = (const float *)(buf + TA::LDS_BYTES);
        // all fragment reads of the stage first, so the LDS latency is paid
        // once per stage rather than once per 16-wide k group
        constexpr int KG = BK / 16;
        float af[KG][TM][8], bf[KG][TN][8];
#pragma unroll
        for (int kg = 0; kg < KG; ++kg) {
#pragma unroll
            for (int i = 0; i < TM; ++i)
                frag_f32<A_KC, TA::PITCH>(fa, (wm * TM + i) * 32 + l32, kg, h, af[kg][i]);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                frag_f32<B_KC, TB::PITCH>(fb, (wn * TN + j) * 32 + l32, kg, h, bf[kg][j]);
        }
#pragma unroll
        for (int kg = 0; kg < KG; ++kg)
#pragma unroll
            for (int t = 0; t < 8; ++t)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[kg][i][t], bf[kg][j][t], acc[i][j],
                                                                         0, 0, 0);
    };

    // instruction counts of one stage, for the scheduling hints
    constexpr int RD_KG = (A_KC ? 2 : 8) * TM + (B_KC ? 2 : 8) * TN;  // LDS reads per k group
    constexpr int MF_KG = 8 * TM * TN;                               // MFMAs per k group
    constexpr int WR = TA::PER + TB::PER;                            // LDS stores per stage

    if (nk > 0) {
        // prologue: stages 0 and 1 in flight, stage 0 into LDS buffer 0
        load(ta0, tb0, kbeg);
        load(ta1, tb1, kbeg + BK);
        store(ta0, tb0, smem);
        __syncthreads();
        load(ta0, tb0, kbeg + 2 * BK);
        // Stage t is computed from LDS buffer t&1.  Register set (t+1)&1 holds
        // stage t+1 and is stored into LDS buffer (t+1)&1 after the compute;
        // it is then refilled with stage t+3.  An odd last stage is peeled.
        // Loads and stores are unconditional (a stage past the end has every
        // k >= kend: it reads nothing and stores zeros), and a scheduling
        // barrier keeps each stage's loads right after the workgroup barrier,
        // so two stages of loads stay in flight during each compute.
        int t = 0;
        // Without the hints (a [k][row] layout), the wavefront raises its
        // issue priority while it computes, so when both wavefronts of a
        // SIMD are ready the one with MFMAs to issue goes first (2-3% on
        // those kernels; neutral with the hints).
        constexpr bool HINTS = A_KC && B_KC;
        for (; t + 1 < nk; t += 2) {
            if constexpr (!HINTS)
                __builtin_amdgcn_s_setprio(1);
            compute(smem);
            store(ta1, tb1, smem + STAGE);
            if constexpr (HINTS)
                sched_stage<RD_KG, MF_KG, WR>();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!HINTS)
                __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            load(ta1, tb1, kbeg + (t + 3) * BK);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!HINTS)
                __builtin_amdgcn_s_setprio(1);
            compute(smem + STAGE);
            store(ta0, tb0, smem);
            if constexpr (HINTS)
                sched_stage<RD_KG, MF_KG, WR>();
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (!HINTS)
                __builtin_amdgcn_s_setprio(0);
            __syncthreads();
            load(ta0, tb0, kbeg + (t + 4) * BK);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t < nk)
            compute(smem);
    }

    // Epilogue.  Accumulator element e of a 32x32 block sits at
    // row 8*(e/4) + 4*h + (e%4), column l32.
    float *C = p.C + (long long)wi.split * p.c_split_stride;

    // Row-major output (split-K partials, dcol, dW, plain GEMMs) with rows
    // of 16-byte aligned columns: the tile goes through LDS, so every lane
    // stores 16-byte vectors of 4 consecutive columns instead of one float
    // per element (a quarter of the store instructions; the short-K data
    // gradient of AlexNet conv1 is bound by its 140 MB of dcol stores).
    constexpr int CP = BN + 4;  // LDS row pitch of the staged tile (floats)
    if constexpr (BM * CP * 4 <= 2 * STAGE) {
        if (p.epi == EPI_ROWMAJOR && (p.ldc & 3) == 0 && (p.N & 3) == 0 && (p.c_split_stride & 3) == 0) {
            float *cs = (float *)smem;
            __syncthreads();  // every wavefront is done reading the stages
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int ml = (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                        cs[ml * CP + (wn * TN + j) * 32 + l32] = acc[i][j][e];
                    }
            __syncthreads();
            constexpr int QR = BN / 4;  // 16-byte vectors per tile row
            for (int q = tid; q < BM * QR; q += NT) {
                const int r = q / QR, c = (q - r * QR) * 4;
                const int m = m_blk + r, n = n_blk + c;
                if (m < p.M && n < p.N) {
                    float4 v = *(const float4 *)(cs + r * CP + c);
                    if (p.bias || p.relu) {
                        v.x = epi_value(v.x, p.bias, p.relu, EPI_ROWMAJOR, m, n);
                        v.y = epi_value(v.y, p.bias, p.relu, EPI_ROWMAJOR, m, n + 1);
                        v.z = epi_value(v.z, p.bias, p.relu, EPI_ROWMAJOR, m, n + 2);
                        v.w = epi_value(v.w, p.bias, p.relu, EPI_ROWMAJOR, m, n + 3);
                    }
                    *(float4 *)(C + (long long)m * p.ldc + n) = v;
                }
            }
            return;
        }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n_blk + (wn * TN + j) * 32 + l32;
        if (n >= p.N)
            continue;
        long long col_off;
        if (p.epi == EPI_NCHW) {
            int b = n / p.P;
            int pix = n - b * p.P;
            col_off = (long long)b * p.M * p.P + pix;
        } else {
            col_off = n;
        }
        const long long row_stride = (p.epi == EPI_NCHW) ? p.P : p.ldc;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                int m = m_blk + (wm * TM + i) * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < p.M)
                    C[col_off + (long long)m * row_stride] = epi_value(acc[i][j][e], p.bias, p.relu, p.epi, m, n);
            }
        }
    }
}

template <int AMODE, int BMODE, int VEC>
hipError_t launch_gemm32_vec(int cfg, const GemmParams &p, hipStream_t s)
{
    TileShape ts = tile_shape(cfg);
    int tiles = ((p.M + ts.bm - 1) / ts.bm) * ((p.N + ts.bn - 1) / ts.bn);
    dim3 grid(tiles * p.splits);
    switch (cfg) {
    case TILE_128x128:
        hipLaunchKernelGGL((gemm_kernel<2, 2, 2, 2, AMODE, BMODE, VEC>), grid, dim3(256), 0, s, p);
        break;
    case TILE_64x64:
        hipLaunchKernelGGL((gemm_kernel<2, 2, 1, 1, AMODE, BMODE, VEC>), grid, dim3(256), 0, s, p);
        break;
    case TILE_32x128:
        hipLaunchKernelGGL((gemm_kernel<1, 4, 1, 1, AMODE, BMODE, VEC>), grid, dim3(256), 0, s, p);
        break;
    case TILE_96x128:
        hipLaunchKernelGGL((gemm_kernel<1, 4, 3, 1, AMODE, BMODE, VEC>), grid, dim3(256), 0, s, p);
        break;
    case TILE_128x64:
        hipLaunchKernelGGL((gemm_kernel<2, 2, 2, 1, AMODE, BMODE, VEC>), grid, dim3(256), 0, s, p);
        break;
    default:
        return hipErrorInvalidValue;  // tile shape not built for f32
    }
    return hipGetLastError();
}

// The vector bits cover the plainly strided operands (OP_ROWS / OP_KC); the
// gathered ones (OP_IMPL, OP_NCHW, OP_NCHW_K) load single elements either
// way, so their bit is fixed at 1 (no extra instantiations).
template <int AMODE, int BMODE>
hipError_t launch_gemm32_modes(int cfg, const GemmParams &p, hipStream_t s)
{
    constexpr bool a_plain = AMODE == OP_ROWS || AMODE == OP_KC;
    constexpr bool b_plain = BMODE == OP_ROWS || BMODE == OP_KC;  // OP_IMPL_T keeps bit 1: its
                                                                  // store applies the zero mask
    const bool va = !a_plain || p.a_vec, vb = !b_plain || p.b_vec;
    if (va && vb)
        return launch_gemm32_vec<AMODE, BMODE, 3>(cfg, p, s);
    if constexpr (a_plain && b_plain) {
        if (va)
            return launch_gemm32_vec<AMODE, BMODE, 1>(cfg, p, s);
        if (vb)
            return launch_gemm32_vec<AMODE, BMODE, 2>(cfg, p, s);
        return launch_gemm32_vec<AMODE, BMODE, 0>(cfg, p, s);
    } else if constexpr (a_plain) {
        return launch_gemm32_vec<AMODE, BMODE, 2>(cfg, p, s);  // A scalar
    } else {
        return launch_gemm32_vec<AMODE, BMODE, 1>(cfg, p, s);  // B scalar
    }
}

}  // namespace d4r
