// MFMA GEMM for 16-bit operands (f16 / bf16, f32 accumulation) on gfx950.
//
// Same contract as the f32 kernel (C = op(A) op(B) with the page's transpose
// flags), specialised for the short K stages of the 16-bit MFMAs:
//  * v_mfma_f32_32x32x16_{f16,bf16}: one 32x32 block per 16 k; a 64-deep K
//    stage is only ~512 MFMA cycles per wave, so global loads are issued two
//    stages ahead: two register sets alternate (loop unrolled by two so each
//    set stays in fixed registers) while two LDS buffers alternate behind
//    them; one barrier per stage.
//  * LDS holds every operand as [row][k] with 128-byte rows (64 halves =
//    eight 16-byte chunks).  Chunk c of row r is stored at chunk
//    c ^ ((r ^ (r >> 3)) & 7): the 16-byte fragment reads of 8 consecutive
//    rows then touch 8 different chunk positions (all banks, no conflict),
//    and so do the transposed 8-byte stores described next.
//  * Operands stored row-contiguous in memory (A[k*lda + m] / B[k*ldb + n])
//    are loaded as 4 k-rows x 8 rows per thread (four 16-byte loads), turned
//    into 8 rows x 4 k in registers (16 half-word permutes) and stored as
//    8-byte LDS writes, so fragment reads are 16-byte reads for every layout.
//  * The 128x256 and 256x128 tiles run eight wavefronts (two per SIMD, one
//    workgroup per CU by LDS), so one wavefront's waits are covered by the
//    other's MFMAs; the smaller tiles run four.
//  * Workgroups are renumbered so that consecutive tiles land on the same
//    XCD (the dispatcher deals workgroups round-robin over the 8 XCDs, each
//    with its own L2): the M tiles that share a B panel then share one L2.
#pragma once

#include <stdlib.h>
#include <type_traits>

#include "internal.hpp"

namespace d4r {

typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ int swz(int row) { return (row ^ (row >> 3)) & 7; }

template <int DTID>
__device__ __forceinline__ f32x16_t mfma16(u32x4_t a, u32x4_t b, f32x16_t c)
{
    if constexpr (DTID == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// One operand tile of BR rows x 64 k, 16-bit elements, loaded by NT threads.
template <int BR, bool KC, int NT_ = 256>
struct Tile16 {
    static constexpr int NT = NT_;
    static constexpr int BK = 64;
    static constexpr int LDS_BYTES = BR * 128;
    // k-contiguous: one 16-byte chunk per slot, 8 slots per row
    static constexpr int KC_SLOTS = BR * 8;
    // row-contiguous: one (8-row group, 4-k quad) block per slot; row groups
    // are padded to a multiple of 8 (slots with rg >= BR/8 do nothing)
    static constexpr int RGH = (BR / 8 + 7) / 8;
    static constexpr int MN_SLOTS = RGH * 8 * 16;
    static constexpr int SLOTS = KC ? KC_SLOTS : MN_SLOTS;
    static constexpr int PER = (SLOTS + NT - 1) / NT;
    static constexpr int NVEC = KC ? PER : 4 * PER;  // 16-byte vectors held per thread

    u32x4_t r[NVEC];
    uint32_t okmask;  // bit i: vector r[i] lies inside the matrix (VEC loads)

    // row-contiguous slot decoding: lanes 0..7 take 8 consecutive row groups,
    // lane bit 3 the low bit of the k quad, so 16 consecutive lanes store to
    // 16 distinct (chunk, half) positions.
    __device__ __forceinline__ static void mn_slot(int id, int &rg, int &kq)
    {
        const int lo = id & 7, b3 = (id >> 3) & 1, rest = id >> 4;
        // rest in [0, RGH*8) enumerates (row-group high part, k-quad high part)
        const int rgh = rest % RGH, kqh = rest / RGH;
        rg = rgh * 8 + lo;
        kq = kqh * 2 + b3;
    }

    // Element offset of (row rr, k kk).  Plain operands: rr*ld + kk
    // (k-contiguous) or kk*ld + rr (row-contiguous).  NC (an NCHW tensor
    // t[b][c][pix], nch channels, P pixels): the (image, pixel) index is k
    // for a k-contiguous operand (rows = c) and the row for a row-contiguous
    // one (k = c), at b*nch*P + c*P + pix.
    template <bool NC>
    __device__ __forceinline__ static long long offset(int rr, int kk, int ld, int nch, int P)
    {
        if constexpr (NC) {
            const int n = KC ? kk : rr, c = KC ? rr : kk;
            const int b = n / P;
            return ((long long)b * nch + c) * P + (n - b * P);
        } else {
            return KC ? (long long)rr * ld + kk : (long long)kk * ld + rr;
        }
    }

    // VEC: the operand's leading dimension and K are multiples of 8 (NC: P
    // is), so every 16-byte vector is either wholly inside or wholly outside
    // the matrix (NC: inside one image).  Then each load is issued
    // unconditionally (from offset 0 when outside) and zeroed by a select:
    // no branches, so the compiler can count the loads in flight and wait
    // only for the register set it stores next.
    template <bool VEC, bool NC = false>
    __device__ __forceinline__ void load(const uint16_t *__restrict__ X, int ld, int R, int K, int r0,
                                         int k0, int tid, int nch = 0, int P = 1)
    {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            if (KC) {
                const int row = (id < SLOTS ? id : 0) >> 3, ch = id & 7;
                const int rr = r0 + row, kk = k0 + ch * 8;
                const bool ok = id < SLOTS && rr < R && kk < K;
                if constexpr (VEC) {
                    const long long off = ok ? offset<NC>(rr, kk, ld, nch, P) : 0;
                    r[s] = *(const u32x4_t *)(X + off);
                    okmask = (s == 0 ? 0u : okmask) | ((ok ? 1u : 0u) << s);
                } else {
                    u32x4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool in = ok && kk + e < K;
                        uint32_t hv = in ? (uint32_t)X[offset<NC>(rr, in ? kk + e : 0, ld, nch, P)] : 0u;
                        v[e >> 1] |= hv << (16 * (e & 1));
                    }
                    r[s] = v;
                }
            } else {
                int rg = 0, kq = 0;
                if (id < SLOTS)
                    mn_slot(id, rg, kq);
                const bool live = id < SLOTS && rg < BR / 8;
                const int rr = r0 + rg * 8;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kk = k0 + kq * 4 + i;
                    const bool ok = live && kk < K && rr < R;
                    if constexpr (VEC) {
                        const long long off = ok ? offset<NC>(rr, kk, ld, nch, P) : 0;
                        r[4 * s + i] = *(const u32x4_t *)(X + off);
                        okmask = (s == 0 && i == 0 ? 0u : okmask) | ((ok ? 1u : 0u) << (4 * s + i));
                    } else {
                        u32x4_t v = {0u, 0u, 0u, 0u};
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const bool in = ok && rr + e < R;
                            uint32_t hv = in ? (uint32_t)X[offset<NC>(in ? rr + e : 0, kk, ld, nch, P)] : 0u;
                            v[e >> 1] |= hv << (16 * (e & 1));
                        }
                        r[4 * s + i] = v;
                    }
                }
            }
        }
    }

    // Writes the held vectors to LDS.  With VEC loads, vectors outside the
    // matrix were loaded from offset 0 and are replaced by zeros here, so the
    // wait for their data happens at the store, not at the load.
    template <bool VEC>
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
        const u32x4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            if constexpr (SLOTS % NT != 0) {
                if (id >= SLOTS)
                    break;
            }
            if (KC) {
                const int row = id >> 3, ch = id & 7;
                const u32x4_t v = (!VEC || ((okmask >> s) & 1u)) ? r[s] : z;
                *(u32x4_t *)(lds + row * 128 + ((ch ^ swz(row)) << 4)) = v;
            } else {
                int rg, kq;
                mn_slot(id, rg, kq);
                if constexpr ((BR / 8) % 8 != 0) {
                    if (rg >= BR / 8)
                        continue;
                }
                const u32x4_t a = (!VEC || ((okmask >> (4 * s + 0)) & 1u)) ? r[4 * s + 0] : z;
                const u32x4_t b = (!VEC || ((okmask >> (4 * s + 1)) & 1u)) ? r[4 * s + 1] : z;
                const u32x4_t c = (!VEC || ((okmask >> (4 * s + 2)) & 1u)) ? r[4 * s + 2] : z;
                const u32x4_t d = (!VEC || ((okmask >> (4 * s + 3)) & 1u)) ? r[4 * s + 3] : z;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    // row rg*8+e: halves k = 4kq..4kq+3 taken from element e of a, b, c, d
                    const int w = e >> 1;
                    uint32_t lo, hi;
                    if (e & 1) {
                        lo = (a[w] >> 16) | (b[w] & 0xffff0000u);
                        hi = (c[w] >> 16) | (d[w] & 0xffff0000u);
                    } else {
                        lo = (a[w] & 0xffffu) | (b[w] << 16);
                        hi = (c[w] & 0xffffu) | (d[w] << 16);
                    }
                    const int row = rg * 8 + e;
                    const int ch = kq >> 1;
                    u32x2_t v = {lo, hi};
                    *(u32x2_t *)(lds + row * 128 + ((ch ^ swz(row)) << 4) + ((kq & 1) << 3)) = v;
                }
            }
        }
    }
};

// Forward-GEMM B operand gathered straight from x (the implicit GEMM), in the
// row-contiguous path of Tile16: a thread gathers 4 kc rows x 8 consecutive
// columns n per slot and stores them through the same in-register transpose.
// The thread's 8 columns are fixed for the whole K loop, so their image
// offsets and window origins are decoded once.
// Image offsets and window origins of a thread's 8 columns (fixed for the
// whole K loop, shared by both register sets).
template <int BR, int NT>
struct ImplicitCols16 {
    int nb[8], nh[8], nw[8];  // image offset (-1 past N or unused), window origin

    __device__ __forceinline__ void setup(const ConvGeom &g, int n_blk, int tid)
    {
        // a thread's row group is the same in every slot: id = s*NT + tid and
        // NT/16 is a multiple of RGH
        constexpr int RGH = Tile16<BR, false, NT>::RGH;
        static_assert((NT / 16) % RGH == 0, "fixed columns per thread");
        const int rg = ((tid >> 4) % RGH) * 8 + (tid & 7);
        const int n0 = n_blk + rg * 8;
        int b = n0 / g.P;
        int rem = n0 - b * g.P;
        int i = rem / g.OW;
        int j = rem - i * g.OW;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            nb[e] = (rg < BR / 8 && n0 + e < g.N) ? b * g.C * g.H * g.W : -1;
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

template <int BR, int NT_>
struct ImplicitTile16 : Tile16<BR, false, NT_> {
    using Base = Tile16<BR, false, NT_>;
    using Base::NT;
    using Base::PER;
    using Base::SLOTS;
    using Base::r;

    __device__ __forceinline__ void gather(const uint16_t *__restrict__ x, const ConvGeom &g,
                                           const ImplicitCols16<BR, NT_> &cols, int K, int k0, int tid)
    {
        const int *nb = cols.nb, *nh = cols.nh, *nw = cols.nw;
        const int khw = g.kH * g.kW;
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            const int id = s * NT + tid;
            int rg = 0, kq = 0;
            if (id < SLOTS)
                Base::mn_slot(id, rg, kq);
            const bool live = id < SLOTS && rg < BR / 8;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k = k0 + kq * 4 + i;
                u32x4_t v = {0u, 0u, 0u, 0u};
                if (live && k < K) {
                    const int c = k / khw;
                    const int rr = k - c * khw;
                    const int u = rr / g.kW;
                    const int vv = rr - u * g.kW;
                    const int plane = c * g.H * g.W;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const int hh = nh[e] + u, ww = nw[e] + vv;
                        const bool ok = nb[e] >= 0 && hh >= 0 && hh < g.H && ww >= 0 && ww < g.W;
                        const uint32_t hv = ok ? (uint32_t)x[nb[e] + plane + hh * g.W + ww] : 0u;
                        v[e >> 1] |= hv << (16 * (e & 1));
                    }
                }
                r[4 * s + i] = v;
            }
        }
    }

    template <bool VEC>
    __device__ __forceinline__ void store(char *lds, int tid) const
    {
        Base::template store<false>(lds, tid);
    }
};

// 16-byte fragment: row `row`, 8 consecutive k = 16q + 8h .. +7.
__device__ __forceinline__ u32x4_t frag16(const char *lds, int row, int q, int h)
{
    const int ch = 2 * q + h;
    return *(const u32x4_t *)(lds + row * 128 + ((ch ^ swz(row)) << 4));
}

// Epilogue of a wavefront's TM x TN accumulator blocks, whose top-left
// output is (m0, n0): accumulator element e of a 32x32 block is row
// 8*(e/4) + 4*h + (e%4), column l32.  Row-major store (the partials of
// split `split`) or the NCHW store, bias and ReLU as p says (epi_value).
template <int TM, int TN>
__device__ __forceinline__ void store_acc(const GemmParams &p, const f32x16_t (&acc)[TM][TN], int m0, int n0,
                                          int h, int l32, int split)
{
    float *C = p.C + (long long)split * p.c_split_stride;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + j * 32 + l32;
        if (n >= p.N)
            continue;
        long long col_off, row_stride;
        if (p.epi == EPI_NCHW) {
            const int b = n / p.P;
            col_off = (long long)b * p.M * p.P + (n - b * p.P);
            row_stride = p.P;
        } else if (p.epi == EPI_PHASE) {
            const int b = n / p.P, r = n - b * p.P;
            const int i = r / p.g.OW, jj = r - i * p.g.OW;
            row_stride = (long long)p.ph_H * p.ph_W;
            col_off = (long long)b * p.M * row_stride + (long long)(p.ph_h0 + p.ph_s * i) * p.ph_W + p.ph_w0 +
                      p.ph_s * jj;
        } else {
            col_off = n;
            row_stride = p.ldc;
        }
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int m = m0 + i * 32 + 8 * (e >> 2) + 4 * h + (e & 3);
                if (m < p.M)
                    C[col_off + (long long)m * row_stride] = epi_value(acc[i][j][e], p.bias, p.relu, p.epi, m, n);
            }
        }
    }
}

// A_NC / B_NC: the operand is an NCHW tensor (OP_NCHW, or OP_NCHW_K for a
// k-contiguous B), addressed through p.a_ch / p.b_ch and p.g.P.
template <int DTID, int NWM, int NWN, int TM, int TN, bool A_KC, bool B_KC, bool VEC, bool IMPL,
          bool A_NC = false, bool B_NC = false>
__global__ __launch_bounds__(NWM *NWN * 64) void gemm16_kernel(GemmParams p)
{
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32, BK = 64;
    constexpr int NT = NWM * NWN * 64;
    static_assert(NWM * NWN == 4 || NWM * NWN == 8, "four or eight wavefronts per workgroup");
    static_assert(!IMPL || !B_KC, "implicit B uses the row-contiguous path");
    using TA = Tile16<BM, A_KC, NT>;
    using TB = std::conditional_t<IMPL, ImplicitTile16<BN, NT>, Tile16<BN, B_KC, NT>>;
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

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    const uint16_t *A = (const uint16_t *)p.A;
    const uint16_t *B = (const uint16_t *)p.B;
    TA ta0, ta1;
    TB tb0, tb1;

    ImplicitCols16<BN, NT> cols;
    if constexpr (IMPL)
        cols.setup(p.g, n_blk, tid);
    auto load_a = [&](TA &t, int k0) {
        t.template load<VEC, A_NC>(A, p.lda, p.M, kend, m_blk, k0, tid, p.a_ch, p.g.P);
    };
    auto load_b = [&](TB &t, int k0) {
        if constexpr (IMPL)
            t.gather(B, p.g, cols, kend, k0, tid);
        else
            t.template load<VEC, B_NC>(B, p.ldb, p.N, kend, n_blk, k0, tid, p.b_ch, p.g.P);
    };

    auto compute = [&](const char *la, const char *lb) {
#pragma unroll
        for (int q = 0; q < BK / 16; ++q) {
            u32x4_t af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i)
                af[i] = frag16(la, (wm * TM + i) * 32 + l32, q, h);
#pragma unroll
            for (int j = 0; j < TN; ++j)
                bf[j] = frag16(lb, (wn * TN + j) * 32 + l32, q, h);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = mfma16<DTID>(af[i], bf[j], acc[i][j]);
        }
    };

    if (nk > 0) {
        // prologue: stages 0 and 1 in flight, stage 0 into LDS buffer 0
        load_a(ta0, kbeg);
        load_b(tb0, kbeg);
        load_a(ta1, kbeg + BK);
        load_b(tb1, kbeg + BK);
        ta0.template store<VEC>(smem, tid);
        tb0.template store<VEC>(smem + TA::LDS_BYTES, tid);
        __syncthreads();
        load_a(ta0, kbeg + 2 * BK);
        load_b(tb0, kbeg + 2 * BK);
        // Stage t is computed from LDS buffer t&1.  Register set (t+1)&1 holds
        // stage t+1 and is stored into LDS buffer (t+1)&1 after the compute;
        // it is then refilled with stage t+3.  Two stages per iteration keep
        // each register set in fixed registers; an odd last stage is peeled.
        // Loads and stores are unconditional (a stage past the end has every
        // k >= kend: it reads nothing and stores zeros), and a scheduling
        // barrier keeps each stage's loads right after the workgroup barrier,
        // so two stages of loads stay in flight during each compute.
        int t = 0;
        for (; t + 1 < nk; t += 2) {
            compute(smem, smem + TA::LDS_BYTES);
            ta1.template store<VEC>(smem + STAGE, tid);
            tb1.template store<VEC>(smem + STAGE + TA::LDS_BYTES, tid);
            __syncthreads();
            load_a(ta1, kbeg + (t + 3) * BK);
            load_b(tb1, kbeg + (t + 3) * BK);
            __builtin_amdgcn_sched_barrier(0);
            compute(smem + STAGE, smem + STAGE + TA::LDS_BYTES);
            ta0.template store<VEC>(smem, tid);
            tb0.template store<VEC>(smem + TA::LDS_BYTES, tid);
            __syncthreads();
            load_a(ta0, kbeg + (t + 4) * BK);
            load_b(tb0, kbeg + (t + 4) * BK);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (t < nk)
            compute(smem, smem + TA::LDS_BYTES);
    }

    store_acc<TM, TN>(p, acc, m_blk + wm * TM * 32, n_blk + wn * TN * 32, h, l32, wi.split);
}

// ---------------------------------------------------------------------------
// Direct-to-LDS variant for two k-contiguous operands (128x256 and 256x128
// tiles, eight wavefronts).  Every 16-byte chunk goes from global memory
// straight into LDS (global_load_lds_dwordx4: lane i of a wavefront writes
// bytes [16i, 16i+16) after the wavefront's LDS base), so no registers stage
// the tiles and no LDS store instructions are issued.  A stage is 64 k deep:
// LDS [row][k] with 128-byte rows, chunk c of row r at position c ^ swz(r);
// the loading lane fetches the permuted global chunk, so the swizzle costs
// nothing and a fragment is one conflict-free 16-byte read.  A ring of NBUF
// LDS stages keeps NBUF-1 stages of loads in flight; one barrier per stage.
// (Row-contiguous operands loaded the same way as [k][row] and read with
// ds_read_b64_tr_b16 measured 5-15% slower than the register-transpose
// path: twice the LDS read instructions per fragment, more waits.)
// Requirements (checked by the launcher): 16-byte aligned rows, every split
// a whole number of stages.  Rows past M or N load a clamped row; they only
// reach outputs that the epilogue masks.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) const void gbl_void_t;

constexpr int kDlBK = 64;  // k per stage, 16-bit operands (f32: 32)

// Element type of the direct-to-LDS kernel's operands: 16-bit halves, or
// f32 words (DT_F32).  A stage is one 128-byte LDS row per tile row, i.e.
// 64 halves or 32 floats; a 16-byte chunk holds EPC elements.
template <int DTID>
struct DlElem {
    using T = std::conditional_t<DTID == DT_F32, uint32_t, uint16_t>;
    static constexpr int EPC = 16 / (int)sizeof(T);
    static constexpr int BK = 8 * EPC;
};

// 16-byte chunk c of row `row` of a tile stage (swizzled position)
__device__ __forceinline__ u32x4_t dl_chunk(const char *lds, int row, int c)
{
    return *(const u32x4_t *)(lds + row * 128 + ((c ^ swz(row)) << 4));
}

// Per-lane load offsets of one k-contiguous operand (BR rows of the tile,
// NW wavefronts): a wavefront load covers 8 rows of 128 bytes.
template <int BR, int NW, int DTID>
struct DlOperand {
    using T = typename DlElem<DTID>::T;
    static constexpr int EPC = DlElem<DTID>::EPC;
    static constexpr int ROWB = 128;                // bytes per LDS row
    static constexpr int LPL = 8;                   // rows per wavefront load
    static constexpr int LD = BR / (LPL * NW);      // loads per wavefront per stage
    static constexpr int BYTES = BR * ROWB;
    static_assert(BR % (LPL * NW) == 0, "whole load groups");

    long long off[LD];  // element offset of this lane's chunk, k0 excluded

    __device__ __forceinline__ void setup(int r0, int R, int ld, int wave, int lane)
    {
#pragma unroll
        for (int j = 0; j < LD; ++j) {
            const int lr = (j * NW + wave) * LPL + lane / 8;  // tile row
            const int gr = min(r0 + lr, R - 1);
            off[j] = (long long)gr * ld + ((lane % 8) ^ swz(lr)) * EPC;
        }
    }

    // stage starting at k0 into LDS stage base `lds`
    __device__ __forceinline__ void issue(const T *X, int k0, char *lds, int wave) const
    {
#pragma unroll
        for (int j = 0; j < LD; ++j)
            __builtin_amdgcn_global_load_lds((gbl_void_t *)(X + off[j] + k0),
                                             (lds_void_t *)(lds + (j * NW + wave) * LPL * ROWB), 16, 0, 0);
    }
};

// B operand of the implicit GEMM over an NHWC tensor t[b][h][w][c] (OP_IMPL_T,
// geometry g, stride 1): tile row n = (b, i, j) is an output pixel and a
// stage covers channels c0 .. c0+BK-1 of one tap (u, v), so each row's stage
// is one contiguous 128-byte run of t at (b, i-p+u, j-p+v, c0), or the zero
// page when that position is in the padding.  The same lane-to-LDS mapping
// and swizzle as DlOperand; a lane decodes its rows' pixels once and each
// stage's tap once.
template <int BR, int NW, int DTID>
struct DlImplNhwc {
    using T = typename DlElem<DTID>::T;
    static constexpr int EPC = DlElem<DTID>::EPC;
    static constexpr int BK = DlElem<DTID>::BK;
    static constexpr int ROWB = 128;
    static constexpr int LPL = 8;
    static constexpr int LD = BR / (LPL * NW);
    static constexpr int BYTES = BR * ROWB;
    static_assert(BR % (LPL * NW) == 0, "whole load groups");

    // per load: window origin (h0 far negative for rows past N, so no tap
    // is ever in range) and the element offset of the origin's channel
    // chunk, ((b*H + h0)*W + w0)*C + chunk*EPC; a stage adds its tap's
    // uniform offset (u*W + v)*C + c0
    int h0[LD], w0[LD];
    long long base[LD];

    __device__ __forceinline__ void setup(int n0, const ConvGeom &g, int wave, int lane)
    {
#pragma unroll
        for (int j = 0; j < LD; ++j) {
            const int lr = (j * NW + wave) * LPL + lane / 8;
            const int n = n0 + lr;
            const int chk = (lane % 8) ^ swz(lr);
            const int bb = n / g.P, r = n - (n / g.P) * g.P;
            const int i = r / g.OW;
            h0[j] = n < g.N ? i - g.p : -(1 << 30);
            w0[j] = r - i * g.OW - g.pw;
            base[j] = (((long long)bb * g.H + (i - g.p)) * g.W + w0[j]) * g.C + chk * EPC;
        }
    }

    __device__ __forceinline__ void issue(const T *X, const T *zero, int k0, char *lds, int wave,
                                          const ConvGeom &g) const
    {
        // k0 is a whole stage: BK channels of one tap, stages ordered by
        // channel block, then tap (so the taps of one block reread its
        // channels at shifted pixels while they are in cache); divisors
        // kH*kW, kW <= 1024 and stage index < 2^20 (checked by the host).
        // The chunk's offset inside the zero page is base mod BK (C is a
        // multiple of BK).
        const int ks = k0 / BK, taps = g.kH * g.kW;
        const int cblk = small_div(ks, taps), tap = ks - cblk * taps, c0 = cblk * BK;
        const int u = small_div(tap, g.kW), v = tap - u * g.kW;
        const long long toff = ((long long)u * g.W + v) * g.C + c0;
#pragma unroll
        for (int j = 0; j < LD; ++j) {
            const bool ok = (unsigned)(h0[j] + u) < (unsigned)g.H && (unsigned)(w0[j] + v) < (unsigned)g.W;
            const T *src = ok ? X + base[j] + toff : zero + (base[j] & (BK - 1));
            __builtin_amdgcn_global_load_lds((gbl_void_t *)src, (lds_void_t *)(lds + (j * NW + wave) * LPL * ROWB),
                                             16, 0, 0);
        }
    }
};

// BI: B is OP_IMPL_T (DlImplNhwc) instead of a k-contiguous matrix.
// 16-bit: one 16-byte fragment per 16 k and one v_mfma_f32_32x32x16; f32
// (DTID == DT_F32): floats k = 16q + 8h .. +7 from two chunks and eight
// v_mfma_f32_32x32x2_f32 (lane half h supplies k = 8h + t of step t for
// both operands, so every k is summed once).
// One output tile (m_blk, n_blk) over k in [kbeg, kend) of split `split`.
template <int DTID, int NWM, int NWN, int TM, int TN, int NBUF, bool BI>
__device__ __forceinline__ void dl_gemm_tile(const GemmParams &p, int m_blk, int n_blk, int kbeg, int kend,
                                             int split)
{
    using E = DlElem<DTID>;
    using T = typename E::T;
    constexpr int NW = NWM * NWN;
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32, BK = E::BK;
    using OA = DlOperand<BM, NW, DTID>;
    using OB = std::conditional_t<BI, DlImplNhwc<BN, NW, DTID>, DlOperand<BN, NW, DTID>>;
    constexpr int STAGE = OA::BYTES + OB::BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % NWM, wn = wave / NWM;
    const int h = lane >> 5, l32 = lane & 31;
    const int nk = (kend - kbeg) / BK;

    const T *A = (const T *)p.A;
    const T *B = (const T *)p.B;
    OA oa;
    OB ob;
    oa.setup(m_blk, p.M, p.lda, wave, lane);
    if constexpr (BI)
        ob.setup(n_blk, p.g, wave, lane);
    else
        ob.setup(n_blk, p.N, p.ldb, wave, lane);
    // stage s (clamped to the first stage past the end: its slot is never
    // read) into ring slot s % NBUF
    auto issue = [&](int s) {
        const int k0 = kbeg + (s < nk ? s : 0) * BK;
        char *base = smem + (s % NBUF) * STAGE;
        oa.issue(A, k0, base, wave);
        if constexpr (BI)
            ob.issue(B, (const T *)p.zero, k0, base + OA::BYTES, wave, p.g);
        else
            ob.issue(B, k0, base + OA::BYTES, wave);
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    // NBUF-1 stages are issued ahead; at the top of iteration t the loads of
    // stages t+1 .. t+NBUF-2 may still be in flight, stage t's must be done
    constexpr int LPS = OA::LD + OB::LD;
    constexpr int VM = (NBUF - 2) * LPS;
    static_assert(VM < 64, "vmcnt range");
    constexpr int WAIT = (VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8);

#pragma unroll
    for (int s0 = 0; s0 < NBUF - 1; ++s0)
        issue(s0);
    for (int t = 0; t < nk; ++t) {
        // Stage t has landed (this wavefront's share; the barrier makes it
        // everyone's) and every wavefront is done reading slot
        // (t+NBUF-1) % NBUF.  A plain s_barrier: the workgroup fence of
        // __syncthreads would wait for all loads in flight, LDS-bound ones
        // included.  The empty asm keeps the compiler from moving LDS
        // accesses across it.
        __builtin_amdgcn_s_waitcnt(WAIT);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        issue(t + NBUF - 1);
        // Raised wave priority over the stage's LDS reads and MFMAs: where
        // two workgroups share a CU, the arbiter then favours the wavefront
        // that has MFMA work over one that is issuing loads or about to
        // wait (fp32 filter gradient 184 -> 180 us, 16-bit 128x128 data
        // gradient 38.0 -> 36.0 us; level on the eight-wavefront tiles).
        __builtin_amdgcn_s_setprio(1);
        const char *la = smem + (t % NBUF) * STAGE;
        const char *lb = la + OA::BYTES;
        if constexpr (DTID == DT_F32) {
#pragma unroll
            for (int q = 0; q < BK / 16; ++q) {
                u32x4_t af[TM][2], bf[TN][2];
#pragma unroll
                for (int i = 0; i < TM; ++i) {
                    af[i][0] = dl_chunk(la, (wm * TM + i) * 32 + l32, 4 * q + 2 * h);
                    af[i][1] = dl_chunk(la, (wm * TM + i) * 32 + l32, 4 * q + 2 * h + 1);
                }
#pragma unroll
                for (int j = 0; j < TN; ++j) {
                    bf[j][0] = dl_chunk(lb, (wn * TN + j) * 32 + l32, 4 * q + 2 * h);
                    bf[j][1] = dl_chunk(lb, (wn * TN + j) * 32 + l32, 4 * q + 2 * h + 1);
                }
#pragma unroll
                for (int tt = 0; tt < 8; ++tt)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(
                                __uint_as_float(af[i][tt >> 2][tt & 3]), __uint_as_float(bf[j][tt >> 2][tt & 3]),
                                acc[i][j], 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int q = 0; q < BK / 16; ++q) {
                u32x4_t af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = dl_chunk(la, (wm * TM + i) * 32 + l32, 2 * q + h);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bf[j] = dl_chunk(lb, (wn * TN + j) * 32 + l32, 2 * q + h);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = mfma16<DTID>(af[i], bf[j], acc[i][j]);
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }
    // drain the loads of the stages past the end before the workgroup exits
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));

    store_acc<TM, TN>(p, acc, m_blk + wm * TM * 32, n_blk + wn * TN * 32, h, l32, split);
}

// 16-bit tile with the fragment reads pipelined one 16-deep k step ahead.
// In the plain loop every wavefront leaves the stage barrier with its
// SIMD partner, and both read a step's fragments and wait for them before
// that step's MFMAs, so the LDS latency is paid with the MFMA units idle
// once per step.  Here step q reads the fragments of step q+1 (into the
// other register set) before its own MFMAs, which use fragments read a step
// earlier; the stage barrier moves into the last step, after which that
// step reads step 0 of the next stage.  Scheduling hints keep that order
// (the compiler otherwise moves each read next to its use).  The loads of
// stage t+NBUF-1 go out in step 0 of stage t, interleaved with its MFMAs,
// into the slot of stage t-1, whose last reads came before the barrier in
// stage t-1's last step (which also waits for this wavefront's reads).
// Stages past the end load stage 0 again into slots never used.
template <int DTID, int NWM, int NWN, int TM, int TN, int NBUF, bool BI>
__device__ __forceinline__ void dl_gemm_tile16p(const GemmParams &p, int m_blk, int n_blk, int kbeg, int kend,
                                                int split)
{
    using E = DlElem<DTID>;
    using T = typename E::T;
    static_assert(DTID != DT_F32, "16-bit operands");
    constexpr int NW = NWM * NWN;
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32, BK = E::BK;
    constexpr int NQ = BK / 16;
    using OA = DlOperand<BM, NW, DTID>;
    using OB = std::conditional_t<BI, DlImplNhwc<BN, NW, DTID>, DlOperand<BN, NW, DTID>>;
    constexpr int STAGE = OA::BYTES + OB::BYTES;
    __shared__ __attribute__((aligned(1024))) char smem[NBUF * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % NWM, wn = wave / NWM;
    const int h = lane >> 5, l32 = lane & 31;
    const int nk = (kend - kbeg) / BK;

    const T *A = (const T *)p.A;
    const T *B = (const T *)p.B;
    OA oa;
    OB ob;
    oa.setup(m_blk, p.M, p.lda, wave, lane);
    if constexpr (BI)
        ob.setup(n_blk, p.g, wave, lane);
    else
        ob.setup(n_blk, p.N, p.ldb, wave, lane);
    auto issue = [&](int st) {
        const int k0 = kbeg + (st < nk ? st : 0) * BK;
        char *base = smem + (st % NBUF) * STAGE;
        oa.issue(A, k0, base, wave);
        if constexpr (BI)
            ob.issue(B, (const T *)p.zero, k0, base + OA::BYTES, wave, p.g);
        else
            ob.issue(B, k0, base + OA::BYTES, wave);
    };

    f32x16_t acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                acc[i][j][e] = 0.0f;

    constexpr int LPS = OA::LD + OB::LD;
    constexpr int VM = (NBUF - 2) * LPS;
    static_assert(VM < 64, "vmcnt range");
    constexpr int VMF = (VM & 15) | ((VM >> 4) << 14);
    constexpr int WAIT_LANDED = VMF | (7 << 4) | (15 << 8);  // vmcnt(VM)
    constexpr int WAIT_STAGE = VMF | (7 << 4);               // vmcnt(VM), lgkmcnt(0)
    u32x4_t fa[2][TM], fb[2][TN];
    auto read = [&](u32x4_t(&ra)[TM], u32x4_t(&rb)[TN], const char *slot, int q) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
            ra[i] = dl_chunk(slot, (wm * TM + i) * 32 + l32, 2 * q + h);
#pragma unroll
        for (int j = 0; j < TN; ++j)
            rb[j] = dl_chunk(slot + OA::BYTES, (wn * TN + j) * 32 + l32, 2 * q + h);
    };

#pragma unroll
    for (int s0 = 0; s0 < NBUF - 1; ++s0)
        issue(s0);
    __builtin_amdgcn_s_waitcnt(WAIT_LANDED);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    read(fa[0], fb[0], smem, 0);
    for (int t = 0; t < nk; ++t) {
        const char *cur = smem + (t % NBUF) * STAGE;
        const char *nxt = smem + ((t + 1) % NBUF) * STAGE;
        auto step = [&](auto qc) {
            constexpr int q = decltype(qc)::value;
            constexpr int RD = TM + TN, MF = TM * TN, H1 = MF / 2;
            constexpr int LD_ = q == 0 ? LPS : 0;
            constexpr int PER = (LD_ + H1 - 1) / H1;  // stage loads per MFMA of the first half
            constexpr int C = q & 1, Nn = (q + 1) & 1;
            // step 0 first issues the stage loads: an LDS-writing load waits
            // for every LDS read in flight, which here are only this step's
            // own fragments
            if constexpr (q == 0)
                issue(t + NBUF - 1);
#pragma unroll
            for (int x = 0; x < H1; ++x)
                acc[x / TN][x % TN] = mfma16<DTID>(fa[C][x / TN], fb[C][x % TN], acc[x / TN][x % TN]);
            if constexpr (q + 1 < NQ) {
                read(fa[Nn], fb[Nn], cur, q + 1);
            } else {
                __builtin_amdgcn_sched_barrier(0);
                __builtin_amdgcn_s_waitcnt(WAIT_STAGE);
                __builtin_amdgcn_s_barrier();
                asm volatile("" ::: "memory");
                __builtin_amdgcn_sched_barrier(0);
                read(fa[Nn], fb[Nn], nxt, 0);
            }
#pragma unroll
            for (int x = H1; x < MF; ++x)
                acc[x / TN][x % TN] = mfma16<DTID>(fa[C][x / TN], fb[C][x % TN], acc[x / TN][x % TN]);
            // order (masks: 0x008 MFMA, 0x100 LDS read, 0x020 global load):
            // first half of the MFMAs (with the stage loads between them in
            // step 0), the next fragments, the second half
            if constexpr (q + 1 < NQ) {
#pragma unroll
                for (int r = 0; r < H1; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if constexpr (PER > 0)
                        __builtin_amdgcn_sched_group_barrier(0x020, PER, 0);
                }
            }
            __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, MF - (q + 1 < NQ ? H1 : 0), 0);
            __builtin_amdgcn_sched_barrier(0);
        };
        static_assert(NQ == 4, "four k steps per stage");
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
    }
    // drain the loads of the stages past the end before the workgroup exits
    __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
    store_acc<TM, TN>(p, acc, m_blk + wm * TM * 32, n_blk + wn * TN * 32, h, l32, split);
}

// PIPE (16-bit): dl_gemm_tile16p instead of dl_gemm_tile.
template <int DTID, int NWM, int NWN, int TM, int TN, int NBUF, bool BI = false, bool PIPE = (DTID != DT_F32)>
__global__ __launch_bounds__(NWM *NWN * 64) void gemm_dl_kernel(GemmParams p)
{
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32;
    const int mt = (p.M + BM - 1) / BM, nt = (p.N + BN - 1) / BN;
    const WorkItem wi = xcd_work(blockIdx.x, mt * nt, p.splits);
    const int kbeg = wi.split * p.k_per_split;
    int tm, tn;
    tile_mn(wi.tile, mt, nt, p.group_m, tm, tn);
    if constexpr (PIPE)
        dl_gemm_tile16p<DTID, NWM, NWN, TM, TN, NBUF, BI>(p, tm * BM, tn * BN, kbeg,
                                                          min(p.K, kbeg + p.k_per_split), wi.split);
    else
        dl_gemm_tile<DTID, NWM, NWN, TM, TN, NBUF, BI>(p, tm * BM, tn * BN, kbeg, min(p.K, kbeg + p.k_per_split),
                                                       wi.split);
}

// Every phase of a strided data gradient in one launch: work item w (after
// the XCD renumbering) belongs to the last phase whose first item is <= w;
// that phase's filter, K, sub-convolution geometry and dx placement replace
// the launch-wide ones.  No split: the phases' K are short.
// PIPE (16-bit): the pipelined tile loop (dl_gemm_tile16p).
template <int DTID, int NWM, int NWN, int TM, int TN, int NBUF, bool PIPE = false>
__global__ __launch_bounds__(NWM *NWN * 64) void gemm_dl_phased_kernel(GemmParams p, PhaseArgs pa)
{
    using T = typename DlElem<DTID>::T;
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32;
    const int w = xcd_tile(blockIdx.x, pa.tiles);
    int k = 0;
    while (k + 1 < pa.n && w >= pa.ph[k + 1].tile0)
        ++k;
    const PhaseItem &it = pa.ph[k];
    GemmParams q = p;
    q.A = (const T *)p.A + it.a_off;
    q.K = it.K;
    q.lda = it.K;
    q.k_per_split = it.K;
    q.splits = 1;
    q.g = it.g;
    q.N = it.g.N;
    q.P = it.g.P;
    q.ph_h0 = it.h0;
    q.ph_w0 = it.w0;
    const int mt = (p.M + BM - 1) / BM;
    const int local = w - it.tile0;
    if constexpr (PIPE)
        dl_gemm_tile16p<DTID, NWM, NWN, TM, TN, NBUF, true>(q, (local % mt) * BM, (local / mt) * BN, 0, it.K, 0);
    else
        dl_gemm_tile<DTID, NWM, NWN, TM, TN, NBUF, true>(q, (local % mt) * BM, (local / mt) * BN, 0, it.K, 0);
}

// Loop of the 16-bit direct-to-LDS kernels: pipelined fragment reads
// (dl_gemm_tile16p) unless D4R_DL16_PIPE=0 (the plain loop, kept for
// comparison and tests).
inline bool dl16_pipe()
{
    const char *e = getenv("D4R_DL16_PIPE");
    return !(e && e[0] == '0');
}

// All phases of a strided data gradient in one launch on 128x128 tiles:
// 16-bit as eight wavefronts of 64x32 with a ring of four stages, f32 as
// four wavefronts of 64x64 with a ring of two (the forms the NHWC data
// gradient uses).  The host checks that every phase's K is a whole number
// of stages and that the NHWC loader's divisions are in range.
template <int DTID>
hipError_t launch_gemm_dl_phased(const GemmParams &p, const PhaseArgs &pa, hipStream_t s)
{
    if (pa.n < 1 || pa.n > kMaxPhases || pa.tiles < 1 || !p.zero)
        return hipErrorInvalidValue;
    if constexpr (DTID == DT_F32) {
        hipLaunchKernelGGL((gemm_dl_phased_kernel<DTID, 2, 2, 2, 2, 2>), dim3(pa.tiles), dim3(256), 0, s, p, pa);
    } else {
        if (dl16_pipe())
            hipLaunchKernelGGL((gemm_dl_phased_kernel<DTID, 2, 4, 2, 1, 4, true>), dim3(pa.tiles), dim3(512), 0, s,
                               p, pa);
        else
            hipLaunchKernelGGL((gemm_dl_phased_kernel<DTID, 2, 4, 2, 1, 4, false>), dim3(pa.tiles), dim3(512), 0, s,
                               p, pa);
    }
    return hipGetLastError();
}

// 64-deep stages in a ring of three (two stages of loads in flight):
// measured level with 32-deep stages in a ring of four, with half the
// barriers.
constexpr int kDlBuf = 3;

// The direct-to-LDS kernel applies to two k-contiguous operands with
// 16-byte aligned rows (the VEC condition) whose splits are whole stages.
inline bool dl_applies(int amode, int bmode, const GemmParams &p)
{
    return amode == OP_KC && bmode == OP_KC && p.a_vec && p.b_vec && p.K % kDlBK == 0 &&
           p.k_per_split % kDlBK == 0;
}

template <int DTID, bool BI, bool PIPE>
hipError_t launch_gemm16_dl_form(int cfg, const GemmParams &p, hipStream_t s)
{
    TileShape ts = tile_shape(cfg);
    const int tiles = ((p.M + ts.bm - 1) / ts.bm) * ((p.N + ts.bn - 1) / ts.bn);
    const dim3 grid(tiles * p.splits), b8(512);
    switch (cfg) {
    case TILE_128x256:
        hipLaunchKernelGGL((gemm_dl_kernel<DTID, 2, 4, 2, 2, kDlBuf, BI, PIPE>), grid, b8, 0, s, p);
        break;
    case TILE_256x128:
        hipLaunchKernelGGL((gemm_dl_kernel<DTID, 4, 2, 2, 2, kDlBuf, BI, PIPE>), grid, b8, 0, s, p);
        break;
    case TILE_256x256:
        // eight wavefronts of 128x64, a ring of two 64 KB stages (one
        // workgroup per CU): a third less operand traffic per flop than
        // 128x256 (4096^3 bf16 780 -> 977 TFLOP/s)
        hipLaunchKernelGGL((gemm_dl_kernel<DTID, 2, 4, 4, 2, 2, BI, PIPE>), grid, b8, 0, s, p);
        break;
    case TILE_128x128: {
        const Dl128Form f = dl128_form();
        if (f.waves == 4)
            // four wavefronts, a ring of two stages (64 KB): two workgroups per CU
            hipLaunchKernelGGL((gemm_dl_kernel<DTID, 2, 2, 2, 2, 2, BI, PIPE>), grid, dim3(256), 0, s, p);
        else if (f.nbuf == 2)
            hipLaunchKernelGGL((gemm_dl_kernel<DTID, 2, 4, 2, 1, 2, BI, PIPE>), grid, b8, 0, s, p);
        else if (f.nbuf == 3)
            hipLaunchKernelGGL((gemm_dl_kernel<DTID, 2, 4, 2, 1, 3, BI, PIPE>), grid, b8, 0, s, p);
        else
            hipLaunchKernelGGL((gemm_dl_kernel<DTID, 2, 4, 2, 1, 4, BI, PIPE>), grid, b8, 0, s, p);
        break;
    }
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DTID, bool BI = false>
hipError_t launch_gemm16_dl(int cfg, const GemmParams &p, hipStream_t s)
{
    if (dl16_pipe())
        return launch_gemm16_dl_form<DTID, BI, true>(cfg, p, s);
    return launch_gemm16_dl_form<DTID, BI, false>(cfg, p, s);
}

template <int DTID, bool A_KC, bool B_KC, bool VEC, bool IMPL = false, bool A_NC = false, bool B_NC = false>
hipError_t launch_gemm16_vec(int cfg, const GemmParams &p, hipStream_t s)
{
    TileShape ts = tile_shape(cfg);
    const int tiles = ((p.M + ts.bm - 1) / ts.bm) * ((p.N + ts.bn - 1) / ts.bn);
    const dim3 grid(tiles * p.splits), b4(256), b8(512);
    switch (cfg) {
    case TILE_128x128:
        hipLaunchKernelGGL((gemm16_kernel<DTID, 2, 2, 2, 2, A_KC, B_KC, VEC, IMPL, A_NC, B_NC>), grid, b4, 0, s,
                           p);
        break;
    case TILE_64x64:
        hipLaunchKernelGGL((gemm16_kernel<DTID, 2, 2, 1, 1, A_KC, B_KC, VEC, IMPL, A_NC, B_NC>), grid, b4, 0, s,
                           p);
        break;
    case TILE_32x128:
        hipLaunchKernelGGL((gemm16_kernel<DTID, 1, 4, 1, 1, A_KC, B_KC, VEC, IMPL, A_NC, B_NC>), grid, b4, 0, s,
                           p);
        break;
    case TILE_96x128:
        hipLaunchKernelGGL((gemm16_kernel<DTID, 1, 4, 3, 1, A_KC, B_KC, VEC, IMPL, A_NC, B_NC>), grid, b4, 0, s,
                           p);
        break;
    // the large tiles run eight wavefronts, two per SIMD, so one wave's
    // waits are covered by the other's MFMAs
    case TILE_128x256:
        hipLaunchKernelGGL((gemm16_kernel<DTID, 2, 4, 2, 2, A_KC, B_KC, VEC, IMPL, A_NC, B_NC>), grid, b8, 0, s,
                           p);
        break;
    case TILE_256x128:
        hipLaunchKernelGGL((gemm16_kernel<DTID, 4, 2, 2, 2, A_KC, B_KC, VEC, IMPL, A_NC, B_NC>), grid, b8, 0, s,
                           p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int DTID, bool A_KC, bool B_KC, bool A_NC = false, bool B_NC = false>
hipError_t launch_gemm16_layout(int cfg, const GemmParams &p, hipStream_t s)
{
    if (p.a_vec && p.b_vec)
        return launch_gemm16_vec<DTID, A_KC, B_KC, true, false, A_NC, B_NC>(cfg, p, s);
    return launch_gemm16_vec<DTID, A_KC, B_KC, false, false, A_NC, B_NC>(cfg, p, s);
}

// Supported (A, B) modes: every pair of OP_ROWS / OP_KC, (OP_KC, OP_IMPL)
// for the implicit forward (VEC then covers A only), and the NCHW pairs of
// a 1x1 stride-1 unpadded convolution: (OP_KC, OP_NCHW) forward, (OP_ROWS,
// OP_NCHW) data gradient, (OP_NCHW, OP_NCHW_K) filter gradient.
template <int DTID>
hipError_t launch_gemm16(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    // 256x256 exists only on the direct-to-LDS kernel: 128x256 elsewhere
    // (the grid follows the tile; the split plan stays valid)
    if (cfg == TILE_256x256 && bmode != OP_IMPL_T && !dl_applies(amode, bmode, p))
        cfg = TILE_128x256;
    if (bmode == OP_IMPL_T) {
        // direct-to-LDS only: a k-contiguous A, whole 64-deep stages, each
        // inside one tap
        if (amode != OP_KC || !p.a_vec || p.K % kDlBK != 0 || p.k_per_split % kDlBK != 0 || p.g.C % kDlBK != 0 ||
            p.g.s != 1 || !p.zero)
            return hipErrorInvalidValue;
        return launch_gemm16_dl<DTID, true>(cfg, p, s);
    }
    if (amode == OP_KC && bmode == OP_IMPL) {
        if (p.a_vec)
            return launch_gemm16_vec<DTID, true, false, true, true>(cfg, p, s);
        return launch_gemm16_vec<DTID, true, false, false, true>(cfg, p, s);
    }
    if (amode == OP_KC && bmode == OP_NCHW)
        return launch_gemm16_layout<DTID, true, false, false, true>(cfg, p, s);
    if (amode == OP_ROWS && bmode == OP_NCHW)
        return launch_gemm16_layout<DTID, false, false, false, true>(cfg, p, s);
    if (amode == OP_NCHW && bmode == OP_NCHW_K)
        return launch_gemm16_layout<DTID, true, true, true, true>(cfg, p, s);
    const bool a_ok = amode == OP_ROWS || amode == OP_KC;
    const bool b_ok = bmode == OP_ROWS || bmode == OP_KC;
    if (!a_ok || !b_ok)
        return hipErrorInvalidValue;
    const bool a_kc = amode == OP_KC, b_kc = bmode == OP_KC;
    if ((cfg == TILE_128x256 || cfg == TILE_256x128 || cfg == TILE_256x256 ||
         (cfg == TILE_128x128 && dl128_enabled())) &&
        dl_applies(amode, bmode, p))
        return launch_gemm16_dl<DTID>(cfg, p, s);
    if (a_kc && b_kc)
        return launch_gemm16_layout<DTID, true, true>(cfg, p, s);
    if (a_kc && !b_kc)
        return launch_gemm16_layout<DTID, true, false>(cfg, p, s);
    if (!a_kc && b_kc)
        return launch_gemm16_layout<DTID, false, true>(cfg, p, s);
    return launch_gemm16_layout<DTID, false, false>(cfg, p, s);
}

}  // namespace d4r
