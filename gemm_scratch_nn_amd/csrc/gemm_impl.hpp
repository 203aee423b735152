// MFMA GEMM for gfx950: C(f32) = op(A) * op(B) with the transpose flags of
// the directcompute-nn page ("Matmul Shaders", "Transpose via Flags").
//
// Design (CDNA4, 64-lane wavefronts):
//  * A workgroup of NWM x NWN wavefronts computes a BM x BN tile; each
//    wavefront owns TM x TN blocks of 32x32 outputs held in MFMA
//    accumulators (16 floats per lane per block).
//  * f32 operands use v_mfma_f32_32x32x2_f32; f16 / bf16 operands use the
//    gfx950 v_mfma_f32_32x32x16_{f16,bf16}.  Accumulation is f32 throughout.
//  * Each K stage (BK = 128 bytes of k per operand row) is loaded from global
//    memory with 16-byte vector loads into registers one stage ahead, then
//    written to one of two LDS buffers, so each stage costs one barrier.
//  * LDS layout follows the global layout: an operand stored with k
//    contiguous is kept as [row][k] (row pitch padded by 16 bytes so the
//    16-byte fragment reads of 8 consecutive rows hit distinct banks); an
//    operand stored row-contiguous is kept as [k][row] and read one element
//    per lane per k.
//  * Only the sum over k matters to the result, so lane-half h of a
//    fragment takes k = 8h..8h+7 of each 16-wide k group, the same mapping
//    for A and B.
//  * Out-of-range rows and k are zero-filled in LDS; the MFMAs run on whole
//    blocks and the epilogue masks the stores.
//  * Workgroups are renumbered so that consecutive tiles share an XCD (and
//    its L2).
#pragma once

#include <type_traits>

#include "internal.hpp"

namespace d4r {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

struct DtF32 { static constexpr int ES = 4; static constexpr int ID = DT_F32; };
struct DtF16 { static constexpr int ES = 2; static constexpr int ID = DT_F16; };
struct DtBF16 { static constexpr int ES = 2; static constexpr int ID = DT_BF16; };

template <class DT>
struct GemmTraits {
    static constexpr int ES = DT::ES;
    static constexpr int VW = 16 / ES;      // elements per 16-byte vector
    static constexpr int BK = 128 / ES;     // k depth of one stage
    static constexpr int PAD = 16 / ES;     // 16 bytes of row padding
};

// One operand's global -> register -> LDS path.
//   KC = true : global X[r*ld + k], LDS [r][k] with pitch BK + PAD
//   KC = false: global X[k*ld + r], LDS [k][r] with pitch BR + PAD
template <class DT, int BR, bool KC, int NT>
struct OperandTile {
    using TR = GemmTraits<DT>;
    static constexpr int ES = TR::ES, VW = TR::VW, BK = TR::BK, PAD = TR::PAD;
    static constexpr int PITCH = KC ? (BK + PAD) : (BR + PAD);
    static constexpr int LDS_BYTES = (KC ? BR : BK) * PITCH * ES;
    static constexpr int NV = BR * BK / VW;
    static constexpr int PER = (NV + NT - 1) / NT;

    u32x4 reg[PER];

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

    __device__ __forceinline__ void load(const char *__restrict__ base, int ld, int R, int K,
                                         int r0, int k0, bool vec_ok, int tid)
    {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            int id = s * NT + tid;
            if (NV % NT != 0 && id >= NV)
                break;
            int row, kk;
            slot(id, row, kk);
            int r = r0 + row, k = k0 + kk;
            bool full;
            long long off;
            if (KC) {
                full = vec_ok && r < R && k + VW <= K;
                off = (long long)r * ld + k;
            } else {
                full = vec_ok && k < K && r + VW <= R;
                off = (long long)k * ld + r;
            }
            if (full) {
                reg[s] = *(const u32x4 *)(base + off * ES);
            } else {
                u32x4 v = {0u, 0u, 0u, 0u};
                if (ES == 4) {
                    const uint32_t *p = (const uint32_t *)base;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        bool ok = KC ? (r < R && k + e < K) : (k < K && r + e < R);
                        long long o = KC ? ((long long)r * ld + k + e) : ((long long)k * ld + r + e);
                        v[e] = ok ? p[o] : 0u;
                    }
                } else {
                    const uint16_t *p = (const uint16_t *)base;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        bool ok = KC ? (r < R && k + e < K) : (k < K && r + e < R);
                        long long o = KC ? ((long long)r * ld + k + e) : ((long long)k * ld + r + e);
                        uint32_t h = ok ? (uint32_t)p[o] : 0u;
                        v[e >> 1] |= h << (16 * (e & 1));
                    }
                }
                reg[s] = v;
            }
        }
    }

    __device__ __forceinline__ void store(char *lds, int tid) const
    {
#pragma unroll
        for (int s = 0; s < PER; ++s) {
            int id = s * NT + tid;
            if (NV % NT != 0 && id >= NV)
                break;
            int row, kk;
            slot(id, row, kk);
            int e = KC ? (row * PITCH + kk) : (kk * PITCH + row);
            *(u32x4 *)(lds + e * ES) = reg[s];
        }
    }
};

// Forward-GEMM B operand gathered straight from x (the implicit GEMM):
// op(B)[kc][n] = xt(b, c, i*s - p + u, j*s - p + v), kc = (c*kH + u)*kW + v,
// n = (b*OH + i)*OW + j, stored in the same [k][n] LDS layout as a
// row-contiguous operand.  A thread's four columns n are the same in every
// K stage, so their image offsets and window origins are decoded once; each
// stage decodes only the thread's kc rows.
template <int BR, int NT>
struct ImplicitTileF32 {
    using Base = OperandTile<DtF32, BR, false, NT>;
    static constexpr int VW = 4, BK = 32;
    static constexpr int PITCH = Base::PITCH, LDS_BYTES = Base::LDS_BYTES;
    static constexpr int NV = Base::NV, PER = Base::PER;
    static_assert(NT % (BR / VW) == 0, "a thread's columns must not change between slots");

    u32x4 reg[PER];
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

    __device__ __forceinline__ void load(const uint32_t *__restrict__ x, const ConvGeom &g, int K, int k0,
                                         int tid)
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
                    const int hh = nh[e] + u, ww = nw[e] + vv;
                    const bool ok = nb[e] >= 0 && hh >= 0 && hh < g.H && ww >= 0 && ww < g.W;
                    v[e] = ok ? x[nb[e] + plane + hh * g.W + ww] : 0u;
                }
            }
            reg[s] = v;
        }
    }

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

// Fragment reads.  f32: 8 consecutive k (one k group of 16, lane half h)
// for one 32-row block; the 8 MFMAs of the group use element t.
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

// 16-bit: 8 consecutive k of k group q for lane half h, packed in 4 dwords.
template <bool KC, int PITCH>
__device__ __forceinline__ u32x4 frag_h(const uint16_t *lds, int row, int q, int h)
{
    if (KC) {
        return *(const u32x4 *)(lds + row * PITCH + q * 16 + h * 8);
    } else {
        u32x4 v;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            uint32_t lo = lds[(q * 16 + h * 8 + 2 * j) * PITCH + row];
            uint32_t hi = lds[(q * 16 + h * 8 + 2 * j + 1) * PITCH + row];
            v[j] = lo | (hi << 16);
        }
        return v;
    }
}

template <class DT>
__device__ __forceinline__ f32x16 mfma_h(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (DT::ID == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <class DT, int NWM, int NWN, int TM, int TN, bool A_KC, bool B_KC, bool IMPL>
__global__ __launch_bounds__(NWM *NWN * 64) void gemm_kernel(GemmParams p)
{
    constexpr int NT = NWM * NWN * 64;
    constexpr int BM = NWM * TM * 32, BN = NWN * TN * 32;
    using TR = GemmTraits<DT>;
    constexpr int BK = TR::BK;
    static_assert(!IMPL || (!B_KC && DT::ID == DT_F32), "implicit B: f32, [k][n] layout");
    using TA = OperandTile<DT, BM, A_KC, NT>;
    using TB = std::conditional_t<IMPL, ImplicitTileF32<BN, NT>, OperandTile<DT, BN, B_KC, NT>>;
    __shared__ __attribute__((aligned(16))) char smem[2 * (TA::LDS_BYTES + TB::LDS_BYTES)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave % NWM, wn = wave / NWM;
    const int h = lane >> 5, l32 = lane & 31;

    const int mt = (p.M + BM - 1) / BM;
    const int tile = xcd_tile(blockIdx.x, mt * ((p.N + BN - 1) / BN));
    const int m_blk = (tile % mt) * BM;
    const int n_blk = (tile / mt) * BN;

    const int kbeg = blockIdx.z * p.k_per_split;
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

    TA ta;
    TB tb;
    const char *Ab = (const char *)p.A;
    const char *Bb = (const char *)p.B;
    // K bound for this split: the loaders zero-fill k >= kend.
    auto load_b = [&](int k0) {
        if constexpr (IMPL)
            tb.load((const uint32_t *)p.B, p.g, kend, k0, tid);
        else
            tb.load(Bb, p.ldb, p.N, kend, n_blk, k0, p.b_vec, tid);
    };
    if constexpr (IMPL)
        tb.setup(p.g, n_blk, tid);
    if (nk > 0) {
        ta.load(Ab, p.lda, p.M, kend, m_blk, kbeg, p.a_vec, tid);
        load_b(kbeg);
    }
    for (int kt = 0; kt < nk; ++kt) {
        char *la = smem + (kt & 1) * (TA::LDS_BYTES + TB::LDS_BYTES);
        char *lb = la + TA::LDS_BYTES;
        ta.store(la, tid);
        tb.store(lb, tid);
        __syncthreads();
        if (kt + 1 < nk) {
            int k0 = kbeg + (kt + 1) * BK;
            ta.load(Ab, p.lda, p.M, kend, m_blk, k0, p.a_vec, tid);
            load_b(k0);
        }
        if constexpr (DT::ID == DT_F32) {
            const float *fa = (const float *)la;
            const float *fb = (const float *)lb;
#pragma unroll
            for (int kg = 0; kg < BK / 16; ++kg) {
                float af[TM][8], bf[TN][8];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    frag_f32<A_KC, TA::PITCH>(fa, (wm * TM + i) * 32 + l32, kg, h, af[i]);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    frag_f32<B_KC, TB::PITCH>(fb, (wn * TN + j) * 32 + l32, kg, h, bf[j]);
#pragma unroll
                for (int t = 0; t < 8; ++t)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int j = 0; j < TN; ++j)
                            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[i][t], bf[j][t],
                                                                             acc[i][j], 0, 0, 0);
            }
        } else {
            const uint16_t *ha = (const uint16_t *)la;
            const uint16_t *hb = (const uint16_t *)lb;
#pragma unroll
            for (int q = 0; q < BK / 16; ++q) {
                u32x4 af[TM], bf[TN];
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[i] = frag_h<A_KC, TA::PITCH>(ha, (wm * TM + i) * 32 + l32, q, h);
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bf[j] = frag_h<B_KC, TB::PITCH>(hb, (wn * TN + j) * 32 + l32, q, h);
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int j = 0; j < TN; ++j)
                        acc[i][j] = mfma_h<DT>(af[i], bf[j], acc[i][j]);
            }
        }
    }

    // Epilogue.  Accumulator element e of a 32x32 block sits at
    // row 8*(e/4) + 4*h + (e%4), column l32.
    float *C = p.C + (long long)blockIdx.z * p.c_split_stride;
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
                if (m < p.M) {
                    float v = acc[i][j][e];
                    if (p.epi == EPI_NCHW && p.bias)
                        v += p.bias[m];
                    C[col_off + (long long)m * row_stride] = v;
                }
            }
        }
    }
}

template <class DT, bool A_KC, bool B_KC, bool IMPL = false>
hipError_t launch_gemm_layout(int cfg, const GemmParams &p, hipStream_t s)
{
    TileShape ts = tile_shape(cfg);
    int tiles = ((p.M + ts.bm - 1) / ts.bm) * ((p.N + ts.bn - 1) / ts.bn);
    dim3 grid(tiles, 1, p.splits);
    switch (cfg) {
    case TILE_128x128:
        hipLaunchKernelGGL((gemm_kernel<DT, 2, 2, 2, 2, A_KC, B_KC, IMPL>), grid, dim3(256), 0, s, p);
        break;
    case TILE_64x64:
        hipLaunchKernelGGL((gemm_kernel<DT, 2, 2, 1, 1, A_KC, B_KC, IMPL>), grid, dim3(256), 0, s, p);
        break;
    case TILE_32x128:
        hipLaunchKernelGGL((gemm_kernel<DT, 1, 4, 1, 1, A_KC, B_KC, IMPL>), grid, dim3(256), 0, s, p);
        break;
    case TILE_96x128:
        hipLaunchKernelGGL((gemm_kernel<DT, 1, 4, 3, 1, A_KC, B_KC, IMPL>), grid, dim3(256), 0, s, p);
        break;
    default:
        return hipErrorInvalidValue;  // tile shape not built for this dtype
    }
    return hipGetLastError();
}

template <class DT>
hipError_t launch_gemm_dt(int cfg, bool a_kc, bool b_kc, const GemmParams &p, hipStream_t s)
{
    if (a_kc && b_kc)
        return launch_gemm_layout<DT, true, true>(cfg, p, s);
    if (a_kc && !b_kc)
        return launch_gemm_layout<DT, true, false>(cfg, p, s);
    if (!a_kc && b_kc)
        return launch_gemm_layout<DT, false, true>(cfg, p, s);
    return launch_gemm_layout<DT, false, false>(cfg, p, s);
}

}  // namespace d4r
