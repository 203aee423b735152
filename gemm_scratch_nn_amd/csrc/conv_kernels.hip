// HBM-bound steps of convolution lowered to GEMM, for gfx950.
//
// Steps (directcompute-nn page, "Convolution: The im2col Approach" and the
// "Convolution Shaders" table): im2col (patches -> column matrix), col2im
// (column matrix -> image, the adjoint of im2col), conv_grad_reshape
// ((batch, C, H, W) gradient -> matrix form), and the bias gradient (a
// per-channel sum of the reshaped gradient).
//
// All of these move data and do at most a few adds per element, so they are
// written for coalesced HBM access: consecutive lanes touch consecutive
// addresses of the larger side, stores are 16-byte vectors where the row
// length allows, and nothing uses atomics (col2im is a gather with a fixed
// summation order; reductions go through per-block partials).
#include "internal.hpp"

namespace d4r {

namespace {

constexpr int NT = 256;

template <typename T>
struct Vec16;
template <>
struct Vec16<uint32_t> { typedef uint32_t type __attribute__((ext_vector_type(4))); static constexpr int N = 4; };
template <>
struct Vec16<uint16_t> { typedef uint16_t type __attribute__((ext_vector_type(8))); static constexpr int N = 8; };

__device__ __forceinline__ float to_f32(uint32_t v, int) { return __uint_as_float(v); }
__device__ __forceinline__ float to_f32(uint16_t v, int dt)
{
    if (dt == DT_BF16)
        return __uint_as_float(((uint32_t)v) << 16);
    return (float)__builtin_bit_cast(_Float16, v);
}

// ---------------------------------------------------------------------------
// im2col: col[r][n] = xt(b, c, i*s - p + u, j*s - p + v) with r = (c*kH+u)*kW+v
// and n = (b*OH + i)*OW + j.  A thread owns VW consecutive n (one 16-byte
// store per row) and one (c, u) pair, and walks the kW rows v = 0..kW-1 of
// that pair: the x row segment it gathers from is the same for every v up
// to a shift, so after the first v it is served from L1 / L2 instead of
// HBM.  Raw bit copy: T is the storage word of the dtype.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void im2col_kernel(const T *__restrict__ x, T *__restrict__ col,
                                                    ConvGeom g, int vec_store)
{
    constexpr int VW = Vec16<T>::N;
    const int n0 = (blockIdx.x * NT + threadIdx.x) * VW;
    if (n0 >= g.N)
        return;
    // per element: image plane offset (b*C*H*W) and the window origin
    int base[VW], h0[VW], w0[VW];
    {
        int b = n0 / g.P;
        int rem = n0 - b * g.P;
        int i = rem / g.OW;
        int j = rem - i * g.OW;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            base[e] = b < g.B ? b * g.C * g.H * g.W : -1;
            h0[e] = i * g.s - g.p;
            w0[e] = j * g.s - g.p;
            if (++j == g.OW) {
                j = 0;
                if (++i == g.OH) {
                    i = 0;
                    ++b;
                }
            }
        }
    }
    const int CU = g.C * g.kH;
    for (int cu = blockIdx.y; cu < CU; cu += gridDim.y) {
        const int c = cu / g.kH;
        const int u = cu - c * g.kH;
        const int plane = c * g.H * g.W;
        for (int v = 0; v < g.kW; ++v) {
            typename Vec16<T>::type out;
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                const int hh = h0[e] + u;
                const int ww = w0[e] + v;
                T val = 0;
                if (base[e] >= 0 && hh >= 0 && hh < g.H && ww >= 0 && ww < g.W)
                    val = x[base[e] + plane + hh * g.W + ww];
                out[e] = val;
            }
            T *dst = col + (long long)(cu * g.kW + v) * g.N + n0;
            if (vec_store) {
                *(typename Vec16<T>::type *)dst = out;
            } else {
#pragma unroll
                for (int e = 0; e < VW; ++e)
                    if (n0 + e < g.N)
                        dst[e] = out[e];
            }
        }
    }
}

// LDS window padding: one 4-byte word after every 32 words.  Threads that own
// 16-byte column vectors read window positions 4 words apart, which without
// padding fall on only 8 of the 32 banks.
template <typename T>
__device__ __forceinline__ int lds_pad(int a)
{
    if constexpr (sizeof(T) == 4)
        return a + (a >> 5);
    else
        return a + ((a >> 6) << 1);
}

template <typename T>
constexpr long long lds_padded_elems(long long n)
{
    return sizeof(T) == 4 ? n + n / 32 + 1 : n + 2 * (n / 64) + 2;
}

// ---------------------------------------------------------------------------
// im2col through LDS.  A block owns one channel c, images [b0, b0+BB) and
// output rows [i0, i1) (a row range only when BB = 1).  It copies the
// zero-padded input window those outputs read into LDS with coalesced loads,
// then writes, for every tap (u, v), the col segment of its outputs, which
// is one contiguous run n = (b0*OH + i0)*OW .. of BB*(i1-i0)*OW elements, with
// 16-byte stores (element stores at the two unaligned ends).  x is read from
// HBM once, col written once in long runs.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void im2col_lds_kernel(const T *__restrict__ x, T *__restrict__ col,
                                                        ConvGeom g, int RB, int BB, int Rl, int Wl,
                                                        int vec_store)
{
    constexpr int VW = Vec16<T>::N;
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    T *lds = (T *)lds_raw;
    const int c = blockIdx.y;
    const int b0 = blockIdx.z * BB;
    const int nbb = min(BB, g.B - b0);
    const int i0 = blockIdx.x * RB;
    const int i1 = min(g.OH, i0 + RB);
    const int rows = i1 - i0;
    const int plane = Rl * Wl;
    const int h_org = i0 * g.s - g.p, w_org = -g.p;

    // Fill: a thread keeps one window column q and walks the window rows
    // (rows_per_pass of them are filled per pass), so no per-element
    // division.  Loads go out FB at a time before their LDS stores, so a
    // thread waits for one batch instead of once per row.
    {
        constexpr int FB = 8;
        const int rpp = Wl <= NT ? NT / Wl : 1;
        const int r_off = Wl <= NT ? threadIdx.x / Wl : 0;
        const int q0 = Wl <= NT ? threadIdx.x - r_off * Wl : threadIdx.x;
        const int qstep = Wl <= NT ? Wl : NT;
        const int total_rows = nbb * Rl;
        if (r_off < rpp) {
            for (int q = q0; q < Wl; q += qstep) {
                const int ww = w_org + q;
                const bool col_ok = ww >= 0 && ww < g.W;
                // (bb, r) of window row rr = bb*Rl + r, stepped by rpp
                // (small_div: r + rpp < 2^20 and Rl <= 1024, checked by the
                // host); out-of-window loads read x[0] and are discarded,
                // so the batch has no branches to wait at
                int bb = small_div(r_off, Rl), r = r_off - bb * Rl;
                for (int rr = r_off; rr < total_rows; rr += FB * rpp) {
                    T val[FB];
                    int dst[FB];
#pragma unroll
                    for (int k = 0; k < FB; ++k) {
                        const bool live = rr + k * rpp < total_rows;
                        const int hh = h_org + r;
                        const bool ok = live && col_ok && (unsigned)hh < (unsigned)g.H;
                        const long long a = (((long long)(b0 + bb) * g.C + c) * g.H + hh) * g.W + ww;
                        const T v = x[ok ? a : 0];
                        val[k] = ok ? v : (T)0;
                        dst[k] = live ? (bb * Rl + r) * Wl + q : -1;
                        r += rpp;
                        const int wr = small_div(r, Rl);
                        r -= wr * Rl;
                        bb += wr;
                    }
#pragma unroll
                    for (int k = 0; k < FB; ++k)
                        if (dst[k] >= 0)
                            lds[lds_pad<T>(dst[k])] = val[k];
                }
            }
        }
    }
    __syncthreads();

    // Output phase: a thread owns one 16-byte vector of columns, resolves its
    // VW LDS offsets once, then walks the taps (u, v): one LDS read per
    // element and one store per tap (the window in LDS already holds the
    // padding zeros).  When the block has fewer vectors than threads, the
    // threads form `groups` sets that share out the kernel rows u (set t
    // takes u = t, t + groups, ...), so no thread sits idle through the taps
    // (AlexNet conv1: 124 vectors per block of 256 threads).
    const int khw = g.kH * g.kW;
    const int n_start = (b0 * g.OH + i0) * g.OW;
    const int per_img = rows * g.OW;
    const int L = nbb * per_img;
    const int n_al = n_start - (n_start % VW);
    const int nvec = (n_start + L - n_al + VW - 1) / VW;
    const long long row_stride = g.N;
    const int span = nvec < NT ? nvec : NT;  // threads per set
    const int groups = min(NT / span, g.kH);
    const int grp = threadIdx.x / span;
    if (grp >= groups)
        return;  // no barrier follows
    for (int q = threadIdx.x - grp * span; q < nvec; q += span) {
        const int n0 = n_al + q * VW;
        const int lo = n0 - n_start;
        int off[VW];
        bool in[VW];
        {
            const int e0 = lo < 0 ? -lo : 0;
            const int loc = lo + e0;
            int bb = loc / per_img;
            const int rem = loc - bb * per_img;
            int il = rem / g.OW;
            int j = rem - il * g.OW;
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                in[e] = e >= e0 && lo + e < L;
                off[e] = in[e] ? bb * plane + il * g.s * Wl + j * g.s : 0;
                if (in[e]) {
                    if (++j == g.OW) {
                        j = 0;
                        if (++il == rows) {
                            il = 0;
                            ++bb;
                        }
                    }
                }
            }
        }
        const bool full = vec_store && lo >= 0 && lo + VW <= L;
        for (int u = grp; u < g.kH; u += groups) {
            T *dst = col + ((long long)c * khw + u * g.kW) * row_stride + n0;
            for (int v = 0; v < g.kW; ++v) {
                const int tap = u * Wl + v;
                typename Vec16<T>::type out;
#pragma unroll
                for (int e = 0; e < VW; ++e)
                    out[e] = lds[lds_pad<T>(off[e] + tap)];
                if (full) {
                    *(typename Vec16<T>::type *)dst = out;
                } else {
#pragma unroll
                    for (int e = 0; e < VW; ++e)
                        if (in[e])
                            dst[e] = out[e];
                }
                dst += row_stride;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// im2col for stride 1 when OW is a multiple of the vector width VW.  A block
// owns channel c, images [b0, b0+BB) and output rows [i0, i0+RB) as above;
// LDS holds, for every column tap v, the Rl window rows restricted to the
// OW columns that tap reads: copy[v][bb][r][j] = x(b0+bb, c, i0-p+r, j+v-p)
// (0 in the padding).  The VW outputs (b, i, j0..j0+VW-1) of tap (u, v) are
// then copy[v][bb][i-i0+u][j0..j0+VW-1]: one aligned 16-byte LDS read per
// 16-byte store (the general kernel reads VW single elements).  The fill
// walks the copies in their LDS order, eight loads in flight per thread.
// Host checks: OW <= 1024, BB*Rl <= 1024 and kW*BB*Rl*OW < 2^20 (small_div),
// LDS within 48 KB.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void im2col_shift_kernel(const T *__restrict__ x, T *__restrict__ col,
                                                          ConvGeom g, int RB, int BB, int Rl)
{
    constexpr int VW = Vec16<T>::N;
    using V = typename Vec16<T>::type;
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    T *lds = (T *)lds_raw;
    const int c = blockIdx.y;
    const int b0 = blockIdx.z * BB;
    const int nbb = min(BB, g.B - b0);
    const int i0 = blockIdx.x * RB;
    const int rows = min(g.OH, i0 + RB) - i0;
    const int OW = g.OW;
    const int rows_c = nbb * Rl;          // window rows of one tap copy
    const int total = g.kW * rows_c * OW;  // LDS elements
    {
        constexpr int FB = 8;
        for (int t0 = threadIdx.x; t0 < total; t0 += FB * NT) {
            T val[FB];
#pragma unroll
            for (int k = 0; k < FB; ++k) {
                const int t = t0 + k * NT;
                const int rid = small_div(t, OW), j = t - rid * OW;
                const int v = small_div(rid, rows_c), rr = rid - v * rows_c;
                const int bb = small_div(rr, Rl), r = rr - bb * Rl;
                const int hh = i0 - g.p + r, ww = j + v - g.p;
                const bool ok = t < total && (unsigned)hh < (unsigned)g.H && (unsigned)ww < (unsigned)g.W;
                const long long a = (((long long)(b0 + bb) * g.C + c) * g.H + hh) * g.W + ww;
                const T xv = x[ok ? a : 0];
                val[k] = ok ? xv : (T)0;
            }
#pragma unroll
            for (int k = 0; k < FB; ++k)
                if (t0 + k * NT < total)
                    lds[t0 + k * NT] = val[k];
        }
    }
    __syncthreads();
    const int khw = g.kH * g.kW;
    const int n_start = (b0 * g.OH + i0) * OW;  // a multiple of OW, so of VW
    const int per_img = rows * OW;
    const int nvec = nbb * per_img / VW;
    for (int q = threadIdx.x; q < nvec; q += NT) {
        const int lo = q * VW;
        const int bb = lo / per_img, rem = lo - bb * per_img;
        const int il = rem / OW, j0 = rem - il * OW;
        T *dst = col + (long long)c * khw * g.N + n_start + lo;
        const T *src0 = lds + (bb * Rl + il) * OW + j0;
        for (int u = 0; u < g.kH; ++u)
            for (int v = 0; v < g.kW; ++v) {
                *(V *)dst = *(const V *)(src0 + (v * rows_c + u) * OW);
                dst += g.N;
            }
    }
}

// ---------------------------------------------------------------------------
// col2im as a gather: one thread per dx element (b, c, h, w) sums the dcol
// entries that im2col copied from (b, c, h, w).  Tap u contributes when
// h + p - u >= 0, divisible by s and (h + p - u)/s < OH, i.e. u runs over one
// residue class mod s between u_lo and u_hi; same for v.  Order: u
// ascending, then v ascending.  TU / TV > 0 fix the number of candidate taps
// per axis (ceil(k / s)) at compile time so every load of a thread is issued
// before the adds; TU = TV = 0 is the general loop.
// ---------------------------------------------------------------------------
// Taps of dx element idx: the candidate (u, v) pairs, their dcol offsets
// and whether each lies inside the tap range (TU x TV candidates).
template <int TU, int TV>
__device__ __forceinline__ void col2im_taps(const ConvGeom &g, int idx, long long (&off)[TU][TV],
                                            bool (&ok)[TU][TV])
{
    const int w = idx % g.W;
    int t = idx / g.W;
    const int h = t % g.H;
    t /= g.H;
    const int c = t % g.C;
    const int b = t / g.C;

    const int hp = h + g.p, wp = w + g.p;
    // smallest u >= max(0, hp - s*(OH-1)) with u = hp (mod s); largest u <= min(kH-1, hp)
    int u_lo = hp - g.s * (g.OH - 1);
    if (u_lo < 0)
        u_lo = 0;
    u_lo += ((hp - u_lo) % g.s);
    const int u_hi = min(g.kH - 1, hp);
    int v_lo = wp - g.s * (g.OW - 1);
    if (v_lo < 0)
        v_lo = 0;
    v_lo += ((wp - v_lo) % g.s);
    const int v_hi = min(g.kW - 1, wp);
    const int nb = b * g.P;
#pragma unroll
    for (int a = 0; a < TU; ++a) {
        const int u = u_lo + a * g.s;
        const int i = (hp - u) / g.s;
#pragma unroll
        for (int q = 0; q < TV; ++q) {
            const int v = v_lo + q * g.s;
            const int j = (wp - v) / g.s;
            ok[a][q] = (u <= u_hi) && (v <= v_hi);
            off[a][q] = ok[a][q] ? (long long)((c * g.kH + u) * g.kW + v) * g.N + nb + i * g.OW + j : 0;
        }
    }
}

// General tap loop (tap counts not fixed at compile time).
__device__ __forceinline__ float col2im_one_general(const float *__restrict__ dcol, const ConvGeom &g, int idx)
{
    const int w = idx % g.W;
    int t = idx / g.W;
    const int h = t % g.H;
    t /= g.H;
    const int c = t % g.C;
    const int b = t / g.C;
    const int hp = h + g.p, wp = w + g.p;
    int u_lo = hp - g.s * (g.OH - 1);
    if (u_lo < 0)
        u_lo = 0;
    u_lo += ((hp - u_lo) % g.s);
    const int u_hi = min(g.kH - 1, hp);
    int v_lo = wp - g.s * (g.OW - 1);
    if (v_lo < 0)
        v_lo = 0;
    v_lo += ((wp - v_lo) % g.s);
    const int v_hi = min(g.kW - 1, wp);
    const long long Nl = g.N;
    const int nb = b * g.P;
    float acc = 0.0f;
    for (int u = u_lo; u <= u_hi; u += g.s) {
        const int i = (hp - u) / g.s;
        const int rbase = (c * g.kH + u) * g.kW;
        for (int v = v_lo; v <= v_hi; v += g.s) {
            const int j = (wp - v) / g.s;
            acc += dcol[(long long)(rbase + v) * Nl + nb + i * g.OW + j];
        }
    }
    return acc;
}

// A thread computes four consecutive dx elements.  With the row width a
// multiple of 4 and the stride 4 (AlexNet conv1), the lanes of a wavefront
// then share one residue class of w for each of the four, so every tap's
// load reads 64 consecutive floats of one dcol row (whole cache lines: the
// form with elements NT apart read each line in 64-byte halves, 1.5x the
// dcol bytes from HBM), and the four sums leave as one 16-byte store.
// Blocks are renumbered so each XCD walks one contiguous range of dx: a
// row segment of dcol that one block reads shares its cache lines with the
// next output row, read by the block a few rows on, which round-robin
// dispatch would put on another XCD (another L2).
// With the tap counts fixed at compile time (TU, TV > 0) the loads of CPT
// elements are all issued before the first add: loads are unconditional
// (offset 0 outside the tap range, the value then dropped), and elements
// past the end repeat the last one.  Each element adds its taps in the
// order u, then v ascending.
template <int TU, int TV>
__global__ __launch_bounds__(NT) void col2im_kernel(const float *__restrict__ dcol,
                                                    float *__restrict__ dx, ConvGeom g, int total)
{
    constexpr int CPT = (TU > 0 && TU * TV > 9) ? 2 : 4;
    const int base = (xcd_tile(blockIdx.x, gridDim.x) * NT + threadIdx.x) * 4;
    float res[4];
    if constexpr (TU > 0) {
#pragma unroll
        for (int half = 0; half < 4 / CPT; ++half) {
            float vals[CPT][TU][TV];
            bool ok[CPT][TU][TV];
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                long long off[TU][TV];
                col2im_taps<TU, TV>(g, min(base + half * CPT + e, total - 1), off, ok[e]);
#pragma unroll
                for (int a = 0; a < TU; ++a)
#pragma unroll
                    for (int q = 0; q < TV; ++q)
                        vals[e][a][q] = dcol[off[a][q]];
            }
#pragma unroll
            for (int e = 0; e < CPT; ++e) {
                float acc = 0.0f;
#pragma unroll
                for (int a = 0; a < TU; ++a)
#pragma unroll
                    for (int q = 0; q < TV; ++q)
                        acc += ok[e][a][q] ? vals[e][a][q] : 0.0f;
                res[half * CPT + e] = acc;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            res[e] = base + e < total ? col2im_one_general(dcol, g, base + e) : 0.0f;
    }
    // dx is 16-byte aligned, so a whole group of four is one aligned vector
    if (base + 4 <= total) {
        *(float4 *)(dx + base) = make_float4(res[0], res[1], res[2], res[3]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (base + e < total)
                dx[base + e] = res[e];
    }
}

// ---------------------------------------------------------------------------
// col2im as the adjoint of the LDS im2col.  A block owns channel c and whole
// images [b0, b0+BB); LDS holds their zero-initialised padded windows (the
// same window im2col reads).  A thread owns up to QMAX 16-byte vectors of
// dcol columns n and resolves their window offsets once; then, tap by tap in
// the order u ascending, v ascending, it loads its dcol vectors (coalesced)
// and adds each value into the window position the column read in im2col.
// Within one tap every column hits a distinct position, and a barrier
// separates taps, so each dx element is summed in the fixed tap order with
// no atomics.  Finally the window interior is written to dx.
// ---------------------------------------------------------------------------
constexpr int C2I_QMAX = 4;

__global__ __launch_bounds__(NT) void col2im_lds_kernel(const float *__restrict__ dcol,
                                                        float *__restrict__ dx, ConvGeom g, int BB,
                                                        int Rl, int Wl, int vec_load)
{
    constexpr int VW = 4;
    extern __shared__ __attribute__((aligned(16))) char lds_raw[];
    float *lds = (float *)lds_raw;
    const int c = blockIdx.y;
    const int b0 = blockIdx.z * BB;
    const int nbb = min(BB, g.B - b0);
    const int plane = Rl * Wl;
    for (int t = threadIdx.x; t < lds_padded_elems<float>((long long)nbb * plane); t += NT)
        lds[t] = 0.0f;

    const int n_start = b0 * g.P;
    const int L = nbb * g.P;
    const int n_al = n_start - (n_start % VW);
    const int nvec = (n_start + L - n_al + VW - 1) / VW;
    int off[C2I_QMAX][VW];
    bool in[C2I_QMAX][VW];
#pragma unroll
    for (int qi = 0; qi < C2I_QMAX; ++qi) {
        const int q = threadIdx.x + qi * NT;
        const int n0 = n_al + q * VW;
        const int lo = n0 - n_start;
        const int e0 = lo < 0 ? -lo : 0;
        const int loc = lo + e0;
        int bb = loc / g.P;
        const int rem = loc - bb * g.P;
        int i = rem / g.OW;
        int j = rem - i * g.OW;
#pragma unroll
        for (int e = 0; e < VW; ++e) {
            in[qi][e] = q < nvec && e >= e0 && lo + e < L;
            off[qi][e] = in[qi][e] ? bb * plane + i * g.s * Wl + j * g.s : 0;
            if (in[qi][e] && ++j == g.OW) {
                j = 0;
                if (++i == g.OH) {
                    i = 0;
                    ++bb;
                }
            }
        }
    }
    __syncthreads();

    const int khw = g.kH * g.kW;
    const float *src = dcol + (long long)c * khw * g.N + n_al;
    for (int u = 0; u < g.kH; ++u) {
        for (int v = 0; v < g.kW; ++v) {
            const int tap = u * Wl + v;
#pragma unroll
            for (int qi = 0; qi < C2I_QMAX; ++qi) {
                const int q = threadIdx.x + qi * NT;
                if (q < nvec) {
                    float val[VW];
                    if (vec_load && in[qi][0] && in[qi][VW - 1]) {
                        const float4 f = *(const float4 *)(src + q * VW);
                        val[0] = f.x;
                        val[1] = f.y;
                        val[2] = f.z;
                        val[3] = f.w;
                    } else {
#pragma unroll
                        for (int e = 0; e < VW; ++e)
                            val[e] = in[qi][e] ? src[q * VW + e] : 0.0f;
                    }
#pragma unroll
                    for (int e = 0; e < VW; ++e)
                        if (in[qi][e])
                            lds[lds_pad<float>(off[qi][e] + tap)] += val[e];
                }
            }
            src += g.N;
            __syncthreads();
        }
    }

    const int hw = g.H * g.W;
    for (int t = threadIdx.x; t < nbb * hw; t += NT) {
        const int bb = t / hw;
        const int r = t - bb * hw;
        const int h = r / g.W;
        const int w = r - h * g.W;
        const int wr = h + g.p, wc = w + g.p;
        const float val = (wr < Rl && wc < Wl) ? lds[lds_pad<float>(bb * plane + wr * Wl + wc)] : 0.0f;
        dx[(((long long)(b0 + bb) * g.C + c) * g.H + h) * g.W + w] = val;
    }
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        v += __shfl_xor(v, off, 64);
    return v;
}

// ---------------------------------------------------------------------------
// conv_grad_reshape: G[o][n] = dy[b][o][pix], n = b*P + pix.  Thread per VW
// consecutive n of one row o: consecutive lanes read consecutive pixels of
// an image plane and write consecutive columns of G.  With bias_part set,
// the same pass also yields the bias gradient's first level: block (x, o)
// sums its elements (fixed wave-shuffle tree, then LDS in wave order) into
// bias_part[o * gridDim.x + x].
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void grad_reshape_kernel(const T *__restrict__ dy, T *__restrict__ G,
                                                          ConvGeom g, int vec_store,
                                                          float *__restrict__ bias_part, int dt)
{
    constexpr int VW = Vec16<T>::N;
    __shared__ float red[NT / 64];
    const int n0 = (blockIdx.x * NT + threadIdx.x) * VW;
    const bool live = n0 < g.N;
    for (int o = blockIdx.y; o < g.O; o += gridDim.y) {
        float sum = 0.0f;
        if (live) {
            int b = n0 / g.P;
            int pix = n0 - b * g.P;
            typename Vec16<T>::type out;
#pragma unroll
            for (int e = 0; e < VW; ++e) {
                out[e] = (b < g.B) ? dy[((long long)b * g.O + o) * g.P + pix] : (T)0;
                if (++pix == g.P) {
                    pix = 0;
                    ++b;
                }
            }
            T *dst = G + (long long)o * g.N + n0;
            if (vec_store) {
                *(typename Vec16<T>::type *)dst = out;
            } else {
#pragma unroll
                for (int e = 0; e < VW; ++e)
                    if (n0 + e < g.N)
                        dst[e] = out[e];
            }
            if (bias_part) {
#pragma unroll
                for (int e = 0; e < VW; ++e)
                    sum += to_f32(out[e], dt);  // zero past N
            }
        }
        if (bias_part) {  // uniform across the block
            sum = wave_sum(sum);
            if ((threadIdx.x & 63) == 0)
                red[threadIdx.x >> 6] = sum;
            __syncthreads();
            if (threadIdx.x == 0) {
                float t = 0.0f;
#pragma unroll
                for (int w = 0; w < NT / 64; ++w)
                    t += red[w];
                bias_part[(long long)o * gridDim.x + blockIdx.x] = t;
            }
            __syncthreads();
        }
    }
}

// ---------------------------------------------------------------------------
// Batched transpose out[b][c][r] = in[b][r][c] through a 64x64 LDS tile
// (one extra column of padding so the column reads hit distinct banks).
// Each wavefront reads 64 consecutive elements of a row and writes 64
// consecutive elements of an output row; a thread's 16 loads are all issued
// before the first is used.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void transpose_tile(const T *__restrict__ in, T *__restrict__ out, int R, int Cc,
                                               int bx, int by, int bz, T (*tile)[65])
{
    const long long base = (long long)bz * R * Cc;
    const int r0 = by * 64, c0 = bx * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    constexpr int ROWS = 64 / (NT / 64);
    T v[ROWS];
    const bool cin = c0 + tx < Cc;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int r = r0 + ty + i * (NT / 64);
        v[i] = (cin && r < R) ? in[base + (long long)r * Cc + c0 + tx] : (T)0;
    }
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
        tile[ty + i * (NT / 64)][tx] = v[i];
    __syncthreads();
    const bool rin = r0 + tx < R;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int c = c0 + ty + i * (NT / 64);
        if (rin && c < Cc)
            out[base + (long long)c * R + r0 + tx] = tile[tx][ty + i * (NT / 64)];
    }
}

template <typename T>
__global__ __launch_bounds__(NT) void transpose_kernel(const T *__restrict__ in, T *__restrict__ out,
                                                       int R, int Cc)
{
    __shared__ T tile[64][65];
    transpose_tile<T>(in, out, R, Cc, blockIdx.x, blockIdx.y, blockIdx.z, tile);
}

// A filter job (FilterJob).  Forward order (flip 0): one 16-byte output
// vector per thread, in output order; its elements are w[o][c..c+VW-1][tap],
// taps apart, so a wavefront reads one contiguous stretch of w.  Data
// gradient order (flip 1): w viewed as O x C*taps is transposed through a
// 64x64 LDS tile (rows o, 64 consecutive (c, tap) columns: 128-byte row
// reads), and element (o, c, tap) is stored at out[c][ob][taps-1-tap][oi]
// (o = ob*kb + oi): 64 consecutive o of a tile are one contiguous run when
// kb = 64, two when kb = 32.  Block 0 clears the zero page.
template <typename T>
__device__ __forceinline__ void filter_job(const FilterJob &f, int block, T (*tile)[65])
{
    using V = typename Vec16<T>::type;
    constexpr int VW = Vec16<T>::N;
    if (f.zero && block == 0 && threadIdx.x < 64)
        f.zero[threadIdx.x] = 0u;
    const T *w = (const T *)f.in;
    if (!f.flip) {
        const long long q = (long long)block * NT + threadIdx.x;
        const long long total = (long long)f.O * f.C * f.taps / VW;
        if (q >= total)
            return;
        const long long e0 = q * VW;
        const int i0 = (int)(e0 % f.kb);  // channel inside the block (first of VW)
        long long r = e0 / f.kb;
        const int t = (int)(r % f.taps);
        r /= f.taps;
        const int cbn = f.C / f.kb;
        const int cb = (int)(r % cbn);
        const long long o = r / cbn;
        const T *src = w + (o * f.C + (long long)cb * f.kb + i0) * f.taps + t;
        V v;
#pragma unroll
        for (int e = 0; e < VW; ++e)
            v[e] = src[(long long)e * f.taps];
        *(V *)((T *)f.out + e0) = v;
        return;
    }
    const int R = f.O, Cc = f.C * f.taps;
    const int gx = (Cc + 63) / 64;
    const int r0 = (block / gx) * 64, c0 = (block % gx) * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    constexpr int ROWS = 64 / (NT / 64);
    T v[ROWS];
    const bool cin = c0 + tx < Cc;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int r = r0 + ty + i * (NT / 64);
        v[i] = (cin && r < R) ? w[(long long)r * Cc + c0 + tx] : (T)0;
    }
#pragma unroll
    for (int i = 0; i < ROWS; ++i)
        tile[ty + i * (NT / 64)][tx] = v[i];
    __syncthreads();
    const int o = r0 + tx;  // the output's inner index runs over o
    const int ob = o / f.kb, oi = o - ob * f.kb;
    const long long opart = (long long)ob * f.kb * f.taps + oi;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int k = c0 + ty + i * (NT / 64);  // (c, tap) column of w
        const int c = k / f.taps, t = f.taps - 1 - (k - c * f.taps);
        if (o < R && k < Cc)
            ((T *)f.out)[(long long)c * R * f.taps + (long long)t * f.kb + opart] = tile[tx][ty + i * (NT / 64)];
    }
}

// A data transpose and a filter job in one launch: blocks [0, a.blocks) run
// the transpose, the rest the filter job (the choice is uniform per block).
template <typename T>
__global__ __launch_bounds__(NT) void transpose_filter_kernel(TransposeJob a, FilterJob f)
{
    __shared__ T tile[64][65];  // one tile for either job
    if ((int)blockIdx.x >= a.blocks) {
        filter_job<T>(f, (int)blockIdx.x - a.blocks, tile);
        return;
    }
    const int local = (int)blockIdx.x;
    const int gx = (a.Cc + 63) / 64, gy = (a.R + 63) / 64;
    if (a.zero && local == 0 && threadIdx.x < 64)
        a.zero[threadIdx.x] = 0u;
    transpose_tile<T>((const T *)a.in, (T *)a.out, a.R, a.Cc, local % gx, (local / gx) % gy, local / (gx * gy),
                      tile);
}

// ---------------------------------------------------------------------------
// dy prepared for both gradients in one pass (combined backward): a block
// reads one 64 (channel) x 64 (pixel) tile of dy[b] once and writes it
//   * as G[o][b*P + pix] (the filter gradient's k-contiguous operand),
//   * transposed as Gt[b][pix][o] (the NHWC data gradient's operand),
//   * and, when bias_part is set, the tile row sums (one wavefront per row,
//     fixed butterfly order) as bias_part[o*parts + b*ceil(P/64) + tile].
// Blocks past the tiles run the filter job w, as transpose_filter_kernel
// does.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void dy_prep_kernel(DyPrep a, FilterJob w)
{
    __shared__ T tile[64][65];  // one tile for either job
    if ((int)blockIdx.x >= a.blocks) {
        filter_job<T>(w, (int)blockIdx.x - a.blocks, tile);
        return;
    }
    const int gx = (a.P + 63) / 64, gy = (a.O + 63) / 64;
    const int bx = (int)blockIdx.x % gx, by = ((int)blockIdx.x / gx) % gy, b = (int)blockIdx.x / (gx * gy);
    const int p0 = bx * 64, o0 = by * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    constexpr int ROWS = 64 / (NT / 64);
    const T *dy = (const T *)a.dy + (long long)b * a.O * a.P;
    const bool pin = p0 + tx < a.P;
    T v[ROWS];
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int o = o0 + ty + i * (NT / 64);
        v[i] = (pin && o < a.O) ? dy[(long long)o * a.P + p0 + tx] : (T)0;
    }
    const long long N = (long long)a.B * a.P;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int o = o0 + ty + i * (NT / 64);
        if (pin && o < a.O)
            ((T *)a.g)[(long long)o * N + (long long)b * a.P + p0 + tx] = v[i];
        tile[ty + i * (NT / 64)][tx] = v[i];
    }
    __syncthreads();
    if (a.bias_part) {
        // row r of the tile: four threads add 16 columns each (zeros past
        // P), then the quarters combine in a fixed order (lanes t^1, t^2)
        const int r = threadIdx.x >> 2, q = threadIdx.x & 3;
        float t = 0.0f;
#pragma unroll
        for (int k = 0; k < 16; ++k)
            t += to_f32(tile[r][q * 16 + k], a.dt);
        t += __shfl_xor(t, 1);
        t += __shfl_xor(t, 2);
        if (q == 0 && o0 + r < a.O)
            a.bias_part[(long long)(o0 + r) * (a.B * gx) + b * gx + bx] = t;
    }
    T *gt = (T *)a.gt + (long long)b * a.O * a.P;
    const bool oin = o0 + tx < a.O;
#pragma unroll
    for (int i = 0; i < ROWS; ++i) {
        const int pix = p0 + ty + i * (NT / 64);
        if (oin && pix < a.P)
            gt[(long long)pix * a.O + o0 + tx] = tile[tx][ty + i * (NT / 64)];
    }
}

// ---------------------------------------------------------------------------
// Bias gradient.  Pass 1: block (s, o) sums images [s*per, (s+1)*per) of
// channel o: its threads stride through the flattened (image, pixel) range
// of those planes, four elements in flight per thread, then the block
// reduces through a fixed wave-shuffle tree and LDS.  Pass 2: one thread per
// channel adds the partials in split order.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void bias_partial_kernel(const T *__restrict__ dy,
                                                          float *__restrict__ partial, ConvGeom g,
                                                          int splits, int per, int dt)
{
    __shared__ float red[NT / 64];
    const int s = blockIdx.x, o = blockIdx.y;
    const int b0 = s * per, nb = min(g.B, b0 + per) - b0;
    const int total = nb * g.P;  // elements of this block
    const long long plane = (long long)g.O * g.P;
    const T *base = dy + ((long long)b0 * g.O + o) * g.P;
    // element i = b*P + pix of the block sits at base[b*O*P + pix]
    int b = threadIdx.x / g.P, pix = threadIdx.x - (threadIdx.x / g.P) * g.P;
    const int step_b = NT / g.P, step_p = NT - (NT / g.P) * g.P;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int i = threadIdx.x;
    for (; i + 3 * NT < total; i += 4 * NT) {
        T v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[u] = base[b * plane + pix];
            pix += step_p;
            b += step_b;
            if (pix >= g.P) {
                pix -= g.P;
                ++b;
            }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
            acc[u] += to_f32(v[u], dt);
    }
    for (; i < total; i += NT) {
        acc[0] += to_f32(base[b * plane + pix], dt);
        pix += step_p;
        b += step_b;
        if (pix >= g.P) {
            pix -= g.P;
            ++b;
        }
    }
    float tot = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
    if ((threadIdx.x & 63) == 0)
        red[threadIdx.x >> 6] = tot;
    __syncthreads();
    if (threadIdx.x == 0) {
        float t = 0.0f;
#pragma unroll
        for (int w = 0; w < NT / 64; ++w)
            t += red[w];
        partial[o * splits + s] = t;
    }
}

__global__ __launch_bounds__(NT) void bias_final_kernel(const float *__restrict__ partial,
                                                        float *__restrict__ db, int O, int splits)
{
    const int o = blockIdx.x * NT + threadIdx.x;
    if (o >= O)
        return;
    float tot = 0.0f;
    for (int s = 0; s < splits; ++s)
        tot += partial[o * splits + s];
    db[o] = tot;
}

// A BiasSum's per-channel sums: one wavefront per channel (block j covers
// channels 4j .. 4j+3); lane l adds partials l, l+64, .. in order, then the
// lanes combine through the fixed butterfly of wave_sum.  Run by extra
// blocks of a split-K reduction, or alone (bias_sum_kernel).
__device__ __forceinline__ void bias_sum_job(const BiasSum &bs, int j)
{
    const int o = j * (NT / 64) + (int)(threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (o >= bs.O)
        return;  // whole wavefront
    float t = 0.0f;
    for (int s = lane; s < bs.parts; s += 64)
        t += bs.partial[(long long)o * bs.parts + s];
    t = wave_sum(t);
    if (lane == 0)
        bs.db[o] = t;
}

__global__ __launch_bounds__(NT) void bias_sum_kernel(BiasSum bs) { bias_sum_job(bs, blockIdx.x); }

// ---------------------------------------------------------------------------
// Split-K reduction: C = sum_{s} part[s], then the GEMM epilogue (row-major
// store, or NCHW store with bias).  Two fixed summation orders:
//  * vector path (N and the split stride multiples of 4): a thread owns four
//    consecutive outputs, loads four splits ahead and adds them in split
//    order;
//  * grouped path (anything else, and few outputs over many splits): a block
//    owns 64 consecutive outputs; its four wavefronts sum contiguous quarters
//    of the split range (lanes along the outputs, so loads coalesce) and the
//    four partial sums are added in quarter order.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void splitk_store(float acc, long long idx, int M, int N, int epi, float *C,
                                             int ldc, const float *bias, int P, int relu)
{
    const int m = (int)(idx / N);
    const int n = (int)(idx - (long long)m * N);
    const float v = epi_value(acc, bias, relu, epi, m, n);
    if (epi == EPI_NCHW) {
        const int b = n / P, pix = n - b * P;
        C[((long long)b * M + m) * P + pix] = v;
    } else {
        C[(long long)m * ldc + n] = v;
    }
}

__global__ __launch_bounds__(NT) void splitk_reduce_vec_kernel(const float *__restrict__ part, int splits,
                                                               int M, int N, long long stride, int epi,
                                                               float *__restrict__ C, int ldc,
                                                               const float *__restrict__ bias, int P, int relu,
                                                               int rblocks, BiasSum bs)
{
    if ((int)blockIdx.x >= rblocks) {
        bias_sum_job(bs, (int)blockIdx.x - rblocks);
        return;
    }
    const long long total = (long long)M * N;
    const long long i0 = ((long long)blockIdx.x * NT + threadIdx.x) * 4;
    if (i0 >= total)
        return;
    // i0 .. i0+3 lie in one row and inside the matrix (N % 4 == 0)
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    int sp = 0;
    for (; sp + 4 <= splits; sp += 4) {
        float4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = *(const float4 *)(part + (sp + u) * stride + i0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            acc[0] += v[u].x;
            acc[1] += v[u].y;
            acc[2] += v[u].z;
            acc[3] += v[u].w;
        }
    }
    if (sp < splits) {
        // the last 1-3 slabs: all loads issued together (a slab past the
        // end re-reads the last one and is not added), added in order
        float4 v[3];
#pragma unroll
        for (int u = 0; u < 3; ++u)
            v[u] = *(const float4 *)(part + (long long)min(sp + u, splits - 1) * stride + i0);
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            if (sp + u < splits) {
                acc[0] += v[u].x;
                acc[1] += v[u].y;
                acc[2] += v[u].z;
                acc[3] += v[u].w;
            }
        }
    }
    // one row m for all four; the NCHW position decoded once and stepped
    const int m = (int)(i0 / N);
    const int n0 = (int)(i0 - (long long)m * N);
    // one 16-byte store when the four outputs are contiguous and aligned
    // (row-major rows; NCHW when they stay in one image), else four
    float out[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
        out[e] = epi_value(acc[e], bias, relu, epi, m, n0 + e);
    if (epi == EPI_NCHW) {
        int b = n0 / P, pix = n0 - b * P;
        float *dst = C + ((long long)b * M + m) * P + pix;
        if (pix + 4 <= P && ((uintptr_t)dst & 15) == 0) {
            *(float4 *)dst = make_float4(out[0], out[1], out[2], out[3]);
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            C[((long long)b * M + m) * P + pix] = out[e];
            if (++pix == P) {
                pix = 0;
                ++b;
            }
        }
    } else {
        float *dst = C + (long long)m * ldc + n0;
        if (((uintptr_t)dst & 15) == 0) {
            *(float4 *)dst = make_float4(out[0], out[1], out[2], out[3]);
            return;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e)
            dst[e] = out[e];
    }
}

__global__ __launch_bounds__(NT) void splitk_reduce_group_kernel(const float *__restrict__ part, int splits,
                                                                 int M, int N, long long stride, int epi,
                                                                 float *__restrict__ C, int ldc,
                                                                 const float *__restrict__ bias, int P, int relu,
                                                                 int rblocks, BiasSum bs)
{
    if ((int)blockIdx.x >= rblocks) {  // uniform per block: no barrier below is split
        bias_sum_job(bs, (int)blockIdx.x - rblocks);
        return;
    }
    constexpr int G = NT / 64;  // split groups per block
    __shared__ float red[G][64];
    const long long total = (long long)M * N;
    const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
    const long long idx = (long long)blockIdx.x * 64 + lane;
    const int per = (splits + G - 1) / G;
    const int s0 = grp * per, s1 = min(splits, s0 + per);
    float acc = 0.0f;
    if (idx < total) {
        int sp = s0;
        for (; sp + 4 <= s1; sp += 4) {
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                v[u] = part[(sp + u) * stride + idx];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                acc += v[u];
        }
        for (; sp < s1; ++sp)
            acc += part[sp * stride + idx];
    }
    red[grp][lane] = acc;
    __syncthreads();
    if (grp == 0 && idx < total) {
        float t = red[0][lane];
#pragma unroll
        for (int g2 = 1; g2 < G; ++g2)
            t += red[g2][lane];
        splitk_store(t, idx, M, N, epi, C, ldc, bias, P, relu);
    }
}

// ---------------------------------------------------------------------------
// Filter for the implicit data gradient: Wf[c][o][u][v] = W[o][c][kH-1-u][kW-1-v]
// (output channels and input channels swapped, taps rotated by 180 degrees).
// One thread per output element; writes coalesced.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(NT) void flip_filter_kernel(const T *__restrict__ w, T *__restrict__ wf, int O,
                                                         int C, int kH, int kW)
{
    const long long total = (long long)O * C * kH * kW;
    const long long i = (long long)blockIdx.x * NT + threadIdx.x;
    if (i >= total)
        return;
    const int khw = kH * kW;
    const int t = (int)(i % khw);
    const long long co = i / khw;  // c*O + o
    const int o = (int)(co % O), c = (int)(co / O);
    const int u = t / kW, v = t - (t / kW) * kW;
    wf[i] = w[((long long)o * C + c) * khw + (kH - 1 - u) * kW + (kW - 1 - v)];
}

inline dim3 grid2(long long x, long long y)
{
    return dim3((unsigned)x, (unsigned)(y < 65535 ? y : 65535), 1);
}

}  // namespace

namespace {

// Phase filters of a strided data gradient: for phase k of pa, element
// e = c*K + ((ob*Tu + u')*Tv + v')*bk + oi of its block (at pa.ph[k].a_off;
// K = Tu*Tv*O, o = ob*bk + oi: the NHWC loader's order of channel block,
// tap, channel) is W[o][c][rh + s*(Tu-1-u')][rw + s*(Tv-1-v')], where the
// phase's first dx row h0 fixes rh = (h0 + p) mod s (likewise rw).  Every
// tap of W lands in exactly one phase, so the blocks together hold |W|
// elements.  One thread per element, writes in order.
template <typename T>
__global__ __launch_bounds__(NT) void phase_filter_kernel(const T *__restrict__ w, T *__restrict__ wph,
                                                          ConvGeom g, PhaseArgs pa, long long total, int bk)
{
    const long long e = (long long)blockIdx.x * NT + threadIdx.x;
    if (e >= total)
        return;
    int k = 0;
    while (k + 1 < pa.n && e >= pa.ph[k + 1].a_off)
        ++k;
    const PhaseItem &it = pa.ph[k];
    const int Tu = it.g.kH, Tv = it.g.kW, O = g.O;
    const int rh = (it.h0 + g.p) % g.s, rw = (it.w0 + g.p) % g.s;
    const long long K = (long long)Tu * Tv * O;
    const long long r = e - it.a_off;
    const int c = (int)(r / K);
    int q = (int)(r - c * K);
    const int oi = q % bk;
    q /= bk;
    const int vv = q % Tv;
    q /= Tv;
    const int uu = q % Tu;
    const int o = (q / Tu) * bk + oi;
    const int u = rh + g.s * (Tu - 1 - uu), v = rw + g.s * (Tv - 1 - vv);
    wph[e] = w[(((long long)o * g.C + c) * g.kH + u) * g.kW + v];
}

}  // namespace

hipError_t launch_phase_filter(int dt, const ConvGeom &g, const PhaseArgs &pa, const void *w, void *wph,
                               hipStream_t s)
{
    const long long total = (long long)g.O * g.C * g.kH * g.kW;
    const dim3 grid((unsigned)((total + NT - 1) / NT));
    if (dt == DT_F32)
        hipLaunchKernelGGL(phase_filter_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)w,
                           (uint32_t *)wph, g, pa, total, gemm_bk(dt));
    else
        hipLaunchKernelGGL(phase_filter_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)w,
                           (uint16_t *)wph, g, pa, total, gemm_bk(dt));
    return hipGetLastError();
}

// experiments, tests: D4R_IM2COL_SHIFT=0 keeps stride-1 layers on the
// general LDS kernel
static bool im2col_shift_enabled()
{
    const char *e = getenv("D4R_IM2COL_SHIFT");
    return !(e && e[0] == '0');
}

// Which im2col kernel a launch runs and its block shape.  LDS-staged path:
// a block covers up to ~128K col elements (whole images of one channel when
// an image is small, else a range of output rows), halved until the grid
// has 2048 blocks (16-bit) or 512 (f32), and its input window must fit in
// 48 KB; otherwise the direct gather.  (16-bit, against 16K and 1024
// blocks: AlexNet conv3-5 bf16 im2col 25.3 -> 22.1 us.  f32 with 512
// instead of 2048: LeNet conv2 11.2 -> 6.4 us, AlexNet conv1 46.7 -> 43.8
// us, conv3-5 32.3 -> 30.0 us.)
Im2colPlan plan_im2col(int dt, const ConvGeom &g)
{
    const int VW = dt == DT_F32 ? 4 : 8;
    const int es = dt == DT_F32 ? 4 : 2;
    Im2colPlan pl{IM2COL_GATHER, g.OH, 1, 0, 0, 0};
    const int khw = g.kH * g.kW;
    const int Wl = (g.OW - 1) * g.s + g.kW;
    const long long per_img = (long long)khw * g.OH * g.OW;
    long long target = 131072;
    long long min_blocks = dt == DT_F32 ? 512 : 2048;
    if (const char *e = getenv("D4R_IM2COL_TARGET"))  // experiments
        target = atoll(e);
    if (const char *e = getenv("D4R_IM2COL_MINBLK"))  // experiments
        min_blocks = atoll(e);
    // f32 row-range blocks at half the size: their windows then fit four
    // blocks per CU in LDS (AlexNet conv1: 10 -> 9 output rows of 11x11
    // stride-4 taps, 42.7 -> 39 KB; im2col 44.0 -> 38.7 us)
    if (dt == DT_F32 && per_img >= target)
        target /= 2;
    int RB = g.OH, BB = 1;
    if (per_img >= target) {
        RB = (int)(target / ((long long)khw * g.OW));
        RB = RB < 1 ? 1 : (RB > g.OH ? g.OH : RB);
    } else {
        BB = (int)(target / per_img);
        BB = BB < 1 ? 1 : (BB > g.B ? g.B : BB);
    }
    // enough blocks to fill the chip: split images, then output rows
    auto blocks = [&](int rb, int bb) {
        return (long long)((g.OH + rb - 1) / rb) * g.C * ((g.B + bb - 1) / bb);
    };
    while (BB > 1 && blocks(RB, BB) < min_blocks)
        BB = (BB + 1) / 2;
    while (RB > 1 && blocks(RB, BB) < min_blocks)
        RB = (RB + 1) / 2;
    if (const char *e = getenv("D4R_IM2COL_RB")) {  // experiments: output rows per block
        RB = std::max(1, std::min(atoi(e), g.OH));
        BB = 1;
    }
    int Rl = (RB - 1) * g.s + g.kH;
    while (BB > 1 && (long long)BB * Rl * Wl * es > 48 * 1024)
        BB = (BB + 1) / 2;
    while (RB > 1 && (long long)Rl * Wl * es > 48 * 1024) {
        RB = (RB + 1) / 2;
        Rl = (RB - 1) * g.s + g.kH;
    }
    const long long win_elems = (long long)BB * Rl * Wl;
    const size_t shm = (size_t)(es == 4 ? lds_padded_elems<uint32_t>(win_elems)
                                        : lds_padded_elems<uint16_t>(win_elems)) * es;
    // stride 1 with whole vectors per output row: the shifted-copy kernel
    // (its LDS holds kW copies of the window's OW-wide part)
    if (g.s == 1 && g.OW % VW == 0 && g.OW <= 1024 && g.C <= 65535 && im2col_shift_enabled()) {
        int rb = RB, bb = BB;
        auto rl = [&](int r) { return r - 1 + g.kH; };
        auto elems = [&](int r, int b) { return (long long)g.kW * b * rl(r) * g.OW; };
        while (bb > 1 && (elems(rb, bb) * es > 48 * 1024 || (long long)bb * rl(rb) > 1024))
            bb = (bb + 1) / 2;
        while (rb > 1 && (elems(rb, bb) * es > 48 * 1024 || (long long)bb * rl(rb) > 1024))
            rb = (rb + 1) / 2;
        if (elems(rb, bb) * es <= 48 * 1024 && (long long)bb * rl(rb) <= 1024 && elems(rb, bb) < (1 << 20) &&
            (g.B + bb - 1) / bb <= 65535)
            return Im2colPlan{IM2COL_SHIFT, rb, bb, rl(rb), g.OW, (size_t)elems(rb, bb) * es};
    }
    if (shm <= 50 * 1024 && g.C <= 65535 && (g.B + BB - 1) / BB <= 65535 && Rl <= 1024)
        return Im2colPlan{IM2COL_LDS, RB, BB, Rl, Wl, shm};
    return pl;
}

hipError_t launch_im2col(int dt, const ConvGeom &g, const void *x, void *col, hipStream_t s)
{
    const int VW = dt == DT_F32 ? 4 : 8;
    const Im2colPlan pl = plan_im2col(dt, g);
    if (pl.kind == IM2COL_SHIFT) {
        dim3 grid((g.OH + pl.RB - 1) / pl.RB, g.C, (g.B + pl.BB - 1) / pl.BB);
        if (dt == DT_F32)
            hipLaunchKernelGGL(im2col_shift_kernel<uint32_t>, grid, dim3(NT), pl.shm, s, (const uint32_t *)x,
                               (uint32_t *)col, g, pl.RB, pl.BB, pl.Rl);
        else
            hipLaunchKernelGGL(im2col_shift_kernel<uint16_t>, grid, dim3(NT), pl.shm, s, (const uint16_t *)x,
                               (uint16_t *)col, g, pl.RB, pl.BB, pl.Rl);
        return hipGetLastError();
    }
    if (pl.kind == IM2COL_LDS) {
        dim3 grid((g.OH + pl.RB - 1) / pl.RB, g.C, (g.B + pl.BB - 1) / pl.BB);
        const int vec = (g.N % VW) == 0;
        if (dt == DT_F32)
            hipLaunchKernelGGL(im2col_lds_kernel<uint32_t>, grid, dim3(NT), pl.shm, s, (const uint32_t *)x,
                               (uint32_t *)col, g, pl.RB, pl.BB, pl.Rl, pl.Wl, vec);
        else
            hipLaunchKernelGGL(im2col_lds_kernel<uint16_t>, grid, dim3(NT), pl.shm, s, (const uint16_t *)x,
                               (uint16_t *)col, g, pl.RB, pl.BB, pl.Rl, pl.Wl, vec);
        return hipGetLastError();
    }
    const long long threads = (g.N + VW - 1) / VW;
    dim3 grid = grid2((threads + NT - 1) / NT, (long long)g.C * g.kH);
    const int vec = (g.N % VW) == 0;
    if (dt == DT_F32)
        hipLaunchKernelGGL(im2col_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)x,
                           (uint32_t *)col, g, vec);
    else
        hipLaunchKernelGGL(im2col_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)x,
                           (uint16_t *)col, g, vec);
    return hipGetLastError();
}

// LDS path of col2im: whole padded image windows of one channel fit in 48
// KB and a block's columns fit in QMAX vectors per thread; BB images per
// block, halved until the grid has 1024 blocks, and at least 256 blocks;
// otherwise the element-parallel gather.
Col2imPlan plan_col2im(const ConvGeom &g)
{
    const int Rl = (g.OH - 1) * g.s + g.kH;
    const int Wl = (g.OW - 1) * g.s + g.kW;
    const long long win = (long long)Rl * Wl * 4;
    const long long max_cols = (long long)C2I_QMAX * NT * 4 - 4;
    if (win <= 48 * 1024 && g.P <= max_cols && g.C <= 65535) {
        long long BB = (48 * 1024) / win;
        const long long by_cols = max_cols / g.P;
        if (BB > by_cols)
            BB = by_cols;
        if (BB > g.B)
            BB = g.B;
        if (BB < 1)
            BB = 1;
        while (BB > 1 && (long long)g.C * ((g.B + BB - 1) / BB) < 1024)
            BB = (BB + 1) / 2;
        if ((long long)g.C * ((g.B + BB - 1) / BB) >= 256 && (g.B + BB - 1) / BB <= 65535)
            return Col2imPlan{COL2IM_LDS, (int)BB, Rl, Wl,
                              (size_t)lds_padded_elems<float>(BB * (long long)Rl * Wl) * 4};
    }
    return Col2imPlan{COL2IM_GATHER, 1, 0, 0, 0};
}

hipError_t launch_col2im(const ConvGeom &g, const float *dcol, float *dx, hipStream_t s)
{
    const Col2imPlan pl = plan_col2im(g);
    if (pl.kind == COL2IM_LDS) {
        dim3 grid(1, g.C, (unsigned)((g.B + pl.BB - 1) / pl.BB));
        const int vec = (g.N % 4) == 0;
        hipLaunchKernelGGL(col2im_lds_kernel, grid, dim3(NT), pl.shm, s, dcol, dx, g, pl.BB, pl.Rl, pl.Wl, vec);
        return hipGetLastError();
    }
    const int total = g.B * g.C * g.H * g.W;
    const int threads = (total + 3) / 4;  // four dx elements per thread
    const dim3 grid((threads + NT - 1) / NT), block(NT);
    const int tu = (g.kH + g.s - 1) / g.s, tv = (g.kW + g.s - 1) / g.s;
    if (tu == 1 && tv == 1)
        hipLaunchKernelGGL((col2im_kernel<1, 1>), grid, block, 0, s, dcol, dx, g, total);
    else if (tu == 2 && tv == 2)
        hipLaunchKernelGGL((col2im_kernel<2, 2>), grid, block, 0, s, dcol, dx, g, total);
    else if (tu == 3 && tv == 3)
        hipLaunchKernelGGL((col2im_kernel<3, 3>), grid, block, 0, s, dcol, dx, g, total);
    else if (tu == 5 && tv == 5)
        hipLaunchKernelGGL((col2im_kernel<5, 5>), grid, block, 0, s, dcol, dx, g, total);
    else
        hipLaunchKernelGGL((col2im_kernel<0, 0>), grid, block, 0, s, dcol, dx, g, total);
    return hipGetLastError();
}

int grad_reshape_blocks(int dt, const ConvGeom &g)
{
    const int VW = dt == DT_F32 ? 4 : 8;
    const long long threads = (g.N + VW - 1) / VW;
    return (int)((threads + NT - 1) / NT);
}

hipError_t launch_grad_reshape(int dt, const ConvGeom &g, const void *dy, void *G, float *bias_part,
                               hipStream_t s)
{
    const int VW = dt == DT_F32 ? 4 : 8;
    dim3 grid = grid2(grad_reshape_blocks(dt, g), g.O);
    const int vec = (g.N % VW) == 0;
    if (dt == DT_F32)
        hipLaunchKernelGGL(grad_reshape_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)dy,
                           (uint32_t *)G, g, vec, bias_part, dt);
    else
        hipLaunchKernelGGL(grad_reshape_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)dy,
                           (uint16_t *)G, g, vec, bias_part, dt);
    return hipGetLastError();
}

hipError_t launch_bias_final(const float *partial, float *db, int O, int splits, hipStream_t s)
{
    hipLaunchKernelGGL(bias_final_kernel, dim3((O + NT - 1) / NT), dim3(NT), 0, s, partial, db, O, splits);
    return hipGetLastError();
}

hipError_t launch_transpose(int dt, int batch, int R, int Cc, const void *in, void *out, hipStream_t s)
{
    dim3 grid((Cc + 63) / 64, (R + 63) / 64, batch);
    if (dt == DT_F32)
        hipLaunchKernelGGL(transpose_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)in,
                           (uint32_t *)out, R, Cc);
    else
        hipLaunchKernelGGL(transpose_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)in,
                           (uint16_t *)out, R, Cc);
    return hipGetLastError();
}

int bias_grad_splits(const ConvGeom &g)
{
    // enough blocks to cover the chip several times (>= ~4096), at least one
    // image per block
    int want = (4096 + g.O - 1) / g.O;
    if (want > g.B)
        want = g.B;
    if (want < 1)
        want = 1;
    int per = (g.B + want - 1) / want;
    return (g.B + per - 1) / per;
}

hipError_t launch_bias_partials(int dt, const ConvGeom &g, const void *dy, float *partial, int splits,
                                hipStream_t s)
{
    const int per = (g.B + splits - 1) / splits;
    dim3 grid(splits, g.O);
    if (dt == DT_F32)
        hipLaunchKernelGGL(bias_partial_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)dy,
                           partial, g, splits, per, dt);
    else
        hipLaunchKernelGGL(bias_partial_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)dy,
                           partial, g, splits, per, dt);
    return hipGetLastError();
}

hipError_t launch_bias_grad(int dt, const ConvGeom &g, const void *dy, float *db, float *partial,
                            int splits, hipStream_t s)
{
    hipError_t e = launch_bias_partials(dt, g, dy, partial, splits, s);
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL(bias_final_kernel, dim3((g.O + NT - 1) / NT), dim3(NT), 0, s, partial, db, g.O,
                       splits);
    return hipGetLastError();
}

hipError_t launch_flip_filter(int dt, const ConvGeom &g, const void *w, void *wf, hipStream_t s)
{
    const long long total = (long long)g.O * g.C * g.kH * g.kW;
    const dim3 grid((unsigned)((total + NT - 1) / NT));
    if (dt == DT_F32)
        hipLaunchKernelGGL(flip_filter_kernel<uint32_t>, grid, dim3(NT), 0, s, (const uint32_t *)w,
                           (uint32_t *)wf, g.O, g.C, g.kH, g.kW);
    else
        hipLaunchKernelGGL(flip_filter_kernel<uint16_t>, grid, dim3(NT), 0, s, (const uint16_t *)w,
                           (uint16_t *)wf, g.O, g.C, g.kH, g.kW);
    return hipGetLastError();
}

// partial bias sums per channel of the one-pass dy preparation: one per
// image and 64-pixel tile
int dy_prep_bias_parts(const ConvGeom &g) { return g.B * ((g.P + 63) / 64); }

namespace {

long long filter_blocks(int dt, const FilterJob &f)
{
    if (f.flip)  // 64x64 tiles of w viewed as O x C*taps
        return (long long)((f.C * f.taps + 63) / 64) * ((f.O + 63) / 64);
    const long long vw = dt == DT_F32 ? 4 : 8;
    return ((long long)f.O * f.C * f.taps / vw + NT - 1) / NT;
}

}  // namespace

hipError_t launch_dy_prep(int dt, DyPrep a, FilterJob w, hipStream_t s)
{
    const long long na = (long long)((a.P + 63) / 64) * ((a.O + 63) / 64) * a.B;
    const long long nw = filter_blocks(dt, w);
    if (na + nw > INT32_MAX)
        return hipErrorInvalidValue;
    a.blocks = (int)na;
    a.dt = dt;
    if (dt == DT_F32)
        hipLaunchKernelGGL(dy_prep_kernel<uint32_t>, dim3((unsigned)(na + nw)), dim3(NT), 0, s, a, w);
    else
        hipLaunchKernelGGL(dy_prep_kernel<uint16_t>, dim3((unsigned)(na + nw)), dim3(NT), 0, s, a, w);
    return hipGetLastError();
}

int bias_sum_blocks(const BiasSum &bs) { return (bs.O + NT / 64 - 1) / (NT / 64); }

hipError_t launch_bias_sum(const BiasSum &bs, hipStream_t s)
{
    hipLaunchKernelGGL(bias_sum_kernel, dim3((unsigned)bias_sum_blocks(bs)), dim3(NT), 0, s, bs);
    return hipGetLastError();
}

hipError_t launch_transpose_filter(int dt, TransposeJob a, FilterJob f, hipStream_t s)
{
    const long long na = (long long)((a.Cc + 63) / 64) * ((a.R + 63) / 64) * a.batch;
    const long long nf = filter_blocks(dt, f);
    if (na + nf > INT32_MAX)
        return hipErrorInvalidValue;
    a.blocks = (int)na;
    if (dt == DT_F32)
        hipLaunchKernelGGL(transpose_filter_kernel<uint32_t>, dim3((unsigned)(na + nf)), dim3(NT), 0, s, a, f);
    else
        hipLaunchKernelGGL(transpose_filter_kernel<uint16_t>, dim3((unsigned)(na + nf)), dim3(NT), 0, s, a, f);
    return hipGetLastError();
}

hipError_t launch_splitk_reduce(const float *part, int splits, int M, int N, long long split_stride,
                                int epi, float *C, int ldc, const float *bias, int P, int relu,
                                const BiasSum &bs, hipStream_t s)
{
    const long long total = (long long)M * N;
    const long long vthreads = (total + 3) / 4;
    const bool vec = (N % 4) == 0 && (split_stride % 4) == 0 && ((uintptr_t)part % 16) == 0;
    const int bblocks = bs.db ? bias_sum_blocks(bs) : 0;
    // the vector path needs enough threads to fill the chip
    if (vec && vthreads >= 64LL * 1024) {
        const int rb = (int)((vthreads + NT - 1) / NT);
        hipLaunchKernelGGL(splitk_reduce_vec_kernel, dim3((unsigned)(rb + bblocks)), dim3(NT), 0, s, part, splits,
                           M, N, split_stride, epi, C, ldc, bias, P, relu, rb, bs);
    } else {
        const int rb = (int)((total + 63) / 64);
        hipLaunchKernelGGL(splitk_reduce_group_kernel, dim3((unsigned)(rb + bblocks)), dim3(NT), 0, s, part,
                           splits, M, N, split_stride, epi, C, ldc, bias, P, relu, rb, bs);
    }
    return hipGetLastError();
}

}  // namespace d4r
