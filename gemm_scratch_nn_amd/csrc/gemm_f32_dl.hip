// Instantiation of the direct-to-LDS MFMA GEMM for f32 operands: two
// k-contiguous operands (the filter-gradient product on a copied dy) and
// the implicit data gradient from dy read as NHWC.  Tiles 128x128 and
// 128x64 with four wavefronts and a ring of two 32-deep stages (64 / 48 KB
// of LDS: two workgroups per CU, as the register-staged f32 kernel).  A
// 32-float stage takes ~4K MFMA cycles per wavefront, so one stage of loads
// in flight covers the latency.
#include <stdlib.h>

#include "gemm16_impl.hpp"

namespace d4r {

namespace {

bool dl_f32_enabled()
{
    // experiments, tests: D4R_F32_DL=0 runs the register-staged kernel
    const char *e = getenv("D4R_F32_DL");
    return !(e && e[0] == '0');
}

template <bool BI>
hipError_t launch_dl_f32(int cfg, const GemmParams &p, hipStream_t s)
{
    TileShape ts = tile_shape(cfg);
    const int tiles = ((p.M + ts.bm - 1) / ts.bm) * ((p.N + ts.bn - 1) / ts.bn);
    const dim3 grid(tiles * p.splits), b4(256);
    switch (cfg) {
    case TILE_128x128:
        hipLaunchKernelGGL((gemm_dl_kernel<DT_F32, 2, 2, 2, 2, 2, BI>), grid, b4, 0, s, p);
        break;
    case TILE_128x64:
        hipLaunchKernelGGL((gemm_dl_kernel<DT_F32, 2, 2, 2, 1, 2, BI>), grid, b4, 0, s, p);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

// Runs the GEMM with the direct-to-LDS kernel when it applies (returns
// true and sets *err), else returns false: (OP_KC, OP_KC) with 16-byte
// aligned rows, or (OP_KC, OP_IMPL_T); K and every split whole 32-deep
// stages; a 128x128 or 128x64 tile.
bool try_gemm_f32_dl(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s, hipError_t *err)
{
    constexpr int BK = DlElem<DT_F32>::BK;
    if (!dl_f32_enabled() || (cfg != TILE_128x128 && cfg != TILE_128x64) || amode != OP_KC || !p.a_vec ||
        p.K % BK != 0 || p.k_per_split % BK != 0)
        return false;
    if (bmode == OP_KC && p.b_vec) {
        *err = launch_dl_f32<false>(cfg, p, s);
        return true;
    }
    if (bmode == OP_IMPL_T && p.g.C % BK == 0 && p.g.s == 1 && p.zero) {
        *err = launch_dl_f32<true>(cfg, p, s);
        return true;
    }
    return false;
}

hipError_t launch_gemm_phased_f32(const GemmParams &p, const PhaseArgs &pa, hipStream_t s)
{
    return launch_gemm_dl_phased<DT_F32>(p, pa, s);
}

}  // namespace d4r
