// Instantiation of the gfx950 MFMA GEMM for f16 operands (f32 accumulation).
#include "gemm16_impl.hpp"

namespace d4r {

hipError_t launch_gemm_f16(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    return launch_gemm16<DT_F16>(cfg, amode, bmode, p, s);
}

hipError_t launch_gemm_phased_f16(const GemmParams &p, const PhaseArgs &pa, hipStream_t s)
{
    return launch_gemm_dl_phased<DT_F16>(p, pa, s);
}

}  // namespace d4r
