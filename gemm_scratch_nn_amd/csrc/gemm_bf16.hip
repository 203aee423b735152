// Instantiation of the gfx950 MFMA GEMM for bf16 operands (f32 accumulation).
#include "gemm16_impl.hpp"

namespace d4r {

hipError_t launch_gemm_bf16(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    return launch_gemm16<DT_BF16>(cfg, amode, bmode, p, s);
}

hipError_t launch_gemm_phased_bf16(const GemmParams &p, const PhaseArgs &pa, hipStream_t s)
{
    return launch_gemm_dl_phased<DT_BF16>(p, pa, s);
}

}  // namespace d4r
