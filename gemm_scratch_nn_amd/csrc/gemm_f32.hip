// Instantiation of the gfx950 MFMA GEMM for f32 operands (f32 accumulation).
#include "gemm_impl.hpp"

namespace d4r {

hipError_t launch_gemm_f32(int cfg, bool a_kc, bool b_kc, const GemmParams &p, hipStream_t s)
{
    return launch_gemm_dt<DtF32>(cfg, a_kc, b_kc, p, s);
}

hipError_t launch_gemm_implicit_f32(int cfg, const GemmParams &p, hipStream_t s)
{
    return launch_gemm_layout<DtF32, true, false, true>(cfg, p, s);
}

}  // namespace d4r
