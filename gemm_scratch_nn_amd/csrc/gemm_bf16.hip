// Instantiation of the gfx950 MFMA GEMM for bf16 operands (f32 accumulation).
#include "gemm16_impl.hpp"

namespace d4r {

hipError_t launch_gemm_bf16(int cfg, bool a_kc, bool b_kc, const GemmParams &p, hipStream_t s)
{
    return launch_gemm16<DT_BF16>(cfg, a_kc, b_kc, p, s);
}

hipError_t launch_gemm_implicit_bf16(int cfg, const GemmParams &p, hipStream_t s)
{
    return launch_gemm16_implicit<DT_BF16>(cfg, p, s);
}

}  // namespace d4r
