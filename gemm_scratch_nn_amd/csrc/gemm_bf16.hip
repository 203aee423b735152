// Instantiation of the gfx950 MFMA GEMM for bf16 operands (f32 accumulation).
#include "gemm16_impl.hpp"

namespace d4r {

hipError_t launch_gemm_bf16(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    return launch_gemm16<DT_BF16>(cfg, amode, bmode, p, s);
}

}  // namespace d4r
