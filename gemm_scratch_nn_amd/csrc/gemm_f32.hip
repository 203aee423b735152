// Instantiation of the gfx950 MFMA GEMM for f32 operands (f32 accumulation):
// the plainly strided operand pairs and the implicit forward.  The pairs
// that read an NCHW gradient are built in gemm_f32_nchw.hip.
#include "gemm_impl.hpp"

namespace d4r {

hipError_t launch_gemm_f32_nchw(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s);
bool try_gemm_f32_dl(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s, hipError_t *err);

hipError_t launch_gemm_f32(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    hipError_t e;
    if (try_gemm_f32_dl(cfg, amode, bmode, p, s, &e))
        return e;
    if (amode == OP_KC && bmode == OP_ROWS)
        return launch_gemm32_modes<OP_KC, OP_ROWS>(cfg, p, s);
    if (amode == OP_KC && bmode == OP_KC)
        return launch_gemm32_modes<OP_KC, OP_KC>(cfg, p, s);
    if (amode == OP_ROWS && bmode == OP_ROWS)
        return launch_gemm32_modes<OP_ROWS, OP_ROWS>(cfg, p, s);
    if (amode == OP_ROWS && bmode == OP_KC)
        return launch_gemm32_modes<OP_ROWS, OP_KC>(cfg, p, s);
    if (amode == OP_KC && bmode == OP_IMPL)
        return launch_gemm32_modes<OP_KC, OP_IMPL>(cfg, p, s);
    return launch_gemm_f32_nchw(cfg, amode, bmode, p, s);
}

}  // namespace d4r
