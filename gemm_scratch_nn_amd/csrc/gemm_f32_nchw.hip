// Instantiation of the gfx950 MFMA GEMM for f32 operands whose A or B is an
// NCHW tensor read in place: the data-gradient product (A = Wmat read
// row-contiguous, B = dy) and the filter-gradient product (A = dy, B = col
// read k-contiguous), and for 1x1 stride-1 unpadded convolutions the forward
// (A = Wmat, B = x) and the filter gradient (A = dy, B = x); and the implicit
// data gradient from dy read as NHWC (A = the flipped filter, B = OP_IMPL_T).
#include "gemm_impl.hpp"

namespace d4r {

hipError_t launch_gemm_f32_nchw(int cfg, int amode, int bmode, const GemmParams &p, hipStream_t s)
{
    if (amode == OP_ROWS && bmode == OP_NCHW)
        return launch_gemm32_modes<OP_ROWS, OP_NCHW>(cfg, p, s);
    if (amode == OP_NCHW && bmode == OP_KC)
        return launch_gemm32_modes<OP_NCHW, OP_KC>(cfg, p, s);
    if (amode == OP_KC && bmode == OP_NCHW)
        return launch_gemm32_modes<OP_KC, OP_NCHW>(cfg, p, s);
    if (amode == OP_NCHW && bmode == OP_NCHW_K)
        return launch_gemm32_modes<OP_NCHW, OP_NCHW_K>(cfg, p, s);
    if (amode == OP_KC && bmode == OP_IMPL_T) {
        // whole 32-deep stages inside one tap
        if (p.g.C % kBK32 != 0 || p.k_per_split % kBK32 != 0 || p.g.s != 1)
            return hipErrorInvalidValue;
        return launch_gemm32_modes<OP_KC, OP_IMPL_T>(cfg, p, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace d4r
