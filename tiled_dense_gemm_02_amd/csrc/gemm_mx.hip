// Instances of the block-scaled FP8 GEMM kernel (E4M3 and E5M2 operands, E8M0 scales).
#include "gemm_mx.hpp"

namespace tlg {

hipError_t launch_mx(const MxParams& p, int fmt, hipStream_t stream)
{
    MxParams args = p;
    void* kargs[] = {&args};
    const void* fn = fmt == 0 ? (const void*)&gemm_mx_kernel<0> : (const void*)&gemm_mx_kernel<1>;
    return hipLaunchKernel(fn, dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(512), kargs, 0, stream);
}

}  // namespace tlg
