// Instances of the block-scaled GEMM kernel (E4M3, E5M2 and E2M1 operands, E8M0 scales).
#include "gemm_mx.hpp"

namespace tlg {

hipError_t launch_mx(const MxParams& p, int fmt, hipStream_t stream)
{
    MxParams args = p;
    void* kargs[] = {&args};
    const void* fn = fmt == 0   ? (const void*)&gemm_mx_kernel<0>
                     : fmt == 1 ? (const void*)&gemm_mx_kernel<1>
                                : (const void*)&gemm_mx_kernel<4>;
    return hipLaunchKernel(fn, dim3((unsigned)(p.tiles_m * p.tiles_n)), dim3(512), kargs, 0, stream);
}

}  // namespace tlg
