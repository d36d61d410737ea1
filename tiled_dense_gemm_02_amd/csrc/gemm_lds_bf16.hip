// Instances of the direct-load ring GEMM kernels (MFMA 16x16x32, 8 wave64s, bf16 operands):
// 256x256x64 tiles with a 2-slot LDS ring and 128x128x64 tiles with a 4-slot ring
// (also with K split over several workgroups per tile).
#include "gemm_lds.hpp"

namespace tlg {

hipError_t launch_lds_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds<DT_BF16>(p, transpose_A, transpose_B, stream);
}

hipError_t launch_lds128_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds128<DT_BF16>(p, transpose_A, transpose_B, stream);
}

hipError_t launch_lds128sk_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds128_sk<DT_BF16>(p, transpose_A, transpose_B, stream);
}

hipError_t launch_lds64_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds64<DT_BF16>(p, transpose_A, transpose_B, stream);
}

}  // namespace tlg
