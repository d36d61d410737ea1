// Instances of the direct-load ring GEMM kernel: 256x256x64 tile, 2-slot LDS ring, 8 wave64s, MFMA 16x16x32, bf16 operands.
#include "gemm_lds.hpp"

namespace tlg {

hipError_t launch_lds_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds<DT_BF16>(p, transpose_A, transpose_B, stream);
}

}  // namespace tlg
