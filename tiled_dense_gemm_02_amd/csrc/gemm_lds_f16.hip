// Instances of the direct-load ring GEMM kernel: 256x256x64 tile, 2-stage LDS ring, 8 wave64s, f16 operands.
#include "gemm_lds.hpp"

namespace tlg {

hipError_t launch_lds_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds<64, 1, 2, false, 2, 4, DT_F16>(p, transpose_A, transpose_B, stream);
}

}  // namespace tlg
