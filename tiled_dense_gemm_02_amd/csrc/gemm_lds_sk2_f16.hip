// Instances of the persistent stream-K schedules of the direct-load ring GEMM
// kernels (f16 operands): 256x256x64 tiles (2-slot ring) and 128x128x64 tiles (4-slot ring).
#include "gemm_lds.hpp"

namespace tlg {

hipError_t launch_lds_sk2_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds_streamk<DT_F16>(p, transpose_A, transpose_B, stream);
}

hipError_t launch_lds128_sk2_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds128_streamk<DT_F16>(p, transpose_A, transpose_B, stream);
}

}  // namespace tlg
