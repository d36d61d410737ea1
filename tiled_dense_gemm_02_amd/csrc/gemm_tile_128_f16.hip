// Instances of the tiled GEMM kernel: 128x128x64 block tile, f16 operands.
#include "gemm_tile.hpp"

namespace tlg {

hipError_t launch_tile_128_f16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a, int vec_b,
                             hipStream_t stream)
{
    return dispatch_layout<128, 128, 2, 1, DT_F16, true>(p, transpose_A, transpose_B, vec_a, vec_b, stream);
}

}  // namespace tlg
