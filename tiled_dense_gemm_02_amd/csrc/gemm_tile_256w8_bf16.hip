// Instances of the tiled GEMM kernel: 256x256x64 block tile, 8 wave64s (2 per SIMD), bf16 operands.
#include "gemm_tile.hpp"

namespace tlg {

hipError_t launch_tile_256w8_bf16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a, int vec_b,
                               hipStream_t stream)
{
    return dispatch_layout<256, 256, 2, 4, DT_BF16, false>(p, transpose_A, transpose_B, vec_a, vec_b, stream);
}

}  // namespace tlg
