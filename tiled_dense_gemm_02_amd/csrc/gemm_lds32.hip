// Instances of the direct-load ring GEMM kernel with 32 x 128 output tiles
// (f16 and bf16 operands): 4 waves of 32 x 32 (one per SIMD), K tiles of 128 in a
// 3-slot ring (120 KiB), barrier after 2 of the last K step's 4 MFMAs, one direct
// load per MFMA.  For grids whose 32 x 128 tiles fit one wave of the chip: twice
// the workgroups of the 64 x 128 tiles, each with half the A rows.  Measured on
// MI355X against the 64 x 128 kernel (same process, operands rotated through
// 1 GiB): 1024^3 10.65 -> 10.14 us, 256^3 ReLU 5.18 -> 4.87, 512 x 1024 x 1024
// 10.5 -> 9.9, 768^2 x 2048 16.5 -> 15.9, 1024^2 x 2048 with B stored [N,K]
// 15.3 -> 13.7; barriers after 1 or 3 MFMAs and 2-slot rings were slower.  Like
// the 64 x 128 kernel, A must be K-contiguous (transpose_A == 0).
#include "gemm_lds.hpp"

namespace tlg {

template <int T>
static hipError_t dispatch_lds32(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    if (tA) return hipErrorInvalidValue;
    if (tB) return launch_lds_inst<32, 128, 3, 2, 1, 1, 4, T, true, true, kModeDP, 128>(p, s);
    return launch_lds_inst<32, 128, 3, 2, 1, 1, 4, T, true, false, kModeDP, 128>(p, s);
}

hipError_t launch_lds32_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds32<DT_F16>(p, transpose_A, transpose_B, stream);
}

hipError_t launch_lds32_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream)
{
    return dispatch_lds32<DT_BF16>(p, transpose_A, transpose_B, stream);
}

}  // namespace tlg
