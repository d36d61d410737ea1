// Instances of the direct-load ring GEMM kernel with 32 x 128 output tiles
// (f16 and bf16 operands): 8 waves of 32 x 16 side by side, K tiles of 128 in a
// 4-slot ring (all 160 KiB of LDS, three tiles in flight), barrier after the first
// of the last K step's 2 MFMAs, one direct load every 2 MFMAs.  For grids whose 32 x 128 tiles fit one wave of the
// chip: twice the workgroups of the 64 x 128 tiles, each with half the A rows.
// Measured on MI355X against the 64 x 128 kernel (same process, operands rotated
// through 1 GiB): 1024^3 10.5 -> 9.6 us, 256^3 ReLU 5.17 -> 4.62, 1024^2 x 512
// 7.44 -> 6.80, 512 x 1024^2 bf16 10.4 -> 9.3, 64 x 16384 x 2048 with B stored
// [N,K] 20.1 -> 18.1.  Four waves of 32 x 32 were 3-5% slower on all of these
// but the last (17.9 us), barriers after 1 or 3 of 4 MFMAs and 2-slot rings
// slower still; the fourth slot gained 1.5% over three (1024^3 9.61 -> 9.46 us,
// 1024^2 x 2048 13.64 -> 13.44; bit-identical).  Like the 64 x 128 kernel, A must be K-contiguous
// (transpose_A == 0).
#include "gemm_lds.hpp"

namespace tlg {

template <int T>
static hipError_t dispatch_lds32(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    if (tA) return hipErrorInvalidValue;
    if (tB) return launch_lds_inst<32, 128, 4, 1, 2, 1, 8, T, true, true, kModeDP, 128>(p, s);
    return launch_lds_inst<32, 128, 4, 1, 2, 1, 8, T, true, false, kModeDP, 128>(p, s);
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
