// Skinny GEMM  C[M x N] = act(A·B)  for M <= 16 rows per workgroup, B stored
// [N, K] (transpose_B = 1), A stored [M, K].  This shape is bound by the HBM
// stream of B (one read of each element), not by MFMA: the roofline bound
// P <= min(P_peak, I * B_mem) of the overview page's "performance model"
// section puts its arithmetic intensity near 16 FLOP/byte.
//
// Each workgroup owns 16 rows x kSkinnyNB columns of C and reads its B rows
// exactly once.  The waves (kSkinnyThreads / 64 of them) split the K range into
// contiguous slices; each wave streams its slice with 16-byte buffer loads
// straight into MFMA 16x16x32 operand registers (B rows are K-contiguous, which
// is the operand layout, so no LDS staging is needed), two register groups of U
// K steps in flight so the next group's loads overlap the current group's
// MFMAs.  The A slice is re-read from L2 (A is 16 x K).  Measured on MI355X for
// 16 x 16384 x 8192: 8 waves with U = 2 stream B at ~4.8 TB/s against ~4.0 TB/s
// for 4 waves with U = 4 (more waves keep more loads in flight per CU).  The
// partial 16 x NB tiles are summed in LDS in a fixed order (deterministic),
// then the epilogue applies
// (+ prior C) -> ReLU -> rounding -> guarded stores.
//
// Out-of-range rows, columns and K steps read as zero through the buffer
// resource's range check ("core primitives" chapter, section 4.2).

#include "tlg_device.hpp"

namespace tlg {

template <int T_IN, int NB, int U>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_kernel(GemmParams p)
{
    constexpr int NS = NB / 16;     // 16-column MFMA tiles per workgroup
    constexpr int WAVES = kSkinnyThreads / 64;
    static_assert(NB % 16 == 0, "NB must be a multiple of 16");

    __shared__ float red[WAVES][NS][4][64];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int m0 = blockIdx.y * kSkinnyRows;
    const int n0 = blockIdx.x * NB;
    const int K = p.K;
    const int KS = (K + 31) / 32;                       // 32-wide K steps
    const int s_begin = wave * KS / WAVES;
    const int s_end = (wave + 1) * KS / WAVES;

    const uint32_t ld = (uint32_t)K * 2u;
    const uint32_t kbyte = (uint32_t)(lane >> 4) * 16u;  // this lane's 8-element K piece
    const int r = lane & 15;

    // A rows m0.., B rows n0..; resources start at those rows.
    const char* a_base = (const char*)p.A + (uint64_t)m0 * ld;
    const char* b_base = (const char*)p.B + (uint64_t)n0 * ld;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(a_base, (uint64_t)(p.M - m0) * ld);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(b_base, (uint64_t)(p.N - n0) * ld);
    const bool a_ok = m0 + r < p.M;
    const uint32_t a_row = (uint32_t)r * ld;
    bool b_ok[NS];
    uint32_t b_row[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) {
        b_ok[j] = n0 + j * 16 + r < p.N;
        b_row[j] = (uint32_t)(j * 16 + r) * ld;
    }

    f32x4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 a0[U], b0[U][NS], a1[U], b1[U][NS];

    auto issue = [&](int s, u32x4 (&av)[U], u32x4 (&bv)[U][NS]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = s + u;
            const bool k_ok = st < s_end && (st * 32 + (lane >> 4) * 8) < K;
            const uint32_t kofs = (uint32_t)st * 64u + kbyte;
            av[u] = buf_load16(ra, (k_ok && a_ok) ? a_row + kofs : kOOB);
#pragma unroll
            for (int j = 0; j < NS; ++j) bv[u][j] = buf_load16(rb, (k_ok && b_ok[j]) ? b_row[j] + kofs : kOOB);
        }
    };
    // MFMA with the B fragment first: the hardware tile is C's transpose, so
    // acc[j][e] is C[m0 + lane%16][n0 + 16j + 4*(lane/16) + e].
    auto compute = [&](const u32x4 (&av)[U], const u32x4 (&bv)[U][NS]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NS; ++j) acc[j] = mfma16x16x32<T_IN>(bv[u][j], av[u], acc[j]);
    };

    issue(s_begin, a0, b0);
    for (int s = s_begin; s < s_end; s += 2 * U) {
        issue(s + U, a1, b1);
        compute(a0, b0);
        issue(s + 2 * U, a0, b0);
        compute(a1, b1);
    }

#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[wave][j][e][lane] = acc[j][e];
    __syncthreads();

    const int m = m0 + r;
    const bool vec_cols = p.c_vec != 0;
    for (int j = wave; j < NS; j += WAVES) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s = red[0][j][e][lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) s += red[w][j][e][lane];
            v[e] = s;
        }
        const int n = n0 + j * 16 + 4 * (lane >> 4);
        if (m >= p.M || n >= p.N) continue;
        const int count = min(4, p.N - n);
        const bool vec_ok = vec_cols && count == 4;
        const int64_t idx = (int64_t)m * p.N + n;
        if (!p.clear_accum) {
            float c[4] = {0.f, 0.f, 0.f, 0.f};
            load_c4(p.C, p.c_dtype, idx, vec_ok, c, count);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = c[e] + v[e];
        }
        if (p.relu) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = relu(v[e]);
        }
        store_c4(p.C, p.c_dtype, idx, vec_ok, v, count);
    }
}

template <int T>
static hipError_t launch_skinny_t(const GemmParams& p, hipStream_t stream)
{
    GemmParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m);
    const dim3 block(kSkinnyThreads);
    return hipLaunchKernel((const void*)&gemm_skinny_kernel<T, kSkinnyNB, 2>, grid, block, kargs, 0, stream);
}

hipError_t launch_skinny(const GemmParams& p, int ab_dtype, hipStream_t stream)
{
    if (ab_dtype == DT_F16) return launch_skinny_t<DT_F16>(p, stream);
    return launch_skinny_t<DT_BF16>(p, stream);
}

}  // namespace tlg
