// Internal interface between the C-ABI layer (tlg_api.cpp) and the kernel
// translation units.  Not installed; not part of the public header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tlg {

enum : int { DT_F16 = 1, DT_BF16 = 2, DT_F32 = 3 };

// Arguments of one launch (passed by value to the kernels).
struct GemmParams {
    const void* A;
    const void* B;
    void* C;
    int M, N, K;
    int relu;         // 1: ReLU epilogue
    int clear_accum;  // 0: add onto C's prior contents
    int c_dtype;      // DT_F16 / DT_BF16 / DT_F32
    int c_vec;        // 1: N % 4 == 0 and C aligned to 4 elements (vector stores allowed)
    int c_vec8;       // 1: N % 8 == 0 and C aligned to 16 bytes (16-byte stores of 8 16-bit outputs)
    int tiles_m;      // output tiles along M (tile kernels) / row blocks (skinny)
    int tiles_n;      // output tiles along N
    // split-K plans only: K is cut into `splits` ranges of whole K tiles, one
    // workgroup per (tile, range); fp32 partial tiles go to ws ([tile][split][BM*BN])
    // and counters[tile] (zero between launches) elects the workgroup that sums them.
    int splits;
    float* ws;
    unsigned* counters;
    // persistent (stream-K) plans only: persistent_grid workgroups; tiles
    // 0 .. dp_tiles-1 (in tile order) are computed whole, the sk_tiles after them
    // in equal shares of K iterations; partial tiles go to ws slots
    // ([persistent_grid + sk_tiles - 1][BM*BN]), counters[0 .. sk_tiles-1].
    int persistent_grid;
    int dp_tiles;
    int sk_tiles;
};

// Block-tile configurations of the tiled kernel.
enum TileConfig : int { TILE_256 = 1, TILE_128 = 2, TILE_256_W8 = 3 };

struct TileShape {
    int bm, bn, bk, waves_m, waves_n, stages;
    int threads() const { return 64 * waves_m * waves_n; }
};

inline TileShape tile_shape(int cfg)
{
    if (cfg == TILE_256) return TileShape{256, 256, 64, 2, 2, 2};
    if (cfg == TILE_256_W8) return TileShape{256, 256, 64, 2, 4, 2};
    return TileShape{128, 128, 64, 2, 1, 2};
}

// Skinny kernel geometry: skinny_rows(M) rows x skinny_cols(rows) columns per
// workgroup (16 x 64, 32 x 64 or 64 x 32: a stage of A and B rows is 40 or 48
// KiB), operands staged through a kSkinnyStages-deep LDS ring of kSkinnyKST-wide
// K stages.
constexpr int kSkinnyRows = 16;       // rows of the M <= 16 instance
constexpr int kSkinnyMaxRows = 64;    // the automatic plan uses the skinny kernel for M <= 64
constexpr int kSkinnyNB = 64;         // columns of the 16- and 32-row instances
__host__ __device__ constexpr int skinny_rows(int64_t M) { return M <= 16 ? 16 : M <= 32 ? 32 : 64; }
__host__ __device__ constexpr int skinny_cols(int rows) { return rows == 64 ? 32 : kSkinnyNB; }
constexpr int kSkinnyThreads = 512;  // 8 waves split the K steps of each stage
constexpr int kSkinnyKST = 256;      // K elements per LDS stage (512-byte row segments)
constexpr int kSkinnyStages = 3;     // LDS ring depth
constexpr int kSkinnyMaxSplits = 8;  // K ranges per column block (grids of few column blocks)

// Launchers (defined in the kernel translation units).  vec_a / vec_b: 8 for
// 128-bit global loads, 1 for 16-bit loads.
hipError_t launch_tile_256_f16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a,
                              int vec_b, hipStream_t stream);
hipError_t launch_tile_256_bf16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a,
                               int vec_b, hipStream_t stream);
hipError_t launch_tile_256w8_f16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a,
                                int vec_b, hipStream_t stream);
hipError_t launch_tile_256w8_bf16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a,
                                 int vec_b, hipStream_t stream);
hipError_t launch_tile_128_f16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a,
                              int vec_b, hipStream_t stream);
hipError_t launch_tile_128_bf16(const GemmParams& p, int transpose_A, int transpose_B, int vec_a,
                               int vec_b, hipStream_t stream);

inline hipError_t launch_tile(int cfg, const GemmParams& p, int ab_dtype, int transpose_A,
                              int transpose_B, int vec_a, int vec_b, hipStream_t stream)
{
    const bool f16 = ab_dtype == DT_F16;
    if (cfg == TILE_256)
        return f16 ? launch_tile_256_f16(p, transpose_A, transpose_B, vec_a, vec_b, stream)
                   : launch_tile_256_bf16(p, transpose_A, transpose_B, vec_a, vec_b, stream);
    if (cfg == TILE_256_W8)
        return f16 ? launch_tile_256w8_f16(p, transpose_A, transpose_B, vec_a, vec_b, stream)
                   : launch_tile_256w8_bf16(p, transpose_A, transpose_B, vec_a, vec_b, stream);
    if (cfg == TILE_128)
        return f16 ? launch_tile_128_f16(p, transpose_A, transpose_B, vec_a, vec_b, stream)
                   : launch_tile_128_bf16(p, transpose_A, transpose_B, vec_a, vec_b, stream);
    return hipErrorInvalidValue;
}
hipError_t launch_skinny(const GemmParams& p, int ab_dtype, hipStream_t stream);

// Direct-load ring kernels (128-bit loads only): 256x256x64 tiles with a 2-slot
// ring, and 128x128x64 tiles with a 4-slot ring for grids too small to fill the
// chip with 256x256 tiles; 64x128x128 and 32x128x128 tiles with 3- and 4-slot rings
// for smaller grids still (8 waves each).
constexpr int kLdsBM = 256, kLdsBN = 256, kLdsBK = 64, kLdsStages = 2, kLdsThreads = 512;
constexpr int kLds128BM = 128, kLds128BN = 128, kLds128Stages = 4;
constexpr int kLds64BM = 64, kLds64BN = 128, kLds64BK = 128, kLds64Stages = 3;
constexpr int kLds32BM = 32, kLds32BN = 128, kLds32BK = 128, kLds32Stages = 4, kLds32Threads = 512;
hipError_t launch_lds_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds128_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds128_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds128sk_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds128sk_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
// Persistent stream-K schedules of the 256 x 256 and 128 x 128 kernels.
hipError_t launch_lds_sk2_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds_sk2_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds128_sk2_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds128_sk2_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
// 64 x 128 tiles; A must be K-contiguous (transpose_A == 0).
hipError_t launch_lds64_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds64_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
// 32 x 128 tiles; A must be K-contiguous (transpose_A == 0).
hipError_t launch_lds32_f16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);
hipError_t launch_lds32_bf16(const GemmParams& p, int transpose_A, int transpose_B, hipStream_t stream);

// Block-scaled FP8 GEMM (gemm_mx.hip).  A [M,K], B [N,K] FP8 bytes; SA [M,K/32],
// SB [N,K/32] E8M0 bytes; K % 128 == 0.
struct MxParams {
    const void* A;
    const void* SA;
    const void* B;
    const void* SB;
    void* C;
    int M, N, K;
    int relu, clear_accum, c_dtype, c_vec;
    int c_vec8;       // N % 8 == 0 and C aligned to 16 bytes
    int tiles_m, tiles_n;
};
hipError_t launch_mx(const MxParams& p, int fmt, hipStream_t stream);   // fmt: 0 = E4M3, 1 = E5M2, 4 = E2M1

// Attention forward (attn_fwd.hip).  Q, K, V, O are [B, S, H, dim] (dim 64 or 128),
// fp16 or bf16, 16-byte aligned; S >= 1; S * H * dim * 2 < 2^31.
struct AttnParams {
    const void* Q;
    const void* K;
    const void* V;
    void* O;
    int B, S, H;
    float scale_log2;   // softmax scale * log2(e)
    int block_q;        // queries per workgroup: 128 or 64
    int nqb;            // query blocks of block_q per (batch, head)
};
hipError_t launch_attn(const AttnParams& p, int dim, int dtype, int causal, hipStream_t stream);

// 4-bit dequant GEMM (gemm_w4.hip): C = act(A W^T), A [M, K] (16-byte aligned,
// K % 32 == 0), Wq [N, K/2] packed codes, S [N, K/G] operand dtype, Z [N, K/G]
// uint8; G % 32 == 0, K % G == 0, K / G <= kW4MaxGroups.
constexpr int kW4NB = 64;                      // columns of C per workgroup
constexpr int kW4Threads = 1024;               // 16 waves
constexpr int kW4TableBytes = 64 * 1024;       // LDS table: one dword per weight row and group
constexpr int kW4MaxGroups = 255;              // the documented limit (the table holds 256 groups)
struct W4Params {
    const void* A;
    const void* Wq;
    const void* S;
    const void* Z;
    void* C;
    int M, N, K, G;
    int relu, c_dtype, c_vec;
    uint32_t nibble_mask;   // 0x000F000F (a kernel argument so that it lives in an SGPR)
};
hipError_t launch_w4(const W4Params& p, int ab_dtype, hipStream_t stream);

// 2:4 structured-sparse GEMM (gemm_sp.hip): C = act(A W^T), A [M, K], Wv [N, K/2]
// compressed values, Wm [N, K/8] positions; K % 64 == 0.
struct SpParams {
    const void* A;
    const void* Wv;
    const void* Wm;
    void* C;
    int M, N, K;
    int relu, c_dtype, c_vec;
    int c_vec8;       // N % 8 == 0 and C aligned to 16 bytes
    int tiles_m, tiles_n;
};
hipError_t launch_sp(const SpParams& p, int ab_dtype, hipStream_t stream);

}  // namespace tlg
