// Tiled, software-pipelined GEMM  C = act(A·B)  on gfx950 MFMA.
//
// One workgroup owns one BM x BN output tile (the tile program's
// T.Kernel(ceildiv(N, bN), ceildiv(M, bM)) grid: "NVIDIA backend codegen"
// chapter, section 1; handbook page "TileLang: a tile language one level below
// Triton", section "first kernel: GEMM").  Its K loop runs over 64-wide K tiles
// as a two-stage software pipeline (T.Pipelined): while the waves multiply the
// tile held in one LDS buffer, the next tile's global loads are in flight in
// registers and are written to the other buffer afterwards (prologue, steady
// state and drain as in the overview page's "software pipelining" section).
//
// Data path per K tile:
//   global --(128-bit buffer loads, zero fill past the matrix edge)--> VGPRs
//     --(ds_write_b128, swizzled rows of 64 K-contiguous elements)--> LDS
//     --(ds_read_b128)--> MFMA 32x32x16 operands --> fp32 accumulators.
// Operands whose K index is not the contiguous one (A stored [K,M], B stored
// [K,N]) are loaded as 8x8 blocks and transposed in registers on the way into
// LDS, so every LDS tile is K-contiguous and every MFMA operand read is one
// 16-byte LDS read.
//
// The MFMA is issued with the B fragment as its first operand and the A
// fragment as its second, so the hardware tile is C's transpose: each lane then
// holds four consecutive columns of one row of C and stores them together.
//
// Epilogue: (+ C's prior value) -> ReLU -> round to the output dtype -> store,
// with stores outside C skipped ("core primitives" chapter, section 4.2).

#pragma once

#include "tlg_device.hpp"

namespace tlg {

// ---------------------------------------------------------------------------
// Tile loaders.  R rows (the tile's M or N extent) x 64 K of one operand.
// ---------------------------------------------------------------------------
template <bool K_CONTIG, int VEC, int R, int THREADS>
struct TileLoader;

// Operand stored [rows_total][K] (K contiguous): A with transpose_A = 0,
// B with transpose_B = 1.  Chunk q of the tile = (row q / 8, 16-byte chunk q % 8);
// eight consecutive lanes read one 128-byte row segment.
template <int VEC, int R, int THREADS>
struct TileLoader<true, VEC, R, THREADS> {
    static constexpr int kChunks = R * (kBK / 8);
    static constexpr int kPer = kChunks / THREADS;
    static_assert(kChunks % THREADS == 0, "tile chunks must divide evenly over the workgroup");

    const char* panel;       // element (r0, 0)
    uint64_t panel_bytes;    // bytes from panel to the end of the matrix
    uint32_t ld_bytes;       // K * 2
    int rows_valid;          // rows_total - r0
    int K;
    u32x4 v[kPer];

    __device__ void init(const void* base, int r0, int rows_total, int K_)
    {
        K = K_;
        ld_bytes = (uint32_t)K_ * 2u;
        panel = (const char*)base + (uint64_t)r0 * ld_bytes;
        panel_bytes = ((uint64_t)rows_total - (uint64_t)r0) * ld_bytes;
        rows_valid = rows_total - r0;
    }

    __device__ void load(int k0)
    {
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(panel + (uint64_t)k0 * 2u, panel_bytes - (uint64_t)k0 * 2u);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int q = i * THREADS + (int)threadIdx.x;
            const int row = q >> 3, c = q & 7;
            const bool row_ok = row < rows_valid;
            if constexpr (VEC == 8) {
                const bool ok = row_ok && (k0 + c * 8 < K);
                v[i] = buf_load16(rs, ok ? (uint32_t)row * ld_bytes + (uint32_t)c * 16u : kOOB);
            } else {
                uint32_t h[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool ok = row_ok && (k0 + c * 8 + e < K);
                    h[e] = buf_load2(rs, ok ? (uint32_t)row * ld_bytes + (uint32_t)(c * 8 + e) * 2u : kOOB);
                }
                v[i] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                             h[6] | (h[7] << 16)};
            }
        }
    }

    __device__ void store(uint16_t* lds) const
    {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int q = i * THREADS + (int)threadIdx.x;
            *(u32x4*)(lds + lds_elem(q >> 3, q & 7)) = v[i];
        }
    }
};

// Operand stored [K][rows_total] (its M or N index contiguous): A with
// transpose_A = 1, B with transpose_B = 0.  Each work-item loads blocks of KR
// K rows x 8 contiguous elements (lanes 0..31 of a wave cover 512 contiguous
// bytes of one K row), transposes each block in registers and writes eight
// K-contiguous pieces of KR elements (16 or 8 bytes).  KR is 8 when there are
// enough 8x8 blocks for every work-item, else 4.
template <int R, int THREADS>
struct MnBlock {
    static constexpr int kKR = ((R / 8) * (kBK / 8)) % THREADS == 0 ? 8 : 4;
};

template <int VEC, int R, int THREADS>
struct TileLoader<false, VEC, R, THREADS> {
    static constexpr int KR = MnBlock<R, THREADS>::kKR;
    static constexpr int kBlocksR = R / 8;
    static constexpr int kBlocks = kBlocksR * (kBK / KR);
    static constexpr int kPer = kBlocks / THREADS;
    static_assert(kBlocks % THREADS == 0 && kPer >= 1, "KR x 8 blocks must divide evenly over the workgroup");

    const char* base;        // element (0, r0)
    uint64_t base_bytes;     // bytes from base to the end of the matrix
    uint32_t ld_bytes;       // rows_total * 2
    int rows_valid;          // rows_total - r0
    int K;
    u32x4 v[kPer][KR];

    __device__ void init(const void* ptr, int r0, int rows_total, int K_)
    {
        K = K_;
        ld_bytes = (uint32_t)rows_total * 2u;
        base = (const char*)ptr + (uint64_t)r0 * 2u;
        base_bytes = (uint64_t)K_ * ld_bytes - (uint64_t)r0 * 2u;
        rows_valid = rows_total - r0;
    }

    __device__ void load(int k0)
    {
        const uint64_t off0 = (uint64_t)k0 * ld_bytes;
        const __amdgpu_buffer_rsrc_t rs = make_rsrc(base + off0, base_bytes - off0);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int q = i * THREADS + (int)threadIdx.x;
            const int rc = q % kBlocksR, kb = q / kBlocksR;
#pragma unroll
            for (int kr = 0; kr < KR; ++kr) {
                const int kl = kb * KR + kr;
                const bool k_ok = k0 + kl < K;
                if constexpr (VEC == 8) {
                    const bool ok = k_ok && (rc * 8 < rows_valid);
                    v[i][kr] = buf_load16(rs, ok ? (uint32_t)kl * ld_bytes + (uint32_t)rc * 16u : kOOB);
                } else {
                    uint32_t h[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const bool ok = k_ok && (rc * 8 + e < rows_valid);
                        h[e] = buf_load2(rs, ok ? (uint32_t)kl * ld_bytes + (uint32_t)(rc * 8 + e) * 2u : kOOB);
                    }
                    v[i][kr] = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                                     h[6] | (h[7] << 16)};
                }
            }
        }
    }

    __device__ void store(uint16_t* lds) const
    {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int q = i * THREADS + (int)threadIdx.x;
            const int rc = q % kBlocksR, kb = q / kBlocksR;
            const int chunk = (kb * KR) >> 3, sub = (kb * KR) & 7;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                // column j of the block: element j of each of the KR K rows
                uint32_t o[KR / 2];
#pragma unroll
                for (int e = 0; e < KR / 2; ++e) {
                    const uint32_t lo = v[i][2 * e][j >> 1], hi = v[i][2 * e + 1][j >> 1];
                    o[e] = (j & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
                }
                uint16_t* dst = lds + lds_elem(rc * 8 + j, chunk) + sub;
                if constexpr (KR == 8)
                    *(u32x4*)dst = u32x4{o[0], o[1], o[2], o[3]};
                else
                    *(u32x2*)dst = u32x2{o[0], o[1]};
            }
        }
    }
};

// ---------------------------------------------------------------------------
// Tile order.  Workgroups are dispatched round-robin over the 8 XCDs; when the
// tile count allows, consecutive tile ids are gathered onto one XCD, and tiles
// are walked in bands of kGroupM tile rows so that the workgroups sharing an
// XCD's L2 reuse few A row panels and B column panels.  Both steps are
// bijections on [0, tiles).
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;
constexpr int kGroupM = 4;

// Tile id -> (tile row, tile column), walking bands of kGroupM tile rows column by
// column.
__device__ inline void band_coords(int id, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int band = kGroupM * tiles_n;
    const int g = id / band;
    const int first = g * kGroupM;
    const int rows = min(tiles_m - first, kGroupM);
    const int r = id - g * band;
    tm = first + r % rows;
    tn = r / rows;
}

// Workgroup id -> tile: the XCD remap (consecutive tile ids onto one XCD), then the bands.
__device__ inline void tile_coords(int bid, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int total = tiles_m * tiles_n;
    int id = bid;
    if (total % kXcds == 0) id = (bid % kXcds) * (total / kXcds) + bid / kXcds;
    band_coords(id, tiles_m, tiles_n, tm, tn);
}

// ---------------------------------------------------------------------------
// The kernel.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, int T_IN, bool A_KC, bool B_KC, int VEC_A, int VEC_B>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_tile_kernel(GemmParams p)
{
    constexpr int THREADS = 64 * WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;   // wave tile
    constexpr int FM = WTM / 32, FN = WTN / 32;              // 32x32 MFMA tiles per wave
    constexpr int A_ELEMS = BM * kRowElems, B_ELEMS = BN * kRowElems;
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be a multiple of 32x32");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2][A_ELEMS + B_ELEMS];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int KT = (p.K + kBK - 1) / kBK;

    TileLoader<A_KC, VEC_A, BM, THREADS> la;
    TileLoader<B_KC, VEC_B, BN, THREADS> lb;
    la.init(p.A, m0, p.M, p.K);
    lb.init(p.B, n0, p.N, p.K);

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Fragment rows of this lane and the chunk half (K 0..7 or 8..15 of a 16-K step).
    const int a_row = wm * WTM + (lane & 31);
    const int b_row = wn * WTN + (lane & 31);
    const int khalf = lane >> 5;

    // One 16-wide K step: FM A fragments and FN B fragments (one 16-byte LDS read each).
    auto load_frags = [&](const uint16_t* st, int kk, u32x4 (&af)[FM], u32x4 (&bf)[FN]) {
        const int c = kk * 2 + khalf;
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = *(const u32x4*)(st + lds_elem(a_row + i * 32, c));
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = *(const u32x4*)(st + A_ELEMS + lds_elem(b_row + j * 32, c));
    };
    auto mma = [&](const u32x4 (&af)[FM], const u32x4 (&bf)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16<T_IN>(bf[j], af[i], acc[i][j]);
    };

    // Software pipeline over K tiles (two LDS buffers).  The fragments of the
    // next 16-wide K step are read while the current step's MFMAs run; the next
    // K tile's global loads are issued at the top of an iteration and land in
    // the other LDS buffer before its closing barrier.
    u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    if (KT > 0) {
        la.load(0);
        lb.load(0);
        la.store(smem[0]);
        lb.store(smem[0] + A_ELEMS);
    }
    __syncthreads();
    if (KT > 0) load_frags(smem[0], 0, fa0, fb0);

    // sched_barrier(0) fences keep the compiler from sinking the global loads
    // next to their use (which would serialise the pipeline) and keep each
    // phase's fragment reads ahead of the MFMAs that overlap them.
    for (int kt = 0; kt < KT - 1; ++kt) {
        const uint16_t* cur = smem[kt & 1];
        uint16_t* nxt = smem[(kt & 1) ^ 1];
        la.load((kt + 1) * kBK);
        lb.load((kt + 1) * kBK);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, 1, fa1, fb1);
        mma(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, 2, fa0, fb0);
        mma(fa1, fb1);
        __builtin_amdgcn_sched_barrier(0);
        load_frags(cur, 3, fa1, fb1);
        mma(fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
        la.store(nxt);
        lb.store(nxt + A_ELEMS);
        mma(fa1, fb1);
        __syncthreads();
        load_frags(nxt, 0, fa0, fb0);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (KT > 0) {
        const uint16_t* cur = smem[(KT - 1) & 1];
        load_frags(cur, 1, fa1, fb1);
        mma(fa0, fb0);
        load_frags(cur, 2, fa0, fb0);
        mma(fa1, fb1);
        load_frags(cur, 3, fa1, fb1);
        mma(fa0, fb0);
        mma(fa1, fb1);
    }

    // Epilogue.  acc[i][j][4g + e] is C[m][n + e] with
    //   m = m0 + wm*WTM + i*32 + lane%32,  n = n0 + wn*WTN + j*32 + 8g + 4*(lane/32).
    const bool vec_cols = p.c_vec != 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + i * 32 + (lane & 31);
        if (m >= p.M) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn * WTN + j * 32 + 8 * g + 4 * (lane >> 5);
                if (n >= p.N) continue;
                const int count = min(4, p.N - n);
                const bool vec_ok = vec_cols && count == 4;
                const int64_t idx = (int64_t)m * p.N + n;
                float v[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
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
    }
}

// ---------------------------------------------------------------------------
// Launch helpers: runtime flags -> template instance.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int T, bool AKC, bool BKC, int VA, int VB>
inline hipError_t launch_inst(const GemmParams& p, hipStream_t stream)
{
    GemmParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const dim3 block(64 * WM * WN);
    return hipLaunchKernel((const void*)&gemm_tile_kernel<BM, BN, WM, WN, T, AKC, BKC, VA, VB>, grid,
                           block, kargs, 0, stream);
}

template <int BM, int BN, int WM, int WN, int T, bool AKC, bool BKC, bool NARROW>
inline hipError_t dispatch_vec(const GemmParams& p, int va, int vb, hipStream_t s)
{
    if constexpr (NARROW) {
        if (va == 8 && vb == 8) return launch_inst<BM, BN, WM, WN, T, AKC, BKC, 8, 8>(p, s);
        if (va == 8) return launch_inst<BM, BN, WM, WN, T, AKC, BKC, 8, 1>(p, s);
        if (vb == 8) return launch_inst<BM, BN, WM, WN, T, AKC, BKC, 1, 8>(p, s);
        return launch_inst<BM, BN, WM, WN, T, AKC, BKC, 1, 1>(p, s);
    } else {
        if (va != 8 || vb != 8) return hipErrorInvalidValue;
        return launch_inst<BM, BN, WM, WN, T, AKC, BKC, 8, 8>(p, s);
    }
}

template <int BM, int BN, int WM, int WN, int T, bool NARROW>
inline hipError_t dispatch_layout(const GemmParams& p, int tA, int tB, int va, int vb, hipStream_t s)
{
    // K-contiguous A <=> transpose_A == 0; K-contiguous B <=> transpose_B == 1.
    if (!tA && tB) return dispatch_vec<BM, BN, WM, WN, T, true, true, NARROW>(p, va, vb, s);
    if (!tA && !tB) return dispatch_vec<BM, BN, WM, WN, T, true, false, NARROW>(p, va, vb, s);
    if (tA && tB) return dispatch_vec<BM, BN, WM, WN, T, false, true, NARROW>(p, va, vb, s);
    return dispatch_vec<BM, BN, WM, WN, T, false, false, NARROW>(p, va, vb, s);
}

}  // namespace tlg
