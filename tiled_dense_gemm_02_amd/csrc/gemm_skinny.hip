// Skinny GEMM  C[M x N] = act(A·B)  for MR = 16, 32 or 64 rows of A per
// workgroup, B stored [N, K] (transpose_B = 1), A stored [M, K].  This shape is
// bound by the HBM stream of B (one read of each element), not by MFMA: the
// roofline bound P <= min(P_peak, I * B_mem) of the overview page's "performance
// model" section puts its arithmetic intensity near 16 FLOP/byte per row of A.
//
// Each workgroup owns MR rows x NB columns of C (16 x 64, 32 x 64 or 64 x 32),
// i.e. NB consecutive rows of B, and streams them exactly once through an
// S-stage LDS ring.  One stage holds KST elements of K of every B row of the
// workgroup and of the MR A rows.  Stages are filled with global->LDS direct
// loads in which each instruction reads 1 KiB of B (or A) rows contiguously, so
// HBM sees long row segments rather than 64-byte pieces of many rows.  The eight
// waves take different 32-wide K steps of a stage and multiply with MFMA
// 16x16x32 (each B fragment against the MR / 16 A fragments); their partial
// MR x NB tiles are summed in LDS in a fixed order (deterministic), then the
// epilogue applies (+ prior C) -> ReLU -> rounding -> guarded stores.
//
// Row layout in a stage: 16-byte chunk c of row r sits at c ^ (r & 15), so the
// sixteen lanes that read sixteen consecutive rows of one chunk for an MFMA
// operand hit 64 distinct banks.  Out-of-range rows, columns and K chunks read
// as zero through the buffer resource's range check ("core primitives"
// chapter, section 4.2).
//
// Measured on MI355X for 16 x 16384 x 8192 fp16: ~6.1 TB/s with the K stage
// order rotated per workgroup (below), ~5.0 TB/s without; the previous design
// that loaded MFMA operands straight from HBM into registers (16 rows x 64
// bytes per load instruction) reached ~4.8 TB/s with 8 waves.

#include "gemm_lds.hpp"

namespace tlg {

template <int T_IN, int NB, int KST, int S, int MR>
__global__ void __launch_bounds__(kSkinnyThreads)
gemm_skinny_kernel(GemmParams p)
{
    constexpr int WAVES = kSkinnyThreads / 64;
    constexpr int MT = MR / 16;                      // 16-row MFMA tiles of A
    constexpr int RB = KST * 2;                      // bytes per row segment of a stage
    constexpr int ROWS = NB + MR;                    // B rows, then A rows
    constexpr int STAGE = ROWS * RB;
    constexpr int NS = NB / 16;                      // 16-column MFMA tiles
    constexpr int KSTEPS = KST / 32;                 // 32-wide MFMA K steps per stage
    constexpr int SPW = KSTEPS / WAVES;              // K steps per wave per stage
    constexpr int CHUNKS = RB / 16;                  // 16-byte chunks per row segment
    constexpr int LPI = 1024 / RB;                   // rows per 1 KiB direct load
    constexpr int LOADS = ROWS / LPI;                // direct loads per stage
    constexpr int LPW = LOADS / WAVES;               // per wave
    static_assert(NB % 16 == 0 && NB % LPI == 0, "NB");
    static_assert(KSTEPS % WAVES == 0 && SPW >= 1, "every wave needs whole K steps of a stage");
    static_assert(LOADS % WAVES == 0, "direct loads must divide evenly over the waves");
    static_assert(CHUNKS >= 16 && 1024 % RB == 0, "row segment of 256 B .. 1 KiB");
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS ring must fit in 160 KiB");
    static_assert((S - 2) * LPW < 64, "vmcnt range");
    static_assert(MR % 16 == 0 && MR % LPI == 0, "MR");
    static_assert(WAVES * MT * NS * 4 * 64 * 4 <= S * STAGE, "reduction area reuses the ring");
    static_assert(MT * NS <= WAVES, "one wave per 16 x 16 output block in the epilogue");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m0 = blockIdx.y * MR, n0 = blockIdx.x * NB;
    const int K = p.K;
    // K stages of the whole K, and this workgroup's range of them: with p.splits > 1
    // (grids of few column blocks) workgroup z of the splits takes stages
    // [z * per, z * per + NST), and the partial tiles are summed below.
    const int NST_ALL = (K + KST - 1) / KST;
    const int splits = p.splits > 1 ? p.splits : 1;
    const int per = (NST_ALL + splits - 1) / splits;
    const int st0 = (int)blockIdx.z * per;
    const int NST = max(0, min(per, NST_ALL - st0));
    const uint32_t ld = (uint32_t)K * 2u;
    const uint32_t lds0 = lds_addr_of(smem);
    const char* b_base = (const char*)p.B + (uint64_t)n0 * ld;
    const char* a_base = (const char*)p.A + (uint64_t)m0 * ld;
    const uint64_t b_bytes = (uint64_t)(p.N - n0) * ld;
    const uint64_t a_bytes = (uint64_t)(p.M - m0) * ld;

    // The workgroups that one XCD holds at a time (dispatch sends workgroup b to XCD
    // b % 8) start at different K stages and wrap around: in step j a workgroup
    // streams stage (j + rot) mod NST.  When every workgroup reads the same K range
    // of its rows at once, a row pitch of a power of two (K = 4096, 8192, 16384)
    // puts those reads on few HBM channels (measured on MI355X, 16 x 16384 x 8192:
    // 5.0 TB/s in step, 6.1 TB/s rotated, as fast as with K = 8320).  Each output
    // still sums every stage once, in an order fixed by its workgroup.
    const unsigned lid = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
    const int rot = NST > 0 ? (int)((lid / 8u) % (unsigned)NST) : 0;
    auto stage_of = [&](int j) { const int x = j + rot; return st0 + (x >= NST ? x - NST : x); };

    // Load i of this wave fills LDS rows q*LPI .. q*LPI + LPI - 1 of the stage
    // (q = i * WAVES + wave); lane -> row q*LPI + lane / CHUNKS, position lane % CHUNKS.
    // Step j of the loop fills ring slot j % S with K stage stage_of(j).
    auto issue = [&](int j) {
        const int k0 = stage_of(j) * KST;
        const uint64_t o = (uint64_t)k0 * 2u;
        const uint32_t slot = lds0 + (uint32_t)((j % S) * STAGE);
        const i32x4 rb = rsrc_words(b_base + o, b_bytes > o ? b_bytes - o : 0);
        const i32x4 ra = rsrc_words(a_base + o, a_bytes > o ? a_bytes - o : 0);
#pragma unroll
        for (int i = 0; i < LPW; ++i) {
            const int q = i * WAVES + wave;
            const int row = q * LPI + lane / CHUNKS;
            const int c = (lane % CHUNKS) ^ (row & 15);
            const bool is_b = q * LPI < NB;          // a load is all B rows or all A rows
            const int r = is_b ? row : row - NB;
            const bool ok = (is_b ? (n0 + r < p.N) : (m0 + r < p.M)) && (k0 + c * 8 < K);
            i32x4 rs;
#pragma unroll
            for (int w = 0; w < 4; ++w) rs[w] = __builtin_amdgcn_readfirstlane(is_b ? rb[w] : ra[w]);
            dma16(rs, ok ? (uint32_t)r * ld + (uint32_t)c * 16u : kOOB,
                  __builtin_amdgcn_readfirstlane(slot + (uint32_t)(q * 1024)));
        }
    };
    auto frag = [&](const char* slot, int row, int c) -> u32x4 {
        return *(const u32x4*)(slot + row * RB + ((c ^ (row & 15)) << 4));
    };

    f32x4 acc[MT][NS];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NS; ++j) acc[mt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
    for (int st = 0; st < S - 1; ++st)
        if (st < NST) issue(st);
    for (int st = 0; st < NST; ++st) {
        // Stage st has landed once at most S-2 newer stages are in flight; the
        // barrier publishes every wave's part and frees the slot refilled next.
        if (st + S - 2 < NST)
            wait_vmcnt<(S - 2) * LPW>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (st + S - 1 < NST) issue(st + S - 1);
        const char* slot = smem + (st % S) * STAGE;
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            const int c = (wave * SPW + u) * 4 + (lane >> 4);
            u32x4 af[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) af[mt] = frag(slot, NB + mt * 16 + (lane & 15), c);
            // B fragment first: the hardware tile is C's transpose, so acc[mt][j][e]
            // is C[m0 + 16mt + lane%16][n0 + 16j + 4*(lane/16) + e].
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const u32x4 bf = frag(slot, j * 16 + (lane & 15), c);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) acc[mt][j] = mfma16x16x32<T_IN>(bf, af[mt], acc[mt][j]);
            }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    // The waves' partial sums meet in LDS; wave w then owns output block
    // (w / NS, w % NS) of the MT x NS blocks of 16 x 16 and sums it in wave order.
    constexpr int NBLK = MT * NS;
    float* red = (float*)smem;   // [WAVES][NBLK][4][64]
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < NS; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((wave * NBLK + mt * NS + j) * 4 + e) * 64 + lane] = acc[mt][j][e];
    __syncthreads();

    const bool owner = wave < NBLK;
    const int mt_o = wave / NS, j_o = wave % NS;
    const int m = m0 + mt_o * 16 + (lane & 15);
    const bool vec_cols = p.c_vec != 0;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    if (owner) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s = red[(wave * 4 + e) * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) s += red[((w * NBLK + wave) * 4 + e) * 64 + lane];
            v[e] = s;
        }
    }
    if (splits > 1) {
        // Publish this K range's MR x NB partial tile (fp32), take a ticket; the last
        // workgroup of the tile sums the partials in K-range order, then runs the
        // epilogue.  The XCDs' L2 caches are separate, so partials are written and
        // read with device-scope (sc1) buffer accesses; each wave waits for its
        // stores before the barrier that precedes the ticket.
        __shared__ unsigned ticket;
        const int tile = (int)(blockIdx.y * gridDim.x + blockIdx.x);
        constexpr int PART = NBLK * 64 * 4;               // floats per partial tile
        const __amdgpu_buffer_rsrc_t wsr = make_rsrc(p.ws + (size_t)tile * splits * PART,
                                                     (uint64_t)splits * PART * 4u);
        if (owner)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v[0], v[1], v[2], v[3]}), wsr,
                                                   (uint32_t)((blockIdx.z * PART + (wave * 64 + lane) * 4) * 4), 0,
                                                   kCoherentDevice);
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0)
            ticket = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(ticket) != (unsigned)(splits - 1)) return;
        if (owner) {
            constexpr int MAXS = kSkinnyMaxSplits;
            u32x4 part[MAXS];
#pragma unroll
            for (int z = 0; z < MAXS; ++z)
                part[z] = __builtin_amdgcn_raw_buffer_load_b128(
                    wsr, z < splits ? (uint32_t)((z * PART + (wave * 64 + lane) * 4) * 4) : kOOB, 0, kCoherentDevice);
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int z = 0; z < MAXS; ++z) t += __builtin_bit_cast(f32x4, part[z]);   // zeros past the last range
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = t[e];
        }
        if (threadIdx.x == 0)   // ready for the next launch
            __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    const int n = n0 + j_o * 16 + 4 * (lane >> 4);
    if (owner && m < p.M && n < p.N) {
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

template <int T, int MR, int NB>
static hipError_t launch_skinny_t(const GemmParams& p, hipStream_t stream)
{
    GemmParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)p.tiles_n, (unsigned)p.tiles_m, (unsigned)(p.splits > 1 ? p.splits : 1));
    const dim3 block(kSkinnyThreads);
    return hipLaunchKernel((const void*)&gemm_skinny_kernel<T, NB, kSkinnyKST, kSkinnyStages, MR>, grid, block,
                           kargs, 0, stream);
}

// Rows of A per block (skinny_rows) and columns per block (skinny_cols) follow M,
// as the plan computed them.
hipError_t launch_skinny(const GemmParams& p, int ab_dtype, hipStream_t stream)
{
    const int mr = skinny_rows(p.M);
    if (ab_dtype == DT_F16) {
        if (mr == 16) return launch_skinny_t<DT_F16, 16, skinny_cols(16)>(p, stream);
        if (mr == 32) return launch_skinny_t<DT_F16, 32, skinny_cols(32)>(p, stream);
        return launch_skinny_t<DT_F16, 64, skinny_cols(64)>(p, stream);
    }
    if (mr == 16) return launch_skinny_t<DT_BF16, 16, skinny_cols(16)>(p, stream);
    if (mr == 32) return launch_skinny_t<DT_BF16, 32, skinny_cols(32)>(p, stream);
    return launch_skinny_t<DT_BF16, 64, skinny_cols(64)>(p, stream);
}

}  // namespace tlg
