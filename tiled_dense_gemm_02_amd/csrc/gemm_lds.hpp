// Tiled GEMM with a multi-stage LDS ring fed by global->LDS direct loads.
//
// The same tile program as gemm_tile.hpp (one 256 x 256 output tile per
// workgroup, K loop over BK-wide tiles, MFMA 32x32x16 into fp32 fragments,
// fused epilogue), with the software pipeline of the tile program's
// T.Pipelined(num_stages = S) realised as an S-stage ring: tile k+S-1 is
// requested while tile k is multiplied ("software pipelining" section of the
// overview page; the handbook page's quickstart uses a 3-stage ring).
//
// Global->LDS copies use buffer_load_dwordx4 ... lds: each lane's 16 bytes go
// straight to LDS at (ring slot block + 16 * lane), with no VGPR staging, no LDS
// write instructions and no VALU work.  Lanes whose chunk lies outside the
// matrix take an out-of-range offset and the hardware writes zeros (the zero
// safe value of out-of-bounds reads, "core primitives" chapter, section 4.2).
// The swizzled LDS layout is produced by choosing which global chunk each lane
// fetches.
//
// Operand layouts in LDS (one ring slot; "rows" are the operand's M or N index):
//   K-contiguous operand (A stored [M,K], B stored [N,K]): 256 rows of BK
//     elements (RB = 2*BK bytes); 16-byte chunk c of row r sits at position
//     c ^ ((r / (16/CH)) % CH), CH = BK/8.  Sixteen lanes reading sixteen
//     consecutive rows of one chunk then touch 64 distinct banks.  MFMA
//     operands are single ds_read_b128s.
//   M/N-contiguous operand (A stored [K,M], B stored [K,N]): BK rows of k, each
//     256 contiguous M/N elements (512 bytes); chunk c of row k sits at
//     c ^ ((k & 3) << 2).  MFMA operands are read with ds_read_b64_tr_b16, which
//     transposes 4 x 16-bit values across each group of 16 lanes: lane i of a
//     group receives element (i & 3) of the 8-byte pieces addressed by lanes
//     (i >> 2) + 4j, j = 0..3.  Addressing row kb + (s >> 2), columns
//     nb + 4 (s & 3) from lane s therefore delivers column nb + i, rows
//     kb..kb+3 to lane i: a K-contiguous MFMA operand.
#pragma once

#include "gemm_tile.hpp"

namespace tlg {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4_t;
typedef int i32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) with the other counters left unconstrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt bits 6:4, lgkmcnt 11:8).
template <int N>
__device__ inline void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Buffer resource as four scalar words (for the inline-asm direct load below).
__device__ inline i32x4 rsrc_words(const void* base, uint64_t bytes_left)
{
    const uint64_t a = (uint64_t)base;
    const uint32_t n = bytes_left > kMaxRecords ? kMaxRecords : (uint32_t)bytes_left;
    i32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
    r[2] = __builtin_amdgcn_readfirstlane((int)n);
    r[3] = kRsrcWord3;
    return r;
}

// 16-byte global->LDS direct load: lane l writes LDS bytes [lds + 16 l, lds + 16 l + 16).
// Issued as inline assembly so that the compiler does not treat the slot being
// filled as aliasing the slot being read (it would otherwise wait for every
// outstanding direct load before each LDS read and serialise the ring).  The
// kernel tracks completion itself with explicit vmcnt waits and issues no other
// vector-memory instruction while direct loads are in flight.
// m0 is a reserved register: the clobber tells the compiler that its value does
// not survive the statement (the compiler re-initialises m0 wherever it needs it).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline uint32_t lds_addr_of(const void* p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ inline u32x2 lds_read_tr16(const char* p)
{
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
    return __builtin_bit_cast(u32x2, v);
}

template <int BK>
__device__ __host__ constexpr int swz_kc(int row)
{
    constexpr int CH = BK / 8;
    return (row / (16 / CH)) % CH;
}

// One operand of the 256 x 256 tile: 256 rows of its M/N index x BK of K.
template <int BK, bool KC>
struct LdsOperand {
    static constexpr int R = 256;
    static constexpr int BYTES = R * BK * 2;
    static constexpr int L = BYTES / (512 * 16);  // direct loads per lane per tile
    static constexpr int RB = BK * 2, CH = BK / 8;

    const char* base;       // element (row r0, k 0)       [K-contig]  /  (k 0, row r0)  [M/N-contig]
    uint64_t base_bytes;    // bytes from base to the end of the matrix
    uint32_t ld;            // row pitch in bytes
    uint32_t off[L];
    int kpos[L];            // K offset of the lane's chunk within a tile
    bool ok[L];

    __device__ void init(const void* ptr, int r0, int rows_total, int K, int lane, int wave)
    {
        if constexpr (KC) {
            ld = (uint32_t)K * 2u;
            base = (const char*)ptr + (uint64_t)r0 * ld;
            base_bytes = (uint64_t)(rows_total - r0) * ld;
        } else {
            ld = (uint32_t)rows_total * 2u;
            base = (const char*)ptr + (uint64_t)r0 * 2u;
            base_bytes = (uint64_t)K * ld - (uint64_t)r0 * 2u;
        }
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const int b = i * 8 + wave;  // 1 KiB block of the slot filled by this load
            if constexpr (KC) {
                const int row = b * (1024 / RB) + lane / CH;
                const int c = (lane % CH) ^ swz_kc<BK>(row);
                ok[i] = r0 + row < rows_total;
                off[i] = (uint32_t)row * ld + (uint32_t)c * 16u;
                kpos[i] = c * 8;
            } else {
                const int k = 2 * b + (lane >> 5);
                const int c = (lane & 31) ^ ((k & 3) << 2);
                ok[i] = r0 + c * 8 < rows_total;
                off[i] = (uint32_t)k * ld + (uint32_t)c * 16u;
                kpos[i] = k;
            }
        }
    }

    // Request the tile starting at k0 into the slot's operand region (wave's block included).
    __device__ void issue(int k0, int K, uint32_t lds_region) const
    {
        const uint64_t o = KC ? (uint64_t)k0 * 2u : (uint64_t)k0 * ld;
        const i32x4 r = rsrc_words(base + o, base_bytes - o);
#pragma unroll
        for (int i = 0; i < L; ++i) {
            const bool valid = ok[i] && (k0 + kpos[i] < K);
            dma16(r, valid ? off[i] : kOOB, lds_region + (uint32_t)(i * 8 * 1024));
        }
    }

    // MFMA operand of rows row0..row0+31 (row0 a multiple of 32), K step kk (16 wide):
    // lane l holds row row0 + l%32 and K elements 8*(l/32) .. +7 of the step.
    __device__ u32x4 frag(const char* region, int row0, int kk, int lane) const
    {
        if constexpr (KC) {
            const int row = row0 + (lane & 31);
            const int c = kk * 2 + (lane >> 5);
            return *(const u32x4*)(region + row * RB + ((c ^ swz_kc<BK>(row)) << 4));
        } else {
            const int g = lane >> 4, s = lane & 15;
            const int n = row0 + (g & 1) * 16 + 4 * (s & 3);
            const int k = kk * 16 + (g >> 1) * 8 + (s >> 2);
            const char* p = region + (((n >> 3) ^ ((k & 3) << 2)) << 4) + ((n >> 2) & 1) * 8;
            const u32x2 lo = lds_read_tr16(p + k * 512);
            const u32x2 hi = lds_read_tr16(p + (k + 4) * 512);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }
};

template <int BK, int S, int T_IN, bool A_KC, bool B_KC>
__global__ void __launch_bounds__(512)
gemm_lds_kernel(GemmParams p)
{
    constexpr int BM = 256, BN = 256, WAVES_N = 4;
    constexpr int WTM = 128, WTN = 64, FM = WTM / 32, FN = WTN / 32;
    using OpA = LdsOperand<BK, A_KC>;
    using OpB = LdsOperand<BK, B_KC>;
    constexpr int STAGE = OpA::BYTES + OpB::BYTES;
    constexpr int L = OpA::L + OpB::L;
    constexpr int KSTEPS = BK / 16;
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS ring must fit in 160 KiB");
    static_assert((S - 2) * L < 64, "vmcnt range");
    static_assert(KSTEPS % 2 == 0, "fragment double buffering steps by two");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int KT = (K + BK - 1) / BK;

    OpA opa;
    OpB opb;
    opa.init(p.A, m0, p.M, K, lane, wave);
    opb.init(p.B, n0, p.N, K, lane, wave);
    const uint32_t lds0 = lds_addr_of(smem);

    auto issue = [&](int t) {
        const uint32_t slot =
            __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t % S) * STAGE) + (uint32_t)wave * 1024u);
        opa.issue(t * BK, K, slot);
        opb.issue(t * BK, K, slot + (uint32_t)OpA::BYTES);
    };
    auto load_frags = [&](const char* slot, int kk, u32x4 (&af)[FM], u32x4 (&bf)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = opa.frag(slot, wm * WTM + i * 32, kk, lane);
#pragma unroll
        for (int j = 0; j < FN; ++j) bf[j] = opb.frag(slot + OpA::BYTES, wn * WTN + j * 32, kk, lane);
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // MFMA with the B fragment first: the hardware tile is C's transpose, so
    // acc[i][j][4g + e] is C[m][n + e] (see the epilogue).
    auto mma = [&](const u32x4 (&af)[FM], const u32x4 (&bf)[FN]) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) acc[i][j] = mfma32x32x16<T_IN>(bf[j], af[i], acc[i][j]);
    };

#pragma unroll
    for (int t = 0; t < S - 1; ++t)
        if (t < KT) issue(t);

    u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    for (int kt = 0; kt < KT; ++kt) {
        // Tile kt has landed once at most min(S-2, KT-1-kt) newer tiles are
        // still in flight; the barrier then publishes every wave's part of it
        // and retires all reads of the slot that the next request overwrites.
        if (kt + S - 2 < KT)
            wait_vmcnt<(S - 2) * L>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (kt + S - 1 < KT) issue(kt + S - 1);
        const char* slot = smem + (kt % S) * STAGE;
        // Waves raise their priority while issuing MFMAs so that a wave in its
        // MFMA run is not starved by the other wave's address/LDS instructions.
        __builtin_amdgcn_s_setprio(1);
        load_frags(slot, 0, fa0, fb0);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; kk += 2) {
            load_frags(slot, kk + 1, fa1, fb1);
            mma(fa0, fb0);
            if (kk + 2 < KSTEPS) load_frags(slot, kk + 2, fa0, fb0);
            mma(fa1, fb1);
        }
        __builtin_amdgcn_s_setprio(0);
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

template <int BK, int S, int T, bool AKC, bool BKC>
inline hipError_t launch_lds_inst(const GemmParams& p, hipStream_t stream)
{
    GemmParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const dim3 block(512);
    return hipLaunchKernel((const void*)&gemm_lds_kernel<BK, S, T, AKC, BKC>, grid, block, kargs, 0, stream);
}

// K-contiguous A <=> transpose_A == 0; K-contiguous B <=> transpose_B == 1.
template <int BK, int S, int T>
inline hipError_t dispatch_lds(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    if (!tA && tB) return launch_lds_inst<BK, S, T, true, true>(p, s);
    if (!tA && !tB) return launch_lds_inst<BK, S, T, true, false>(p, s);
    if (tA && tB) return launch_lds_inst<BK, S, T, false, true>(p, s);
    return launch_lds_inst<BK, S, T, false, false>(p, s);
}

}  // namespace tlg
