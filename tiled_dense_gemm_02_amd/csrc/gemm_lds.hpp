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

// Scheduling groups for one K step: MPS MFMAs, each followed by its share of the
// RPS LDS reads of the next step (sched_group_barrier masks: 0x008 MFMA, 0x100 DS read).
template <int RPS, int MPS, int R>
__device__ inline void sched_mfma_with_reads()
{
    if constexpr (R < MPS) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        constexpr int nr = RPS * (R + 1) / MPS - RPS * R / MPS;
        if constexpr (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);
        sched_mfma_with_reads<RPS, MPS, R + 1>();
    }
}

template <int BK>
__device__ __host__ constexpr int swz_kc(int row)
{
    constexpr int CH = BK / 8;
    return (row / (16 / CH)) % CH;
}

// One operand of the 256 x 256 tile: 256 rows of its M/N index x BK of K,
// filled by NW waves (each direct load fills one 1 KiB block).
template <int BK, bool KC, int NW>
struct LdsOperand {
    static constexpr int R = 256;
    static constexpr int BYTES = R * BK * 2;
    static constexpr int L = BYTES / (NW * 64 * 16);  // direct loads per lane per tile
    static_assert(BYTES % (NW * 1024) == 0, "blocks must divide evenly over the waves");
    static constexpr int RB = BK * 2, CH = BK / 8;

    // Load i of a lane covers block b = i * NW + wave.  Along i the lane's row
    // (K-contiguous) or k (M/N-contiguous) advances by a constant step, and the
    // swizzle term is unchanged by that step, so one base offset per lane
    // describes all L loads.
    static constexpr int DROW = NW * (1024 / RB);   // K-contiguous: rows per load step
    static constexpr int DK = 2 * NW;               // M/N-contiguous: k rows per load step
    static_assert(!KC || (4 * NW) % CH == 0, "swizzle must be invariant along the load step");
    static_assert(KC || NW % 2 == 0, "swizzle must be invariant along the load step");

    const char* base;       // element (row r0, k 0)       [K-contig]  /  (k 0, row r0)  [M/N-contig]
    uint64_t base_bytes;    // bytes from base to the end of the matrix
    uint32_t ld;            // row pitch in bytes
    uint32_t off0;          // byte offset of load 0 relative to base
    int idx0;               // K-contig: row of load 0 (relative to r0); M/N-contig: k of load 0
    int kc;                 // K-contig: first K element of the lane's chunk
    int rows_left;          // rows_total - r0
    bool col_ok;            // M/N-contig: the lane's 8 columns lie inside the matrix

    __device__ void init(const void* ptr, int r0, int rows_total, int K, int lane, int wave)
    {
        rows_left = rows_total - r0;
        if constexpr (KC) {
            ld = (uint32_t)K * 2u;
            base = (const char*)ptr + (uint64_t)r0 * ld;
            base_bytes = (uint64_t)(rows_total - r0) * ld;
            idx0 = wave * (1024 / RB) + lane / CH;
            const int c = (lane % CH) ^ swz_kc<BK>(idx0);
            off0 = (uint32_t)idx0 * ld + (uint32_t)c * 16u;
            kc = c * 8;
            col_ok = true;
        } else {
            ld = (uint32_t)rows_total * 2u;
            base = (const char*)ptr + (uint64_t)r0 * 2u;
            base_bytes = (uint64_t)K * ld - (uint64_t)r0 * 2u;
            idx0 = 2 * wave + (lane >> 5);
            const int c = (lane & 31) ^ ((idx0 & 3) << 2);
            off0 = (uint32_t)idx0 * ld + (uint32_t)c * 16u;
            kc = 0;
            col_ok = c * 8 < rows_left;
        }
    }

    // Request the tile starting at k0 into the slot's operand region (wave's block included).
    __device__ void issue(int k0, int K, uint32_t lds_region) const
    {
        const uint64_t o = KC ? (uint64_t)k0 * 2u : (uint64_t)k0 * ld;
        // Slots past the end of K (padding of the last iteration) get an empty
        // resource; all their lanes are out of range and receive zeros.
        const i32x4 r = rsrc_words(base + o, o < base_bytes ? base_bytes - o : 0);
#pragma unroll
        for (int i = 0; i < L; ++i) {
            bool valid;
            uint32_t off;
            if constexpr (KC) {
                valid = (idx0 + i * DROW < rows_left) && (k0 + kc < K);
                off = off0 + (uint32_t)(i * DROW) * ld;
            } else {
                valid = col_ok && (k0 + idx0 + i * DK < K);
                off = off0 + (uint32_t)(i * DK) * ld;
            }
            dma16(r, valid ? off : kOOB, lds_region + (uint32_t)(i * NW * 1024));
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

// BKS: K width of one ring slot; SPI: slots consumed per barrier; S: ring slots.
// Slot t holds K tile t (t % S).  Iteration j multiplies tiles j*SPI .. j*SPI+SPI-1
// and requests tiles up to j*SPI + S - 1, so every request has S - SPI slots of
// time to land while the barrier count stays at one per SPI*BKS of K.
// PF (needs S >= 2*SPI + 1): an iteration's barrier also publishes the first
// tile of the next iteration, whose first fragments are then read before the
// next barrier, so no wave starts an iteration waiting on LDS.
template <int BKS, int SPI, int S, bool PF, int WAVES_M, int WAVES_N, int T_IN, bool A_KC, bool B_KC>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_lds_kernel(GemmParams p)
{
    constexpr int BM = 256, BN = 256, NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 32, FN = WTN / 32;
    using OpA = LdsOperand<BKS, A_KC, NW>;
    using OpB = LdsOperand<BKS, B_KC, NW>;
    constexpr int STAGE = OpA::BYTES + OpB::BYTES;
    constexpr int L = OpA::L + OpB::L;              // direct loads per lane per slot
    constexpr int KS = BKS / 16;                     // 16-wide K steps per slot
    constexpr int STEPS = SPI * KS;                  // K steps per iteration
    // Slots allowed in flight when an iteration starts (the ones it does not read).
    constexpr int AHEAD = PF ? S - 2 * SPI - 1 : S - 2 * SPI;
    static_assert(BKS == 32 || BKS == 64, "slot width");
    static_assert(SPI >= 1 && S * STAGE <= 160 * 1024, "LDS ring must fit in 160 KiB");
    static_assert(AHEAD >= 0, "ring too short for the requested prefetch");
    static_assert(AHEAD * L < 64, "vmcnt range");
    static_assert(STEPS % 2 == 0, "fragment double buffering steps by two");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int J = (K + SPI * BKS - 1) / (SPI * BKS);   // iterations
    const int TP = J * SPI;                             // slots requested (tail slots zero-filled)

    OpA opa;
    OpB opb;
    opa.init(p.A, m0, p.M, K, lane, wave);
    opb.init(p.B, n0, p.N, K, lane, wave);
    const uint32_t lds0 = lds_addr_of(smem);

    auto issue = [&](int t) {
        const uint32_t slot =
            __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t % S) * STAGE) + (uint32_t)wave * 1024u);
        opa.issue(t * BKS, K, slot);
        opb.issue(t * BKS, K, slot + (uint32_t)OpA::BYTES);
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
    for (int t = 0; t < S - SPI; ++t)
        if (t < TP) issue(t);

    // Wait until the slots read before the next barrier have landed: at most
    // AHEAD newer slots may still be in flight (fewer near the end, where
    // everything is drained).  The caller's barrier then publishes every wave's
    // part and retires all reads of the slots that get overwritten next.
    auto wait_ring = [&](int j) {
        if ((j + 1) * SPI + (PF ? 1 : 0) + AHEAD <= TP)
            wait_vmcnt<AHEAD * L>();
        else
            wait_vmcnt<0>();
    };
    auto slot_of = [&](int t) { return smem + (t % S) * STAGE; };

    u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
    if constexpr (PF) {
        if (J > 0) {
            wait_ring(0);
            __syncthreads();
            load_frags(slot_of(0), 0, fa0, fb0);
        }
    }
    for (int j = 0; j < J; ++j) {
        if (!PF || j > 0) {
            wait_ring(j);
            __syncthreads();
        }
#pragma unroll
        for (int u = 0; u < SPI; ++u) {
            const int t = j * SPI + S - SPI + u;
            if (t < TP) issue(t);
        }
        const int t0 = j * SPI;
        // Waves raise their priority while issuing MFMAs so that a wave in its
        // MFMA run is not starved by the other wave's address/LDS instructions.
        __builtin_amdgcn_s_setprio(1);
        if constexpr (!PF) load_frags(slot_of(t0), 0, fa0, fb0);
#pragma unroll
        for (int q = 0; q < STEPS; q += 2) {
            load_frags(slot_of(t0 + (q + 1) / KS), (q + 1) % KS, fa1, fb1);
            mma(fa0, fb0);
            if (q + 2 < STEPS)
                load_frags(slot_of(t0 + (q + 2) / KS), (q + 2) % KS, fa0, fb0);
            else if constexpr (PF)
                load_frags(slot_of(t0 + SPI), 0, fa0, fb0);   // next iteration's first step (stale after the last)
            mma(fa1, fb1);
        }
        // Issue order for the iteration: each step's MFMAs interleaved with the
        // next step's fragment reads, so LDS latency hides behind MFMA issue
        // instead of being waited on before each MFMA (left alone, the
        // scheduler sinks every read next to its use).
        {
            constexpr int RPS = (A_KC ? FM : 2 * FM) + (B_KC ? FN : 2 * FN);   // LDS reads per K step
            constexpr int MPS = FM * FN;                                       // MFMAs per K step
            if constexpr (!PF) __builtin_amdgcn_sched_group_barrier(0x100, RPS, 0);
#pragma unroll
            for (int q = 0; q < STEPS - 1; ++q) sched_mfma_with_reads<RPS, MPS, 0>();
            if constexpr (PF)
                sched_mfma_with_reads<RPS, MPS, 0>();
            else
                __builtin_amdgcn_sched_group_barrier(0x008, MPS, 0);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    // No direct load may still be writing LDS when the workgroup ends.
    wait_vmcnt<0>();

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

template <int BKS, int SPI, int S, bool PF, int WM, int WN, int T, bool AKC, bool BKC>
inline hipError_t launch_lds_inst(const GemmParams& p, hipStream_t stream)
{
    GemmParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n));
    const dim3 block(64 * WM * WN);
    return hipLaunchKernel((const void*)&gemm_lds_kernel<BKS, SPI, S, PF, WM, WN, T, AKC, BKC>, grid, block,
                           kargs, 0, stream);
}

// K-contiguous A <=> transpose_A == 0; K-contiguous B <=> transpose_B == 1.
template <int BKS, int SPI, int S, bool PF, int WM, int WN, int T>
inline hipError_t dispatch_lds(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    if (!tA && tB) return launch_lds_inst<BKS, SPI, S, PF, WM, WN, T, true, true>(p, s);
    if (!tA && !tB) return launch_lds_inst<BKS, SPI, S, PF, WM, WN, T, true, false>(p, s);
    if (tA && tB) return launch_lds_inst<BKS, SPI, S, PF, WM, WN, T, false, true>(p, s);
    return launch_lds_inst<BKS, SPI, S, PF, WM, WN, T, false, false>(p, s);
}

}  // namespace tlg
