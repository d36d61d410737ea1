// Tiled GEMM with an LDS ring fed by global->LDS direct loads.
//
// The tile program of the overview page's GEMM example (one output tile per
// workgroup, a K loop over K tiles, fp32 register fragments, fused epilogue),
// with the software pipeline of T.Pipelined realised as a ring of S slots: while
// tile j is multiplied, tiles j+1 .. j+S-1 are in flight ("software pipelining"
// section of the overview page).  Instances: 256 x 256 tiles with 64-wide K
// tiles and 2 slots (the large-shape default, described below), 128 x 128 with
// 64-wide K tiles and 4 slots, 64 x 128 with 128-wide K tiles and 3 slots.
//
// Global->LDS copies use buffer_load_dwordx4 ... lds: each lane's 16 bytes go
// straight to LDS at (1 KiB block + 16 * lane), with no VGPR staging and no LDS
// write instructions.  Lanes whose chunk lies outside the matrix take an
// out-of-range offset and the hardware writes zeros (the zero safe value of
// out-of-bounds reads, "core primitives" chapter, section 4.2).  The swizzled
// LDS layout is produced by choosing which global chunk each lane fetches.
// K-contiguous rows need not be 16-byte aligned (K % 8 != 0): gfx950 buffer
// loads accept 2-byte aligned addresses, and the one chunk per row that
// straddles K is trimmed in LDS before the last K tile is published (for the
// matrix's last row, whose chunk runs past the buffer, it is refetched).
// M/N-contiguous rows must hold a multiple of 8 elements.
//
// Operand layouts in LDS (one ring slot of a 256 x 256 tile; "rows" are the
// operand's M or N index; LdsOperand below gives the general rule):
//   K-contiguous operand (A stored [M,K], B stored [N,K]): 256 rows of 64
//     elements (128 bytes); 16-byte chunk c of row r sits at c ^ ((r / 2) % 8).
//     A fragment (16 consecutive rows, one chunk) is one ds_read_b128 per lane
//     and touches every bank once.
//   M/N-contiguous operand (A stored [K,M], B stored [K,N]): 64 rows of k, each
//     256 contiguous M/N elements (512 bytes); chunk c of row k sits at
//     c ^ ((k & 3) << 2) ^ (((k >> 3) & 1) << 1).  Fragments are read with
//     ds_read_b64_tr_b16, which transposes 4 x 16-bit values across each group
//     of 16 lanes: lane i of a group receives element (i & 3) of the 8-byte
//     pieces addressed by lanes (i >> 2) + 4j, j = 0..3.  Addressing row
//     kb + (s >> 2), columns nb + 4 (s & 3) from lane s therefore delivers
//     column nb + i, rows kb..kb+3 to lane i.  The second swizzle term keeps
//     the lane groups that read rows 8 apart on different banks.
//
// MFMA shape.  The wave tiles are multiplied with v_mfma_f32_16x16x32 (f16 or
// bf16 in, fp32 accumulate).  Under the MI355X power limit a stream of
// 16x16x32 instructions on changing data sustains a ~14% higher clock than
// the same FLOPs as 32x32x16 (measured ~1.93 vs ~1.68 GHz), and the kernel is
// power-bound, so the smaller shape is the faster one.  Issuing the B fragment
// as the first operand makes the hardware tile C's transpose: lane l holds
// C[m0 + l%16][n0 + 4 (l/16) + e], e = 0..3 (four consecutive columns).
//
// Schedule (per K tile, per wave).  8 waves in a 2 x 4 grid, 128 x 64 outputs
// each (8 x 4 fragments, 64 MFMAs per K tile).  The instruction order is fixed
// at compile time, one MFMA at a time:
//   - A fragment i is reloaded for the next K step right after its last use;
//     B fragments are double-buffered and read during the preceding step;
//   - the ring barrier sits inside the last K step, after SPLIT of its MFMAs:
//     the remaining MFMAs cover the latency of the next tile's first fragment
//     reads, so no wave starts a tile waiting on LDS;
//   - right after that barrier the tile's slot is free and the loads of the
//     tile S ahead (two ahead with 2 slots) are issued, one every R MFMAs, so
//     each load has at least a full K tile of MFMA work to land and the
//     vector-memory queue never blocks the MFMA stream.
#pragma once

#include <utility>

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

// s_waitcnt vmcnt(N) lgkmcnt(0).
template <int N>
__device__ inline void wait_vmcnt_lgkm0()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
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
// kernels track completion themselves with explicit vmcnt waits and issue no
// other vector-memory load while direct loads are in flight.  The whole offset
// is in the VGPR operand, so the range check (zero fill) covers all of it.
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

// f(std::integral_constant<int, 0>{}), ..., f(std::integral_constant<int, N-1>{}):
// a loop whose index is a compile-time constant in every iteration.
template <typename F, int... Ms>
__device__ inline void static_for_impl(F&& f, std::integer_sequence<int, Ms...>)
{
    (f(std::integral_constant<int, Ms>{}), ...);
}
template <int N, typename F>
__device__ inline void static_for(F&& f)
{
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// One operand of a tile: R rows of its M/N index x BK of K, filled by NW waves
// (each direct load fills one 1 KiB block).
template <int R, int BK, bool KC, int NW>
struct LdsOperand {
    static constexpr int BYTES = R * BK * 2;
    static constexpr int L = BYTES / (NW * 64 * 16);  // direct loads per lane per tile
    static_assert(BYTES % (NW * 1024) == 0, "blocks must divide evenly over the waves");
    static constexpr int RB = BK * 2, CH = BK / 8;   // K-contiguous: row bytes, chunks per row
    static constexpr int KRB = R * 2, KCH = R / 8;   // M/N-contiguous: bytes and chunks per row of k
    static constexpr int KPB = 1024 / KRB;           // M/N-contiguous: rows of k per 1 KiB block
    static_assert(KC || (KPB >= 1 && KCH >= 16), "M/N-contiguous rows of 128..512 elements");

    // Load i of a lane covers block b = i * NW + wave.  Along i the lane's row
    // (K-contiguous) or k (M/N-contiguous) advances by a constant step, and the
    // swizzle term is unchanged by that step, so one base offset per lane
    // describes all L loads.
    static constexpr int DROW = NW * (1024 / RB);   // K-contiguous: rows per load step
    static constexpr int DK = NW * KPB;             // M/N-contiguous: k rows per load step
    static_assert(!KC || (4 * NW) % CH == 0, "swizzle must be invariant along the load step");
    static_assert(KC || DK % 16 == 0, "swizzle must be invariant along the load step");

    __device__ static int swz_kc(int row) { return (row / (16 / CH)) % CH; }
    __device__ static int swz_mn(int k) { return ((k & 3) << 2) ^ (((k >> 3) & 1) << 1); }

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
            const int c = (lane % CH) ^ swz_kc(idx0);
            off0 = (uint32_t)idx0 * ld + (uint32_t)c * 16u;
            kc = c * 8;
            col_ok = true;
        } else {
            ld = (uint32_t)rows_total * 2u;
            base = (const char*)ptr + (uint64_t)r0 * 2u;
            base_bytes = (uint64_t)K * ld - (uint64_t)r0 * 2u;
            idx0 = KPB * wave + lane / KCH;
            const int c = (lane % KCH) ^ swz_mn(idx0);
            off0 = (uint32_t)idx0 * ld + (uint32_t)c * 16u;
            kc = 0;
            col_ok = c * 8 < rows_left;
        }
    }

    // Resource for the tile starting at k0 (tiles at or past the end of K get an
    // empty resource: every lane reads zeros).
    __device__ i32x4 rsrc(int k0) const
    {
        const uint64_t o = KC ? (uint64_t)k0 * 2u : (uint64_t)k0 * ld;
        return rsrc_words(base + o, o < base_bytes ? base_bytes - o : 0);
    }

    // Lane offset of load i of the tile starting at k0, or kOOB.
    __device__ uint32_t voff(int i, int k0, int K) const
    {
        if constexpr (KC) {
            const bool valid = (idx0 + i * DROW < rows_left) && (k0 + kc < K);
            return valid ? off0 + (uint32_t)(i * DROW) * ld : kOOB;
        } else {
            const bool valid = col_ok && (k0 + idx0 + i * DK < K);
            return valid ? off0 + (uint32_t)(i * DK) * ld : kOOB;
        }
    }

    // K-contiguous operand with K % 8 != 0: in the last K tile the chunk holding
    // element K-1 also holds up to 7 elements past K (the next row's first ones).
    // Once the lane's own loads of that tile have landed, it zeroes them in LDS
    // (wave_base: the tile's slot region of this operand + 1 KiB * wave).  The
    // matrix's last row is different: its chunk runs past the end of the buffer,
    // and the range check returns the whole 16-byte load as zeros, so its valid
    // elements (at most 7) are fetched again with 16-bit loads.
    __device__ void fix_k_tail(char* wave_base, int k0, int K, int lane) const
    {
        if constexpr (KC) {
            const int nvalid = K - (k0 + kc);
            if (nvalid > 0 && nvalid < 8) {
                u32x4 keep;
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    keep[w] = 2 * w + 1 < nvalid ? 0xffffffffu : (2 * w < nvalid ? 0x0000ffffu : 0u);
                const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (uint64_t)k0 * 2u, base_bytes - (uint64_t)k0 * 2u);
#pragma unroll
                for (int i = 0; i < L; ++i) {
                    const int row = idx0 + i * DROW;
                    u32x4* q = (u32x4*)(wave_base + i * NW * 1024 + lane * 16);
                    u32x4 v = *q & keep;
                    if (row == rows_left - 1) {
                        uint32_t h[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e)
                            h[e] = e < nvalid ? buf_load2(r, (uint32_t)row * ld + (uint32_t)(kc + e) * 2u) : 0u;
                        v = u32x4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
                    }
                    *q = v;
                }
            }
        }
    }

    // MFMA 16x16x32 operand of rows row0..row0+15 (row0 a multiple of 16), K step
    // kk (32 wide): lane l holds row row0 + l%16 and K elements 8*(l/16) .. +7.
    __device__ u32x4 frag(const char* region, int row0, int kk, int lane) const
    {
        if constexpr (KC) {
            const int row = row0 + (lane & 15);
            const int c = kk * 4 + (lane >> 4);
            return *(const u32x4*)(region + row * RB + ((c ^ swz_kc(row)) << 4));
        } else {
            const int g = lane >> 4, s = lane & 15;
            const int n = row0 + 4 * (s & 3);
            const int k = kk * 32 + g * 8 + (s >> 2);
            const int half = ((n >> 2) & 1) * 8;
            const u32x2 lo = lds_read_tr16(region + k * KRB + (((n >> 3) ^ swz_mn(k)) << 4) + half);
            const u32x2 hi = lds_read_tr16(region + (k + 4) * KRB + (((n >> 3) ^ swz_mn(k + 4)) << 4) + half);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        }
    }
};

// Work decomposition (MODE):
//   kModeDP      one output tile per workgroup, whole K (the tile program's grid).
//   kModeSplitK  workgroup b handles tile b / splits and K range b % splits.
//   kModeStreamK persistent: a fixed grid of G workgroups (one per CU); workgroup g
//                first computes the whole-K tiles g, g + G, ... below p.dp_tiles,
//                then an equal share of the remaining p.sk_tiles x (K tiles)
//                iterations, cut at tile boundaries into segments (the "persistent"
//                schedule of the overview page: a tile scheduler that balances the
//                tail of the grid over every CU).
// A tile whose K range is split over several workgroups has its fp32 partial
// tiles summed, in K order, by whichever of them finishes last (a counter per tile
// elects it), so the result does not depend on the order in which they finish.
enum : int { kModeDP = 0, kModeSplitK = 1, kModeStreamK = 2 };

template <int BM, int BN, int S, int SPLIT, int R, int WAVES_M, int WAVES_N, int T_IN, bool A_KC, bool B_KC,
          int MODE = kModeDP, int BK = 64>
__global__ void __launch_bounds__(64 * WAVES_M * WAVES_N)
gemm_lds_kernel(GemmParams p)
{
    constexpr int NW = WAVES_M * WAVES_N;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 16, FN = WTN / 16;
    using OpA = LdsOperand<BM, BK, A_KC, NW>;
    using OpB = LdsOperand<BN, BK, B_KC, NW>;
    constexpr int STAGE = OpA::BYTES + OpB::BYTES;
    constexpr int LA = OpA::L, LB = OpB::L, L = LA + LB;
    constexpr int KS = BK / 32;                       // MFMA K steps per tile
    constexpr int MPS = FM * FN;                      // MFMAs per K step
    constexpr int MI = KS * MPS;                      // MFMAs per tile
    constexpr int BPOS = (KS - 1) * MPS + SPLIT;      // the barrier precedes MFMA BPOS
    // D loads of tile j+S are issued after tile j's barrier (their slot has just
    // been freed), the other L-D at the start of the next tile.
    constexpr int D0 = (MI - 1 - BPOS) / R + 1;
    constexpr int D = D0 < L ? D0 : L;
    static_assert(S >= 2 && S * STAGE <= 160 * 1024, "LDS ring must fit in 160 KiB");
    static_assert(KS == 2 || (KS == 4 && MODE == kModeDP), "K tiles of 64, or of 128 without a split K");
    static_assert(FM >= 2, "B fragments of the next K step are read at MFMAs jj * FM + 1 of a step");
    static_assert(SPLIT >= 1 && SPLIT < MPS, "barrier inside the last K step");
    static_assert(L - D == 0 || (L - D - 1) * R < BPOS, "early loads precede the barrier");
    static_assert((S - 2) * L + D < 64, "vmcnt range");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];
    __shared__ unsigned ticket;

    const int lane_id = threadIdx.x & 63;
    const int wave_id = threadIdx.x >> 6;
    const int K = p.K;
    const int TPALL = (K + BK - 1) / BK;              // K tiles (the last one zero-padded)

    // One segment: output tile tile_id over K tiles kt0 .. kt0+TP-1.  When the tile's
    // K range is shared by nslots > 1 segments, their partial tiles go to workspace
    // slots counted from slot_base: segment s (in K order) uses slot
    // slot_base + (s == 0 ? first_off : s * stride), this one slot_base + self_off;
    // counters[counter] elects the segment that sums them.
    auto segment = [&](int tile_id, int kt0, int TP, int slot_base, int nslots, int self_off, int first_off,
                       int stride, int counter) {
    // In the persistent loop the lane and wave indices pass through empty asm
    // statements: this keeps the compiler from hoisting the lane-dependent address
    // arithmetic out of the loop, where it would stay live across the K loop and spill.
    int lane = lane_id, wave = __builtin_amdgcn_readfirstlane(wave_id);
    if constexpr (MODE == kModeStreamK) {
        asm volatile("" : "+v"(lane));
        asm volatile("" : "+s"(wave));
        lane &= 63;   // the compiler's knowledge of the ranges, lost through the asm
        wave &= 7;
        // The segment's parameters are the same in every lane: say so, so that the
        // K loop's counters and buffer resources stay in scalar registers.
        tile_id = __builtin_amdgcn_readfirstlane(tile_id);
        kt0 = __builtin_amdgcn_readfirstlane(kt0);
        TP = __builtin_amdgcn_readfirstlane(TP);
        slot_base = __builtin_amdgcn_readfirstlane(slot_base);
        nslots = __builtin_amdgcn_readfirstlane(nslots);
        self_off = __builtin_amdgcn_readfirstlane(self_off);
        first_off = __builtin_amdgcn_readfirstlane(first_off);
        counter = __builtin_amdgcn_readfirstlane(counter);
    }
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    int tm, tn;
    if constexpr (MODE == kModeStreamK)
        band_coords(tile_id, p.tiles_m, p.tiles_n, tm, tn);   // the worker numbering groups XCDs
    else
        tile_coords(tile_id, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // Loads stop at the end of the segment's K range (elements past it read as zeros).
    const int KLIM = min(K, (kt0 + TP) * BK);

    OpA opa;
    OpB opb;
    opa.init(p.A, m0, p.M, K, lane, wave);
    opb.init(p.B, n0, p.N, K, lane, wave);
    const uint32_t lds0 = lds_addr_of(smem);

    // Load i of tile t into its slot.  Every tile index gets its loads, also the
    // ones past the end of K (their resource is empty and they write zeros into a
    // slot nobody reads again), so every K tile issues exactly L loads and the
    // vmcnt bookkeeping below needs no special cases.
    struct TileRes {
        i32x4 ra, rb;
        int k0;
        uint32_t slot;
    };
    auto tile_res = [&](int t) {
        TileRes r;
        r.k0 = (kt0 + t) * BK;
        r.ra = opa.rsrc(r.k0);
        r.rb = opb.rsrc(r.k0);
        r.slot = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t % S) * STAGE) + (uint32_t)wave * 1024u);
        return r;
    };
    auto issue_one = [&](const TileRes& r, int i) {
        if (i < LA)
            dma16(r.ra, opa.voff(i, r.k0, KLIM), r.slot + (uint32_t)(i * NW * 1024));
        else
            dma16(r.rb, opb.voff(i - LA, r.k0, KLIM), r.slot + (uint32_t)OpA::BYTES + (uint32_t)((i - LA) * NW * 1024));
    };

    // Last K tile with K % 8 != 0: trim the elements past K that this lane's
    // loads brought into LDS (called after they landed, before the barrier that
    // publishes the tile).  The asm statements keep the compiler from moving LDS
    // accesses across the preceding wait.
    const bool k_tail = (K & 7) != 0 && kt0 + TP == TPALL;   // this range ends at K
    auto fix_k_tail = [&](int t) {
        asm volatile("" ::: "memory");
        char* region = smem + (t % S) * STAGE + wave * 1024;
        opa.fix_k_tail(region, (kt0 + t) * BK, K, lane);
        opb.fix_k_tail(region + OpA::BYTES, (kt0 + t) * BK, K, lane);
        asm volatile("" ::: "memory");
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 fa[FM], fb[2][FN];
    const int arow = wm * WTM, bcol = wn * WTN;

    // Prologue: tiles 0 .. S-2 whole, the first D loads of tile S-1; wait for tile 0.
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        const TileRes r0 = tile_res(t);
#pragma unroll
        for (int i = 0; i < L; ++i) issue_one(r0, i);
    }
    {
        const TileRes r1 = tile_res(S - 1);
#pragma unroll
        for (int i = 0; i < D; ++i) issue_one(r1, i);
    }
    wait_vmcnt<(S - 2) * L + D>();
    if (k_tail && TP == 1) {
        fix_k_tail(0);
        wait_vmcnt_lgkm0<(S - 2) * L + D>();
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = opa.frag(smem, arow + i * 16, 0, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[0][j] = opb.frag(smem + OpA::BYTES, bcol + j * 16, 0, lane);

    for (int j = 0; j < TP; ++j) {
        const char* cur = smem + (j % S) * STAGE;
        const char* nxt = smem + ((j + 1) % S) * STAGE;
        const TileRes re = tile_res(j + S - 1);     // the rest of this tile's loads
        const TileRes rl = tile_res(j + S);         // loads issued after this tile's barrier
        // Waves raise their priority while issuing MFMAs so that a wave in its
        // MFMA run is not starved by the other wave's address/LDS instructions.
        __builtin_amdgcn_s_setprio(1);
        // Events placed before MFMA m (m = MI: after the last one).
        static_for<MI + 1>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            constexpr int q = m / MPS, r = m % MPS;
            if constexpr (m == BPOS) {
                // Own fragment reads of this slot retired and tile j+1 landed (at
                // most the (S-2) newer tiles in flight); the barrier then publishes
                // every wave's part of tile j+1 and frees tile j's slot.
                __builtin_amdgcn_s_setprio(0);
                wait_vmcnt_lgkm0<(S - 2) * L>();
                if (k_tail && j + 2 == TP) {
                    fix_k_tail(j + 1);
                    wait_vmcnt_lgkm0<(S - 2) * L>();
                }
                __syncthreads();
                __builtin_amdgcn_s_setprio(1);
            }
            if constexpr (m % R == 0 && m / R < L - D) issue_one(re, D + m / R);
            if constexpr (m >= BPOS && (m - BPOS) % R == 0 && (m - BPOS) / R < D) issue_one(rl, (m - BPOS) / R);
            // A fragment i: its last use in step qs is MFMA qs*MPS + i*FN + FN - 1; it
            // is reloaded right after that (for the next tile: not before the barrier).
            if constexpr (m > 0) {
                constexpr int qs = (m - 1) / MPS;
                static_for<FM>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    constexpr int pos = qs * MPS + i * FN + FN;
                    if constexpr (qs + 1 < KS) {
                        if constexpr (m == pos) fa[i] = opa.frag(cur, arow + i * 16, qs + 1, lane);
                    } else {
                        constexpr int pos2 = pos > BPOS ? pos : BPOS;
                        if constexpr (m == pos2) fa[i] = opa.frag(nxt, arow + i * 16, 0, lane);
                    }
                });
            }
            if constexpr (m < MI) {
                // B fragments of the next step into the other buffer, spread over the step.
                static_for<FN>([&](auto jc) {
                    constexpr int jj = decltype(jc)::value;
                    if constexpr (q + 1 < KS) {
                        if constexpr (r == jj * (MPS / FN) + 1)
                            fb[(q + 1) % 2][jj] = opb.frag(cur + OpA::BYTES, bcol + jj * 16, q + 1, lane);
                    } else {
                        if constexpr (r == SPLIT + (jj * (MPS - SPLIT)) / FN)
                            fb[0][jj] = opb.frag(nxt + OpA::BYTES, bcol + jj * 16, 0, lane);
                    }
                });
                constexpr int i = r / FN, jj = r % FN;
                acc[i][jj] = mfma16x16x32<T_IN>(fb[q % 2][jj], fa[i], acc[i][jj]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_setprio(0);
    }
    // No direct load may still be writing LDS when the segment ends.
    wait_vmcnt<0>();

    if constexpr (MODE != kModeDP) if (nslots > 1) {
        // Publish this range's fp32 partial tile, then take a ticket; the last
        // workgroup of the tile sums the partials in range order and goes on to the
        // epilogue, the others are done.  The XCDs have separate L2 caches, so the
        // partials are written and read with device-scope (sc1) buffer accesses,
        // which the hardware keeps coherent across XCDs (the same accesses the
        // compiler emits for agent-scope atomic loads and stores).  Every wave waits
        // for its partial stores to complete before the barrier that precedes the
        // ticket, and the partials are read only after the ticket, so no cache
        // write-back or invalidation is needed.
        const __amdgpu_buffer_rsrc_t wsr =
            make_rsrc(p.ws + (size_t)slot_base * (BM * BN), (uint64_t)((nslots - 1) * stride + 1) * BM * BN * 4u);
        auto ws_off = [&](int s2, int i, int jj) {
            const int ml = arow + i * 16 + (lane & 15), nl = bcol + jj * 16 + 4 * (lane >> 4);
            return (uint32_t)((s2 * (BM * BN) + ml * BN + nl) * 4);
        };
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jj = 0; jj < FN; ++jj)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][jj]), wsr,
                                                       ws_off(self_off, i, jj), 0, kCoherentDevice);
        wait_vmcnt<0>();
        __syncthreads();
        if (threadIdx.x == 0)
            ticket = __hip_atomic_fetch_add(p.counters + counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (__builtin_amdgcn_readfirstlane(ticket) != (unsigned)(nslots - 1)) return;
        // acc = partial 0 + partial 1 + ... in K order (this workgroup's own partial is
        // read back from the workspace too, which keeps the code free of branches).
        // The loads of up to four partials are in flight together (slots past the
        // last one read zeros: their offsets lie beyond the resource), RBI row blocks
        // of fragments at a time so that at most 128 registers hold loaded values.
        constexpr int G = 4;
        constexpr int RBI = (32 / (G * FN)) < FM ? (32 / (G * FN) > 0 ? 32 / (G * FN) : 1) : FM;
        static_assert(FM % RBI == 0, "row blocks of the reduction");
#pragma unroll
        for (int i0 = 0; i0 < FM; i0 += RBI) {
#pragma unroll
            for (int i = i0; i < i0 + RBI; ++i)
#pragma unroll
                for (int jj = 0; jj < FN; ++jj) acc[i][jj] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int s0 = 0; s0 < nslots; s0 += G) {
                u32x4 part[G][RBI][FN];
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int i = 0; i < RBI; ++i)
#pragma unroll
                        for (int jj = 0; jj < FN; ++jj)
                            part[g][i][jj] = __builtin_amdgcn_raw_buffer_load_b128(
                                wsr,
                                s0 + g < nslots ? ws_off(s0 + g == 0 ? first_off : (s0 + g) * stride, i0 + i, jj)
                                                : kOOB,
                                0, kCoherentDevice);
#pragma unroll
                for (int g = 0; g < G; ++g)
#pragma unroll
                    for (int i = 0; i < RBI; ++i)
#pragma unroll
                        for (int jj = 0; jj < FN; ++jj) acc[i0 + i][jj] += __builtin_bit_cast(f32x4, part[g][i][jj]);
            }
        }
        if (threadIdx.x == 0)   // ready for the next launch
            __hip_atomic_store(p.counters + counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // Epilogue.  acc[i][j][e] is C[m][n + e] with
    //   m = m0 + wm*WTM + i*16 + lane%16,  n = n0 + wn*WTN + j*16 + 4*(lane/16).
    store_blocks<FM, FN>(p.C, p.M, p.N, p.c_dtype, p.c_vec != 0, p.c_vec8 != 0, p.relu != 0, p.clear_accum != 0, acc,
                         m0 + arow, n0 + bcol, lane);
    };   // segment

    if constexpr (MODE == kModeDP) {
        segment(blockIdx.x, 0, TPALL, 0, 1, 0, 0, 1, 0);
    } else if constexpr (MODE == kModeSplitK) {
        const int tile_id = blockIdx.x / p.splits, split = blockIdx.x % p.splits;
        const int per = (TPALL + p.splits - 1) / p.splits;
        const int kt0 = split * per;
        segment(tile_id, kt0, min(per, TPALL - kt0), tile_id * p.splits, p.splits, split, 0, 1, tile_id);
    } else {
        // Persistent.  Workgroup g first takes the whole-K tiles g, g + G, ... below
        // dp_tiles, then its share of the stream-K iterations [0, W) of the sk_tiles
        // remaining tiles: [beg(g), beg(g + 1)) with beg(g) = g W / G.  Iteration i
        // belongs to workgroup owner(i) = ((i + 1) G - 1) / W, the largest g with
        // beg(g) <= i.  A workgroup has at most two partial segments: the one that
        // starts at beg(g) (slot 2g) and, if its range crosses a tile boundary, the
        // one that ends at beg(g + 1) (slot 2g + 1); the segments in between cover
        // whole tiles.  So the partials of stream-K tile r, made by workgroups
        // gf .. gl, sit in slots 2gf + (r starts at beg(gf) ? 0 : 1), then 2g for
        // g = gf+1 .. gl.  The loop ends: every trip either takes one of the finitely
        // many whole tiles or advances `it` by at least one K tile towards its end.
        // (One call site of `segment`, so its code is instantiated once.)
        // W = sk_tiles x (K tiles) < 2^9 x 2^16 fits 32 bits (the plan bounds both).
        // The loop state (trip j, iteration `it`) lives in LDS and is read back with
        // volatile loads at the top of every trip, so nothing derived from it can be
        // hoisted out of the loop and held in registers across the K loop.
        __shared__ int sched[2];
        if (threadIdx.x == 0) {
            const int G = (int)gridDim.x;
            const int g = G % kXcds == 0 ? ((int)blockIdx.x % kXcds) * (G / kXcds) + (int)blockIdx.x / kXcds
                                         : (int)blockIdx.x;
            sched[0] = 0;
            sched[1] = (int)((int64_t)g * (p.sk_tiles * TPALL) / G);
        }
        __syncthreads();
        for (;;) {
            // Worker index: workgroups are dispatched round-robin over the 8 XCDs, so
            // numbering the workers XCD by XCD gives each XCD's workgroups consecutive
            // whole tiles and consecutive shares of the iterations, i.e. neighbouring
            // tiles (tile ids walk bands of tile rows, no further remap) that reuse the
            // same A and B panels from that XCD's L2.  (A bijection on [0, G) when
            // G % 8 == 0; the schedule below is correct for any numbering.)
            const int G = (int)gridDim.x;
            const int g = G % kXcds == 0 ? ((int)blockIdx.x % kXcds) * (G / kXcds) + (int)blockIdx.x / kXcds
                                         : (int)blockIdx.x;
            const int j = __builtin_amdgcn_readfirstlane(*(volatile int*)&sched[0]);
            const int itv = __builtin_amdgcn_readfirstlane(*(volatile int*)&sched[1]);
            const int ndp = g < p.dp_tiles ? (p.dp_tiles - g + G - 1) / G : 0;
            const int W = p.sk_tiles * TPALL;
            const int beg = (int)((int64_t)g * W / G), end = (int)((int64_t)(g + 1) * W / G);
            int tile, k0, tp, base, ns, self, first, ctr, next = itv;
            if (j < ndp) {
                tile = g + j * G; k0 = 0; tp = TPALL; base = 0; ns = 1; self = 0; first = 0; ctr = 0;
            } else {
                if (itv >= end) break;
                const int r = itv / TPALL;
                k0 = itv - r * TPALL;
                const int k1 = min(TPALL, k0 + (end - itv));
                const int64_t tb = (int64_t)r * TPALL;
                const int gf = (int)(((tb + 1) * G - 1) / W), gl = (int)(((tb + TPALL) * G - 1) / W);
                tile = p.dp_tiles + r; tp = k1 - k0; ns = gl - gf + 1; ctr = r;
                base = 2 * gf;
                first = tb == (int64_t)gf * W / G ? 0 : 1;
                self = 2 * (g - gf) + (itv == beg ? 0 : 1);
                next = itv + tp;
            }
            segment(tile, k0, tp, base, ns, self, first, 2, ctr);
            // Every thread read the state before the segment's barriers; the next trip
            // reads it after the barrier below.
            if (threadIdx.x == 0) {
                sched[0] = j + 1;
                sched[1] = next;
            }
            __syncthreads();   // every wave is done with the LDS ring before the next prologue
        }
    }
}

template <int BM, int BN, int S, int SPLIT, int R, int WM, int WN, int T, bool AKC, bool BKC, int MODE, int BK = 64>
inline hipError_t launch_lds_inst(const GemmParams& p, hipStream_t stream)
{
    GemmParams args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)(MODE == kModeStreamK ? p.persistent_grid
                                                    : p.tiles_m * p.tiles_n * (MODE == kModeSplitK ? p.splits : 1)));
    const dim3 block(64 * WM * WN);
    return hipLaunchKernel((const void*)&gemm_lds_kernel<BM, BN, S, SPLIT, R, WM, WN, T, AKC, BKC, MODE, BK>, grid,
                           block, kargs, 0, stream);
}

// K-contiguous A <=> transpose_A == 0; K-contiguous B <=> transpose_B == 1.
template <int BM, int BN, int S, int SPLIT, int R, int WM, int WN, int T, int MODE = kModeDP>
inline hipError_t dispatch_lds_layout(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    if (!tA && tB) return launch_lds_inst<BM, BN, S, SPLIT, R, WM, WN, T, true, true, MODE>(p, s);
    if (!tA && !tB) return launch_lds_inst<BM, BN, S, SPLIT, R, WM, WN, T, true, false, MODE>(p, s);
    if (tA && tB) return launch_lds_inst<BM, BN, S, SPLIT, R, WM, WN, T, false, true, MODE>(p, s);
    return launch_lds_inst<BM, BN, S, SPLIT, R, WM, WN, T, false, false, MODE>(p, s);
}

// 256 x 256 tiles: 8 waves of 128 x 64, 2-slot ring, barrier after 8 of the last
// K step's 32 MFMAs, then the next tile's eight direct loads one every 3 MFMAs
// (measured on MI355X against one every 2: 8192^3 -2%, 4096^3 -3%; every 1, 4 or 5
// MFMAs and barriers after 2-24 MFMAs were slower).
template <int T>
inline hipError_t dispatch_lds(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    return dispatch_lds_layout<256, 256, 2, 8, 3, 2, 4, T>(p, tA, tB, s);
}

// 128 x 128 tiles (grids too small for 256 x 256): 8 waves of 64 x 32, 4-slot ring,
// barrier after 4 of the last K step's 8 MFMAs, one direct load every 2 MFMAs.
template <int T>
inline hipError_t dispatch_lds128(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    return dispatch_lds_layout<128, 128, 4, 4, 2, 2, 4, T>(p, tA, tB, s);
}

// 64 x 128 tiles (grids of at most 128 tiles of 128 x 128: twice the workgroups
// in one wave): 8 waves of 32 x 32, K tiles of 128 in a 3-slot ring (144 KiB),
// barrier after 1 of the last K step's 4 MFMAs, one direct load every 2 MFMAs.
// These small grids are bound by each K step's barrier and LDS round trip, not by
// the loads: with K tiles of 64 a wave has only 8 MFMAs per barrier (deeper rings
// of 5 or 6 slots are slower).  K tiles of 128 halve the barriers, and three
// MFMAs after the barrier hide the next tile's fragment reads better than two
// (measured on MI355X: 1024^3 11.9 -> 10.0 us, 64 x 128 x 4096 34.6 -> 25.3 us).
// The LDS layout takes M/N-contiguous rows of 128..512 elements only, so A must
// be K-contiguous (transpose_A == 0).
template <int T>
inline hipError_t dispatch_lds64(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    if (tA) return hipErrorInvalidValue;
    if (tB) return launch_lds_inst<64, 128, 3, 1, 2, 2, 4, T, true, true, kModeDP, 128>(p, s);
    return launch_lds_inst<64, 128, 3, 1, 2, 2, 4, T, true, false, kModeDP, 128>(p, s);
}

// The same 128 x 128 kernel with K split over p.splits workgroups per tile.
template <int T>
inline hipError_t dispatch_lds128_sk(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    return dispatch_lds_layout<128, 128, 4, 4, 2, 2, 4, T, kModeSplitK>(p, tA, tB, s);
}

// Persistent stream-K schedules of the 256 x 256 and 128 x 128 kernels.
template <int T>
inline hipError_t dispatch_lds_streamk(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    return dispatch_lds_layout<256, 256, 2, 8, 2, 2, 4, T, kModeStreamK>(p, tA, tB, s);
}

template <int T>
inline hipError_t dispatch_lds128_streamk(const GemmParams& p, int tA, int tB, hipStream_t s)
{
    return dispatch_lds_layout<128, 128, 4, 4, 2, 2, 4, T, kModeStreamK>(p, tA, tB, s);
}

}  // namespace tlg
