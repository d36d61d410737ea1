// Block-scaled ("MX") GEMM: FP8 operands (E4M3 or E5M2) in which every 32
// consecutive elements along K share one E8M0 power-of-two scale, fp32
// accumulation, on the gfx950 scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4.  This is the block-scaled MMA of the codegen
// chapter (sections 3.4 and 4.6.3: FP8 elements in shared memory, E8M0 scale
// factors per 32 of K, fp32 accumulator), on the same tile program as the 16-bit
// kernels: 256 x 256 output tiles, a K loop over 128-wide K tiles, a two-slot
// LDS ring filled by global->LDS direct loads, fused epilogue.
//
// Operands.  A is stored [M, K] and B [N, K] (both K-contiguous, the layout of
// the pages' 1d1d block-scaled example); SA is [M, K/32] and SB [N, K/32]
// bytes.  K must be a multiple of 128 (whole K tiles, so the per-row scale
// words of a tile are dword-aligned).
//
// One ring slot holds, for a 128-wide K tile:
//   A 256 rows x 128 bytes, B 256 rows x 128 bytes (the byte layout of the
//   16-bit kernels' 64-element rows: 16-byte chunk c of row r at c ^ ((r/2)%8)),
//   then SA and SB, 256 rows x 4 scale bytes each (row r's four blocks at 4 r).
// The data are filled with 16-byte direct loads, the scales with 4-byte ones.
//
// Instruction layout (measured on MI355X with one-hot probes of every operand
// byte): for a 16 x 128 operand, lane l holds row l % 16 and, with g = l / 16,
// the K elements 16 g .. 16 g + 15 in bytes 0..15 and 64 + 16 g .. 64 + 16 g + 15
// in bytes 16..31 -- LDS chunks g and 4 + g of the row; the scale operand of
// lane s is the scale of row s % 16, K block s / 16.
//
// Per wave (8 waves in a 2 x 4 grid, 128 x 64 outputs each) a K tile is 32
// scaled MFMAs, issued row-block-major (MFMA m uses A fragment m / 4 and B
// fragment m % 4).  Register budget (2 waves per SIMD, 256 registers each, 128
// of them accumulators) allows the four B fragments to stay resident while the
// eight A fragments rotate through four buffers: A fragment i is read 12 MFMAs
// before its first use, into the buffer of fragment i-4; the first four A
// fragments and the B fragments of the next tile are read from the next slot.
// The ring barrier sits after MFMA 20, once every read of the current slot has
// been issued; after it the tile two ahead is loaded into the freed slot, its
// loads spread evenly over the remaining 12 MFMAs.
//
// MXFP4 (FMT 4: E2M1 elements, two per byte).  A 128-byte K tile row then holds
// 256 elements, so the tile program, the LDS layout and the fragment reads are
// the FP8 kernel's byte for byte; what changes is the instruction's view of a
// fragment.  With FP4 operands the instruction reads four registers per lane:
// lane l holds row l % 16 and K elements 32 g .. 32 g + 31 (g = l / 16), 16
// consecutive bytes (measured on MI355X: one wave, random codes and scales,
// compared with the host's sums under each candidate layout).  LDS chunk g of a
// row is therefore the operand of the tile's first 128 K elements and chunk 4 + g
// that of the second: each fragment pair (i, j) of a tile is two MFMAs, one per
// K half, each with its own scale byte (blocks 0..3 and 4..7 of the tile, kept in
// two scale planes of 4 bytes per row).  Per A fragment the eight MFMAs are
// issued as the four first halves, then the four second halves, so an
// accumulator's two MFMAs are four instructions apart.
#pragma once

#include "gemm_lds.hpp"

namespace tlg {

typedef int i32x8 __attribute__((ext_vector_type(8)));

// 4-byte global->LDS direct load: lane l writes LDS bytes [lds + 4 l, lds + 4 l + 4).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma4(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ inline uint32_t lds_u8(const char* p) { return *(const unsigned char*)p; }

// FMT: operand format code of the scaled instruction (0 = E4M3, 1 = E5M2, 4 = E2M1).
// SEL: which byte of the scale registers holds the E8M0 scales (the instruction's
// scale byte select).
template <int FMT, int SEL = 0>
__device__ inline f32x4 mfma_scale16x16x128(const i32x8& a, const i32x8& b, f32x4 c, int sa, int sb)
{
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, SEL, sa, SEL, sb);
}

// FP4 operands occupy the low four registers; the upper half is not read.
__device__ inline i32x8 fp4_operand(const u32x4& x)
{
    const i32x4 v = __builtin_bit_cast(i32x4, x);
    return __builtin_shufflevector(v, v, 0, 1, 2, 3, -1, -1, -1, -1);
}

template <int FMT>
__global__ void __launch_bounds__(512) gemm_mx_kernel(MxParams p)
{
    constexpr bool FP4 = FMT == 4;
    constexpr int BM = 256, BN = 256;                    // K tile: 128 bytes per row (128 FP8 / 256 FP4 elements)
    constexpr int PLANES = FP4 ? 2 : 1;                  // scale planes of 4 bytes per row per tile
    constexpr int WAVES_M = 2, WAVES_N = 4, NW = 8;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 16, FN = WTN / 16;
    // A K-tile row has the byte layout of a 64-element 16-bit row: the operand
    // helper works in 16-bit units (K/2 of them per row).
    using OpA = LdsOperand<BM, 64, true, NW>;
    using OpB = LdsOperand<BN, 64, true, NW>;
    constexpr int SCB = BM * 4;                          // scale bytes per operand per plane per tile
    constexpr int STAGE = OpA::BYTES + OpB::BYTES + 2 * PLANES * SCB;
    constexpr int LD = OpA::L + OpB::L;                  // 16-byte data loads per wave per tile
    constexpr int L = LD + PLANES;                       // plus one 4-byte scale load per plane
    constexpr int MI = FM * FN;                          // MFMAs per tile
    constexpr int NBUF = 4;                              // rotating A fragment buffers
    constexpr int LEAD = 3 * FN;                         // A fragment i is read before MFMA FN*i - LEAD
    constexpr int BPOS = FN * FM - LEAD;                 // the barrier precedes MFMA BPOS
    static_assert(FM % NBUF == 0 && LEAD == FN * (NBUF - 1), "rotation of the A fragment buffers");
    static_assert(2 * STAGE <= 160 * 1024, "two ring slots must fit in 160 KiB");
    static_assert(MI - BPOS >= L, "all loads of a tile fit after the barrier, at most one per MFMA");
    static_assert(2 * SCB / 256 == NW, "one 4-byte scale load per wave covers 64 rows");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K, KB = K / 32;
    const int K16 = FP4 ? K / 4 : K / 2;                 // row length in 16-bit units
    const int TP = (K16 + 63) / 64;                      // K tiles (an FP4 K of 128 mod 256: last tile half full)

    OpA opa;
    OpB opb;
    opa.init(p.A, m0, p.M, K16, lane, wave);
    opb.init(p.B, n0, p.N, K16, lane, wave);
    const uint32_t lds0 = lds_addr_of(smem);

    // Scale load of this wave: waves 0-3 load SA rows 64 w .. 64 w + 63, waves 4-7
    // SB rows 64 (w-4) ...; lane l fetches the tile's four block scales of one row.
    const bool sc_a = wave < 4;
    const int sc_row = (wave & 3) * 64 + lane;
    const char* sc_base = (const char*)(sc_a ? p.SA : p.SB) + (uint64_t)(sc_a ? m0 : n0) * KB;
    const int sc_rows_left = sc_a ? p.M - m0 : p.N - n0;
    const uint64_t sc_bytes = (uint64_t)sc_rows_left * KB;
    const uint32_t sc_voff = sc_row < sc_rows_left ? (uint32_t)sc_row * (uint32_t)KB : kOOB;
    // plane h of the tile: A's planes, then B's
    const uint32_t sc_dst_off = (uint32_t)(OpA::BYTES + OpB::BYTES + (sc_a ? 0 : PLANES * SCB) + (wave & 3) * 256);

    struct TileRes {
        i32x4 ra, rb, rs;
        int k0;          // in 16-bit units
        uint32_t slot, sslot;
        uint32_t soff[PLANES];
    };
    auto tile_res = [&](int t) {
        TileRes r;
        r.k0 = t * 64;
        r.ra = opa.rsrc(r.k0);
        r.rb = opb.rsrc(r.k0);
        const uint64_t so = (uint64_t)t * 4u * PLANES;
        r.rs = rsrc_words(sc_base + so, so < sc_bytes ? sc_bytes - so : 0);
        r.slot = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t & 1) * STAGE) + (uint32_t)wave * 1024u);
        r.sslot = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t & 1) * STAGE) + sc_dst_off);
        // plane h covers scale blocks 4 (PLANES t + h) .. +3; past the row's KB blocks it reads zeros
#pragma unroll
        for (int h = 0; h < PLANES; ++h)
            r.soff[h] = (t < TP && (t * PLANES + h) * 4 < KB) ? sc_voff + (uint32_t)(4 * h) : kOOB;
        return r;
    };
    auto issue_one = [&](const TileRes& r, int i) {
        if (i < OpA::L)
            dma16(r.ra, opa.voff(i, r.k0, K16), r.slot + (uint32_t)(i * NW * 1024));
        else if (i < LD)
            dma16(r.rb, opb.voff(i - OpA::L, r.k0, K16), r.slot + (uint32_t)OpA::BYTES + (uint32_t)((i - OpA::L) * NW * 1024));
        else
            dma4(r.rs, r.soff[i - LD], r.sslot + (uint32_t)((i - LD) * SCB));
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int arow = wm * WTM, bcol = wn * WTN;
    i32x8 fa[NBUF], fb[FN];
    int sa[NBUF], sb[FN];
    // fragment (two 16-byte chunks g and 4+g of the row) and its scale byte(s): the
    // lane's row and K block (lane >> 4); with two planes, plane h's byte goes to
    // byte h of the register (selected per MFMA by the instruction)
    auto read_a = [&](const char* slot, int i) {
        const u32x4 lo = opa.frag(slot, arow + i * 16, 0, lane), hi = opa.frag(slot, arow + i * 16, 1, lane);
        fa[i % NBUF] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const char* sp = slot + OpA::BYTES + OpB::BYTES + (arow + i * 16 + (lane & 15)) * 4 + (lane >> 4);
        int v = (int)lds_u8(sp);
        if constexpr (PLANES == 2) v |= (int)lds_u8(sp + SCB) << 8;
        sa[i % NBUF] = v;
    };
    auto read_b = [&](const char* slot, int j) {
        const char* bs = slot + OpA::BYTES;
        const u32x4 lo = opb.frag(bs, bcol + j * 16, 0, lane), hi = opb.frag(bs, bcol + j * 16, 1, lane);
        fb[j] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        const char* sp = slot + OpA::BYTES + OpB::BYTES + PLANES * SCB + (bcol + j * 16 + (lane & 15)) * 4 + (lane >> 4);
        int v = (int)lds_u8(sp);
        if constexpr (PLANES == 2) v |= (int)lds_u8(sp + SCB) << 8;
        sb[j] = v;
    };
    // FP4: the K half (0: chunk g, 1: chunk 4+g) of a fragment as the instruction's operand
    auto half_of = [](const i32x8& f, int h) {
        const u32x4 x = h == 0 ? u32x4{(unsigned)f[0], (unsigned)f[1], (unsigned)f[2], (unsigned)f[3]}
                               : u32x4{(unsigned)f[4], (unsigned)f[5], (unsigned)f[6], (unsigned)f[7]};
        return fp4_operand(x);
    };

    // Prologue: tile 0 whole; tile 1 is loaded in tile 0's iteration (after its
    // barrier), so it is never in flight with tile 0's loads.
    {
        const TileRes r0 = tile_res(0);
#pragma unroll
        for (int i = 0; i < L; ++i) issue_one(r0, i);
    }
    wait_vmcnt<0>();
    __syncthreads();
    // tile 1 goes to slot 1 before the loop (slot 1 is free)
    {
        const TileRes r1 = tile_res(1);
#pragma unroll
        for (int i = 0; i < L; ++i) issue_one(r1, i);
    }
#pragma unroll
    for (int i = 0; i < NBUF; ++i) read_a(smem, i);
#pragma unroll
    for (int j = 0; j < FN; ++j) read_b(smem, j);

    for (int t = 0; t < TP; ++t) {
        const char* cur = smem + (t & 1) * STAGE;
        const char* nxt = smem + ((t + 1) & 1) * STAGE;
        const TileRes rl = tile_res(t + 2);         // loads issued after this tile's barrier
        __builtin_amdgcn_s_setprio(1);
        static_for<MI + 1>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if constexpr (m == BPOS) {
                // Every read of this tile's slot has been issued; once they have
                // returned and tile t+1 has landed (its loads are the only ones in
                // flight), the barrier publishes tile t+1 and frees this slot for
                // tile t+2.
                __builtin_amdgcn_s_setprio(0);
                wait_vmcnt_lgkm0<0>();
                __syncthreads();
                __builtin_amdgcn_s_setprio(1);
            }
            // The next tile's L loads, spread evenly over the MFMAs after the barrier
            // (measured on MI355X against one per MFMA: 2-3% faster, bit-identical).
            static_for<L>([&](auto kc) {
                constexpr int kq = decltype(kc)::value;
                if constexpr (m == BPOS + (kq * (MI - BPOS)) / L) issue_one(rl, kq);
            });
            // A fragment i is read before MFMA FN*i - LEAD (its buffer's previous
            // fragment, i - NBUF, has had its last use): fragments NBUF.. of this
            // tile, then fragments 0..NBUF-1 of the next one.
            if constexpr (m % FN == 0 && m >= FN) {
                constexpr int g = m / FN + NBUF - 1;           // A fragment index, counting on into the next tile
                if constexpr (g < FM) read_a(cur, g);
                else if (g < FM + NBUF) read_a(nxt, g - FM);
            }
            if constexpr (!FP4) {
                if constexpr (m > (FM - 1) * FN) read_b(nxt, m - (FM - 1) * FN - 1);   // after the last use of B fragment
            } else {
                // last uses in the last row block: fragments 0, 1 at step 2 (second half),
                // fragments 2, 3 at step 3
                if constexpr (m == (FM - 1) * FN + 3) { read_b(nxt, 0); read_b(nxt, 1); }
                if constexpr (m == MI) { read_b(nxt, 2); read_b(nxt, 3); }
            }
            if constexpr (m < MI) {
                constexpr int i = m / FN, q = m % FN;
                // B fragment first: the hardware tile is C's transpose (lane l holds
                // C[m0 + l%16][n0 + 4 (l/16) + e]).
                if constexpr (!FP4) {
                    acc[i][q] = mfma_scale16x16x128<FMT>(fb[q], fa[i % NBUF], acc[i][q], sb[q], sa[i % NBUF]);
                } else {
                    // steps q = 0, 1: first K half of (i, 2q), (i, 2q+1); q = 2, 3: second half of (i, 2q-4), (i, 2q-3)
                    constexpr int h = (2 * q) / FN, j0 = (2 * q) % FN;
                    static_assert(FN == 4, "two MFMAs per step over four B fragments");
                    acc[i][j0] = mfma_scale16x16x128<FMT, h>(half_of(fb[j0], h), half_of(fa[i % NBUF], h), acc[i][j0],
                                                             sb[j0], sa[i % NBUF]);
                    acc[i][j0 + 1] = mfma_scale16x16x128<FMT, h>(half_of(fb[j0 + 1], h), half_of(fa[i % NBUF], h),
                                                                 acc[i][j0 + 1], sb[j0 + 1], sa[i % NBUF]);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_setprio(0);
    }
    // No direct load may still be writing LDS when the workgroup ends (the last
    // iterations load zero-filled tiles past K into free slots).
    wait_vmcnt<0>();

    store_blocks<FM, FN>(p.C, p.M, p.N, p.c_dtype, p.c_vec != 0, p.c_vec8 != 0, p.relu != 0, p.clear_accum != 0, acc,
                         m0 + arow, n0 + bcol, lane);
}

}  // namespace tlg
