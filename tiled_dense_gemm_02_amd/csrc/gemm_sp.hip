// 2:4 structured-sparse GEMM, C = act(A W^T): the pages' T.gemm_sp (a "2:4
// structured sparse GEMM" that depends on the hardware's sparse matrix
// instructions, overview page, table of compute primitives).  W [N, K] holds at
// most two values in every group of four consecutive k and is given compressed
// (include/tlg.h states the format): Wv [N, K/2] values, two per group in order;
// Wm [N, K/8] bytes, group q's two 2-bit positions at bits 4(q%2) and 4(q%2)+2 of
// byte q/2.  On gfx950 this is v_smfmac_f32_16x16x64_{f16,bf16}.
//
// Instruction layout (measured on MI355X with one-hot and random probes): the
// sparse operand's lane l holds row l%16 and, with g = l/16, the eight stored
// values of k = 16g .. 16g+15 (value v belongs to the group of k = 16g + 4(v/2)
// and sits at position (idx >> 2v) & 3 of it); the dense operand's lane l holds
// column l%16 with k = 8g .. 8g+7 in elements 0..7 and k = 32+8g .. 32+8g+7 in
// elements 8..15; the result tile has the dense instructions' layout.  So the
// compressed weights of a lane are 16 consecutive bytes of Wv and its index word
// is 16 consecutive bits of Wm -- the format above is the instruction's own --
// and the dense fragment is chunks g and 4+g of a 64-wide row of A, exactly as
// in the block-scaled kernel.
//
// The tile program is the block-scaled kernel's: 256 x 256 output tiles, a K
// loop over 64-wide K tiles, a three-slot LDS ring filled by direct loads, 8 waves
// of 128 x 64 outputs, 32 sparse MFMAs per wave and K tile issued row-block-major
// with the eight A fragments rotating through four buffers and the four weight
// fragments resident, the ring barrier after MFMA 20, then the loads of the
// tile three ahead, spread over the MFMAs after it.  A K tile takes 50 KiB (A 32, values 16,
// positions 2), so three slots fit in 160 KiB and two tiles stay in flight.
#include "gemm_lds.hpp"

namespace tlg {

namespace {

typedef _Float16 h16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 h16x16 __attribute__((ext_vector_type(16)));
typedef __bf16 b16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 b16x16 __attribute__((ext_vector_type(16)));
typedef int sp_i32x8 __attribute__((ext_vector_type(8)));

// 4-byte global->LDS direct load: lane l writes LDS bytes [lds + 4 l, lds + 4 l + 4).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma4_sp(i32x4 rsrc, uint32_t voff, uint32_t lds_addr)
{
    asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds"
                 :
                 : "v"(voff), "s"(rsrc), "s"(lds_addr)
                 : "memory", "m0");
}
#pragma clang diagnostic pop

template <int T>
__device__ inline f32x4 smfmac16x16x64(const u32x4& w, const sp_i32x8& a, f32x4 c, int idx)
{
    if constexpr (T == DT_F16)
        return __builtin_amdgcn_smfmac_f32_16x16x64_f16(__builtin_bit_cast(h16x8, w), __builtin_bit_cast(h16x16, a),
                                                        c, idx, 0, 0);
    else
        return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(__builtin_bit_cast(b16x8, w), __builtin_bit_cast(b16x16, a),
                                                         c, idx, 0, 0);
}

}  // namespace

template <int T>
__global__ void __launch_bounds__(512) gemm_sp_kernel(SpParams p)
{
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int WAVES_M = 2, WAVES_N = 4, NW = 8;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N, FM = WTM / 16, FN = WTN / 16;
    using OpA = LdsOperand<BM, BK, true, NW>;
    constexpr int WVB = BN * BK;                       // compressed weight bytes per tile (BK/2 values of 2 bytes)
    constexpr int WMB = BN * BK / 8;                   // metadata bytes per tile
    constexpr int STAGE = OpA::BYTES + WVB + WMB;
    constexpr int LW = WVB / (NW * 1024);              // 16-byte weight loads per wave per tile
    constexpr int L = OpA::L + LW + 1;                 // plus one 4-byte metadata load
    constexpr int MI = FM * FN;                        // MFMAs per tile
    constexpr int NBUF = 4;
    constexpr int LEAD = 3 * FN;
    constexpr int BPOS = FN * FM - LEAD;
    constexpr int S = 3;                               // ring slots
    static_assert(FM % NBUF == 0 && LEAD == FN * (NBUF - 1), "rotation of the A fragment buffers");
    static_assert(S * STAGE <= 160 * 1024, "the ring must fit in 160 KiB");
    static_assert((S - 2) * L < 64, "vmcnt range");
    static_assert(MI - BPOS >= L, "all loads of a tile fit after the barrier, at most one per MFMA");
    static_assert(WMB == NW * 256 && LW >= 1, "one 4-byte metadata load per wave covers 32 rows");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;
    const int wm = wave / WAVES_N, wn = wave % WAVES_N;

    int tm, tn;
    tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int K = p.K;
    const int TP = K / BK;

    OpA opa;
    opa.init(p.A, m0, p.M, K, lane, wave);
    const uint32_t lds0 = lds_addr_of(smem);

    // Weight values: row r of a tile is 64 bytes (four 16-byte chunks), chunk c at
    // position c ^ ((r/4) % 4).  Load i of a wave fills rows 16 q .. 16 q + 15 with
    // q = i * NW + wave; lane -> row 16 q + lane/4, position lane%4.
    const int wrows = p.N - n0;
    const uint32_t wld = (uint32_t)K;                  // bytes per compressed row
    const i32x4 rwv = rsrc_words((const char*)p.Wv + (uint64_t)n0 * wld, wrows > 0 ? (uint64_t)wrows * wld : 0);
    // Metadata: 8 bytes per row and tile, row-major; wave w loads rows 32 w .. 32 w + 31
    // (lane -> row 32 w + lane/2, dword lane%2).
    const uint32_t mld = (uint32_t)K / 8u;
    const i32x4 rwm = rsrc_words((const char*)p.Wm + (uint64_t)n0 * mld, wrows > 0 ? (uint64_t)wrows * mld : 0);
    const int mrow = wave * 32 + lane / 2;
    const uint32_t moff0 = mrow < wrows ? (uint32_t)mrow * mld + (uint32_t)(lane & 1) * 4u : kOOB;

    struct TileRes {
        i32x4 ra;
        int k0;
        uint32_t slot;
        bool ok;
    };
    auto tile_res = [&](int t) {
        TileRes r;
        r.k0 = t * BK;
        r.ra = opa.rsrc(r.k0);
        r.slot = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)((t % S) * STAGE));
        r.ok = t < TP;
        return r;
    };
    auto issue_one = [&](const TileRes& r, int i) {
        if (i < OpA::L) {
            dma16(r.ra, opa.voff(i, r.k0, K),
                  __builtin_amdgcn_readfirstlane(r.slot + (uint32_t)wave * 1024u + (uint32_t)(i * NW * 1024)));
        } else if (i < OpA::L + LW) {
            const int q = (i - OpA::L) * NW + wave;
            const int row = q * 16 + lane / 4;
            const int c = (lane & 3) ^ ((row >> 2) & 3);
            const uint32_t off = (r.ok && row < wrows) ? (uint32_t)row * wld + (uint32_t)r.k0 + (uint32_t)c * 16u : kOOB;
            dma16(rwv, off, __builtin_amdgcn_readfirstlane(r.slot + (uint32_t)(OpA::BYTES + q * 1024)));
        } else {
            const uint32_t off = (r.ok && moff0 != kOOB) ? moff0 + (uint32_t)(r.k0 / 8) : kOOB;
            dma4_sp(rwm, off, __builtin_amdgcn_readfirstlane(r.slot + (uint32_t)(OpA::BYTES + WVB + wave * 256)));
        }
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int arow = wm * WTM, bcol = wn * WTN;
    sp_i32x8 fa[NBUF];
    u32x4 fw[FN];
    int fi[FN];
    auto read_a = [&](const char* slot, int i) {
        const u32x4 lo = opa.frag(slot, arow + i * 16, 0, lane), hi = opa.frag(slot, arow + i * 16, 1, lane);
        fa[i % NBUF] = sp_i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    };
    auto read_w = [&](const char* slot, int j) {
        const int row = bcol + j * 16 + r16;
        fw[j] = *(const u32x4*)(slot + OpA::BYTES + row * 64 + ((g ^ ((row >> 2) & 3)) << 4));
        fi[j] = (int)*(const unsigned short*)(slot + OpA::BYTES + WVB + row * 8 + 2 * g);
    };

    // Prologue: tiles 0 .. S-2 in flight; once tile 0 has landed, tile S-1 too.
#pragma unroll
    for (int t = 0; t < S - 1; ++t) {
        const TileRes r0 = tile_res(t);
#pragma unroll
        for (int i = 0; i < L; ++i) issue_one(r0, i);
    }
    wait_vmcnt<(S - 2) * L>();
    __syncthreads();
    {
        const TileRes r1 = tile_res(S - 1);
#pragma unroll
        for (int i = 0; i < L; ++i) issue_one(r1, i);
    }
#pragma unroll
    for (int i = 0; i < NBUF; ++i) read_a(smem, i);
#pragma unroll
    for (int j = 0; j < FN; ++j) read_w(smem, j);

    for (int t = 0; t < TP; ++t) {
        const char* cur = smem + (t % S) * STAGE;
        const char* nxt = smem + ((t + 1) % S) * STAGE;
        const TileRes rl = tile_res(t + S);
        __builtin_amdgcn_s_setprio(1);
        static_for<MI + 1>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if constexpr (m == BPOS) {
                // Every read of this tile's slot has been issued; once they have
                // returned and tile t+1 has landed (tiles up to t+S-1 may still be
                // in flight), the barrier publishes tile t+1 and frees this slot
                // for tile t+S.
                __builtin_amdgcn_s_setprio(0);
                wait_vmcnt_lgkm0<(S - 2) * L>();
                __syncthreads();
                __builtin_amdgcn_s_setprio(1);
            }
            // The next tile's L loads, spread evenly over the MFMAs after the barrier
            // (measured on MI355X against one per MFMA: 2-3% faster, bit-identical).
            static_for<L>([&](auto kc) {
                constexpr int kq = decltype(kc)::value;
                if constexpr (m == BPOS + (kq * (MI - BPOS)) / L) issue_one(rl, kq);
            });
            if constexpr (m % FN == 0 && m >= FN) {
                constexpr int gi = m / FN + NBUF - 1;
                if constexpr (gi < FM) read_a(cur, gi);
                else if (gi < FM + NBUF) read_a(nxt, gi - FM);
            }
            if constexpr (m > (FM - 1) * FN) read_w(nxt, m - (FM - 1) * FN - 1);
            if constexpr (m < MI) {
                constexpr int i = m / FN, j = m % FN;
                // Weight fragment first: lane l holds C[m0 + l%16][n0 + 4(l/16) + e].
                acc[i][j] = smfmac16x16x64<T>(fw[j], fa[i % NBUF], acc[i][j], fi[j]);
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        __builtin_amdgcn_s_setprio(0);
    }
    wait_vmcnt<0>();

    store_blocks<FM, FN>(p.C, p.M, p.N, p.c_dtype, p.c_vec != 0, p.c_vec8 != 0, p.relu != 0, true, acc, m0 + arow,
                         n0 + bcol, lane);
}

hipError_t launch_sp(const SpParams& p, int ab_dtype, hipStream_t stream)
{
    const dim3 grid((unsigned)(p.tiles_m * p.tiles_n)), block(512);
    if (ab_dtype == DT_F16)
        hipLaunchKernelGGL(gemm_sp_kernel<DT_F16>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(gemm_sp_kernel<DT_BF16>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace tlg
