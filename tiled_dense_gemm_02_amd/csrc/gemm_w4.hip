// Dequant GEMM with 4-bit weights, C[M x N] = act(A W^T): the "dequant GEMM" of
// the representative-operators table on the overview page (load packed
// weights, apply scale and zero point, convert, then multiply), shaped for
// decoding: few rows of A, a long stream of weights.
//
// Format (include/tlg.h states it in full): W is N x K unsigned 4-bit codes,
// [N, K/2] bytes; the eight codes of k = 8w .. 8w+7 of a row form one
// little-endian 32-bit word with the even k in the low half-word (nibbles 0..3)
// and the odd k in the high half-word (nibbles 4..7).  Per row and group of G
// consecutive k there is a scale s (operand dtype) and a zero point z (uint8);
// the weight is the operand-type value nearest to (q - z) * s.
//
// gfx950 mapping.  A workgroup owns 16 rows x 64 columns of C and streams the
// 64 packed weight rows once, like the fp16 skinny kernel, through an LDS ring
// of three 32 KiB stages filled by 1 KiB direct loads: a stage holds 512 of K,
// i.e. 256 bytes of each weight row and 1 KiB of each A row.  The workgroup's
// scales and zero points are gathered into an LDS table (one dword per group and
// row) while the first stages load; the table takes the other 64 KiB of the
// 160 KiB.
// The sixteen waves (four per SIMD, to hide the latency of each wave's chain of
// LDS read, dequantization and MFMA) take different 32-wide K steps of a stage.  For an MFMA
// 16x16x32 weight fragment a lane needs eight consecutive codes of one row --
// exactly one packed dword -- which it turns into four operand pairs:
//   fp16: x = (d >> 4i) & 0x000F000F | 0x64006400 is the pair (1024 + q0, 1024 + q1)
//         in fp16; x - (1024 + z) is q - z exactly; one packed fp16 multiply by s
//         rounds (q - z) * s to nearest even;
//   bf16: 2^23 + q built the same way in fp32, minus 2^23 + z, times s is exact in
//         fp32; v_cvt_pk_bf16_f32 rounds the pair to nearest even.
// The per-wave partial tiles are summed through LDS in a fixed order, then the
// epilogue (ReLU, conversion, guarded stores) runs.
#include "gemm_lds.hpp"

namespace tlg {

namespace {

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// mask (0x000F000F, in an SGPR) and magic (0x64006400, in a VGPR) come in as
// opaque values: with literal constants the compiler cannot fuse the mask and
// the or into one v_and_or_b32 (a VOP3 instruction takes no literal on gfx950).
// e is the table entry of the fragment's row and group: for fp16 the fp16 value
// 1024 + z in the low half and s in the high half (the packed subtract and
// multiply read each half for both lanes through their operand selects); for
// bf16, z in the low half and s in the high half.
template <int T>
__device__ inline u32x4 dequant8(uint32_t d, uint32_t e, uint32_t mask, uint32_t magic)
{
    u32x4 w;
    if constexpr (T == DT_F16) {
        const h16x2 ev = __builtin_bit_cast(h16x2, e);
        const h16x2 mz = ev.xx, s2 = ev.yy;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const h16x2 x = __builtin_bit_cast(h16x2, ((d >> (4 * i)) & mask) | magic);
            w[i] = __builtin_bit_cast(uint32_t, (x - mz) * s2);
        }
    } else {
        const float zf = (float)(e & 0xffffu) + 8388608.0f;
        const float s = __builtin_bit_cast(float, e & 0xffff0000u);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float lo = __builtin_bit_cast(float, 0x4b000000u | ((d >> (4 * i)) & 15u)) - zf;
            const float hi = __builtin_bit_cast(float, 0x4b000000u | ((d >> (16 + 4 * i)) & 15u)) - zf;
            const f32x2 v = {lo * s, hi * s};
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
        }
    }
    return w;
}

}  // namespace

// S: ring slots (S-1 stages in flight) of KST-wide stages; the scale / zero table
// gets the rest of the 160 KiB.
template <int T_IN, int S, int KST>
__global__ void __launch_bounds__(kW4Threads) gemm_w4_kernel(W4Params p)
{
    constexpr int WAVES = kW4Threads / 64, MR = 16, NB = kW4NB;
    constexpr int BRB = KST / 2;                 // bytes of a weight row per stage
    constexpr int ARB = KST * 2;                 // bytes of an A row per stage
    constexpr int BCH = BRB / 16;                // 16-byte chunks of a weight row per stage
    constexpr int BBYTES = NB * BRB, ABYTES = MR * ARB;
    constexpr int STAGE = BBYTES + ABYTES;
    constexpr int BRPL = 1024 / BRB;             // weight rows per 1 KiB direct load
    constexpr int APL = ARB / 1024;              // 1 KiB direct loads per A row
    constexpr int BL = BBYTES / 1024, AL = ABYTES / 1024;
    constexpr int LPW = (BL + AL) / WAVES;       // direct loads per wave per stage
    constexpr int NS = NB / 16;                  // 16-column MFMA tiles
    constexpr int KSTEPS = KST / 32, SPW = KSTEPS / WAVES;
    static_assert(BRB >= 256 && BRB <= 1024 && ARB >= 1024 && BL % WAVES == 0 && AL % WAVES == 0, "stage layout");
    static_assert(KSTEPS % WAVES == 0 && SPW >= 1, "every wave takes whole K steps of a stage");
    constexpr int TABLE = 160 * 1024 - S * STAGE;
    static_assert(S >= 2, "at least one stage in flight");
    static_assert(TABLE >= 16 * 1024 && TABLE <= kW4TableBytes, "ring and table must fit in 160 KiB");
    static_assert(WAVES * NS * 4 * 64 * 4 <= S * STAGE, "reduction area reuses the ring");

    __shared__ __attribute__((aligned(1024))) char smem[S * STAGE];
    // Scale / zero table, [group][row of the workgroup], row r of group gi at
    // gi * NB + (r ^ (gi & 15)): the 16 rows a fragment reads at one group are a
    // permutation of 16 consecutive dwords (16 banks), and the gather below, whose
    // consecutive threads take consecutive groups of one row, writes 16 banks.
    __shared__ __attribute__((aligned(16))) uint32_t tab[TABLE / 4];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 4, r16 = lane & 15;
    const int m0 = blockIdx.y * MR, n0 = blockIdx.x * NB;
    const int K = p.K, G = p.G, KG = K / G;
    const int NST = (K + KST - 1) / KST;

    const uint32_t bld = (uint32_t)K / 2u, ald = (uint32_t)K * 2u;
    const char* b_base = (const char*)p.Wq + (uint64_t)n0 * bld;
    const char* a_base = (const char*)p.A + (uint64_t)m0 * ald;
    const uint64_t b_bytes = (uint64_t)(p.N - n0) * bld;
    const uint64_t a_bytes = (uint64_t)(p.M - m0) * ald;
    const uint32_t lds0 = lds_addr_of(smem);

    // Load q = i * WAVES + wave of a stage: q < BL fills weight rows q*BRPL ..
    // (lane -> row q*BRPL + lane/BCH, chunk position lane%BCH); otherwise 1 KiB of
    // A row (q-BL)/APL (lane -> chunk position ((q-BL)%APL)*64 + lane).  Chunk c of
    // row r sits at c ^ (r & 15).  A lane's offset inside the stage and the first k
    // of its chunk do not change from stage to stage; rows past M or N read zeros.
    uint32_t voff[LPW], kc[LPW];
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
        const int q = i * WAVES + wave;
        if (q < BL) {
            const int row = q * BRPL + lane / BCH;
            const int c = (lane % BCH) ^ (row & 15);
            voff[i] = n0 + row < p.N ? (uint32_t)row * bld + (uint32_t)c * 16u : kOOB;
            kc[i] = (uint32_t)c * 32u;
        } else {
            const int row = (q - BL) / APL;
            const int c = (((q - BL) % APL) * 64 + lane) ^ (row & 15);
            voff[i] = m0 + row < p.M ? (uint32_t)row * ald + (uint32_t)c * 16u : kOOB;
            kc[i] = (uint32_t)c * 8u;
        }
    }
    auto issue = [&](int st) {
        const int k0 = st * KST;
        const uint64_t ob = (uint64_t)st * BRB, oa = (uint64_t)st * ARB;
        const uint32_t slot = lds0 + (uint32_t)((st % S) * STAGE);
        // st < NST, so ob < K/2 <= b_bytes and oa < 2K <= a_bytes (n0 < N, m0 < M).
        const i32x4 rb = rsrc_words(b_base + ob, b_bytes - ob);
        const i32x4 ra = rsrc_words(a_base + oa, a_bytes - oa);
        if (k0 + KST <= K) {
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int q = i * WAVES + wave;
                if (q < BL)
                    dma16(rb, voff[i], __builtin_amdgcn_readfirstlane(slot + (uint32_t)(q * 1024)));
                else
                    dma16(ra, voff[i], __builtin_amdgcn_readfirstlane(slot + (uint32_t)(BBYTES + (q - BL) * 1024)));
            }
        } else {
            // The stage reaches past K: chunks at or past K read zeros.
#pragma unroll
            for (int i = 0; i < LPW; ++i) {
                const int q = i * WAVES + wave;
                const uint32_t off = k0 + (int)kc[i] < K ? voff[i] : kOOB;
                if (q < BL)
                    dma16(rb, off, __builtin_amdgcn_readfirstlane(slot + (uint32_t)(q * 1024)));
                else
                    dma16(ra, off, __builtin_amdgcn_readfirstlane(slot + (uint32_t)(BBYTES + (q - BL) * 1024)));
            }
        }
    };

    f32x4 acc[NS];
#pragma unroll
    for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t mask = __builtin_amdgcn_readfirstlane(p.nibble_mask);
    uint32_t magic;
    asm volatile("v_mov_b32 %0, 0x64006400" : "=v"(magic));

    // Stages 0 .. S-3 go out before the table gather, stage S-2 after the wait
    // below (the prologue then waits for one stage fewer; stage S-2 is first
    // needed S-2 stages later).
#pragma unroll
    for (int st = 0; st < S - 2; ++st)
        if (st < NST) issue(st);
    // Scale / zero table of this workgroup's rows (rows past N: zero weights).
    // Every gather is issued before the first is waited for: entry i of the table
    // is thread i % 1024's gather number i / 1024 (at most GMAX of them), read
    // through range-checked resources (entries past the rows' end read zeros).
    {
        constexpr int GMAX = (NB * kW4MaxGroups + WAVES * 64 - 1) / (WAVES * 64);
        const int nent = NB * KG;
        const int rows = min(NB, p.N - n0);
        const __amdgpu_buffer_rsrc_t rz = make_rsrc((const uint8_t*)p.Z + (uint64_t)n0 * KG, (uint64_t)rows * KG);
        const __amdgpu_buffer_rsrc_t rs = make_rsrc((const uint16_t*)p.S + (uint64_t)n0 * KG, (uint64_t)rows * KG * 2u);
        uint32_t zv[GMAX], sv[GMAX];
#pragma unroll
        for (int it = 0; it < GMAX; ++it) {
            const int i = (int)threadIdx.x + it * WAVES * 64;
            zv[it] = sv[it] = 0u;
            if (it * WAVES * 64 < nent) {
                // i = r * KG + gi is the entry's offset in both arrays (row-major [N, K/G]).
                const uint32_t off = i < nent ? (uint32_t)i : kOOB;
                zv[it] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(rz, off, 0, 0);
                sv[it] = buf_load2(rs, off == kOOB ? kOOB : off * 2u);
            }
        }
#pragma unroll
        for (int it = 0; it < GMAX; ++it) {
            const int i = (int)threadIdx.x + it * WAVES * 64;
            if (it * WAVES * 64 < nent) {
                // Keeps the use of the loaded values here, after every gather has gone out.
                asm volatile("" : "+v"(zv[it]), "+v"(sv[it]));
                if (i < nent) {
                    const int r = i / KG, gi = i - r * KG;
                    const uint32_t e =
                        n0 + r < p.N ? ((T_IN == DT_F16 ? 0x6400u + zv[it] : zv[it]) | (sv[it] << 16)) : 0u;
                    tab[gi * NB + (r ^ (gi & 15))] = e;
                }
            }
        }
    }
    // The gathers above overlap the first stages' direct loads.  They are waited
    // for here, together with everything issued before them: the ring's vmcnt
    // accounting below counts direct loads only.
    wait_vmcnt<0>();
    if (S - 2 < NST) issue(S - 2);

    // Per K step u of this wave: LDS offsets of its A and weight fragments inside
    // a slot, and its group index, advanced stage by stage (the quotient and
    // remainder of st * KST + ks * 32 by G).
    uint32_t aoff[SPW], woff[SPW];
    int gq[SPW], gr[SPW];
    const int kst_q = KST / G, kst_r = KST - kst_q * G;
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
        const int ks = wave * SPW + u;
        aoff[u] = (uint32_t)(BBYTES + r16 * ARB + (((ks * 4 + g) ^ r16) << 4));
        woff[u] = (uint32_t)(r16 * BRB + ((ks ^ r16) << 4) + 4 * g);
        gq[u] = (ks * 32) / G;
        gr[u] = ks * 32 - gq[u] * G;
    }

    for (int st = 0; st < NST; ++st) {
        // Stage st has landed once at most S-2 newer stages are in flight; the
        // barrier publishes every wave's part (and, the first time, the table)
        // and frees the slot refilled next.
        if (st + S - 2 < NST)
            wait_vmcnt<(S - 2) * LPW>();
        else
            wait_vmcnt<0>();
        __syncthreads();
        if (st + S - 1 < NST) issue(st + S - 1);
        const char* slot = smem + (st % S) * STAGE;
#pragma unroll
        for (int u = 0; u < SPW; ++u) {
            // K steps past the end of K read zeros from A and W (range-checked
            // loads); their group index is clamped so the table read stays inside.
            const int gi = min(gq[u], KG - 1);
            const uint32_t* trow = tab + gi * NB + (r16 ^ (gi & 15));
            const u32x4 af = *(const u32x4*)(slot + aoff[u]);
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                const uint32_t d = *(const uint32_t*)(slot + woff[u] + j * 16 * BRB);
                const u32x4 wf = dequant8<T_IN>(d, trow[j * 16], mask, magic);
                // Weight fragment first: acc[j][e] is C[m0 + lane%16][n0 + 16j + 4(lane/16) + e].
                acc[j] = mfma16x16x32<T_IN>(wf, af, acc[j]);
            }
            gq[u] += kst_q;
            gr[u] += kst_r;
            if (gr[u] >= G) { gr[u] -= G; ++gq[u]; }
        }
    }
    wait_vmcnt<0>();
    __syncthreads();

    float* red = (float*)smem;   // [WAVES][NS][4][64]
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((wave * NS + j) * 4 + e) * 64 + lane] = acc[j][e];
    __syncthreads();

    const int m = m0 + r16;
    for (int j = wave; j < NS; j += WAVES) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float s = red[(j * 4 + e) * 64 + lane];
#pragma unroll
            for (int w = 1; w < WAVES; ++w) s += red[((w * NS + j) * 4 + e) * 64 + lane];
            v[e] = s;
        }
        const int n = n0 + j * 16 + 4 * g;
        if (m >= p.M || n >= p.N) continue;
        const int count = min(4, p.N - n);
        const bool vec_ok = p.c_vec != 0 && count == 4;
        if (p.relu) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = relu(v[e]);
        }
        store_c4(p.C, p.c_dtype, (int64_t)m * p.N + n, vec_ok, v, count);
    }
}

template <int S, int KST>
static hipError_t launch_w4_s(const W4Params& p, int ab_dtype, hipStream_t stream)
{
    W4Params args = p;
    void* kargs[] = {&args};
    const dim3 grid((unsigned)((p.N + kW4NB - 1) / kW4NB), (unsigned)((p.M + 15) / 16)), block(kW4Threads);
    const void* fn = ab_dtype == DT_F16 ? (const void*)&gemm_w4_kernel<DT_F16, S, KST>
                                        : (const void*)&gemm_w4_kernel<DT_BF16, S, KST>;
    return hipLaunchKernel(fn, grid, block, kargs, 0, stream);
}

// Three slots of 512-wide stages leave a 64 KiB table (K/G <= 256).  On the
// 16 x 16384 x 8192 decode shape they beat two slots of 1024-wide stages (one
// stage in flight) and four of 512 (less work per wave between barriers).
hipError_t launch_w4(const W4Params& p, int ab_dtype, hipStream_t stream)
{
    static_assert(kW4NB * kW4MaxGroups * 4 <= kW4TableBytes, "table");
    return launch_w4_s<3, 512>(p, ab_dtype, stream);
}

}  // namespace tlg
