// Attention forward with online softmax (FlashAttention), on the same building
// blocks as the GEMM kernels: the tile program of the handbook page "TileLang: a
// tile language one level below Triton", section "FlashAttention: online softmax
// as tile code".  One workgroup owns a block of queries of one (batch, head),
// walks the keys in blocks, and per block
//   scores = Q K^T (fp32), scaled by scale * log2(e), masked;
//   m_new  = max(m_old, row max of the block);   alpha = exp2(m_old - m_new);
//   P      = exp2(scores - m_new), rounded to the operand type;
//   l      = l * alpha + row sum of P;   O = O * alpha + P V;
// and finally O / l is rounded to the operand type and stored.  The causal rule
// is the page's: the query at position i sees the keys at positions j <= i; key
// blocks wholly to the right of a query block are never visited.
//
// Tensors Q, K, V and O are [batch, seq, heads, dim], dim 64 or 128, fp16 or
// bf16, 16-byte aligned; element (b, t, h, d) sits at ((b*S + t)*H + h)*D + d.
//
// gfx950 mapping.
//   - Workgroup: 4 waves, 128 queries (32 per wave: two 16-row MFMA tiles), or
//     64 queries (16 per wave, one row tile) for grids that would not give every
//     CU a workgroup: each wave's chain per key block (scores, softmax, P V) is
//     then half as long, and twice the workgroups share the work.  Q fragments
//     are loaded once into registers.  Key blocks of 64 keys (K and V tiles)
//     stream through a two-slot LDS ring filled by global->LDS direct loads; the
//     loads of block j+1 are in flight while block j is computed.
//   - Both products run on v_mfma_f32_16x16x32 with the key-side operand first,
//     so the score tile lands as S[q][key] with lane l holding query l%16 and
//     keys 4(l/16)..+3 of each 16-key tile.  That is already the A-operand
//     layout of the P V product once the keys of two adjacent 16-key tiles are
//     taken as one 32-wide K step in the order {4g..4g+3, 16+4g..16+4g+3}
//     (g = l/16); the V fragment is read in the same key order, so P never
//     leaves the registers.  Row statistics need a reduction over the four lanes
//     that share a query (lanes l, l^16, l^32, l^48) only for the maximum; the
//     row sum is kept per lane and reduced once at the end.
//   - LDS layouts (row = one key, 2*dim bytes, 16-byte chunks):
//       K: chunk c of row r at c ^ ((r / RPB) % CH)  -- a fragment read (16 rows
//          of one chunk per 16 lanes) touches every bank once;
//       V: chunk c of row r at c ^ 2((r / RPB) % (CH/2)) -- the transposing
//          reads (ds_read_b64_tr_b16: 16 consecutive rows, 32 bytes each) spread
//          over all banks; the XOR is even, so the two chunks a read needs stay
//          adjacent;
//     with CH = dim/8 chunks per row and RPB = rows per 256 bytes.
//   - Grid: (query blocks) x heads x batch workgroups.  The query blocks of one
//     (batch, head) go to one XCD (its L2 then holds that head's K and V), the
//     causal ones heaviest first.
#pragma once

#include "gemm_lds.hpp"

namespace tlg {

template <int D>
struct AttnLds {
    static constexpr int RB = 2 * D;                    // bytes per key row
    static constexpr int CH = D / 8;                    // 16-byte chunks per row
    static constexpr int RPB = RB >= 256 ? 1 : 256 / RB;
    static constexpr int RPK = 1024 / RB;               // rows per 1 KiB direct-load block
    __device__ static int swz_k(int r) { return (r / RPB) % CH; }
    __device__ static int swz_v(int r) { return 2 * ((r / RPB) % (CH / 2)); }
};

// Extremes over the lanes l, l^16, l^32 and l^48 (one score row's four key
// groups).  gfx950's row swaps do it in registers: with the value in both
// operands, v_permlane16_swap leaves lane l with x[l] and x[l^16] in its two
// results, v_permlane32_swap with x[l] and x[l^32].  (A lane shuffle would be a
// round trip through LDS, waited for twice per row tile and key block.)
__device__ inline u32x2 swap16(float x)
{
    return __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
}
__device__ inline u32x2 swap32(float x)
{
    return __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
}

__device__ inline float wave_max4(float x)
{
    const u32x2 a = swap16(x);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const u32x2 b = swap32(x);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline float wave_min4(float x)
{
    const u32x2 a = swap16(x);
    x = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const u32x2 b = swap32(x);
    return fminf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest even in the operand type, packed (one
// v_cvt_pk_{f16,bf16}_f32 on gfx950).
template <int T>
__device__ inline uint32_t pack_op(float a, float b)
{
    const f32x2 v = {a, b};
    if constexpr (T == DT_F16)
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
    else
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

template <int T>
__device__ inline float round_op(float x, uint32_t& bits)
{
    if constexpr (T == DT_F16) {
        const _Float16 h = (_Float16)x;
        bits = __builtin_bit_cast(uint16_t, h);
        return (float)h;
    } else {
        const __bf16 h = (__bf16)x;
        bits = __builtin_bit_cast(uint16_t, h);
        return (float)h;
    }
}

// NEG: the softmax scale is negative (the row maximum of the scaled scores is
// then the scale times the row minimum of the raw scores).  RT: 16-row tiles of
// queries per wave (2: 128 queries per workgroup, 1: 64).
template <int D, int T, bool CAUSAL, bool NEG, int RT>
__global__ void __launch_bounds__(256, 2) attn_fwd_kernel(AttnParams p)
{
    constexpr int NW = 4, WROWS = 16 * RT, BM = NW * WROWS, BN = 64;
    static_assert(RT == 1 || RT == 2, "one or two 16-row query tiles per wave");
    using Lay = AttnLds<D>;
    constexpr int RB = Lay::RB, CH = Lay::CH, RPK = Lay::RPK;
    constexpr int TILE = BN * RB;                 // bytes of one K (or V) tile
    constexpr int SLOT = 2 * TILE;
    constexpr int LK = TILE / (NW * 1024);        // direct loads per lane per tile
    constexpr int KS = D / 32;                    // MFMA K steps of the score product
    constexpr int DT = D / 16;                    // 16-wide output column tiles
    static_assert(TILE % (NW * 1024) == 0 && LK >= 1, "tile must split into 1 KiB blocks per wave");
    static_assert(2 * SLOT <= 64 * 1024, "two slots per workgroup, two workgroups per CU");

    __shared__ __attribute__((aligned(1024))) char smem[2 * SLOT];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, r16 = lane & 15;

    // Work item: (batch, head, query block).
    const int total = p.nqb * p.H * p.B;
    int id = blockIdx.x;
    if (total % kXcds == 0) id = (id % kXcds) * (total / kXcds) + id / kXcds;
    const int bh = id / p.nqb;
    const int qi = id - bh * p.nqb;
    const int qb = CAUSAL ? p.nqb - 1 - qi : qi;
    const int b = bh / p.H, h = bh - b * p.H;
    const int S = p.S;
    const int q0 = qb * BM;
    const uint32_t stride = (uint32_t)p.H * (uint32_t)RB;            // bytes between consecutive positions
    const uint64_t head_off = ((uint64_t)b * (uint64_t)S * (uint64_t)p.H + (uint64_t)h) * (uint64_t)RB;
    const uint64_t head_bytes = (uint64_t)(S - 1) * stride + RB;    // up to the end of position S-1

    const int q_last = min(q0 + BM, S) - 1;
    const int nkb = CAUSAL ? q_last / BN + 1 : (S + BN - 1) / BN;

    // Q fragments of this wave's rows (rows past S read as zeros).
    u32x4 qf[RT][KS];
    {
        const __amdgpu_buffer_rsrc_t rq = make_rsrc((const char*)p.Q + head_off, head_bytes);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int q = q0 + wave * WROWS + rt * 16 + r16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const uint32_t off = q < S ? (uint32_t)q * stride + (uint32_t)(ks * 4 + g) * 16u : kOOB;
                qf[rt][ks] = buf_load16(rq, off);
            }
        }
    }

    // Direct loads: load i of this lane fills row r0 + 4 i RPK of a tile, chunk
    // position lane % CH; the swizzle of that row is the same for every i.  The
    // block's first key goes into the buffer resource, so the lane offsets do not
    // change from block to block; the resource ends with position S-1's row of
    // this head, so keys at or past S (whose rows start at least a row stride
    // further on) read zeros.
    const int r0 = wave * RPK + lane / CH;
    const int ck = (lane % CH) ^ Lay::swz_k(r0);
    const int cv = (lane % CH) ^ Lay::swz_v(r0);
    uint32_t offk[LK], offv[LK];
#pragma unroll
    for (int i = 0; i < LK; ++i) {
        const uint32_t base = (uint32_t)(r0 + i * NW * RPK) * stride;
        offk[i] = base + (uint32_t)ck * 16u;
        offv[i] = base + (uint32_t)cv * 16u;
    }
    const char* kbase = (const char*)p.K + head_off;
    const char* vbase = (const char*)p.V + head_off;
    const uint32_t lds0 = lds_addr_of(smem);
    auto issue = [&](int kb) {
        const uint32_t slot = lds0 + (uint32_t)((kb & 1) * SLOT) + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 1024u;
        const uint64_t ob = (uint64_t)kb * BN * stride;   // < head_bytes: block kb starts before S
        const i32x4 rk = rsrc_words(kbase + ob, head_bytes - ob);
        const i32x4 rv = rsrc_words(vbase + ob, head_bytes - ob);
#pragma unroll
        for (int i = 0; i < LK; ++i) {
            dma16(rk, offk[i], __builtin_amdgcn_readfirstlane(slot + (uint32_t)(i * NW * 1024)));
            dma16(rv, offv[i], __builtin_amdgcn_readfirstlane(slot + (uint32_t)(TILE + i * NW * 1024)));
        }
    };

    f32x4 oacc[RT][DT];
    f32x4 lacc[RT];                       // row sums of P (all four entries equal)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        lacc[rt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[rt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float m_run[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) m_run[rt] = -INFINITY;
    // All-ones operand: P times it gives the row sums of the rounded P on the
    // matrix cores, exactly as the page sums its fp16 probability tile.
    const uint32_t one2 = T == DT_F16 ? 0x3C003C00u : 0x3F803F80u;
    const u32x4 ones = u32x4{one2, one2, one2, one2};
    const float c = p.scale_log2;
    constexpr float SENT = NEG ? INFINITY : -INFINITY;   // masked raw score, ignored by the row extreme
    constexpr float kSlack = 8.0f;                        // P <= 2^8 between moves of the reference

    const int wq0 = q0 + wave * WROWS;          // first query row of this wave
    issue(0);
    wait_vmcnt<0>();
    __syncthreads();

    for (int kb = 0; kb < nkb; ++kb) {
        if (kb + 1 < nkb) issue(kb + 1);
        const int kb0 = kb * BN;
        // Under the causal rule a wave whose rows all precede the block sees none of it.
        const bool active = !CAUSAL || kb0 <= wq0 + WROWS - 1;
        if (active) {
            const char* kt_base = smem + (kb & 1) * SLOT;
            const char* vt_base = kt_base + TILE;

            f32x4 sacc[RT][4];
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) sacc[rt][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
            // K fragments of step ks+1 are read while step ks's 8 MFMAs run (two
            // register buffers; the fences keep the compiler from moving a read
            // next to its first use, where its LDS latency would be exposed).
            u32x4 kf[2][4];
            auto read_k = [&](int ks, u32x4* dst) {
#pragma unroll
                for (int kt = 0; kt < 4; ++kt) {
                    const int row = kt * 16 + r16;
                    const int cc = ks * 4 + g;
                    dst[kt] = *(const u32x4*)(kt_base + row * RB + ((cc ^ Lay::swz_k(row)) << 4));
                }
            };
            read_k(0, kf[0]);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if (ks + 1 < KS) read_k(ks + 1, kf[(ks + 1) & 1]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt) sacc[rt][kt] = mfma16x16x32<T>(kf[ks & 1][kt], qf[rt][ks], sacc[rt][kt]);
                __builtin_amdgcn_sched_barrier(0);
            }

            const bool need_mask = (kb0 + BN > S) || (CAUSAL && kb0 + BN - 1 > wq0);
            u32x4 pf[RT][2];
            float alpha[RT];
            bool rescale = false;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int q = wq0 + rt * 16 + r16;
                // Score t of this lane is key kb0 + 4g + 16(t/4) + t%4; it is masked
                // when that key lies past the row's last allowed key.
                const int lim = (CAUSAL ? min(q, S - 1) : S - 1) - (kb0 + 4 * g);
                float sv[16];
#pragma unroll
                for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                    for (int e = 0; e < 4; ++e) sv[kt * 4 + e] = sacc[rt][kt][e];
                if (need_mask) {          // uniform: only the diagonal and the last key block
#pragma unroll
                    for (int t = 0; t < 16; ++t) sv[t] = (t >> 2) * 16 + (t & 3) > lim ? SENT : sv[t];
                }
                // Row maximum of the scaled scores, from the raw scores: the scale
                // is applied once per row, and once per score inside the FMA below.
                float mloc = sv[0];
#pragma unroll
                for (int t = 1; t < 16; ++t) mloc = NEG ? fminf(mloc, sv[t]) : fmaxf(mloc, sv[t]);
                mloc = NEG ? wave_min4(mloc) : wave_max4(mloc);
                const float mblk = mloc == SENT ? -INFINITY : mloc * c;
                // The row's reference maximum moves only when the block's maximum
                // exceeds it by more than kSlack (log2 units, from -inf always).
                // Until then P = 2^(s*c - reference) stays at or below 2^kSlack,
                // well inside the operand type, and O and l keep the same
                // reference, so O / l is unchanged; O is rescaled far less often.
                const bool move = mblk > m_run[rt] + kSlack;
                const float m_ref = move ? mblk : m_run[rt];
                const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
                alpha[rt] = __builtin_amdgcn_exp2f(m_run[rt] - m_use);
                rescale = rescale || move;
                m_run[rt] = m_ref;
                float pv[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) pv[t] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[t], c, -m_use));
                if (need_mask) {
#pragma unroll
                    for (int t = 0; t < 16; ++t) pv[t] = (t >> 2) * 16 + (t & 3) > lim ? 0.f : pv[t];
                }
                // K step kk of the P V product: keys {4g..4g+3} of tile 2kk, then of tile 2kk+1.
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
                    pf[rt][kk] = u32x4{pack_op<T>(pv[8 * kk + 0], pv[8 * kk + 1]), pack_op<T>(pv[8 * kk + 2], pv[8 * kk + 3]),
                                       pack_op<T>(pv[8 * kk + 4], pv[8 * kk + 5]), pack_op<T>(pv[8 * kk + 6], pv[8 * kk + 7])};
            }
            // O and the row sums are rescaled only when some row's reference
            // maximum moved (alpha is exactly 1 for the others).
            if (__any(rescale)) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) lacc[rt][e] *= alpha[rt];
#pragma unroll
                    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                        for (int e = 0; e < 4; ++e) oacc[rt][dt][e] *= alpha[rt];
                }
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt)
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) lacc[rt] = mfma16x16x32<T>(ones, pf[rt][kk], lacc[rt]);

            // V fragments of output tile dt+VPD are read while tile dt's 4 MFMAs
            // run (a ring of VPD+1 register buffers, fenced as above).
            constexpr int VPD = D == 128 ? 2 : 1;
            u32x4 vfr[VPD + 1][2];
            auto read_v = [&](int dt, u32x4* dst) {
                const int sx = r16;
                const int chunk = 2 * dt + ((sx & 3) >> 1);
                const int half = (sx & 1) * 8;
#pragma unroll
                for (int kk = 0; kk < 2; ++kk) {
                    const int klo = kk * 32 + 4 * g + (sx >> 2), khi = klo + 16;
                    const u32x2 lo = lds_read_tr16(vt_base + klo * RB + ((chunk ^ Lay::swz_v(klo)) << 4) + half);
                    const u32x2 hi = lds_read_tr16(vt_base + khi * RB + ((chunk ^ Lay::swz_v(khi)) << 4) + half);
                    dst[kk] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                }
            };
#pragma unroll
            for (int dt = 0; dt < VPD; ++dt) read_v(dt, vfr[dt]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                if (dt + VPD < DT) read_v(dt + VPD, vfr[(dt + VPD) % (VPD + 1)]);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                    for (int rt = 0; rt < RT; ++rt)
                        oacc[rt][dt] = mfma16x16x32<T>(vfr[dt % (VPD + 1)][kk], pf[rt][kk], oacc[rt][dt]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // The next block has landed (this lane's loads) and every wave is done
        // with this slot (the barrier), so the slot can be refilled.
        wait_vmcnt<0>();
        __syncthreads();
    }

    // Epilogue: O / l, rounded to the operand type.  A lane holds four consecutive
    // dims of each 16-dim block; pairs of blocks go out as one 16-byte store per
    // lane (store_pair16: 64 contiguous bytes of each row per instruction).  O and
    // its rows are 16-byte aligned (the entry point checks O; a row is 128 or 256
    // bytes of a head).
    static_assert(DT % 2 == 0, "pairs of 16-dim blocks");
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
        const int q = wq0 + rt * 16 + r16;
        const float inv = 1.0f / lacc[rt][0];
        if (q >= S) continue;
        uint16_t* orow = (uint16_t*)((char*)p.O + head_off + (uint64_t)q * stride);
#pragma unroll
        for (int dp = 0; dp < DT / 2; ++dp) {
            float v[4], w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = oacc[rt][2 * dp][e] * inv;
                w[e] = oacc[rt][2 * dp + 1][e] * inv;
            }
            store_pair16(orow + dp * 32, T, lane, v, w);
        }
    }
}

}  // namespace tlg
