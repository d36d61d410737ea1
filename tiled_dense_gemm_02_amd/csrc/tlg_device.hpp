// Device-side building blocks shared by the gfx950 GEMM kernels:
// buffer-resource loads with hardware zero fill, the swizzled LDS tile layout,
// MFMA wrappers and the fp32 -> output conversions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tlg_internal.h"

namespace tlg {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Global loads through a buffer resource.  A lane whose element lies outside
// the matrix gets the offset kOOB, which is beyond the resource's record count:
// the hardware returns zeros and touches no memory.  This is the zero "safe
// value" for out-of-bounds source elements of a tile copy ("core primitives"
// chapter, section 4.2), applied to both operands so that padding contributes
// exact zeros to the sum.
// ---------------------------------------------------------------------------
constexpr uint32_t kOOB = 0x80000000u;
constexpr uint32_t kMaxRecords = 0x7fffffffu;
// Word 3 of a gfx9 buffer descriptor: DATA_FORMAT = 32-bit, everything else 0.
constexpr int kRsrcWord3 = 0x00020000;
// Cache-policy operand of the buffer builtins: sc1, device scope (coherent
// across the XCDs' separate L2 caches).
constexpr int kCoherentDevice = 16;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes_left)
{
    const uint32_t n = bytes_left > kMaxRecords ? kMaxRecords : (uint32_t)bytes_left;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, kRsrcWord3);
}

__device__ inline u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ inline uint32_t buf_load2(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS tile layout.  Every operand tile is stored as rows of its M (or N) index
// with 64 K-contiguous 16-bit elements per row (128 bytes = 8 chunks of 16 B).
// Chunk c of row r sits at chunk position c ^ swz(r).  swz is a permutation of
// 0..7 within every 8 consecutive rows (MFMA operand reads: 8 lanes read 8
// consecutive rows of one chunk) and also across rows 8 apart (the transposing
// writes: 8 lanes write rows r, r+8, ..., r+56 of one chunk), so both access
// patterns spread 8 lanes over all 32 banks.
// ---------------------------------------------------------------------------
constexpr int kBK = 64;            // K extent of one tile (elements)
constexpr int kRowElems = kBK;     // 16-bit elements per LDS row

__device__ __host__ constexpr int swz(int row) { return (row ^ (row >> 3)) & 7; }

__device__ inline int lds_elem(int row, int chunk) { return row * kRowElems + ((chunk ^ swz(row)) << 3); }

// ---------------------------------------------------------------------------
// MFMA wrappers (fp16 / bf16 operands, fp32 accumulator).
// ---------------------------------------------------------------------------
template <int T>
__device__ inline f32x16 mfma32x32x16(u32x4 a, u32x4 b, f32x16 c)
{
    if constexpr (T == DT_F16)
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

template <int T>
__device__ inline f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c)
{
    if constexpr (T == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Conversions (round to nearest even) and the epilogue activation.
// ---------------------------------------------------------------------------
__device__ inline uint32_t f32_to_f16_bits(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
__device__ inline uint32_t f32_to_bf16_bits(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ inline float f16_bits_to_f32(uint32_t b) { return (float)__builtin_bit_cast(_Float16, (uint16_t)b); }
__device__ inline float bf16_bits_to_f32(uint32_t b) { return __builtin_bit_cast(float, b << 16); }

// ReLU as max(x, 0) on the fp32 accumulator: non-positive (and NaN) -> +0.
__device__ inline float relu(float x) { return x > 0.0f ? x : 0.0f; }

// Read four consecutive outputs' prior values (clear_accum == 0), all in range.
__device__ inline void load_c4(const void* C, int c_dtype, int64_t idx, bool vec_ok, float* v,
                               int count)
{
    if (c_dtype == DT_F32) {
        const float* c = (const float*)C + idx;
        if (vec_ok) {
            f32x4 t = *(const f32x4*)c;
            v[0] = t[0]; v[1] = t[1]; v[2] = t[2]; v[3] = t[3];
        } else {
            for (int e = 0; e < count; ++e) v[e] = c[e];
        }
    } else {
        const uint16_t* c = (const uint16_t*)C + idx;
        for (int e = 0; e < count; ++e)
            v[e] = c_dtype == DT_F16 ? f16_bits_to_f32(c[e]) : bf16_bits_to_f32(c[e]);
    }
}

// Store up to four consecutive outputs of one row.  vec_ok: all four in range
// and the address aligned for one vector store.
__device__ inline void store_c4(void* C, int c_dtype, int64_t idx, bool vec_ok, const float* v,
                                int count)
{
    if (c_dtype == DT_F32) {
        float* c = (float*)C + idx;
        if (vec_ok) {
            f32x4 t = {v[0], v[1], v[2], v[3]};
            *(f32x4*)c = t;
        } else {
            for (int e = 0; e < count; ++e) c[e] = v[e];
        }
        return;
    }
    uint32_t h[4];
    for (int e = 0; e < 4; ++e)
        h[e] = c_dtype == DT_F16 ? f32_to_f16_bits(v[e]) : f32_to_bf16_bits(v[e]);
    uint16_t* c = (uint16_t*)C + idx;
    if (vec_ok) {
        u32x2 t = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        *(u32x2*)c = t;
    } else {
        for (int e = 0; e < count; ++e) c[e] = (uint16_t)h[e];
    }
}

// Two adjacent 16 x 16 output blocks of an MFMA 16x16 result, written with one
// 16-byte store per lane.  In the result layout lane l holds four consecutive
// columns 4 (l / 16) .. +3 of row l % 16 in each block (p: the left block, q: the
// right one), so a plain store writes 8 bytes per lane and 32-byte pieces of each
// row.  gfx950's v_permlane16_swap exchanges the odd 16-lane rows of its first
// operand with the even rows of its second; applied to (q, p) it leaves lanes
// 0-15 with columns 0-7 of q, lanes 16-31 with columns 0-7 of p, lanes 32-47 with
// columns 8-15 of q and lanes 48-63 with columns 8-15 of p.  Each lane then
// stores 8 consecutive 16-bit outputs, and every row receives 64 contiguous
// bytes from one instruction.  16-bit outputs written 8 bytes per lane reach
// about half the bandwidth of fp32 outputs written 16 bytes per lane (measured
// on MI355X: 8192^2 outputs with K = 0, 2.5-3.1 against 5.1-5.4 TB/s).
// c16: the first of the pair's 32 columns in row m (16-byte aligned).  All four
// lanes sharing a row must be active together.
__device__ inline void store_pair16(uint16_t* c16, int c_dtype, int lane, const float* p, const float* q)
{
    uint32_t ph[4], qh[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        ph[e] = c_dtype == DT_F16 ? f32_to_f16_bits(p[e]) : f32_to_bf16_bits(p[e]);
        qh[e] = c_dtype == DT_F16 ? f32_to_f16_bits(q[e]) : f32_to_bf16_bits(q[e]);
    }
    const u32x2 s01 = __builtin_amdgcn_permlane16_swap(qh[0] | (qh[1] << 16), ph[0] | (ph[1] << 16), false, false);
    const u32x2 s23 = __builtin_amdgcn_permlane16_swap(qh[2] | (qh[3] << 16), ph[2] | (ph[3] << 16), false, false);
    const int g = lane >> 4;
    const int col = ((g & 1) ? 0 : 16) + (g >> 1) * 8;
    *(u32x4*)(c16 + col) = u32x4{s01[0], s23[0], s01[1], s23[1]};
}

// Epilogue of a wave's FM x FN blocks of 16 x 16 outputs in the MFMA 16x16 result
// layout: acc[i][j][e] is C[m][n + e] with m = m_base + 16 i + lane % 16 and
// n = n_base + 16 j + 4 (lane / 16).  Adds C's prior value (clear_accum == 0),
// applies ReLU on the fp32 sum, rounds to C's type and stores what lies inside
// M x N.  16-bit outputs of a fresh sum go out through store_pair16 where a pair of
// blocks lies wholly inside N (c_vec8: N % 8 == 0 and C 16-byte aligned).
template <int FM, int FN>
__device__ inline void store_blocks(void* C, int M, int N, int c_dtype, bool c_vec, bool c_vec8, bool relu_on,
                                    bool clear_accum, const f32x4 (&acc)[FM][FN], int m_base, int n_base, int lane)
{
    const bool pairs = (FN % 2 == 0) && c_vec8 && clear_accum && c_dtype != DT_F32;
    auto store_block = [&](int i, int jj, int m) {
        const int n = n_base + jj * 16 + 4 * (lane >> 4);
        if (n >= N) return;
        const int count = min(4, N - n);
        const bool vec_ok = c_vec && count == 4;
        const int64_t idx = (int64_t)m * N + n;
        float v[4] = {acc[i][jj][0], acc[i][jj][1], acc[i][jj][2], acc[i][jj][3]};
        if (!clear_accum) {
            float c[4] = {0.f, 0.f, 0.f, 0.f};
            load_c4(C, c_dtype, idx, vec_ok, c, count);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = c[e] + v[e];
        }
        if (relu_on) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = relu(v[e]);
        }
        store_c4(C, c_dtype, idx, vec_ok, v, count);
    };
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m_base + i * 16 + (lane & 15);
        if (m >= M) continue;
        if (pairs) {
#pragma unroll
            for (int jp = 0; jp < FN / 2; ++jp) {
                const int nb = n_base + jp * 32;
                if (nb + 32 <= N) {
                    float v[4], w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        v[e] = relu_on ? relu(acc[i][2 * jp][e]) : acc[i][2 * jp][e];
                        w[e] = relu_on ? relu(acc[i][2 * jp + 1][e]) : acc[i][2 * jp + 1][e];
                    }
                    store_pair16((uint16_t*)C + (int64_t)m * N + nb, c_dtype, lane, v, w);
                } else {
                    store_block(i, 2 * jp, m);
                    store_block(i, 2 * jp + 1, m);
                }
            }
        } else {
#pragma unroll
            for (int jj = 0; jj < FN; ++jj) store_block(i, jj, m);
        }
    }
}

}  // namespace tlg
