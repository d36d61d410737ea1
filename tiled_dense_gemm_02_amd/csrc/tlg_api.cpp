// C-ABI layer of libtlg.so: argument validation, plan (variant) selection and
// launch.  Mirrors the pages' generated host wrapper (an extern "C" call that
// launches the kernel on the caller's stream: "NVIDIA backend codegen"
// chapter, section 4.2) and its host-side checks of pointers, dtypes and
// shapes before launch (overview page, "JIT and ABI" section).  Invalid or
// unsupported requests are rejected with a status code; nothing falls back
// silently.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <mutex>
#include <new>
#include <tuple>
#include <vector>

#include "../../include/tlg.h"
#include "tlg_internal.h"

using namespace tlg;

struct tlg_gemm_s {
    int64_t M, N, K;
    int ab, c, tA, tB, clear, relu;
    int variant;
    int vec_a, vec_b;
    int align_a, align_b;  // byte alignment run() requires of A and B
    // split-K plans: workspace = [tiles][splits][128*128] (skinny: [rows*cols of a
    // block]) fp32 partials, then one counter per tile (zero between launches);
    // allocated on `device` at create
    int splits = 1;
    void* ws = nullptr;
    size_t ws_partials_bytes = 0, ws_bytes = 0;
    int64_t dp_tiles = 0, sk_tiles = 0, grid = 0;   // stream-K plans (grid: persistent workgroups)
    int device = -1;
    tlg_plan_info info;
    char desc[256];
    ~tlg_gemm_s()
    {
        if (ws) (void)hipFree(ws);
    }
};

namespace {

constexpr int64_t kMaxMN = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 22;

int elem_bytes(int dt) { return dt == TLG_F32 ? 4 : (dt == TLG_E4M3 || dt == TLG_E5M2 || dt == TLG_E2M1) ? 1 : 2; }

bool is_mx(int dt) { return dt == TLG_E4M3 || dt == TLG_E5M2 || dt == TLG_E2M1; }

const char* dt_name(int dt)
{
    switch (dt) {
    case TLG_F16: return "f16";
    case TLG_BF16: return "bf16";
    case TLG_F32: return "f32";
    case TLG_E4M3: return "e4m3";
    case TLG_E5M2: return "e5m2";
    case TLG_E2M1: return "e2m1";
    default: return "?";
    }
}

const char* variant_name(int v)
{
    switch (v) {
    case TLG_VARIANT_TILE_256: return "tile256";
    case TLG_VARIANT_TILE_128: return "tile128";
    case TLG_VARIANT_SKINNY: return "skinny";
    case TLG_VARIANT_EMPTY: return "empty";
    case TLG_VARIANT_TILE_256_W8: return "tile256w8";
    case TLG_VARIANT_TILE_256_DMA: return "tile256dma";
    case TLG_VARIANT_TILE_128_DMA: return "tile128dma";
    case TLG_VARIANT_TILE_128_DMA_SPLITK: return "tile128dma_sk";
    case TLG_VARIANT_MX_256: return "mx256";
    case TLG_VARIANT_TILE_64_DMA: return "tile64dma";
    case TLG_VARIANT_TILE_256_DMA_STREAMK: return "tile256dma_streamk";
    case TLG_VARIANT_TILE_128_DMA_STREAMK: return "tile128dma_streamk";
    case TLG_VARIANT_TILE_32_DMA: return "tile32dma";
    default: return "?";
    }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The register-staged kernels' 128-bit loads need the contiguous dimension of
// the operand to be a multiple of 8 elements (every 16-byte chunk lies inside one
// row and is 16-byte aligned when the base is); otherwise the operand is loaded
// element by element (the narrow-load fallback for unaligned rows, "core
// primitives" chapter, T.copy notes on alignment).  The direct-load kernels
// relax this for K-contiguous operands (see dma_ok below).
int vec_for(int64_t contiguous_len) { return contiguous_len % 8 == 0 ? 8 : 1; }

bool flag_ok(int v) { return v == 0 || v == 1; }

constexpr int64_t kSplitMinKTiles = 48;
constexpr int kMaxSplits = 8;

// Split-K factor for `tiles` 128x128 output tiles and `ktiles` 64-wide K tiles:
// about 256 workgroups (one per CU), at most 8 ranges, at least 2 K tiles per
// range, and no empty last range.
int choose_splits(int64_t tiles, int64_t ktiles)
{
    int64_t s = std::min<int64_t>(8, std::max<int64_t>(1, 256 / std::max<int64_t>(tiles, 1)));
    s = std::min<int64_t>(s, std::max<int64_t>(1, ktiles / 2));
    while (s > 1 && (s - 1) * ((ktiles + s - 1) / s) >= ktiles) --s;
    return (int)s;
}

// K ranges of the skinny kernel for `tiles` blocks of outputs (16 x 64, 32 x 64 or
// 64 x 32) and `nst` 256-wide K stages.  A block streams its rows of B with at most
// two stages in flight, so a grid of few blocks cannot keep HBM busy (16 x 4096 x
// 8192, 64 blocks: 2.7 TB/s).  Grids of fewer than 256 blocks split K over up to 8
// workgroups per block (about 256 in all), at least 4 stages each, no empty range.
constexpr int64_t kSkinnyMinStagesPerSplit = 4;
int choose_skinny_splits(int64_t tiles, int64_t nst)
{
    if (tiles >= 256) return 1;
    int64_t s = std::min<int64_t>(kSkinnyMaxSplits, std::max<int64_t>(1, 256 / std::max<int64_t>(tiles, 1)));
    s = std::min<int64_t>(s, std::max<int64_t>(1, nst / kSkinnyMinStagesPerSplit));
    while (s > 1 && (s - 1) * ((nst + s - 1) / s) >= nst) --s;
    return (int)s;
}

// Whether the automatic plan takes the skinny kernel for M <= 64 (A stored [M,K],
// B stored [N,K]).  Measured on MI355X against the 64 x 128 tile kernel: with 16 <
// M <= 32 (32 x 64 blocks) it wins from K = 1024 on (32 x 16384 x 1024: 8.4 against
// 9.5 us; 32 x 16384 x 8192: 44.6 against 62.8 us) and loses at K = 512; with
// 32 < M <= 64 (64 x 32 blocks) it wins while the blocks fit about 1.5 rounds of
// the CUs (64 x 8192 x 8192: 30.2 against 54.5 us; 64 x 12288 x 4096: 30.8 against
// 32.3 us), or two rounds with a long K (64 x 16384 x 8192: 58 against 66 us), and
// loses beyond (64 x 16384 x 2048: 20.8 against 19.8 us; 48 x 28672 x 8192: 102
// against 85 us).
bool skinny_pays(int64_t M, int64_t N, int64_t K)
{
    if (M <= kSkinnyRows) return true;
    if (K < 1024) return false;
    if (M <= 32) return true;
    const int64_t blocks = ceil_div(N, skinny_cols(skinny_rows(M)));
    return blocks <= 384 || (blocks <= 512 && K >= 4096);
}

bool is_streamk(int v) { return v == TLG_VARIANT_TILE_256_DMA_STREAMK || v == TLG_VARIANT_TILE_128_DMA_STREAMK; }

// The direct-load variants with K tiles of 128 and 128-column tiles (64 x 128, 32 x 128).
bool is_narrow_dma(int v) { return v == TLG_VARIANT_TILE_64_DMA || v == TLG_VARIANT_TILE_32_DMA; }

// Persistent grid of the stream-K variants: one workgroup per CU of an MI355X
// (each takes 128 KiB of LDS, so one fits a CU).
constexpr int kPersistentGrid = 256;

// Tiles computed whole vs shared out by K iterations, and the persistent grid.
// Every wave but the last full one is data-parallel; the last full wave and the
// remainder (G .. 2G-1 tiles) are stream-K, so every workgroup gets at least one
// tile's worth of K iterations and a tile has at most three partial segments.
// Fewer tiles than workgroups: all stream-K, on min(G, iterations) workgroups so
// that no workgroup's share is empty (the workgroups sharing a tile must be
// consecutive).  K == 0: every tile is "whole" (the epilogue alone).
void streamk_split(int64_t tiles, int64_t ktiles, int64_t* dp, int64_t* sk, int64_t* grid)
{
    const int64_t G = kPersistentGrid;
    if (ktiles == 0) {
        *dp = tiles;
        *sk = 0;
        *grid = std::min(G, tiles);
        return;
    }
    const int64_t waves = tiles / G;
    *dp = waves >= 2 ? (waves - 1) * G : 0;
    *sk = tiles - *dp;
    *grid = *dp > 0 ? G : std::min(G, *sk * ktiles);
}

bool is_tile(int v)
{
    return v == TLG_VARIANT_TILE_256 || v == TLG_VARIANT_TILE_128 || v == TLG_VARIANT_TILE_256_W8;
}

int tile_config(int v)
{
    if (v == TLG_VARIANT_TILE_256) return TILE_256;
    if (v == TLG_VARIANT_TILE_256_W8) return TILE_256_W8;
    return TILE_128;
}

// Validation, variant choice and launch geometry: everything a plan holds except
// its device workspace.  Host only.
tlg_status plan_build(tlg_gemm_s* p, int64_t M, int64_t N, int64_t K, int ab, int c, int tA, int tB, int clear,
                      int epi, int forced, int forced_splits = 0)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxMN || N > kMaxMN || K > kMaxK) return TLG_ERR_INVALID_ARG;
    if (!flag_ok(tA) || !flag_ok(tB) || !flag_ok(clear)) return TLG_ERR_INVALID_ARG;
    if (epi != TLG_EPI_NONE && epi != TLG_EPI_RELU) return TLG_ERR_INVALID_ARG;
    if (ab != TLG_F16 && ab != TLG_BF16 && ab != TLG_F32 && !is_mx(ab))
        return TLG_ERR_INVALID_ARG;
    if (c != TLG_F16 && c != TLG_BF16 && c != TLG_F32) return TLG_ERR_INVALID_ARG;
    if (ab == TLG_F32) return TLG_ERR_UNSUPPORTED;
    if (forced < TLG_VARIANT_AUTO || forced > TLG_VARIANT_TILE_32_DMA || forced == TLG_VARIANT_EMPTY)
        return TLG_ERR_INVALID_ARG;
    if (is_mx(ab)) {
        // Block-scaled FP8 / FP4: A stored [M, K], B stored [N, K], K a multiple of
        // 128 (whole scale words of four blocks); anything else is refused rather
        // than run without its scales.  An FP4 K tile is 256 elements (128 bytes).
        if (tA || !tB || K % 128 != 0) return TLG_ERR_UNSUPPORTED;
        if (forced != TLG_VARIANT_AUTO && forced != TLG_VARIANT_MX_256) return TLG_ERR_UNSUPPORTED;
        const int variant = (M == 0 || N == 0) ? TLG_VARIANT_EMPTY : TLG_VARIANT_MX_256;
        if (ceil_div(M, 256) * ceil_div(N, 256) > INT32_MAX) return TLG_ERR_INVALID_ARG;
        p->M = M; p->N = N; p->K = K;
        p->ab = ab; p->c = c; p->tA = tA; p->tB = tB; p->clear = clear; p->relu = epi == TLG_EPI_RELU;
        p->variant = variant;
        p->vec_a = p->vec_b = 16;
        p->align_a = p->align_b = 16;
        tlg_plan_info& in = p->info;
        in = tlg_plan_info{};
        in.variant = variant;
        in.vec_a = in.vec_b = 16;
        if (variant == TLG_VARIANT_MX_256) {
            const int planes = ab == TLG_E2M1 ? 2 : 1;
            in.block_m = 256; in.block_n = 256; in.block_k = 128 * planes;
            in.stages = 2;
            in.threads = 512;
            in.grid = ceil_div(M, 256) * ceil_div(N, 256);
            in.lds_bytes = 2 * (2 * 256 * 128 + 2 * planes * 256 * 4);
            in.k_tiles = (int32_t)ceil_div(K, in.block_k);
        }
        in.splits = 1;
        std::snprintf(p->desc, sizeof(p->desc),
                      "%s M=%lld N=%lld K=%lld ab=%s c=%s tA=%d tB=%d clear=%d relu=%d block=%dx%dx%d "
                      "stages=%d threads=%d grid=%lld lds=%lld scale_block=32",
                      variant_name(variant), (long long)M, (long long)N, (long long)K, dt_name(ab), dt_name(c), tA,
                      tB, clear, p->relu, in.block_m, in.block_n, in.block_k, in.stages, in.threads,
                      (long long)in.grid, (long long)in.lds_bytes);
        return TLG_OK;
    }
    if (forced == TLG_VARIANT_MX_256) return TLG_ERR_UNSUPPORTED;

    const int va = vec_for(tA ? M : K);
    const int vb = vec_for(tB ? K : N);
    const bool skinny_ok = !tA && tB && K % 8 == 0;
    // Direct-load kernels: a K-contiguous operand may have any K (unaligned 128-bit
    // loads, tail trimmed in LDS); an M/N-contiguous one needs rows of 8k elements.
    const bool dma_ok = (!tA || M % 8 == 0) && (tB || N % 8 == 0);

    int variant;
    if (M == 0 || N == 0) {
        variant = TLG_VARIANT_EMPTY;
    } else if (forced != TLG_VARIANT_AUTO) {
        variant = forced;
        if (forced == TLG_VARIANT_SKINNY && !skinny_ok) return TLG_ERR_UNSUPPORTED;
        if ((forced == TLG_VARIANT_TILE_256 || forced == TLG_VARIANT_TILE_256_W8) && (va != 8 || vb != 8))
            return TLG_ERR_UNSUPPORTED;
        if ((forced == TLG_VARIANT_TILE_256_DMA || forced == TLG_VARIANT_TILE_128_DMA ||
             forced == TLG_VARIANT_TILE_128_DMA_SPLITK || is_narrow_dma(forced) || is_streamk(forced)) && !dma_ok)
            return TLG_ERR_UNSUPPORTED;
        if (is_narrow_dma(forced) && tA) return TLG_ERR_UNSUPPORTED;
        // Their K tiles are 128 rows of k: with B stored [K,N] a lane's direct-load
        // offset reaches 127 rows of 2N bytes (plus a chunk), which must stay below
        // 2^31 (offsets from 2^31 up read as out of range).  The automatic choice
        // takes these variants only for N <= 128 * 128.
        if (is_narrow_dma(forced) && !tB && 127 * 2 * N + 256 > (int64_t)INT32_MAX)
            return TLG_ERR_UNSUPPORTED;
    } else if (M <= kSkinnyMaxRows && skinny_ok && skinny_pays(M, N, K)) {
        variant = TLG_VARIANT_SKINNY;
    } else if (dma_ok) {
        // 256x256 tiles once they fill every CU, else 128x128 tiles (4x the workgroups);
        // fewer than 128 of those with a long K: split K as well.  The exchange of
        // partial tiles costs ~5-10 us per launch (measured on MI355X), which a
        // split repays only from about 48 K tiles (K >= 3072) on.  Otherwise, at
        // most 128 tiles of 128x128 and A stored [M,K]: 64x128 tiles, twice the
        // workgroups in one wave (measured on MI355X: 1024^3 13.5 -> 10.0 us,
        // 1000x1500x777 bf16 13.5 -> 10.8 us; at 2048^3, 256 tiles of 128x128,
        // they are 1.5x slower), or 32x128 tiles where those still fit one wave of
        // 256 workgroups (1024^3 10.5 -> 9.6 us, 256^3 5.17 -> 4.62 us; with 384
        // of them, 1024x1536x1024, 9.8 -> 15.6 us).
        //
        // Once 256x256 tiles fill at least half the chip, the wave count decides
        // between the two tile sizes: a wave of 128x128 tiles costs about 0.37 of a
        // wave of 256x256 tiles (measured on MI355X: 8192^3 82 vs 222 us per wave,
        // 4096^3 43 vs 122, 6144^3 43 vs 107), so a grid whose last wave of 256x256
        // tiles is nearly empty runs faster in 128x128 tiles (4600x4350x4100: 306
        // tiles of 256x256, 2 waves, 293 us; 1224 of 128x128, 5 waves, 260 us), and
        // one partial wave of more than 128 tiles of 256x256 beats three waves of
        // 128x128 (8192x1536x8192: 194 against 246 us), while 128 of them lose to
        // two waves of 128x128 (8192x1024x8192: 184 against 168 us).
        const int64_t t128 = ceil_div(M, 128) * ceil_div(N, 128), kt = ceil_div(K, 64);
        const int64_t t256 = ceil_div(M, 256) * ceil_div(N, 256);
        if (t256 >= 128 && 37 * ceil_div(t128, 256) < 97 * ceil_div(t256, 256))
            variant = TLG_VARIANT_TILE_128_DMA;
        else if (t256 >= 128)
            variant = TLG_VARIANT_TILE_256_DMA;
        else if (t128 < 128 && kt >= kSplitMinKTiles && choose_splits(t128, kt) >= 2)
            variant = TLG_VARIANT_TILE_128_DMA_SPLITK;
        else if (t128 <= 128 && !tA)
            variant = ceil_div(M, kLds32BM) * ceil_div(N, kLds32BN) <= 256 ? TLG_VARIANT_TILE_32_DMA
                                                                          : TLG_VARIANT_TILE_64_DMA;
        else
            variant = TLG_VARIANT_TILE_128_DMA;
    } else {
        variant = TLG_VARIANT_TILE_128;
    }

    // Launch-grid limits: the tile kernels use a 1-D grid of tile ids (int), the
    // skinny kernel a 2-D grid with row blocks in y.
    int splits = 1;
    if (variant == TLG_VARIANT_TILE_128_DMA_SPLITK) {
        const int64_t kt = ceil_div(K, 64);
        if (forced_splits > 0) {
            // a split count asked for by the tuner: whole K tiles per range, none empty
            if (forced_splits > kMaxSplits || (forced_splits - 1) * ceil_div(kt, forced_splits) >= kt)
                return TLG_ERR_UNSUPPORTED;
            splits = forced_splits;
        } else {
            splits = choose_splits(ceil_div(M, 128) * ceil_div(N, 128), kt);
        }
    }
    if (is_tile(variant) || variant == TLG_VARIANT_TILE_256_DMA || variant == TLG_VARIANT_TILE_128_DMA ||
        variant == TLG_VARIANT_TILE_128_DMA_SPLITK || is_narrow_dma(variant) || is_streamk(variant)) {
        const int64_t b = (variant == TLG_VARIANT_TILE_256 || variant == TLG_VARIANT_TILE_256_W8 ||
                           variant == TLG_VARIANT_TILE_256_DMA || variant == TLG_VARIANT_TILE_256_DMA_STREAMK) ? 256 : 128;
        const int64_t bm = variant == TLG_VARIANT_TILE_64_DMA ? kLds64BM : variant == TLG_VARIANT_TILE_32_DMA ? kLds32BM : b;
        if (ceil_div(M, bm) * ceil_div(N, b) * splits > INT32_MAX) return TLG_ERR_INVALID_ARG;
    } else if (variant == TLG_VARIANT_SKINNY) {
        const int mr = skinny_rows(M);
        if (ceil_div(M, mr) > 65535 || ceil_div(N, skinny_cols(mr)) > INT32_MAX) return TLG_ERR_INVALID_ARG;
    }

    p->M = M; p->N = N; p->K = K;
    p->ab = ab; p->c = c; p->tA = tA; p->tB = tB; p->clear = clear; p->relu = epi == TLG_EPI_RELU;
    p->variant = variant;
    const bool dma = variant == TLG_VARIANT_TILE_256_DMA || variant == TLG_VARIANT_TILE_128_DMA ||
                     variant == TLG_VARIANT_TILE_128_DMA_SPLITK || is_narrow_dma(variant) || is_streamk(variant);
    p->vec_a = (variant == TLG_VARIANT_SKINNY || dma) ? 8 : va;
    p->vec_b = (variant == TLG_VARIANT_SKINNY || dma) ? 8 : vb;
    if (dma) {
        p->align_a = tA ? 16 : 2;   // K-contiguous operands take unaligned 128-bit loads
        p->align_b = tB ? 2 : 16;
    } else {
        p->align_a = p->vec_a == 8 ? 16 : 2;
        p->align_b = p->vec_b == 8 ? 16 : 2;
    }

    tlg_plan_info& in = p->info;
    in = tlg_plan_info{};
    in.variant = variant;
    in.vec_a = p->vec_a;
    in.vec_b = p->vec_b;
    if (is_tile(variant)) {
        const TileShape ts = tile_shape(tile_config(variant));
        in.block_m = ts.bm; in.block_n = ts.bn; in.block_k = ts.bk;
        in.stages = ts.stages;
        in.threads = ts.threads();
        in.grid = ceil_div(M, ts.bm) * ceil_div(N, ts.bn);
        in.lds_bytes = (int64_t)ts.stages * (ts.bm + ts.bn) * ts.bk * 2;
        in.k_tiles = (int32_t)ceil_div(K, ts.bk);
    } else if (variant == TLG_VARIANT_TILE_256_DMA) {
        in.block_m = kLdsBM; in.block_n = kLdsBN; in.block_k = kLdsBK;
        in.stages = kLdsStages;
        in.threads = kLdsThreads;
        in.grid = ceil_div(M, kLdsBM) * ceil_div(N, kLdsBN);
        in.lds_bytes = (int64_t)kLdsStages * (kLdsBM + kLdsBN) * kLdsBK * 2;
        in.k_tiles = (int32_t)ceil_div(K, kLdsBK);
    } else if (variant == TLG_VARIANT_TILE_128_DMA || variant == TLG_VARIANT_TILE_128_DMA_SPLITK) {
        const int64_t tiles = ceil_div(M, kLds128BM) * ceil_div(N, kLds128BN);
        in.block_m = kLds128BM; in.block_n = kLds128BN; in.block_k = kLdsBK;
        in.stages = kLds128Stages;
        in.threads = kLdsThreads;
        in.grid = tiles * splits;
        in.lds_bytes = (int64_t)kLds128Stages * (kLds128BM + kLds128BN) * kLdsBK * 2;
        in.k_tiles = (int32_t)ceil_div(ceil_div(K, kLdsBK), splits);
        if (variant == TLG_VARIANT_TILE_128_DMA_SPLITK) {
            p->splits = splits;
            p->ws_partials_bytes = (size_t)tiles * splits * kLds128BM * kLds128BN * sizeof(float);
            p->ws_bytes = p->ws_partials_bytes + (size_t)((tiles * sizeof(unsigned) + 255) / 256 * 256);
        }
    } else if (is_streamk(variant)) {
        const bool big = variant == TLG_VARIANT_TILE_256_DMA_STREAMK;
        const int64_t bm = big ? kLdsBM : kLds128BM, bn = big ? kLdsBN : kLds128BN;
        const int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn);
        streamk_split(tiles, ceil_div(K, kLdsBK), &p->dp_tiles, &p->sk_tiles, &p->grid);
        in.block_m = (int32_t)bm; in.block_n = (int32_t)bn; in.block_k = kLdsBK;
        in.stages = big ? kLdsStages : kLds128Stages;
        in.threads = kLdsThreads;
        in.grid = p->grid;
        in.lds_bytes = (int64_t)in.stages * (bm + bn) * kLdsBK * 2;
        in.k_tiles = (int32_t)ceil_div(K, kLdsBK);
        in.dp_tiles = (int32_t)p->dp_tiles;
        in.sk_tiles = (int32_t)p->sk_tiles;
        if (p->sk_tiles > 0) {
            p->ws_partials_bytes = (size_t)2 * (size_t)p->grid * (size_t)(bm * bn) * sizeof(float);
            p->ws_bytes = p->ws_partials_bytes + (size_t)((p->sk_tiles * sizeof(unsigned) + 255) / 256 * 256);
        }
    } else if (variant == TLG_VARIANT_TILE_64_DMA) {
        in.block_m = kLds64BM; in.block_n = kLds64BN; in.block_k = kLds64BK;
        in.stages = kLds64Stages;
        in.threads = kLdsThreads;
        in.grid = ceil_div(M, kLds64BM) * ceil_div(N, kLds64BN);
        in.lds_bytes = (int64_t)kLds64Stages * (kLds64BM + kLds64BN) * kLds64BK * 2;
        in.k_tiles = (int32_t)ceil_div(K, kLds64BK);
    } else if (variant == TLG_VARIANT_TILE_32_DMA) {
        in.block_m = kLds32BM; in.block_n = kLds32BN; in.block_k = kLds32BK;
        in.stages = kLds32Stages;
        in.threads = kLds32Threads;
        in.grid = ceil_div(M, kLds32BM) * ceil_div(N, kLds32BN);
        in.lds_bytes = (int64_t)kLds32Stages * (kLds32BM + kLds32BN) * kLds32BK * 2;
        in.k_tiles = (int32_t)ceil_div(K, kLds32BK);
    } else if (variant == TLG_VARIANT_SKINNY) {
        const int mr = skinny_rows(M), nb = skinny_cols(mr);
        const int64_t tiles = ceil_div(M, mr) * ceil_div(N, nb);
        const int64_t nst = ceil_div(K, kSkinnyKST);
        const int sp = choose_skinny_splits(tiles, nst);
        in.block_m = mr; in.block_n = nb; in.block_k = kSkinnyKST;
        in.stages = kSkinnyStages;
        in.threads = kSkinnyThreads;
        in.grid = tiles * sp;
        in.lds_bytes = (int64_t)kSkinnyStages * (nb + mr) * kSkinnyKST * 2;
        in.k_tiles = (int32_t)ceil_div(nst, sp);
        if (sp > 1) {
            p->splits = sp;
            p->ws_partials_bytes = (size_t)tiles * sp * mr * nb * sizeof(float);
            p->ws_bytes = p->ws_partials_bytes + (size_t)((tiles * sizeof(unsigned) + 255) / 256 * 256);
        }
    }
    in.splits = p->splits;
    in.workspace_bytes = (int64_t)p->ws_bytes;
    char sk_desc[64] = "";
    if (is_streamk(variant))
        std::snprintf(sk_desc, sizeof(sk_desc), " dp_tiles=%lld sk_tiles=%lld", (long long)p->dp_tiles,
                      (long long)p->sk_tiles);
    std::snprintf(p->desc, sizeof(p->desc),
                  "%s M=%lld N=%lld K=%lld ab=%s c=%s tA=%d tB=%d clear=%d relu=%d block=%dx%dx%d "
                  "stages=%d threads=%d grid=%lld lds=%lld vec=%d/%d splits=%d%s",
                  variant_name(variant), (long long)M, (long long)N, (long long)K, dt_name(ab), dt_name(c), tA,
                  tB, clear, p->relu, in.block_m, in.block_n, in.block_k, in.stages, in.threads,
                  (long long)in.grid, (long long)in.lds_bytes, in.vec_a, in.vec_b, in.splits, sk_desc);
    return TLG_OK;
}

tlg_status plan_create(tlg_gemm_t* out, int64_t M, int64_t N, int64_t K, int ab, int c, int tA, int tB,
                       int clear, int epi, int forced, int forced_splits = 0)
{
    if (!out) return TLG_ERR_NULL;
    *out = nullptr;
    tlg_gemm_s* p = new (std::nothrow) tlg_gemm_s();
    if (!p) return TLG_ERR_NOMEM;
    const tlg_status st = plan_build(p, M, N, K, ab, c, tA, tB, clear, epi, forced, forced_splits);
    if (st != TLG_OK) {
        delete p;
        return st;
    }
    if (p->ws_bytes) {
        // Split-K workspace on the current device; the per-tile counters start at
        // zero (the kernel returns each one to zero after use).
        if (hipGetDevice(&p->device) != hipSuccess || hipMalloc(&p->ws, p->ws_bytes) != hipSuccess) {
            p->ws = nullptr;
            delete p;
            return TLG_ERR_HIP;
        }
        if (hipMemset((char*)p->ws + p->ws_partials_bytes, 0, p->ws_bytes - p->ws_partials_bytes) != hipSuccess ||
            hipStreamSynchronize(nullptr) != hipSuccess) {
            delete p;
            return TLG_ERR_HIP;
        }
    }
    *out = p;
    return TLG_OK;
}

bool ranges_overlap(uintptr_t a, uint64_t an, uintptr_t b, uint64_t bn)
{
    if (an == 0 || bn == 0) return false;
    return a < b + bn && b < a + an;
}

}  // namespace

extern "C" {

tlg_status tlg_gemm_create(tlg_gemm_t* out, int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                           int32_t transpose_A, int32_t transpose_B, int32_t clear_accum, int32_t epilogue)
{
    return plan_create(out, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                       TLG_VARIANT_AUTO);
}

tlg_status tlg_gemm_create_variant(tlg_gemm_t* out, int64_t M, int64_t N, int64_t K, int32_t ab_dtype,
                                   int32_t c_dtype, int32_t transpose_A, int32_t transpose_B,
                                   int32_t clear_accum, int32_t epilogue, int32_t variant)
{
    return plan_create(out, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                       variant);
}

tlg_status tlg_gemm_select(tlg_plan_info* info, int64_t M, int64_t N, int64_t K, int32_t ab_dtype,
                           int32_t c_dtype, int32_t transpose_A, int32_t transpose_B, int32_t clear_accum,
                           int32_t epilogue, int32_t variant)
{
    if (!info) return TLG_ERR_NULL;
    tlg_gemm_s p;
    const tlg_status st =
        plan_build(&p, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue, variant);
    if (st == TLG_OK) *info = p.info;
    return st;
}

}  // extern "C"

namespace {

// The host checks of a run (pointers, alignment, overlap); TLG_OK when the plan may
// be launched on these buffers.
tlg_status check_run(const tlg_gemm_s& p, const void* A, const void* B, const void* C)
{
    if (is_mx(p.ab)) return TLG_ERR_INVALID_ARG;   // needs its scales: tlg_gemm_run_mx
    if (p.variant == TLG_VARIANT_EMPTY) return TLG_OK;
    if (!C) return TLG_ERR_NULL;
    if (p.K > 0 && (!A || !B)) return TLG_ERR_NULL;
    const uintptr_t a = (uintptr_t)A, b = (uintptr_t)B, c = (uintptr_t)C;
    const int cb = elem_bytes(p.c);
    if (c % (uintptr_t)cb) return TLG_ERR_MISALIGNED;
    if (p.K > 0) {
        if ((a % (uintptr_t)p.align_a) || (b % (uintptr_t)p.align_b)) return TLG_ERR_MISALIGNED;
    }
    const uint64_t a_bytes = p.K > 0 ? (uint64_t)p.M * (uint64_t)p.K * 2u : 0;
    const uint64_t b_bytes = p.K > 0 ? (uint64_t)p.K * (uint64_t)p.N * 2u : 0;
    const uint64_t c_bytes = (uint64_t)p.M * (uint64_t)p.N * (uint64_t)cb;
    if (ranges_overlap(c, c_bytes, a, a_bytes) || ranges_overlap(c, c_bytes, b, b_bytes))
        return TLG_ERR_INVALID_ARG;
    return TLG_OK;
}

// One launch of a checked 16-bit plan.  ws / counters: the split-K partial tiles
// and per-tile counters (the plan's own workspace, or the static scratch of
// tlg_gemm_run_noalloc); unused by the other variants.
tlg_status launch_plan(const tlg_gemm_s& p, const void* A, const void* B, void* C, void* stream, float* ws,
                       unsigned* counters)
{
    if (p.variant == TLG_VARIANT_EMPTY) return TLG_OK;
    const uintptr_t c = (uintptr_t)C;
    const int cb = elem_bytes(p.c);
    GemmParams gp{};
    gp.A = A; gp.B = B; gp.C = C;
    gp.M = (int)p.M; gp.N = (int)p.N; gp.K = (int)p.K;
    gp.relu = p.relu;
    gp.clear_accum = p.clear;
    gp.c_dtype = p.c;
    gp.c_vec = (p.N % 4 == 0) && (c % (uintptr_t)(4 * cb) == 0);
    gp.c_vec8 = (p.N % 8 == 0) && (c % 16u == 0);

    hipError_t err;
    if (p.variant == TLG_VARIANT_SKINNY) {
        gp.tiles_m = (int)ceil_div(p.M, skinny_rows(p.M));
        gp.tiles_n = (int)ceil_div(p.N, skinny_cols(skinny_rows(p.M)));
        gp.splits = p.splits;
        gp.ws = ws;
        gp.counters = counters;
        err = launch_skinny(gp, p.ab, (hipStream_t)stream);
    } else if (p.variant == TLG_VARIANT_TILE_256_DMA) {
        gp.tiles_m = (int)ceil_div(p.M, kLdsBM);
        gp.tiles_n = (int)ceil_div(p.N, kLdsBN);
        err = p.ab == TLG_F16 ? launch_lds_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                              : launch_lds_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
    } else if (p.variant == TLG_VARIANT_TILE_128_DMA) {
        gp.tiles_m = (int)ceil_div(p.M, kLds128BM);
        gp.tiles_n = (int)ceil_div(p.N, kLds128BN);
        err = p.ab == TLG_F16 ? launch_lds128_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                              : launch_lds128_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
    } else if (is_streamk(p.variant)) {
        const bool big = p.variant == TLG_VARIANT_TILE_256_DMA_STREAMK;
        gp.tiles_m = (int)ceil_div(p.M, big ? kLdsBM : kLds128BM);
        gp.tiles_n = (int)ceil_div(p.N, big ? kLdsBN : kLds128BN);
        gp.persistent_grid = (int)p.grid;
        gp.dp_tiles = (int)p.dp_tiles;
        gp.sk_tiles = (int)p.sk_tiles;
        gp.ws = ws;
        gp.counters = counters;
        if (big)
            err = p.ab == TLG_F16 ? launch_lds_sk2_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                                  : launch_lds_sk2_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
        else
            err = p.ab == TLG_F16 ? launch_lds128_sk2_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                                  : launch_lds128_sk2_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
    } else if (p.variant == TLG_VARIANT_TILE_64_DMA) {
        gp.tiles_m = (int)ceil_div(p.M, kLds64BM);
        gp.tiles_n = (int)ceil_div(p.N, kLds64BN);
        err = p.ab == TLG_F16 ? launch_lds64_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                              : launch_lds64_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
    } else if (p.variant == TLG_VARIANT_TILE_32_DMA) {
        gp.tiles_m = (int)ceil_div(p.M, kLds32BM);
        gp.tiles_n = (int)ceil_div(p.N, kLds32BN);
        err = p.ab == TLG_F16 ? launch_lds32_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                              : launch_lds32_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
    } else if (p.variant == TLG_VARIANT_TILE_128_DMA_SPLITK) {
        gp.tiles_m = (int)ceil_div(p.M, kLds128BM);
        gp.tiles_n = (int)ceil_div(p.N, kLds128BN);
        gp.splits = p.splits;
        gp.ws = ws;
        gp.counters = counters;
        err = p.ab == TLG_F16 ? launch_lds128sk_f16(gp, p.tA, p.tB, (hipStream_t)stream)
                              : launch_lds128sk_bf16(gp, p.tA, p.tB, (hipStream_t)stream);
    } else {
        const int cfg = tile_config(p.variant);
        const TileShape ts = tile_shape(cfg);
        gp.tiles_m = (int)ceil_div(p.M, ts.bm);
        gp.tiles_n = (int)ceil_div(p.N, ts.bn);
        err = launch_tile(cfg, gp, p.ab, p.tA, p.tB, p.vec_a, p.vec_b, (hipStream_t)stream);
    }
    return err == hipSuccess ? TLG_OK : TLG_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Static scratch of tlg_gemm_run_noalloc: the split-K partial tiles and per-tile
// counters of a request, in a file-scope device array instead of a plan-owned
// allocation.  Every GPU the library runs on holds one copy of it (at its own
// address) until the process ends.  Host code never passes the array's name to a
// kernel (in host code that name is a host-side stand-in, not a device address):
// the device address is looked up once per device with hipGetSymbolAddress, with
// that device current, and kept in g_scratch_ptr.
//   [0, kScratchPartialBytes)                  fp32 partial tiles
//   [kScratchPartialBytes, + kScratchCounterBytes)  one counter per output tile
// The automatic plan never needs more: it splits K only for fewer than 128 tiles
// of 128 x 128, into at most 256 / tiles ranges (tiles x ranges <= 256 partial
// tiles of 64 KiB), and in the skinny kernel for fewer than 256 blocks (at most
// 256 partial blocks of 4 or 8 KiB).
// ---------------------------------------------------------------------------
constexpr size_t kScratchPartialBytes = size_t(256) * kLds128BM * kLds128BN * sizeof(float);   // 16 MiB
constexpr size_t kScratchCounterBytes = 4096;                                                 // 1024 counters
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) char scratch[kScratchPartialBytes + kScratchCounterBytes];

// Zero n 32-bit words (a kernel rather than hipMemsetAsync, so that the clear
// may be recorded into a captured graph).
__global__ void tlg_fill_zero_u32(unsigned* p, int n)
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

namespace {

std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device (nullptr: not set up)

// Device address of the current device's scratch.  First call on a device: look
// the address up and zero the counters with a kernel on `stream` (ordered before
// the caller's launch).  The split-K kernel returns every counter it uses to zero,
// so the counters stay zero between calls.
tlg_status scratch_for_current_device(void* stream, char** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TLG_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return TLG_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return TLG_ERR_HIP;
        constexpr int n = (int)(kScratchCounterBytes / sizeof(unsigned));
        void* args_p = (char*)ptr + kScratchPartialBytes;
        int args_n = n;
        void* kargs[] = {&args_p, &args_n};
        if (hipLaunchKernel((const void*)&tlg_fill_zero_u32, dim3((n + 255) / 256), dim3(256), kargs, 0,
                            (hipStream_t)stream) != hipSuccess)
            return TLG_ERR_HIP;
        g_scratch_ptr[dev] = (char*)ptr;
    }
    *out = g_scratch_ptr[dev];
    return TLG_OK;
}

}  // namespace

extern "C" {

tlg_status tlg_gemm_run(tlg_gemm_t plan, const void* A, const void* B, void* C, void* stream)
{
    if (!plan) return TLG_ERR_NULL;
    const tlg_gemm_s& p = *plan;
    const tlg_status st = check_run(p, A, B, C);
    if (st != TLG_OK || p.variant == TLG_VARIANT_EMPTY) return st;
    if (p.ws) {
        int dev = -1;
        if (hipGetDevice(&dev) != hipSuccess) return TLG_ERR_HIP;
        if (dev != p.device) return TLG_ERR_INVALID_ARG;   // the workspace lives on the plan's device
    }
    return launch_plan(p, A, B, C, stream, (float*)p.ws, (unsigned*)((char*)p.ws + p.ws_partials_bytes));
}

tlg_status tlg_gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                                int32_t transpose_A, int32_t transpose_B, int32_t clear_accum, int32_t epilogue,
                                const void* A, const void* B, void* C, void* stream)
{
    if (is_mx(ab_dtype)) return TLG_ERR_UNSUPPORTED;   // block-scaled: tlg_gemm_run_mx
    tlg_gemm_s p;   // on the stack: plan_build is host work only and allocates nothing
    tlg_status st = plan_build(&p, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                               TLG_VARIANT_AUTO);
    if (st != TLG_OK) return st;
    st = check_run(p, A, B, C);
    if (st != TLG_OK || p.variant == TLG_VARIANT_EMPTY) return st;
    float* ws = nullptr;
    unsigned* counters = nullptr;
    if (p.ws_bytes) {
        if (p.ws_partials_bytes > kScratchPartialBytes || p.ws_bytes - p.ws_partials_bytes > kScratchCounterBytes)
            return TLG_ERR_TOO_LARGE;
        char* base = nullptr;
        st = scratch_for_current_device(stream, &base);
        if (st != TLG_OK) return st;
        ws = (float*)base;
        counters = (unsigned*)(base + kScratchPartialBytes);
    }
    return launch_plan(p, A, B, C, stream, ws, counters);
}

tlg_status tlg_gemm_run_mx(tlg_gemm_t plan, const void* A, const void* SA, const void* B, const void* SB, void* C,
                           void* stream)
{
    if (!plan) return TLG_ERR_NULL;
    const tlg_gemm_s& p = *plan;
    if (!is_mx(p.ab)) return TLG_ERR_INVALID_ARG;
    if (p.variant == TLG_VARIANT_EMPTY) return TLG_OK;
    if (!C) return TLG_ERR_NULL;
    if (p.K > 0 && (!A || !B || !SA || !SB)) return TLG_ERR_NULL;
    const uintptr_t a = (uintptr_t)A, b = (uintptr_t)B, c = (uintptr_t)C, sa = (uintptr_t)SA, sb = (uintptr_t)SB;
    const int cb = elem_bytes(p.c);
    if (c % (uintptr_t)cb) return TLG_ERR_MISALIGNED;
    if (p.K > 0 && ((a % 16) || (b % 16) || (sa % 4) || (sb % 4))) return TLG_ERR_MISALIGNED;
    const uint64_t a_elems = p.K > 0 ? (uint64_t)p.M * (uint64_t)p.K : 0;
    const uint64_t b_elems = p.K > 0 ? (uint64_t)p.N * (uint64_t)p.K : 0;
    const uint64_t per_byte = p.ab == TLG_E2M1 ? 2 : 1;   // FP4: two elements per byte
    const uint64_t a_bytes = a_elems / per_byte, b_bytes = b_elems / per_byte;
    const uint64_t sa_bytes = a_elems / 32, sb_bytes = b_elems / 32;
    const uint64_t c_bytes = (uint64_t)p.M * (uint64_t)p.N * (uint64_t)cb;
    if (ranges_overlap(c, c_bytes, a, a_bytes) || ranges_overlap(c, c_bytes, b, b_bytes) ||
        ranges_overlap(c, c_bytes, sa, sa_bytes) || ranges_overlap(c, c_bytes, sb, sb_bytes))
        return TLG_ERR_INVALID_ARG;
    MxParams mp{};
    mp.A = A; mp.SA = SA; mp.B = B; mp.SB = SB; mp.C = C;
    mp.M = (int)p.M; mp.N = (int)p.N; mp.K = (int)p.K;
    mp.relu = p.relu;
    mp.clear_accum = p.clear;
    mp.c_dtype = p.c;
    mp.c_vec = (p.N % 4 == 0) && (c % (uintptr_t)(4 * cb) == 0);
    mp.c_vec8 = (p.N % 8 == 0) && (c % 16u == 0);
    mp.tiles_m = (int)ceil_div(p.M, 256);
    mp.tiles_n = (int)ceil_div(p.N, 256);
    const hipError_t err = launch_mx(mp, p.ab == TLG_E4M3 ? 0 : p.ab == TLG_E5M2 ? 1 : 4, (hipStream_t)stream);
    return err == hipSuccess ? TLG_OK : TLG_ERR_HIP;
}

int32_t tlg_attn_query_block(int64_t batch, int64_t seq, int64_t heads, int64_t dim, int32_t causal)
{
    if (batch <= 0 || seq <= 0 || heads <= 0) return 0;
    // Queries per workgroup: 128, or 64 when blocks of 128 would leave CUs without
    // a workgroup (at most 256 of them), and for causal dim 64 up to 1024 blocks.
    // Measured on MI355X (fp16, one process): with 64 queries, the page's instance
    // 1x1024x8x64 causal (64 blocks of 128) goes from 19.6 to 13.2 us, 2x777x3x128
    // non-causal (42) from 21.5 to 15.0, 1x2048x8x128 causal (128) from 48.8 to
    // 37.7; causal dim 64 with 512-1024 blocks gains 2-6% (1x8192x16x64: 217.8 ->
    // 206.6 us, 2x4096x16x64: 119.6 -> 112.9, 2x2048x16x64: 47.9 -> 47.1); other
    // grids of 512 or more blocks gain at most 1% or lose up to 24% (non-causal
    // 1x4096x16x128: 142 against 177 us; causal 1x4096x32x128: 178 against 193),
    // and 4x4096x32x{64,128} causal lose 7% and 18%.
    const int64_t blocks128 = ceil_div(seq, 128);
    if (blocks128 > 1024 || heads > 1024 || batch > 1024) return 128;   // (each factor is at least 1)
    const int64_t blocks = blocks128 * heads * batch;
    return blocks <= 256 || (causal && dim == 64 && blocks <= 1024) ? 64 : 128;
}

tlg_status tlg_attn_fwd_block(const void* Q, const void* K, const void* V, void* O, int64_t batch, int64_t seq,
                              int64_t heads, int64_t dim, int32_t dtype, int32_t causal, float softmax_scale,
                              int32_t block_q, void* stream)
{
    if (block_q != 0 && block_q != 64 && block_q != 128) return TLG_ERR_INVALID_ARG;
    if (batch < 0 || seq < 0 || heads < 0 || dim <= 0) return TLG_ERR_INVALID_ARG;
    if (!flag_ok(causal) || !std::isfinite(softmax_scale)) return TLG_ERR_INVALID_ARG;
    if (dtype != TLG_F16 && dtype != TLG_BF16) {
        if (dtype == TLG_F32 || is_mx(dtype)) return TLG_ERR_UNSUPPORTED;
        return TLG_ERR_INVALID_ARG;
    }
    if (dim != 64 && dim != 128) return TLG_ERR_UNSUPPORTED;
    if (batch == 0 || seq == 0 || heads == 0) return TLG_OK;
    const uint64_t per_batch = (uint64_t)seq * (uint64_t)heads * (uint64_t)dim * 2u;
    if (per_batch >= (uint64_t(1) << 31)) return TLG_ERR_UNSUPPORTED;
    const int64_t bq = block_q ? block_q : tlg_attn_query_block(batch, seq, heads, dim, causal);
    const int64_t nqb = ceil_div(seq, bq);
    if (batch > INT32_MAX || nqb * heads > INT32_MAX || nqb * heads * batch > INT32_MAX) return TLG_ERR_UNSUPPORTED;
    if (!Q || !K || !V || !O) return TLG_ERR_NULL;
    const uintptr_t q = (uintptr_t)Q, k = (uintptr_t)K, v = (uintptr_t)V, o = (uintptr_t)O;
    if ((q | k | v | o) % 16) return TLG_ERR_MISALIGNED;
    const uint64_t bytes = per_batch * (uint64_t)batch;
    if (ranges_overlap(o, bytes, q, bytes) || ranges_overlap(o, bytes, k, bytes) || ranges_overlap(o, bytes, v, bytes))
        return TLG_ERR_INVALID_ARG;
    AttnParams ap{};
    ap.Q = Q; ap.K = K; ap.V = V; ap.O = O;
    ap.B = (int)batch; ap.S = (int)seq; ap.H = (int)heads;
    ap.scale_log2 = (float)((double)softmax_scale * 1.4426950408889634);   // log2(e)
    ap.block_q = (int)bq;
    ap.nqb = (int)nqb;
    const hipError_t err = launch_attn(ap, (int)dim, dtype == TLG_F16 ? DT_F16 : DT_BF16, causal, (hipStream_t)stream);
    return err == hipSuccess ? TLG_OK : TLG_ERR_HIP;
}

tlg_status tlg_attn_fwd(const void* Q, const void* K, const void* V, void* O, int64_t batch, int64_t seq,
                        int64_t heads, int64_t dim, int32_t dtype, int32_t causal, float softmax_scale, void* stream)
{
    return tlg_attn_fwd_block(Q, K, V, O, batch, seq, heads, dim, dtype, causal, softmax_scale, 0, stream);
}

tlg_status tlg_gemm_w4(const void* A, const void* Wq, const void* S, const void* Z, void* C, int64_t M, int64_t N,
                       int64_t K, int64_t G, int32_t ab_dtype, int32_t c_dtype, int32_t epilogue, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxMN || N > kMaxMN || K > kMaxK) return TLG_ERR_INVALID_ARG;
    if (G <= 0 || G % 32 != 0 || K % G != 0) return TLG_ERR_INVALID_ARG;
    if (ab_dtype != TLG_F16 && ab_dtype != TLG_BF16) return TLG_ERR_INVALID_ARG;
    if (c_dtype != TLG_F16 && c_dtype != TLG_BF16 && c_dtype != TLG_F32) return TLG_ERR_INVALID_ARG;
    if (epilogue != TLG_EPI_NONE && epilogue != TLG_EPI_RELU) return TLG_ERR_INVALID_ARG;
    if (K / G > kW4MaxGroups) return TLG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return TLG_OK;
    if (ceil_div(M, 16) > 65535) return TLG_ERR_INVALID_ARG;   // row blocks of 16 go in the grid's y dimension
    if (!C || (K > 0 && (!A || !Wq || !S || !Z))) return TLG_ERR_NULL;
    const uintptr_t a = (uintptr_t)A, w = (uintptr_t)Wq, sc = (uintptr_t)S, z = (uintptr_t)Z, c = (uintptr_t)C;
    const int cb = elem_bytes(c_dtype);
    if (c % (uintptr_t)cb) return TLG_ERR_MISALIGNED;
    if (K > 0 && ((a % 16) || (w % 16) || (sc % 2))) return TLG_ERR_MISALIGNED;
    const uint64_t kg = K > 0 ? (uint64_t)(K / G) : 0;
    const uint64_t a_bytes = (uint64_t)M * (uint64_t)K * 2u, w_bytes = (uint64_t)N * (uint64_t)K / 2u;
    const uint64_t s_bytes = (uint64_t)N * kg * 2u, z_bytes = (uint64_t)N * kg;
    const uint64_t c_bytes = (uint64_t)M * (uint64_t)N * (uint64_t)cb;
    if (ranges_overlap(c, c_bytes, a, a_bytes) || ranges_overlap(c, c_bytes, w, w_bytes) ||
        ranges_overlap(c, c_bytes, sc, s_bytes) || ranges_overlap(c, c_bytes, z, z_bytes))
        return TLG_ERR_INVALID_ARG;
    W4Params wp{};
    wp.A = A; wp.Wq = Wq; wp.S = S; wp.Z = Z; wp.C = C;
    wp.M = (int)M; wp.N = (int)N; wp.K = (int)K; wp.G = K > 0 ? (int)G : 32;
    wp.relu = epilogue == TLG_EPI_RELU;
    wp.c_dtype = c_dtype;
    wp.c_vec = (N % 4 == 0) && (c % (uintptr_t)(4 * cb) == 0);
    wp.nibble_mask = 0x000F000Fu;
    const hipError_t err = launch_w4(wp, ab_dtype == TLG_F16 ? DT_F16 : DT_BF16, (hipStream_t)stream);
    return err == hipSuccess ? TLG_OK : TLG_ERR_HIP;
}

tlg_status tlg_gemm_sp(const void* A, const void* Wv, const void* Wm, void* C, int64_t M, int64_t N, int64_t K,
                       int32_t ab_dtype, int32_t c_dtype, int32_t epilogue, void* stream)
{
    if (M < 0 || N < 0 || K < 0 || M > kMaxMN || N > kMaxMN || K > kMaxK) return TLG_ERR_INVALID_ARG;
    if (ab_dtype != TLG_F16 && ab_dtype != TLG_BF16) return TLG_ERR_INVALID_ARG;
    if (c_dtype != TLG_F16 && c_dtype != TLG_BF16 && c_dtype != TLG_F32) return TLG_ERR_INVALID_ARG;
    if (epilogue != TLG_EPI_NONE && epilogue != TLG_EPI_RELU) return TLG_ERR_INVALID_ARG;
    if (K % 64 != 0) return TLG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return TLG_OK;
    if (ceil_div(M, 256) * ceil_div(N, 256) > INT32_MAX) return TLG_ERR_INVALID_ARG;
    if (!C || (K > 0 && (!A || !Wv || !Wm))) return TLG_ERR_NULL;
    const uintptr_t a = (uintptr_t)A, wv = (uintptr_t)Wv, wm = (uintptr_t)Wm, c = (uintptr_t)C;
    const int cb = elem_bytes(c_dtype);
    if (c % (uintptr_t)cb) return TLG_ERR_MISALIGNED;
    if (K > 0 && ((a % 16) || (wv % 16) || (wm % 4))) return TLG_ERR_MISALIGNED;
    const uint64_t a_bytes = (uint64_t)M * (uint64_t)K * 2u, wv_bytes = (uint64_t)N * (uint64_t)K;
    const uint64_t wm_bytes = (uint64_t)N * (uint64_t)K / 8u, c_bytes = (uint64_t)M * (uint64_t)N * (uint64_t)cb;
    if (ranges_overlap(c, c_bytes, a, a_bytes) || ranges_overlap(c, c_bytes, wv, wv_bytes) ||
        ranges_overlap(c, c_bytes, wm, wm_bytes))
        return TLG_ERR_INVALID_ARG;
    SpParams sp{};
    sp.A = A; sp.Wv = Wv; sp.Wm = Wm; sp.C = C;
    sp.M = (int)M; sp.N = (int)N; sp.K = (int)K;
    sp.relu = epilogue == TLG_EPI_RELU;
    sp.c_dtype = c_dtype;
    sp.c_vec = (N % 4 == 0) && (c % (uintptr_t)(4 * cb) == 0);
    sp.c_vec8 = (N % 8 == 0) && (c % 16u == 0);
    sp.tiles_m = (int)ceil_div(M, 256);
    sp.tiles_n = (int)ceil_div(N, 256);
    const hipError_t err = launch_sp(sp, ab_dtype == TLG_F16 ? DT_F16 : DT_BF16, (hipStream_t)stream);
    return err == hipSuccess ? TLG_OK : TLG_ERR_HIP;
}

tlg_status tlg_gemm_destroy(tlg_gemm_t plan)
{
    delete plan;
    return TLG_OK;
}

tlg_status tlg_gemm_query(tlg_gemm_t plan, tlg_plan_info* info)
{
    if (!plan || !info) return TLG_ERR_NULL;
    *info = plan->info;
    return TLG_OK;
}

const char* tlg_gemm_describe(tlg_gemm_t plan) { return plan ? plan->desc : "(null plan)"; }

const char* tlg_status_string(int32_t status)
{
    switch (status) {
    case TLG_OK: return "TLG_OK";
    case TLG_ERR_INVALID_ARG: return "TLG_ERR_INVALID_ARG";
    case TLG_ERR_UNSUPPORTED: return "TLG_ERR_UNSUPPORTED";
    case TLG_ERR_NULL: return "TLG_ERR_NULL";
    case TLG_ERR_MISALIGNED: return "TLG_ERR_MISALIGNED";
    case TLG_ERR_HIP: return "TLG_ERR_HIP";
    case TLG_ERR_NOMEM: return "TLG_ERR_NOMEM";
    case TLG_ERR_TOO_LARGE: return "TLG_ERR_TOO_LARGE";
    default: return "TLG_ERR_UNKNOWN";
    }
}

const char* tlg_version(void) { return "tlg 0.2.0 (gfx950)"; }

}  // extern "C"

// Autotuning, after the pages' autotuner (overview page, "autotuning" section):
// a search space of kernel configurations pruned by what each can serve, every
// candidate run on the same real inputs, warmed up, timed over repeated runs,
// and the best configuration kept in a cache keyed by device and problem.
namespace {

// The alignment class of the buffers is part of the key: a choice timed on
// 16-byte-aligned operands may be a variant that refuses 2-byte-aligned ones.
struct TuneKey {
    int dev;
    int64_t M, N, K;
    int ab, c, tA, tB, clear, epi;
    int align;   // bit 0: A 16-byte aligned, bit 1: B, bit 2: C
    bool operator<(const TuneKey& o) const
    {
        return std::tie(dev, M, N, K, ab, c, tA, tB, clear, epi, align) <
               std::tie(o.dev, o.M, o.N, o.K, o.ab, o.c, o.tA, o.tB, o.clear, o.epi, o.align);
    }
};

int align_class(const void* A, const void* B, const void* C)
{
    return (((uintptr_t)A % 16 == 0) ? 1 : 0) | (((uintptr_t)B % 16 == 0) ? 2 : 0) |
           (((uintptr_t)C % 16 == 0) ? 4 : 0);
}

std::mutex g_tune_mu;
std::map<TuneKey, std::pair<int, int>> g_tune_cache;   // -> (variant, forced splits)

struct TuneCandidate {
    int variant, splits;   // splits: 0 = the plan's own choice
};

// The search space for a request: every kernel family, and for output grids that
// leave CUs idle (fewer than 256 tiles of 128 x 128) the split-K kernel with each
// split count from 2 to kMaxSplits.  Candidates that cannot serve the request are
// dropped when their plan is refused.
std::vector<TuneCandidate> tune_space(int64_t M, int64_t N)
{
    std::vector<TuneCandidate> c = {{TLG_VARIANT_TILE_256_DMA, 0}, {TLG_VARIANT_TILE_128_DMA, 0},
                                    {TLG_VARIANT_TILE_64_DMA, 0},  {TLG_VARIANT_TILE_32_DMA, 0},
                                    {TLG_VARIANT_SKINNY, 0},
                                    {TLG_VARIANT_TILE_256_W8, 0},  {TLG_VARIANT_TILE_256, 0},
                                    {TLG_VARIANT_TILE_128, 0}};
    c.push_back({TLG_VARIANT_TILE_256_DMA_STREAMK, 0});
    c.push_back({TLG_VARIANT_TILE_128_DMA_STREAMK, 0});
    if (ceil_div(M, 128) * ceil_div(N, 128) < 256)
        for (int s = 2; s <= kMaxSplits; ++s) c.push_back({TLG_VARIANT_TILE_128_DMA_SPLITK, s});
    return c;
}

}  // namespace

extern "C" {

tlg_status tlg_gemm_tune(tlg_gemm_t* out, int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                         int32_t transpose_A, int32_t transpose_B, int32_t clear_accum, int32_t epilogue,
                         const void* A, const void* B, void* C, void* stream, int32_t iters,
                         tlg_tune_result* results, int32_t max_results, int32_t* n_results)
{
    if (!out) return TLG_ERR_NULL;
    *out = nullptr;
    if (n_results) *n_results = 0;
    if (iters < 1 || iters > 1000 || max_results < 0) return TLG_ERR_INVALID_ARG;
    if (max_results > 0 && !results) return TLG_ERR_NULL;
    // The request itself must be valid (the automatic plan's checks).
    tlg_gemm_s probe;
    tlg_status st = plan_build(&probe, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                               TLG_VARIANT_AUTO);
    if (st != TLG_OK) return st;
    if (is_mx(ab_dtype)) return TLG_ERR_UNSUPPORTED;   // one kernel serves block-scaled GEMM: nothing to tune
    if (probe.variant == TLG_VARIANT_EMPTY)
        return plan_create(out, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                           TLG_VARIANT_AUTO);
    if (!C || (K > 0 && (!A || !B))) return TLG_ERR_NULL;

    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return TLG_ERR_HIP;
    const TuneKey key{dev, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                      align_class(A, B, C)};
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        auto it = g_tune_cache.find(key);
        if (it != g_tune_cache.end())
            return plan_create(out, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum, epilogue,
                               it->second.first, it->second.second);
    }

    hipEvent_t e0 = nullptr, e1 = nullptr;
    if (hipEventCreate(&e0) != hipSuccess || hipEventCreate(&e1) != hipSuccess) {
        if (e0) (void)hipEventDestroy(e0);
        return TLG_ERR_HIP;
    }
    tlg_gemm_t best = nullptr;
    TuneCandidate best_c{0, 0};
    float best_ms = 0.f;
    int32_t count = 0;
    st = TLG_OK;
    for (const TuneCandidate& cand : tune_space(M, N)) {
        tlg_gemm_t pl = nullptr;
        const tlg_status cs = plan_create(&pl, M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B, clear_accum,
                                          epilogue, cand.variant, cand.splits);
        if (cs == TLG_ERR_UNSUPPORTED) continue;
        if (cs != TLG_OK) {
            st = cs;
            break;
        }
        // one untimed run (also checks the buffers for this plan), then `iters` timed
        st = tlg_gemm_run(pl, A, B, C, stream);
        if (st == TLG_ERR_MISALIGNED) {   // this candidate needs an alignment the buffers lack
            tlg_gemm_destroy(pl);
            st = TLG_OK;
            continue;
        }
        if (st == TLG_OK && hipEventRecord(e0, (hipStream_t)stream) != hipSuccess) st = TLG_ERR_HIP;
        for (int i = 0; i < iters && st == TLG_OK; ++i) st = tlg_gemm_run(pl, A, B, C, stream);
        float ms = 0.f;
        if (st == TLG_OK && (hipEventRecord(e1, (hipStream_t)stream) != hipSuccess ||
                             hipEventSynchronize(e1) != hipSuccess || hipEventElapsedTime(&ms, e0, e1) != hipSuccess))
            st = TLG_ERR_HIP;
        if (st != TLG_OK) {
            tlg_gemm_destroy(pl);
            break;
        }
        ms /= (float)iters;
        if (count < max_results) results[count] = tlg_tune_result{pl->variant, pl->splits, ms};
        ++count;
        if (!best || ms < best_ms) {
            tlg_gemm_destroy(best);
            best = pl;
            best_ms = ms;
            best_c = TuneCandidate{cand.variant, cand.splits};
        } else {
            tlg_gemm_destroy(pl);
        }
    }
    (void)hipEventDestroy(e0);
    (void)hipEventDestroy(e1);
    if (n_results) *n_results = std::min(count, max_results);
    if (st != TLG_OK) {
        tlg_gemm_destroy(best);
        return st;
    }
    if (!best) return TLG_ERR_UNSUPPORTED;
    {
        std::lock_guard<std::mutex> lock(g_tune_mu);
        g_tune_cache[key] = {best_c.variant, best_c.splits};
    }
    *out = best;
    return TLG_OK;
}

}  // extern "C"
