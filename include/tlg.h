/*
 * tlg — tiled, software-pipelined dense GEMM  C = act(A·B)  for AMD MI355X (gfx950).
 *
 * C-ABI boundary of libtlg.so.  Plain pointers and sizes only.
 *
 * The operation is the tile program of the TileLang quickstart GEMM(+ReLU):
 *   - "NVIDIA backend codegen" chapter, section 1: a grid of block_M x block_N
 *     output tiles, a K loop of block_K steps run as a software pipeline
 *     (T.Pipelined, num_stages), global->shared copies of the A and B tiles, a
 *     block GEMM into an fp32 register fragment, then a copy back to C;
 *   - handbook page "TileLang: a tile language one level below Triton",
 *     section "first kernel: GEMM" (block 128x128x64, 3 stages, fp16 in, fp32
 *     accumulate, fp16 out);
 *   - "core primitives" chapter, section 3.3 (T.gemm): transpose_A means A is
 *     stored [K, M], transpose_B means B is stored [N, K]; clear_accum starts
 *     the accumulator at zero instead of C's prior contents; the accumulator
 *     type is C's fragment type (fp32 here, always);
 *   - "core primitives" chapter, sections 3.8 and 4.6: the ReLU epilogue is
 *     max(x, 0) on the fp32 tile before the write-out;
 *   - "core primitives" chapter, section 4.2: out-of-bounds source elements
 *     read as 0, stores outside C are skipped.
 *
 * Value computed, for 0 <= m < M, 0 <= n < N:
 *   acc(m,n) = (clear_accum ? 0 : (float)C[m*N + n]) + sum_k a(m,k) * b(k,n)   (fp32 accumulate)
 *   C[m*N + n] = convert_rne(epilogue == RELU ? max(acc, +0) : acc)
 * with a(m,k) = transpose_A ? A[k*M + m] : A[m*K + k]
 *      b(k,n) = transpose_B ? B[n*K + k] : B[k*N + n].
 * The order of the fp32 additions is unspecified but fixed for a plan: two runs
 * of one plan on the same inputs give bit-identical C.
 *
 * Layout: all matrices are dense and packed (leading dimension = row length).
 * Dtypes: A and B share ab_dtype in {TLG_F16, TLG_BF16}; c_dtype in {TLG_F16,
 * TLG_BF16, TLG_F32}.
 *
 * Ownership: the caller owns A, B and C (device memory) and keeps them alive
 * until the work queued on the stream has finished.  The library owns the
 * plan, and the device workspace of a split-K plan (see tlg_plan_info.splits).
 * tlg_gemm_run allocates nothing, does not synchronise, and enqueues at most
 * one kernel on the given stream.  A plan is immutable after create; runs of a
 * plan without a workspace may overlap on different streams, runs of a split-K
 * plan may not (they share its workspace).
 */
#ifndef TLG_H
#define TLG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tlg_gemm_s *tlg_gemm_t;

/* TLG_E4M3 / TLG_E5M2: FP8 operands, TLG_E2M1: FP4 operands (two per byte) of the
 * block-scaled GEMM (tlg_gemm_run_mx). */
typedef enum { TLG_F16 = 1, TLG_BF16 = 2, TLG_F32 = 3, TLG_E4M3 = 4, TLG_E5M2 = 5, TLG_E2M1 = 6 } tlg_dtype;

typedef enum { TLG_EPI_NONE = 0, TLG_EPI_RELU = 1 } tlg_epilogue;

/* Kernel variants.  AUTO lets create choose; the others force one (tests). */
typedef enum {
    TLG_VARIANT_AUTO = 0,
    TLG_VARIANT_TILE_256 = 1,  /* 256x256x64 block tile, 4 wave64s, 2-stage LDS ring */
    TLG_VARIANT_TILE_128 = 2,  /* 128x128x64 block tile, 2 wave64s, 2-stage LDS ring */
    TLG_VARIANT_SKINNY = 3,    /* 16/32/64 rows of A per block, B stored [N,K], streaming */
    TLG_VARIANT_EMPTY = 4,     /* M == 0 or N == 0: nothing to launch (chosen by create) */
    TLG_VARIANT_TILE_256_W8 = 5, /* 256x256x64 block tile, 8 wave64s (2 per SIMD), 2-stage ring */
    TLG_VARIANT_TILE_256_DMA = 6, /* 256x256x64, 8 wave64s, LDS ring filled by global->LDS direct loads */
    TLG_VARIANT_TILE_128_DMA = 7, /* 128x128x64, 8 wave64s, 4-slot ring of direct loads (grids too small for 256x256) */
    TLG_VARIANT_TILE_128_DMA_SPLITK = 8, /* as 7, K split over several workgroups per tile (plan owns a workspace) */
    TLG_VARIANT_MX_256 = 9,    /* block-scaled FP8 / FP4: 256x256 x 128 bytes of K, 8 wave64s, scaled MFMA 16x16x128 */
    TLG_VARIANT_TILE_64_DMA = 10, /* 64x128x128, 8 wave64s, 3-slot ring of direct loads; A stored [M,K] only
                                    (transpose_A == 0); grids of at most 128 tiles of 128x128 */
    TLG_VARIANT_TILE_256_DMA_STREAMK = 11, /* as 6, persistent: 256 workgroups (one per CU) take the tiles
                                    of all but the last wave whole, then equal shares of the remaining
                                    tiles' K iterations (stream-K); the plan owns a workspace */
    TLG_VARIANT_TILE_128_DMA_STREAMK = 12, /* as 7, with the persistent stream-K schedule of 11 */
    TLG_VARIANT_TILE_32_DMA = 13  /* 32x128x128, 8 wave64s, 4-slot ring of direct loads; A stored [M,K] only
                                    (transpose_A == 0); grids whose 32x128 tiles fit one wave (256) */
} tlg_variant;

typedef enum {
    TLG_OK = 0,
    TLG_ERR_INVALID_ARG = -1,  /* bad dimension, enum or flag; C overlaps A or B   */
    TLG_ERR_UNSUPPORTED = -2,  /* valid request this library does not implement  */
    TLG_ERR_NULL = -3,         /* null plan, output handle or data pointer        */
    TLG_ERR_MISALIGNED = -4,   /* pointer not aligned as the plan requires        */
    TLG_ERR_HIP = -5,          /* the HIP runtime reported an error at launch     */
    TLG_ERR_NOMEM = -6,        /* host allocation of the plan failed              */
    TLG_ERR_TOO_LARGE = -7     /* tlg_gemm_run_noalloc: the request needs more scratch
                                  than the library's static buffer holds           */
} tlg_status;

/* Plan facts, for tests and the benchmark. */
typedef struct {
    int32_t variant;       /* tlg_variant actually chosen                            */
    int32_t block_m, block_n, block_k;
    int32_t stages;        /* LDS ring depth                                          */
    int32_t threads;       /* work-items per workgroup                                */
    int32_t vec_a, vec_b;  /* elements per global load of A / B (8 = 128-bit, 1 = 16-bit) */
    int64_t grid;          /* workgroups per launch                                   */
    int64_t lds_bytes;     /* LDS bytes per workgroup                                 */
    int32_t k_tiles;       /* trips of the K loop per workgroup (at most)             */
    int32_t splits;        /* workgroups per output tile along K (1: no split)        */
    int64_t workspace_bytes; /* device workspace the plan owns (0 unless splits > 1 or stream-K) */
    int32_t dp_tiles;      /* stream-K plans: output tiles computed whole (the first waves)  */
    int32_t sk_tiles;      /* stream-K plans: output tiles shared out by K iterations         */
} tlg_plan_info;

/*
 * Create a plan for C[M,N] = act(A·B).
 *
 * create / run / destroy are this library's counterpart of the host wrapper the
 * pages' compiler generates around a tile program ("NVIDIA backend codegen"
 * chapter, section 4.2 "host/device split and wrapper generation": an extern "C"
 * init() that does the one-time set-up and an extern "C" call() that launches
 * the kernel on the caller's stream, both returning an int status).  Here the
 * one-time part is create (validation, variant choice, launch geometry, the
 * workspace of a split-K plan) and the launch part is run.  The argument checks
 * that the pages' generated host stub performs before a launch (overview page,
 * "automatically generated host checks": null data pointers, dtypes, shapes,
 * alignment/contiguity assumptions) are performed by create (sizes, enums,
 * flags) and run (pointers, alignment, overlap, device) and reported as a
 * status instead of a launch.
 *
 *   M, N, K      : 0 <= M, N <= 2^24, 0 <= K <= 2^22.  M or N == 0 is a no-op plan;
 *                  K == 0 gives C = act(clear_accum ? 0 : C) (the empty sum).
 *   ab_dtype     : TLG_F16 or TLG_BF16 (A and B); TLG_E4M3 / TLG_E5M2 for the
 *                  block-scaled GEMM (see tlg_gemm_run_mx).
 *   c_dtype      : TLG_F16, TLG_BF16 or TLG_F32.
 *   transpose_A  : 0 -> A stored [M,K];  1 -> A stored [K,M].
 *   transpose_B  : 0 -> B stored [K,N];  1 -> B stored [N,K].
 *   clear_accum  : 1 -> start from zero; 0 -> add onto C's prior contents.
 *   epilogue     : TLG_EPI_NONE or TLG_EPI_RELU.
 * Returns TLG_ERR_NULL if out is NULL, TLG_ERR_INVALID_ARG for a bad dimension,
 * enum or flag, TLG_ERR_UNSUPPORTED for an operand dtype other than F16/BF16 (or a
 * block-scaled request other than the one tlg_gemm_run_mx describes),
 * TLG_ERR_NOMEM if the plan cannot be allocated.  Plans with K split over
 * several workgroups per tile (tlg_plan_info.splits > 1, chosen for output grids
 * of fewer than 128 tiles of 128x128 with at least 48 K tiles of 64, and for the
 * skinny kernel when it has fewer than 256 blocks of outputs and at least
 * 8 K stages of 256) allocate a device workspace here
 * (tlg_plan_info.workspace_bytes: fp32 partial tiles plus one counter per tile),
 * on the device current at the call, zero its counters and wait for that to
 * finish (TLG_ERR_HIP if any of it fails); other plans do no device work.  On
 * failure *out is set to NULL.
 */
tlg_status tlg_gemm_create(tlg_gemm_t *out, int64_t M, int64_t N, int64_t K,
                           int32_t ab_dtype, int32_t c_dtype, int32_t transpose_A,
                           int32_t transpose_B, int32_t clear_accum, int32_t epilogue);

/*
 * Fill *info with the plan that tlg_gemm_create_variant (variant ==
 * TLG_VARIANT_AUTO: tlg_gemm_create) would make for these arguments, without
 * making it: host work only, no device is needed.  Lets a caller learn the
 * chosen variant, launch grid and workspace size in advance.  Returns the
 * status create would return for the same arguments, except that it never
 * returns TLG_ERR_HIP or TLG_ERR_NOMEM; TLG_ERR_NULL for a NULL info.
 */
tlg_status tlg_gemm_select(tlg_plan_info *info, int64_t M, int64_t N, int64_t K,
                           int32_t ab_dtype, int32_t c_dtype, int32_t transpose_A,
                           int32_t transpose_B, int32_t clear_accum, int32_t epilogue,
                           int32_t variant);

/*
 * As tlg_gemm_create, but forces a kernel variant (tlg_variant).  Returns
 * TLG_ERR_UNSUPPORTED when the forced variant cannot run the request (the
 * skinny variant needs transpose_A == 0, transpose_B == 1 and K % 8 == 0;
 * TILE_64_DMA and TILE_32_DMA need transpose_A == 0, and with transpose_B == 0
 * N <= 8454656, so that a direct load's lane offset, up to 127 rows of B apart,
 * stays below 2^31).
 */
tlg_status tlg_gemm_create_variant(tlg_gemm_t *out, int64_t M, int64_t N, int64_t K,
                                   int32_t ab_dtype, int32_t c_dtype, int32_t transpose_A,
                                   int32_t transpose_B, int32_t clear_accum, int32_t epilogue,
                                   int32_t variant);

/*
 * Enqueue C = act(A·B) on `stream` (a hipStream_t; NULL is the null stream): the
 * launch half of the host wrapper (codegen chapter, section 4.2.2: call() runs
 * the host checks, then launches on the given stream and returns a status).
 *   A, B : device pointers to the packed operands (read only).  May be NULL only
 *          when K == 0 or M*N == 0.
 *   C    : device pointer to the packed M x N output (read when clear_accum == 0).
 * A and B must be aligned to their element size, and to 16 bytes when the plan
 * uses 128-bit loads for them (tlg_plan_info.vec_a / vec_b == 8), except that
 * the direct-load variants (TILE_256_DMA, TILE_128_DMA, TILE_128_DMA_SPLITK, TILE_64_DMA, TILE_32_DMA and
 * the stream-K variants) take K-contiguous
 * operands (A with transpose_A == 0, B with transpose_B == 1) at element
 * alignment and any K; C to its element size.  C must not overlap A or B.
 * Returns TLG_ERR_NULL, TLG_ERR_MISALIGNED, TLG_ERR_INVALID_ARG (overlap) or
 * TLG_ERR_HIP (launch failure); TLG_OK once the kernel is queued.  Execution
 * errors surface on the stream, as for any HIP kernel.
 * Plans without a workspace may run concurrently on several streams.  A plan
 * with a workspace (splits > 1) must run on the device it was created on
 * (TLG_ERR_INVALID_ARG otherwise), and its runs must not overlap in time: they
 * share the workspace, so issue them on one stream or order them by events.
 */
tlg_status tlg_gemm_run(tlg_gemm_t plan, const void *A, const void *B, void *C, void *stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): plan and run in one call,
 * allocating nothing.  Same arguments and result as tlg_gemm_create (automatic
 * variant) followed by tlg_gemm_run of that plan; the same kernel runs, so C is
 * bit-identical to that pair's.
 *
 * The plan is built on the stack and discarded.  When the automatic choice splits
 * K (tlg_plan_info.splits > 1), its fp32 partial tiles and per-tile counters live
 * in a static device buffer of the library instead of a plan workspace: 16 MiB of
 * partial tiles plus 4 KiB of counters, one copy per GPU, held until the process
 * ends.  The automatic choice always fits (it splits only grids of fewer than 128
 * tiles of 128 x 128, into at most 256 partial tiles, and skinny grids of fewer
 * than 256 blocks, into at most 256 partial blocks of 4 or 8 KiB); a request that would
 * need more is refused with TLG_ERR_TOO_LARGE.  The first call on a device looks up
 * the buffer's device address and enqueues a small kernel on `stream` that zeroes
 * the counters; every split-K launch returns the counters it uses to zero.
 *
 * All calls on one GPU share that GPU's buffer, which keeps the last call's
 * contents: two calls whose split-K launches overlap in time on one GPU (on
 * different streams, or one captured in a graph replayed concurrently with
 * another) race on it and give wrong results; order them on one stream or by
 * events.  Calls whose automatic plan does not split K use no scratch and may
 * overlap freely.
 *
 * Errors: those of tlg_gemm_create (except TLG_ERR_NOMEM) and tlg_gemm_run, plus
 * TLG_ERR_UNSUPPORTED for block-scaled dtypes (use tlg_gemm_run_mx) or a device
 * index of 64 or more, TLG_ERR_TOO_LARGE as above.  Nothing is enqueued on error.
 */
tlg_status tlg_gemm_run_noalloc(int64_t M, int64_t N, int64_t K, int32_t ab_dtype, int32_t c_dtype,
                                int32_t transpose_A, int32_t transpose_B, int32_t clear_accum,
                                int32_t epilogue, const void *A, const void *B, void *C, void *stream);

/*
 * Block-scaled ("MX") GEMM: the block-scaled MMA of the codegen chapter
 * (sections 3.4 and 4.6.3, MXFP8 / MXFP4): FP8 or FP4 elements in which every 32
 * consecutive elements along K share one E8M0 scale factor, fp32 accumulation.
 * A plan is made by tlg_gemm_create with ab_dtype TLG_E4M3, TLG_E5M2 or TLG_E2M1
 * (both operands in that format), transpose_A = 0 and transpose_B = 1, and K a
 * multiple of 128; any other combination is refused with TLG_ERR_UNSUPPORTED (a
 * scaled operand is never run without its scales).  Value computed:
 *   acc(m,n) = (clear_accum ? 0 : (float)C[m*N + n])
 *              + sum_k (A[m*K + k] * 2^(SA[m*(K/32) + k/32] - 127))
 *                      * (B[n*K + k] * 2^(SB[n*(K/32) + k/32] - 127))
 *   C[m*N + n] = convert_rne(epilogue == RELU ? max(acc, +0) : acc)
 * where A[.] and B[.] are decoded as E4M3 (1 sign, 4 exponent bits with bias 7,
 * 3 fraction bits, no infinity), E5M2 (IEEE-style, 5/2 bits, bias 15) or E2M1
 * (1 sign, 2 exponent bits with bias 1, 1 fraction bit, no infinity or NaN;
 * element k of a row in the low nibble of byte k/2 when k is even, the high
 * nibble when odd).
 *   A  : device pointer, M x K bytes (M x K/2 for E2M1), row-major (16-byte aligned).
 *   SA : device pointer, M x K/32 E8M0 bytes (4-byte aligned).
 *   B  : device pointer, N x K bytes (N x K/2 for E2M1), row-major (16-byte aligned).
 *   SB : device pointer, N x K/32 E8M0 bytes (4-byte aligned).
 *   C  : as for tlg_gemm_run.
 * Returns TLG_ERR_INVALID_ARG for a plan that is not block-scaled (or C
 * overlapping an input), TLG_ERR_NULL, TLG_ERR_MISALIGNED, TLG_ERR_HIP; TLG_OK
 * once the kernel is queued.  tlg_gemm_run refuses block-scaled plans with
 * TLG_ERR_INVALID_ARG, and tlg_gemm_tune refuses block-scaled requests with
 * TLG_ERR_UNSUPPORTED.  NaN scales or elements: unspecified.
 */
tlg_status tlg_gemm_run_mx(tlg_gemm_t plan, const void *A, const void *SA, const void *B,
                           const void *SB, void *C, void *stream);

/* One timed candidate of tlg_gemm_tune. */
typedef struct {
    int32_t variant;   /* tlg_variant */
    int32_t splits;    /* K ranges per output tile (split-K variant, split skinny plans), else 1 */
    float ms;          /* average time of one run, milliseconds */
} tlg_tune_result;

/*
 * Autotune (the pages' autotuner: overview page, "autotuning" section): make a
 * plan for the same request as tlg_gemm_create, choosing the kernel variant,
 * and for the split-K variant the number of K ranges, by timing every
 * candidate that can serve the request on the caller's buffers.  Candidates:
 * the fp16/bf16 variants of tlg_variant (TILE_256_DMA, TILE_128_DMA, TILE_64_DMA,
 * TILE_32_DMA, SKINNY, TILE_256_W8, TILE_256, TILE_128, TILE_256_DMA_STREAMK,
 * TILE_128_DMA_STREAMK), and the split-K variant with 2..8
 * ranges when the output has fewer than 256 tiles of 128 x 128 (block-scaled
 * requests are refused, see tlg_gemm_run_mx).  A candidate
 * that refuses the request (TLG_ERR_UNSUPPORTED) or the buffers' alignment
 * (TLG_ERR_MISALIGNED) is skipped.
 *   A, B, C, stream : as for tlg_gemm_run.  C is overwritten, and with
 *                     clear_accum == 0 its prior contents are lost (the runs
 *                     accumulate into it).
 *   iters           : timed runs per candidate, 1..1000, after one untimed run.
 *   results         : receives up to max_results entries (may be NULL when
 *                     max_results == 0), one per candidate timed, in the order
 *                     timed; *n_results (may be NULL) gets the number written.
 * The choice is cached per (current device, M, N, K, dtypes, flags, epilogue,
 * whether each of A, B and C is 16-byte aligned) for the life of the process: a later call with the same key times nothing
 * (*n_results = 0) and returns a new plan of the cached choice.  The choice
 * depends on timings and so may differ between processes.  Synchronises the
 * stream.  Returns the errors of tlg_gemm_create and tlg_gemm_run,
 * TLG_ERR_INVALID_ARG for iters or max_results out of range, TLG_ERR_HIP if
 * timing fails.  On failure *out is set to NULL.
 */
tlg_status tlg_gemm_tune(tlg_gemm_t *out, int64_t M, int64_t N, int64_t K,
                         int32_t ab_dtype, int32_t c_dtype, int32_t transpose_A,
                         int32_t transpose_B, int32_t clear_accum, int32_t epilogue,
                         const void *A, const void *B, void *C, void *stream, int32_t iters,
                         tlg_tune_result *results, int32_t max_results, int32_t *n_results);

/*
 * Attention forward with online softmax: the FlashAttention tile program of the
 * handbook page "TileLang: a tile language one level below Triton", section
 * "FlashAttention: online softmax as tile code".
 *
 * Value computed, for every batch b, head h and query position i (0 <= i < seq):
 *   keys allowed:  j in [0, seq), and j <= i when causal != 0 (the page's rule)
 *   s_j  = softmax_scale * sum_d Q[b,i,h,d] * K[b,j,h,d]          (fp32)
 *   O[b,i,h,:] = convert_rne( sum_j p_j V[b,j,h,:] / sum_j p_j ),
 *   p_j  = exp(s_j - m), rounded to the operand type before the second product
 *          (the page rounds its probability tile to fp16), fp32 sums; m is a
 *          reference maximum that the kernel keeps within 8 (log2 units) below
 *          max_j s_j * log2(e), so p_j <= 256 and O is the softmax whatever m is.
 * The page's scale is 1/sqrt(dim); the caller passes it (any finite value).
 *
 * Layout: Q, K, V and O are dense [batch, seq, heads, dim] tensors; element
 * (b, t, h, d) sits at ((b*seq + t)*heads + h)*dim + d.  All four share dtype
 * (TLG_F16 or TLG_BF16) and must be 16-byte aligned.  dim must be 64 or 128.
 * seq * heads * dim * 2 must stay below 2^31 bytes (per-batch offsets are 32-bit).
 * O must not overlap Q, K or V (Q, K and V may overlap each other).
 *
 * Ownership: the caller owns all four tensors (device memory) and keeps them
 * alive until the queued work has finished.  The call allocates nothing, does
 * not synchronise and enqueues at most one kernel on `stream`; calls with
 * disjoint outputs may overlap.  batch, seq or heads == 0 enqueues nothing.
 *
 * Errors: TLG_ERR_INVALID_ARG (negative sizes, dim <= 0, causal not 0/1,
 * non-finite scale, unknown dtype, O overlapping an input), TLG_ERR_UNSUPPORTED
 * (dim other than 64/128, FP32 or FP8 operands, sizes past the limits above),
 * TLG_ERR_NULL (a null tensor with non-empty sizes), TLG_ERR_MISALIGNED,
 * TLG_ERR_HIP (launch failure).  Nothing is enqueued on error.
 */
tlg_status tlg_attn_fwd(const void *Q, const void *K, const void *V, void *O, int64_t batch, int64_t seq,
                        int64_t heads, int64_t dim, int32_t dtype, int32_t causal, float softmax_scale,
                        void *stream);

/*
 * The number of queries one workgroup of tlg_attn_fwd takes for this shape
 * (host only, no device needed): 128, or 64 when blocks of 128 queries would
 * number at most 256 over all (batch, head) pairs (a grid too small to give
 * every CU a workgroup), or at most 1024 with causal != 0 and dim == 64.  The
 * choice changes no result: every query's sums are formed in the same order
 * either way.  0 for a non-positive batch, seq or heads.
 */
int32_t tlg_attn_query_block(int64_t batch, int64_t seq, int64_t heads, int64_t dim, int32_t causal);

/*
 * As tlg_attn_fwd, with the number of queries per workgroup given: block_q = 64
 * or 128, or 0 for the choice of tlg_attn_query_block (tlg_attn_fwd is this call
 * with 0).  O does not depend on it; it is there for tests and tuning.  Returns
 * TLG_ERR_INVALID_ARG for any other block_q, else as tlg_attn_fwd.
 */
tlg_status tlg_attn_fwd_block(const void *Q, const void *K, const void *V, void *O, int64_t batch,
                              int64_t seq, int64_t heads, int64_t dim, int32_t dtype, int32_t causal,
                              float softmax_scale, int32_t block_q, void *stream);

/*
 * Dequant GEMM with 4-bit weights: the "dequant GEMM" of the overview page's
 * table of representative operators (load packed weights, apply scale and zero
 * point, convert, then multiply).  Shaped for decoding (few rows of A, one
 * stream of the weights per 16 rows of A).
 *
 * Value computed, for 0 <= m < M, 0 <= n < N:
 *   w(n,k)   = convert_rne((q(n,k) - Z[n*(K/G) + k/G]) * S[n*(K/G) + k/G])   (operand dtype)
 *   acc(m,n) = sum_k A[m*K + k] * w(n,k)                                   (fp32 accumulate)
 *   C[m*N + n] = convert_rne(epilogue == RELU ? max(acc, +0) : acc)
 * Weight format: q(n,k) in 0..15 are stored [N, K/2] bytes; the eight codes of
 * k = 8j .. 8j+7 of row n form the little-endian 32-bit word at bytes 4j..4j+3 of
 * the row, code k = 8j + i at bits 4*(i/2) .. +3 for even i and at bits
 * 16 + 4*(i/2) .. +3 for odd i.  S [N, K/G] holds scales in the operand dtype, Z
 * [N, K/G] zero points (uint8, any value 0..255).
 *
 * A [M, K], S and C are dense row-major.  ab_dtype (A and S) in {TLG_F16,
 * TLG_BF16}; c_dtype in {TLG_F16, TLG_BF16, TLG_F32}; epilogue NONE or RELU.
 * Limits: G a positive multiple of 32, K % G == 0, K / G <= 255, M and N <= 2^24.
 * A and Wq must be 16-byte aligned, S 2-byte aligned, C aligned to its element.
 * C must not overlap A, Wq, S or Z.
 *
 * Ownership as tlg_gemm_run: the caller owns all buffers; the call allocates
 * nothing, does not synchronise and enqueues at most one kernel on `stream`.
 * M == 0 or N == 0 enqueues nothing.  Errors: TLG_ERR_INVALID_ARG (sizes,
 * enums, group, overlap), TLG_ERR_UNSUPPORTED (K / G > 255), TLG_ERR_NULL,
 * TLG_ERR_MISALIGNED, TLG_ERR_HIP.  Nothing is enqueued on error.
 */
tlg_status tlg_gemm_w4(const void *A, const void *Wq, const void *S, const void *Z, void *C, int64_t M, int64_t N,
                       int64_t K, int64_t G, int32_t ab_dtype, int32_t c_dtype, int32_t epilogue, void *stream);

/*
 * 2:4 structured-sparse GEMM: the pages' T.gemm_sp (a "2:4 structured sparse
 * GEMM" on the hardware's sparse matrix instructions; overview page, table of
 * compute primitives), here on gfx950's v_smfmac_f32_16x16x64.  The sparse
 * operand is the weight matrix W [N, K] of C = act(A W^T): every group of four
 * consecutive k of a row holds two stored values (the others are zero).
 *
 * Format: Wv [N, K/2] holds the stored values in the operand dtype, two per
 * group in order (Wv[n*(K/2) + 2q], Wv[n*(K/2) + 2q + 1] for group q, which
 * covers k = 4q .. 4q+3).  Wm [N, K/8] bytes hold their positions inside the
 * group: byte n*(K/8) + q/2 carries group q's first position at bits
 * 4*(q%2) .. +1 and its second at bits 4*(q%2) + 2 .. +3.  Two values at one
 * position add.
 *
 * Value computed, for 0 <= m < M, 0 <= n < N:
 *   acc(m,n) = sum_k A[m*K + k] * w(n,k)      (fp32 accumulate)
 *   C[m*N + n] = convert_rne(epilogue == RELU ? max(acc, +0) : acc)
 * A [M, K] and C are dense row-major.  ab_dtype (A and Wv) in {TLG_F16,
 * TLG_BF16}; c_dtype in {TLG_F16, TLG_BF16, TLG_F32}; epilogue NONE or RELU.
 * Limits: K % 64 == 0 (whole K tiles), M and N <= 2^24, K <= 2^22.  A and Wv
 * must be 16-byte aligned, Wm 4-byte aligned, C aligned to its element; C must
 * not overlap A, Wv or Wm.
 *
 * Ownership as tlg_gemm_run: the call allocates nothing, does not synchronise
 * and enqueues at most one kernel on `stream`.  M == 0 or N == 0 enqueues
 * nothing; K == 0 writes act(0).  Errors: TLG_ERR_INVALID_ARG (sizes, enums,
 * overlap), TLG_ERR_UNSUPPORTED (K % 64 != 0), TLG_ERR_NULL, TLG_ERR_MISALIGNED,
 * TLG_ERR_HIP.  Nothing is enqueued on error.
 */
tlg_status tlg_gemm_sp(const void *A, const void *Wv, const void *Wm, void *C, int64_t M, int64_t N, int64_t K,
                       int32_t ab_dtype, int32_t c_dtype, int32_t epilogue, void *stream);

/* Release a plan (and its workspace, if any; the caller first makes sure no run of
 * the plan is still in flight).  NULL is accepted (no-op, TLG_OK).  The pages'
 * generated wrapper has no counterpart (its module lives as long as the
 * process); a plan here owns host memory and possibly a device workspace, so it
 * is released explicitly. */
tlg_status tlg_gemm_destroy(tlg_gemm_t plan);

/* Fill *info with the plan's launch facts.  TLG_ERR_NULL for a NULL argument. */
tlg_status tlg_gemm_query(tlg_gemm_t plan, tlg_plan_info *info);

/* Human-readable one-line description of a plan (static storage owned by the plan). */
const char *tlg_gemm_describe(tlg_gemm_t plan);

/* Name of a status code (static string). */
const char *tlg_status_string(int32_t status);

/* Library version string (static). */
const char *tlg_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TLG_H */
