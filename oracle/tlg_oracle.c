/*
 * CPU oracle for the tiled dense GEMM  C = act(A·B)  — TEST INFRASTRUCTURE ONLY.
 * Further sections below hold the block-scaled (MX) GEMM, the attention
 * forward pass, the 4-bit dequant GEMM and the 2:4 structured-sparse GEMM,
 * each with its own statement of what it computes.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
 * load this library.  It shares no code, header, table or helper with the HIP
 * path: it has its own IEEE-754 binary16 / bfloat16 decoders and its own
 * round-to-nearest-even encoder, written from the format definitions.
 *
 * What it computes (plain definition, double precision, ascending k):
 *
 *   a(m,k) = dec(transpose_A ? A[k*M + m] : A[m*K + k])
 *   b(k,n) = dec(transpose_B ? B[n*K + k] : B[k*N + n])
 *   s(m,n) = (clear_accum ? 0 : dec_c(C_in[m*N + n])) + sum_{k=0}^{K-1} a(m,k) * b(k,n)
 *   o(m,n) = relu ? (s > 0 ? s : +0.0) : s
 *
 * Passages followed:
 *   - the tile program (grid of block_M x block_N output tiles, K loop of
 *     block_K steps, gemm into an fp32 fragment, copy back to C):
 *     "NVIDIA backend codegen" chapter, section 1 (origin of the problem);
 *     handbook page "TileLang: a tile language one level below Triton",
 *     section "first kernel: GEMM".  Tiling and pipelining do not change the
 *     mathematical result, so the oracle is the untiled sum.
 *   - fp16 inputs, fp32 accumulation, conversion back to the output dtype:
 *     overview page "TileLang: from tile dataflow to controllable AI kernels",
 *     section "minimal but complete GEMM skeleton".  The oracle keeps the sum
 *     in double; the comparison tolerance absorbs the fp32 accumulation.
 *   - transpose_A / transpose_B only change which dimension is M/N and which is
 *     K; clear_accum starts from zero instead of C's prior contents; the
 *     accumulator type is C's fragment type: "core primitives" chapter,
 *     section 3.3 (T.gemm).
 *   - T.clear is T.fill(..., 0): "core primitives" chapter, section 3.6.
 *   - ReLU is max(x, 0) applied to the fp32 tile before it is written out:
 *     "core primitives" chapter, section 3.8 (the GEMM+ReLU chain) and
 *     section 4.6.  Non-positive values give +0.0; NaN gives +0.0 (reading of
 *     an unspecified case; "parity unpinned" for NaN, which no workload makes).
 *   - out-of-bounds source elements read as the safe value 0 and stores
 *     outside C are skipped: "core primitives" chapter, section 4.2.  The
 *     untiled sum never touches padding, which is exactly what zero fill
 *     must reproduce.
 *
 * Output conversion (oracle_encode) is IEEE round-to-nearest-even with
 * overflow to infinity; the pages name no rounding mode for the cast that
 * the copy inserts, and this is the plain reading.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_F16 = 1, ORACLE_BF16 = 2, ORACLE_F32 = 3 };

/* ---------------------------------------------------------------------------
 * Decoders, from the interchange-format definitions.
 *   binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 *   bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits.
 *   binary32: 1 sign, 8 exponent (bias 127), 23 fraction bits.
 * Exponent field 0 -> subnormal  frac * 2^(1 - bias - p);
 * all ones -> Inf (frac == 0) or NaN; otherwise (2^p + frac) * 2^(e - bias - p).
 * ------------------------------------------------------------------------- */
static double dec_ieee(uint32_t bits, int p, int ebits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const uint32_t frac = bits & ((1u << p) - 1u);
    const uint32_t e = (bits >> p) & ((1u << ebits) - 1u);
    const int neg = (bits >> (p + ebits)) & 1u;
    double v;
    if (e == 0)
        v = ldexp((double)frac, 1 - bias - p);
    else if (e == (1u << ebits) - 1u)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)((1u << p) + frac), (int)e - bias - p);
    return neg ? -v : v;
}

static double dec(int dtype, uint32_t bits)
{
    switch (dtype) {
    case ORACLE_F16: return dec_ieee(bits & 0xffffu, 10, 5);
    case ORACLE_BF16: return dec_ieee(bits & 0xffffu, 7, 8);
    default: return dec_ieee(bits, 23, 8);
    }
}

/* Round-half-to-even of a non-negative double below 2^53 (all steps exact). */
static double round_half_even(double q)
{
    double fl = floor(q);
    double d = q - fl;
    if (d > 0.5) return fl + 1.0;
    if (d < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* Encode a double into a format with p fraction bits and ebits exponent bits,
 * rounding to nearest, ties to even; overflow gives infinity; NaN gives the
 * positive quiet NaN. */
static uint32_t enc_ieee(double x, int p, int ebits)
{
    const int bias = (1 << (ebits - 1)) - 1;
    const int emin = 1 - bias, emax = bias;
    const uint32_t sign = signbit(x) ? (1u << (p + ebits)) : 0u;
    const uint32_t expall = ((1u << ebits) - 1u) << p;
    if (isnan(x)) return expall | (1u << (p - 1));
    if (isinf(x)) return sign | expall;
    double a = fabs(x);
    if (a == 0.0) return sign;
    int e;
    (void)frexp(a, &e);
    e -= 1;                           /* a in [2^e, 2^(e+1)) */
    if (e < emin) e = emin;           /* subnormal: fixed quantum 2^(emin-p) */
    double q = ldexp(a, p - e);       /* exact power-of-two scaling, q < 2^(p+1) */
    double r = round_half_even(q);
    uint32_t ri = (uint32_t)r;
    if (ri == (2u << p)) { ri = 1u << p; e += 1; }
    if (e > emax) return sign | expall;
    if (ri < (1u << p)) return sign | ri;                 /* subnormal or zero */
    return sign | ((uint32_t)(e + bias) << p) | (ri - (1u << p));
}

static uint32_t enc(int dtype, double x)
{
    switch (dtype) {
    case ORACLE_F16: return enc_ieee(x, 10, 5);
    case ORACLE_BF16: return enc_ieee(x, 7, 8);
    default: return enc_ieee(x, 23, 8);
    }
}

static int valid_dtype(int d) { return d == ORACLE_F16 || d == ORACLE_BF16 || d == ORACLE_F32; }

/* Fetch of the stored prior value of C(m,n) (16- or 32-bit patterns). */
static uint32_t c_bits(const void *C_in, int c_dtype, int64_t idx)
{
    if (c_dtype == ORACLE_F32) return ((const uint32_t *)C_in)[idx];
    return ((const uint16_t *)C_in)[idx];
}

/* ---------------------------------------------------------------------------
 * Full GEMM over the output rows [m0, m1).
 * The operands are first decoded to double (a as an M-major row per m, b stored
 * per column n so that both inner reads are contiguous).  Storage order of the
 * decoded values does not change any arithmetic: every s(m,n) is the sum of the
 * same products in ascending k.
 * ------------------------------------------------------------------------- */
struct job {
    int64_t M, N, K, m0, m1;
    int ab, cd, tA, tB, clear, relu;
    const uint16_t *A;
    const double *bcol;   /* N x K decoded b, bcol[n*K + k] = b(k, n) */
    const void *C_in;
    double *out;          /* (m1-m0) x N */
    int64_t r_begin, r_end;
};

static void *run_rows(void *arg)
{
    struct job *j = (struct job *)arg;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    if (!arow) return (void *)1;
    for (int64_t m = j->r_begin; m < j->r_end; ++m) {
        for (int64_t k = 0; k < j->K; ++k) {
            uint16_t bits = j->tA ? j->A[k * j->M + m] : j->A[m * j->K + k];
            arow[k] = dec(j->ab, bits);
        }
        for (int64_t n = 0; n < j->N; ++n) {
            double s = j->clear ? 0.0 : dec(j->cd, c_bits(j->C_in, j->cd, m * j->N + n));
            const double *bc = j->bcol + n * j->K;
            for (int64_t k = 0; k < j->K; ++k)
                s += arow[k] * bc[k];
            if (j->relu) s = (s > 0.0) ? s : 0.0;
            j->out[(m - j->m0) * j->N + n] = s;
        }
    }
    free(arow);
    return NULL;
}

/* Returns 0 on success, -1 on bad arguments, -2 on allocation failure. */
int oracle_gemm_rows(int64_t M, int64_t N, int64_t K, int ab_dtype, int c_dtype,
                     int transpose_A, int transpose_B, int clear_accum, int relu,
                     const uint16_t *A, const uint16_t *B, const void *C_in,
                     int64_t m0, int64_t m1, double *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || m0 < 0 || m1 < m0 || m1 > M) return -1;
    if (ab_dtype != ORACLE_F16 && ab_dtype != ORACLE_BF16) return -1;
    if (!valid_dtype(c_dtype)) return -1;
    if (!clear_accum && !C_in && M * N > 0) return -1;
    if (m1 == m0 || N == 0) return 0;
    if (K > 0 && (!A || !B)) return -1;
    if (nthreads < 1) nthreads = 1;

    double *bcol = (double *)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
    if (!bcol) return -2;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) {
            uint16_t bits = transpose_B ? B[n * K + k] : B[k * N + n];
            bcol[n * K + k] = dec(ab_dtype, bits);
        }

    int64_t rows = m1 - m0;
    if (nthreads > rows) nthreads = (int)rows;
    struct job *jobs = (struct job *)calloc((size_t)nthreads, sizeof(struct job));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(bcol); free(jobs); free(th); return -2; }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        struct job *j = &jobs[t];
        j->M = M; j->N = N; j->K = K; j->m0 = m0; j->m1 = m1;
        j->ab = ab_dtype; j->cd = c_dtype; j->tA = transpose_A; j->tB = transpose_B;
        j->clear = clear_accum; j->relu = relu;
        j->A = A; j->bcol = bcol; j->C_in = C_in; j->out = out;
        j->r_begin = m0 + rows * t / nthreads;
        j->r_end = m0 + rows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run_rows, &jobs[t]) != 0) { rc = -2; th[t] = 0; }
    if (run_rows(&jobs[0]) != NULL) rc = -2;
    for (int t = 1; t < nthreads; ++t) {
        void *ret = NULL;
        if (th[t]) { pthread_join(th[t], &ret); if (ret) rc = -2; }
        else run_rows(&jobs[t]);
    }
    free(bcol); free(jobs); free(th);
    return rc;
}

int oracle_gemm(int64_t M, int64_t N, int64_t K, int ab_dtype, int c_dtype,
                int transpose_A, int transpose_B, int clear_accum, int relu,
                const uint16_t *A, const uint16_t *B, const void *C_in,
                double *out, int nthreads)
{
    return oracle_gemm_rows(M, N, K, ab_dtype, c_dtype, transpose_A, transpose_B,
                            clear_accum, relu, A, B, C_in, 0, M, out, nthreads);
}

/* The same definition evaluated at selected output coordinates (pm[i], pn[i]),
 * decoding each operand element where it is used. */
int oracle_gemm_points(int64_t M, int64_t N, int64_t K, int ab_dtype, int c_dtype,
                       int transpose_A, int transpose_B, int clear_accum, int relu,
                       const uint16_t *A, const uint16_t *B, const void *C_in,
                       int64_t npts, const int64_t *pm, const int64_t *pn, double *out)
{
    if (M < 0 || N < 0 || K < 0 || npts < 0) return -1;
    if (ab_dtype != ORACLE_F16 && ab_dtype != ORACLE_BF16) return -1;
    if (!valid_dtype(c_dtype)) return -1;
    for (int64_t i = 0; i < npts; ++i) {
        int64_t m = pm[i], n = pn[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double s = clear_accum ? 0.0 : dec(c_dtype, c_bits(C_in, c_dtype, m * N + n));
        for (int64_t k = 0; k < K; ++k) {
            uint16_t ab = transpose_A ? A[k * M + m] : A[m * K + k];
            uint16_t bb = transpose_B ? B[n * K + k] : B[k * N + n];
            s += dec(ab_dtype, ab) * dec(ab_dtype, bb);
        }
        if (relu) s = (s > 0.0) ? s : 0.0;
        out[i] = s;
    }
    return 0;
}

/* Element-wise format conversions exposed for the comparisons. */
int oracle_decode(int dtype, const uint32_t *bits, int64_t n, double *out)
{
    if (!valid_dtype(dtype) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = dec(dtype, bits[i]);
    return 0;
}

int oracle_encode(int dtype, const double *x, int64_t n, uint32_t *bits)
{
    if (!valid_dtype(dtype) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) bits[i] = enc(dtype, x[i]);
    return 0;
}

/* ===========================================================================
 * Block-scaled ("MX") GEMM: the codegen chapter's block-scaled MMA (sections
 * 3.4 and 4.6.3): low-precision elements in which every 32 consecutive
 * elements along K share one power-of-two scale factor (E8M0), fp32
 * accumulation.  Element formats, from their definitions:
 *   E4M3: 1 sign, 4 exponent (bias 7), 3 fraction bits; exponent field 0 is
 *         subnormal (frac * 2^-9); S.1111.111 is NaN; there is no infinity
 *         (largest finite 1.75 * 2^8 = 448).
 *   E5M2: 1 sign, 5 exponent (bias 15), 2 fraction bits, IEEE-style:
 *         subnormal at field 0, Inf / NaN at field 31.
 *   E2M1 (the 4-bit element of MXFP4): 1 sign, 2 exponent (bias 1), 1 fraction
 *         bit; exponent field 0 is subnormal (frac * 2^-1); no infinity or NaN
 *         (largest 1.5 * 2^2 = 6).  Two elements per byte: element k of a row is
 *         the low nibble of byte k/2 when k is even, the high nibble when odd.
 *   E8M0 (scale): an 8-bit biased exponent, value 2^(e - 127); 255 is NaN.
 * Value computed (A stored [M, K], B stored [N, K], both K-contiguous, as the
 * pages' "1d1d" block-scaled example has it; E2M1 rows hold K/2 bytes):
 *   a(m,k) = elem(A, m, k) * 2^(SA[m*(K/32) + k/32] - 127)
 *   b(k,n) = elem(B, n, k) * 2^(SB[n*(K/32) + k/32] - 127)
 *   s(m,n) = (clear_accum ? 0 : C_in(m,n)) + sum_k a(m,k) * b(k,n)   (double)
 *   o(m,n) = relu ? max(s, +0) : s
 * K must be a multiple of 32 (whole scale blocks).  NaN inputs: parity unpinned.
 * ======================================================================== */
enum { ORACLE_E4M3 = 10, ORACLE_E5M2 = 11, ORACLE_E8M0 = 12, ORACLE_E2M1 = 13 };

static double dec_e4m3(uint32_t b)
{
    const uint32_t frac = b & 7u, e = (b >> 3) & 15u;
    const int neg = (b >> 7) & 1u;
    double v;
    if (e == 15u && frac == 7u) return NAN;
    if (e == 0) v = ldexp((double)frac, 1 - 7 - 3);
    else v = ldexp((double)(8u + frac), (int)e - 7 - 3);
    return neg ? -v : v;
}

static double dec_e5m2(uint32_t b) { return dec_ieee(b & 0xffu, 2, 5); }

static double dec_e2m1(uint32_t b)
{
    const uint32_t frac = b & 1u, e = (b >> 1) & 3u;
    const int neg = (b >> 3) & 1u;
    const double v = e == 0 ? ldexp((double)frac, 1 - 1 - 1) : ldexp((double)(2u + frac), (int)e - 1 - 1);
    return neg ? -v : v;
}

static double dec_e8m0(uint32_t b)
{
    b &= 0xffu;
    return b == 255u ? NAN : ldexp(1.0, (int)b - 127);
}

static double dec_mx(int fmt, uint32_t b)
{
    switch (fmt) {
    case ORACLE_E4M3: return dec_e4m3(b);
    case ORACLE_E5M2: return dec_e5m2(b);
    case ORACLE_E2M1: return dec_e2m1(b);
    default: return dec_e8m0(b);
    }
}

static int valid_elem_fmt(int f) { return f == ORACLE_E4M3 || f == ORACLE_E5M2 || f == ORACLE_E2M1; }

/* Element k of row r of an MX operand with K elements per row: one byte per
 * element for the 8-bit formats, two per byte (low nibble first) for E2M1. */
static double mx_elem(int fmt, const uint8_t *X, int64_t K, int64_t r, int64_t k)
{
    if (fmt == ORACLE_E2M1) {
        const uint32_t byte = X[r * (K / 2) + k / 2];
        return dec_e2m1((k & 1) ? byte >> 4 : byte & 15u);
    }
    return dec_mx(fmt, X[r * K + k]);
}

struct mxjob {
    int64_t M, N, K, m0;
    int cd, clear, relu, fa;
    const uint8_t *A, *SA;
    const double *bcol;   /* N x K decoded and scaled b: bcol[n*K + k] = b(k, n) */
    const void *C_in;
    double *out;
    int64_t r_begin, r_end;
};

static void *run_mx_rows(void *arg)
{
    struct mxjob *j = (struct mxjob *)arg;
    const int64_t KB = j->K / 32;
    double *arow = (double *)malloc(sizeof(double) * (size_t)(j->K > 0 ? j->K : 1));
    if (!arow) return (void *)1;
    for (int64_t m = j->r_begin; m < j->r_end; ++m) {
        for (int64_t k = 0; k < j->K; ++k)
            arow[k] = mx_elem(j->fa, j->A, j->K, m, k) * dec_e8m0(j->SA[m * KB + k / 32]);
        for (int64_t n = 0; n < j->N; ++n) {
            const double prior = j->clear ? 0.0 : dec(j->cd, c_bits(j->C_in, j->cd, m * j->N + n));
            const double *bc = j->bcol + n * j->K;
            double s = prior;
            for (int64_t kk = 0; kk < j->K; ++kk)
                s += arow[kk] * bc[kk];
            if (j->relu && !(s > 0.0)) s = 0.0;
            j->out[(m - j->m0) * j->N + n] = s;
        }
    }
    free(arow);
    return NULL;
}

/* Output rows [m0, m1) of the block-scaled GEMM.  Returns 0 on success, -1 on
 * bad arguments, -2 on allocation failure. */
int oracle_mxgemm_rows(int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b, int c_dtype, int clear_accum,
                       int relu, const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                       const void *C_in, int64_t m0, int64_t m1, double *out, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || m0 < 0 || m1 < m0 || m1 > M) return -1;
    if (!valid_elem_fmt(fmt_a) || !valid_elem_fmt(fmt_b) || !valid_dtype(c_dtype)) return -1;
    if (!clear_accum && !C_in && M * N > 0) return -1;
    if (m1 == m0 || N == 0) return 0;
    if (K > 0 && (!A || !SA || !B || !SB)) return -1;
    if (nthreads < 1) nthreads = 1;
    const int64_t KB = K / 32;
    double *bcol = (double *)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
    if (!bcol) return -2;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            bcol[n * K + k] = mx_elem(fmt_b, B, K, n, k) * dec_e8m0(SB[n * KB + k / 32]);
    int64_t rows = m1 - m0;
    if (nthreads > rows) nthreads = (int)rows;
    struct mxjob *jobs = (struct mxjob *)calloc((size_t)nthreads, sizeof(struct mxjob));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(bcol); free(jobs); free(th); return -2; }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        struct mxjob *j = &jobs[t];
        j->M = M; j->N = N; j->K = K; j->m0 = m0;
        j->cd = c_dtype; j->clear = clear_accum; j->relu = relu; j->fa = fmt_a;
        j->A = A; j->SA = SA; j->bcol = bcol; j->C_in = C_in; j->out = out;
        j->r_begin = m0 + rows * t / nthreads;
        j->r_end = m0 + rows * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run_mx_rows, &jobs[t]) != 0) { rc = -2; th[t] = 0; }
    if (run_mx_rows(&jobs[0]) != NULL) rc = -2;
    for (int t = 1; t < nthreads; ++t) {
        void *ret = NULL;
        if (th[t]) { pthread_join(th[t], &ret); if (ret) rc = -2; }
        else run_mx_rows(&jobs[t]);
    }
    free(bcol); free(jobs); free(th);
    return rc;
}

/* The same definition at selected output coordinates (pm[i], pn[i]). */
int oracle_mxgemm_points(int64_t M, int64_t N, int64_t K, int fmt_a, int fmt_b, int c_dtype, int clear_accum,
                         int relu, const uint8_t *A, const uint8_t *SA, const uint8_t *B, const uint8_t *SB,
                         const void *C_in, int64_t npts, const int64_t *pm, const int64_t *pn, double *out)
{
    if (M < 0 || N < 0 || K < 0 || K % 32 != 0 || npts < 0) return -1;
    if (!valid_elem_fmt(fmt_a) || !valid_elem_fmt(fmt_b) || !valid_dtype(c_dtype)) return -1;
    const int64_t KB = K / 32;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t m = pm[i], n = pn[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double s = clear_accum ? 0.0 : dec(c_dtype, c_bits(C_in, c_dtype, m * N + n));
        for (int64_t k = 0; k < K; ++k)
            s += (mx_elem(fmt_a, A, K, m, k) * dec_e8m0(SA[m * KB + k / 32])) *
                 (mx_elem(fmt_b, B, K, n, k) * dec_e8m0(SB[n * KB + k / 32]));
        if (relu) s = (s > 0.0) ? s : 0.0;
        out[i] = s;
    }
    return 0;
}

/* Decode of E4M3 / E5M2 / E8M0 bytes, or of E2M1 codes (one code 0..15 per byte),
 * for the comparisons and the pins. */
int oracle_mx_decode(int fmt, const uint8_t *bytes, int64_t n, double *out)
{
    if ((!valid_elem_fmt(fmt) && fmt != ORACLE_E8M0) || n < 0) return -1;
    for (int64_t i = 0; i < n; ++i) out[i] = dec_mx(fmt, bytes[i]);
    return 0;
}

/* ===========================================================================
 * Attention forward (the FlashAttention tile program of the handbook page
 * "TileLang: a tile language one level below Triton", section "FlashAttention:
 * online softmax as tile code").  The tile program walks the keys in blocks
 * and keeps a running row maximum and row sum; that online rescaling reaches
 * the ordinary softmax exactly (up to rounding), so the oracle is the plain
 * definition, in double:
 *
 *   element (b, t, h, d) of Q, K, V and O sits at ((b*S + t)*H + h)*D + d
 *   keys allowed for query i:  j in [0, S), and j <= i when causal
 *   s_j   = scale * sum_d q(b,i,h,d) * k(b,j,h,d)
 *   w_j   = exp(s_j - max_j s_j)
 *   o(d)  = sum_j w_j * v(b,j,h,d) / sum_j w_j
 *
 * The page folds log2(e) into its scale and uses exp2; exp2(x*log2 e) is
 * exp(x), so the oracle uses exp with the plain scale (the page sets
 * scale = 1/sqrt(dim); here it is an input).  The causal rule is the page's:
 * a query at position i sees the keys at positions j <= i.  Subtracting the
 * row maximum changes nothing mathematically and keeps exp finite.
 * ======================================================================== */
struct attnjob {
    int64_t S, H, D, i0, i1;
    int dt, causal;
    double scale;
    const uint16_t *Q, *K, *V;
    double *out;            /* [B, i1-i0, H, D] */
    int64_t w_begin, w_end; /* work items: (b, i, h) flattened over [B, i1-i0, H] */
};

static void attn_row(const struct attnjob *j, int64_t b, int64_t i, int64_t h, double *s, double *o)
{
    const int64_t S = j->S, H = j->H, D = j->D;
    const int64_t nkeys = j->causal ? i + 1 : S;
    const uint16_t *q = j->Q + ((b * S + i) * H + h) * D;
    double mx = -INFINITY;
    for (int64_t t = 0; t < nkeys; ++t) {
        const uint16_t *k = j->K + ((b * S + t) * H + h) * D;
        double dot = 0.0;
        for (int64_t d = 0; d < D; ++d) dot += dec(j->dt, q[d]) * dec(j->dt, k[d]);
        s[t] = j->scale * dot;
        if (s[t] > mx) mx = s[t];
    }
    double denom = 0.0;
    for (int64_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t t = 0; t < nkeys; ++t) {
        const double w = exp(s[t] - mx);
        const uint16_t *v = j->V + ((b * S + t) * H + h) * D;
        denom += w;
        for (int64_t d = 0; d < D; ++d) o[d] += w * dec(j->dt, v[d]);
    }
    for (int64_t d = 0; d < D; ++d) o[d] /= denom;
}

static void *run_attn(void *arg)
{
    struct attnjob *j = (struct attnjob *)arg;
    double *s = (double *)malloc(sizeof(double) * (size_t)(j->S > 0 ? j->S : 1));
    if (!s) return (void *)1;
    const int64_t rows = j->i1 - j->i0;
    for (int64_t w = j->w_begin; w < j->w_end; ++w) {
        const int64_t h = w % j->H, r = (w / j->H) % rows, b = w / (j->H * rows);
        attn_row(j, b, j->i0 + r, h, s, j->out + ((b * rows + r) * j->H + h) * j->D);
    }
    free(s);
    return NULL;
}

static int attn_args_ok(int64_t B, int64_t S, int64_t H, int64_t D, int dtype, double scale)
{
    return B >= 0 && S >= 0 && H >= 0 && D > 0 && (dtype == ORACLE_F16 || dtype == ORACLE_BF16) && isfinite(scale);
}

/* Query positions [i0, i1) of every batch and head.  Returns 0 on success, -1 on
 * bad arguments, -2 on allocation failure. */
int oracle_attn_rows(int64_t B, int64_t S, int64_t H, int64_t D, int dtype, int causal, double scale,
                     const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t i0, int64_t i1,
                     double *out, int nthreads)
{
    if (!attn_args_ok(B, S, H, D, dtype, scale) || i0 < 0 || i1 < i0 || i1 > S) return -1;
    const int64_t items = B * (i1 - i0) * H;
    if (items == 0) return 0;
    if (!Q || !K || !V || !out) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > items) nthreads = (int)items;
    struct attnjob *jobs = (struct attnjob *)calloc((size_t)nthreads, sizeof(struct attnjob));
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return -2; }
    int rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        struct attnjob *j = &jobs[t];
        j->S = S; j->H = H; j->D = D; j->i0 = i0; j->i1 = i1;
        j->dt = dtype; j->causal = causal != 0; j->scale = scale;
        j->Q = Q; j->K = K; j->V = V; j->out = out;
        j->w_begin = items * t / nthreads;
        j->w_end = items * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        if (pthread_create(&th[t], NULL, run_attn, &jobs[t]) != 0) { rc = -2; th[t] = 0; }
    if (run_attn(&jobs[0]) != NULL) rc = -2;
    for (int t = 1; t < nthreads; ++t) {
        void *ret = NULL;
        if (th[t]) { pthread_join(th[t], &ret); if (ret) rc = -2; }
        else if (run_attn(&jobs[t]) != NULL) rc = -2;
    }
    free(jobs); free(th);
    return rc;
}

/* The same definition for the output rows (pb[n], pi[n], ph[n]); out is [npts, D]. */
int oracle_attn_points(int64_t B, int64_t S, int64_t H, int64_t D, int dtype, int causal, double scale,
                       const uint16_t *Q, const uint16_t *K, const uint16_t *V, int64_t npts,
                       const int64_t *pb, const int64_t *pi, const int64_t *ph, double *out)
{
    if (!attn_args_ok(B, S, H, D, dtype, scale) || npts < 0) return -1;
    if (npts == 0) return 0;
    if (!Q || !K || !V || !out || !pb || !pi || !ph) return -1;
    struct attnjob j;
    memset(&j, 0, sizeof j);
    j.S = S; j.H = H; j.D = D; j.dt = dtype; j.causal = causal != 0; j.scale = scale;
    j.Q = Q; j.K = K; j.V = V;
    double *s = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    if (!s) return -2;
    for (int64_t n = 0; n < npts; ++n) {
        if (pb[n] < 0 || pb[n] >= B || pi[n] < 0 || pi[n] >= S || ph[n] < 0 || ph[n] >= H) { free(s); return -1; }
        attn_row(&j, pb[n], pi[n], ph[n], s, out + n * D);
    }
    free(s);
    return 0;
}

/* ===========================================================================
 * Dequant GEMM (the pages' table of representative operators, "dequant GEMM":
 * load packed weights, apply scale and zero point, convert, then multiply).
 * Weight format read here (the pages name the steps, not a format):
 *   - W is N x K 4-bit unsigned codes q(n, k) in 0..15, stored [N, K/2] bytes;
 *     the 8 codes of k = 8w .. 8w+7 of a row form one little-endian 32-bit word
 *     (bytes 4w .. 4w+3 of the row), in which code k = 8w + j sits at bits
 *     4*(j/2) .. +3 for even j and at bits 16 + 4*(j/2) .. +3 for odd j (even
 *     codes in the low half-word, odd codes in the high half-word);
 *   - per row n and group g of G consecutive k: a scale s(n, g) in the operand
 *     dtype (fp16 / bf16 bits, [N, K/G]) and a zero point z(n, g) (uint8, [N, K/G]);
 *   - the weight is the operand-type value nearest (ties to even) to
 *     (q - z) * s; the multiplication then runs on those values:
 *       c(m, n) = sum_k a(m, k) * w(n, k)      (double, ascending k)
 *       o(m, n) = relu ? max(c, +0) : c
 * ======================================================================== */
static uint32_t w4_code(const uint8_t *row, int64_t k)
{
    const int64_t w = k / 8;
    const int j = (int)(k % 8);
    const uint32_t word = (uint32_t)row[4 * w] | ((uint32_t)row[4 * w + 1] << 8) |
                          ((uint32_t)row[4 * w + 2] << 16) | ((uint32_t)row[4 * w + 3] << 24);
    const int shift = (j % 2 == 0) ? 4 * (j / 2) : 16 + 4 * (j / 2);
    return (word >> shift) & 15u;
}

static double w4_weight(int dt, const uint8_t *Wq, const uint16_t *S, const uint8_t *Z, int64_t K, int64_t G,
                        int64_t n, int64_t k)
{
    const int64_t KG = K / G;
    const double q = (double)w4_code(Wq + n * (K / 2), k);
    const double z = (double)Z[n * KG + k / G];
    const double s = dec(dt, S[n * KG + k / G]);
    return dec(dt, enc(dt, (q - z) * s));
}

static int w4_args_ok(int64_t M, int64_t N, int64_t K, int64_t G, int dt)
{
    return M >= 0 && N >= 0 && K >= 0 && G > 0 && K % G == 0 && K % 8 == 0 &&
           (dt == ORACLE_F16 || dt == ORACLE_BF16);
}

/* Dequantized weights w(n, k) as doubles, [N, K]. */
int oracle_w4_dequant(int64_t N, int64_t K, int64_t G, int ab_dtype, const uint8_t *Wq, const uint16_t *S,
                      const uint8_t *Z, double *out)
{
    if (!w4_args_ok(0, N, K, G, ab_dtype)) return -1;
    if (N * K == 0) return 0;
    if (!Wq || !S || !Z || !out) return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) out[n * K + k] = w4_weight(ab_dtype, Wq, S, Z, K, G, n, k);
    return 0;
}

/* Output rows [m0, m1) of C = act(A W^T); A [M, K] 16-bit bits of ab_dtype. */
int oracle_w4gemm_rows(int64_t M, int64_t N, int64_t K, int64_t G, int ab_dtype, int relu, const uint16_t *A,
                       const uint8_t *Wq, const uint16_t *S, const uint8_t *Z, int64_t m0, int64_t m1, double *out)
{
    if (!w4_args_ok(M, N, K, G, ab_dtype) || m0 < 0 || m1 < m0 || m1 > M) return -1;
    if (m1 == m0 || N == 0) return 0;
    if (K > 0 && (!A || !Wq || !S || !Z)) return -1;
    double *w = (double *)malloc(sizeof(double) * (size_t)(N * (K > 0 ? K : 1)));
    double *arow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!w || !arow) { free(w); free(arow); return -2; }
    if (K > 0) oracle_w4_dequant(N, K, G, ab_dtype, Wq, S, Z, w);
    for (int64_t m = m0; m < m1; ++m) {
        for (int64_t k = 0; k < K; ++k) arow[k] = dec(ab_dtype, A[m * K + k]);
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            const double *wr = w + n * K;
            for (int64_t k = 0; k < K; ++k) acc += arow[k] * wr[k];
            if (relu && !(acc > 0.0)) acc = 0.0;
            out[(m - m0) * N + n] = acc;
        }
    }
    free(w); free(arow);
    return 0;
}

/* The same definition at selected outputs (pm[i], pn[i]), dequantizing each weight where used. */
int oracle_w4gemm_points(int64_t M, int64_t N, int64_t K, int64_t G, int ab_dtype, int relu, const uint16_t *A,
                         const uint8_t *Wq, const uint16_t *S, const uint8_t *Z, int64_t npts, const int64_t *pm,
                         const int64_t *pn, double *out)
{
    if (!w4_args_ok(M, N, K, G, ab_dtype) || npts < 0) return -1;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t m = pm[i], n = pn[i];
        if (m < 0 || m >= M || n < 0 || n >= N) return -1;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += dec(ab_dtype, A[m * K + k]) * w4_weight(ab_dtype, Wq, S, Z, K, G, n, k);
        if (relu && !(acc > 0.0)) acc = 0.0;
        out[i] = acc;
    }
    return 0;
}

/* ===========================================================================
 * 2:4 structured-sparse GEMM (the pages' T.gemm_sp: "2:4 structured sparse
 * GEMM" in the overview page's table of compute primitives, tied there to the
 * hardware's sparse matrix instructions).  Reading used here: the sparse
 * operand is the weight matrix W [N, K] of C = act(A W^T), given compressed:
 *   - every group of four consecutive k of a row holds two stored values,
 *     Wv[n, 2q] and Wv[n, 2q+1] for group q (Wv is [N, K/2] in the operand dtype);
 *   - their positions inside the group, two 2-bit fields per value pair, in
 *     Wm [N, K/8] bytes: byte n*(K/8) + q/2 holds group q's positions at bits
 *     4*(q%2) (first value) and 4*(q%2) + 2 (second value);
 *   - the dense w(n, k) is the sum of the stored values whose position is k
 *     (two values at one position add; positions without a value are zero).
 *   c(m, n) = sum_k a(m, k) * w(n, k)      (double, ascending k)
 *   o(m, n) = relu ? max(c, +0) : c
 * ======================================================================== */
static void sp_expand_row(int dt, const uint16_t *Wv, const uint8_t *Wm, int64_t K, int64_t n, double *w)
{
    for (int64_t k = 0; k < K; ++k) w[k] = 0.0;
    for (int64_t q = 0; q < K / 4; ++q) {
        const uint32_t byte = Wm[n * (K / 8) + q / 2];
        const int sh = 4 * (int)(q % 2);
        const int p0 = (int)((byte >> sh) & 3u), p1 = (int)((byte >> (sh + 2)) & 3u);
        w[4 * q + p0] += dec(dt, Wv[n * (K / 2) + 2 * q]);
        w[4 * q + p1] += dec(dt, Wv[n * (K / 2) + 2 * q + 1]);
    }
}

static int sp_args_ok(int64_t M, int64_t N, int64_t K, int dt)
{
    return M >= 0 && N >= 0 && K >= 0 && K % 8 == 0 && (dt == ORACLE_F16 || dt == ORACLE_BF16);
}

/* Dense w(n, k), [N, K]. */
int oracle_sp_expand(int64_t N, int64_t K, int ab_dtype, const uint16_t *Wv, const uint8_t *Wm, double *out)
{
    if (!sp_args_ok(0, N, K, ab_dtype)) return -1;
    if (N * K == 0) return 0;
    if (!Wv || !Wm || !out) return -1;
    for (int64_t n = 0; n < N; ++n) sp_expand_row(ab_dtype, Wv, Wm, K, n, out + n * K);
    return 0;
}

/* Output rows [m0, m1) of C = act(A W^T). */
int oracle_spgemm_rows(int64_t M, int64_t N, int64_t K, int ab_dtype, int relu, const uint16_t *A,
                       const uint16_t *Wv, const uint8_t *Wm, int64_t m0, int64_t m1, double *out)
{
    if (!sp_args_ok(M, N, K, ab_dtype) || m0 < 0 || m1 < m0 || m1 > M) return -1;
    if (m1 == m0 || N == 0) return 0;
    if (K > 0 && (!A || !Wv || !Wm)) return -1;
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    double *arow = (double *)malloc(sizeof(double) * (size_t)((m1 - m0) * (K > 0 ? K : 1)));
    if (!w || !arow) { free(w); free(arow); return -2; }
    for (int64_t m = m0; m < m1; ++m)
        for (int64_t k = 0; k < K; ++k) arow[(m - m0) * K + k] = dec(ab_dtype, A[m * K + k]);
    for (int64_t n = 0; n < N; ++n) {
        sp_expand_row(ab_dtype, Wv, Wm, K, n, w);
        for (int64_t m = m0; m < m1; ++m) {
            double acc = 0.0;
            const double *ar = arow + (m - m0) * K;
            for (int64_t k = 0; k < K; ++k) acc += ar[k] * w[k];
            if (relu && !(acc > 0.0)) acc = 0.0;
            out[(m - m0) * N + n] = acc;
        }
    }
    free(w); free(arow);
    return 0;
}

/* The same definition at selected outputs (pm[i], pn[i]). */
int oracle_spgemm_points(int64_t M, int64_t N, int64_t K, int ab_dtype, int relu, const uint16_t *A,
                         const uint16_t *Wv, const uint8_t *Wm, int64_t npts, const int64_t *pm,
                         const int64_t *pn, double *out)
{
    if (!sp_args_ok(M, N, K, ab_dtype) || npts < 0) return -1;
    double *w = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
    if (!w) return -2;
    for (int64_t i = 0; i < npts; ++i) {
        const int64_t m = pm[i], n = pn[i];
        if (m < 0 || m >= M || n < 0 || n >= N) { free(w); return -1; }
        sp_expand_row(ab_dtype, Wv, Wm, K, n, w);
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) acc += dec(ab_dtype, A[m * K + k]) * w[k];
        if (relu && !(acc > 0.0)) acc = 0.0;
        out[i] = acc;
    }
    free(w);
    return 0;
}
