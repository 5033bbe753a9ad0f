/*
 * oracle.c -- the plain, slow CPU oracle for the FP16 and BF16 GEMM and GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library, and never calls it.
 *
 * What it computes (the plain definition, written out):
 *
 *   GEMM   D[m,n] = RNE_fp16( sum_{k=0}^{K-1} A[m,k] * B[n,k] )
 *          A [M,K] and B [N,K] row-major (K-contiguous), D [M,N] row-major.
 *          Layout and the fp16-in / fp32-accumulate / fp16-out contract:
 *          "使用 TMA 为 GEMM 建立 Pipeline" (TVM TIRx chapter), step 4
 *          full kernel (A (M,K), B (N,K), D (M,N), fp16) and the Croqtile
 *          tutorial ch. 7 pipelined matmul (lhs [M,K], rhs [N,K]).
 *
 *   GEMV   y[n] = RNE_fp16( sum_{k=0}^{K-1} x[k] * W[n,k] )
 *          W [N,K] row-major as nn.Linear stores it; "Learning TileLang
 *          with GEMV", §01 GEMV and the kernels of §04 (FP32 accumulation,
 *          never FP16: the hazard is spelled out in §5.2 block_split_k).
 *
 * The pages accumulate in FP32; this oracle accumulates in FP64 with k
 * ascending, which is at least as accurate, and rounds once to fp16 with
 * round-to-nearest, ties-to-even (the `_rn` conversion of the SM120 TMA GEMM
 * walk-through, §2.3 epilogue).  fp16 x fp16 products are exact in FP64.
 *
 * The fp16 <-> fp64 conversions are written here from the IEEE 754 binary16
 * definition (1 sign bit, 5 exponent bits with bias 15, 10 fraction bits;
 * subnormals; overflow to infinity), not taken from any library.
 *
 * BF16 (bfloat16: 1 sign bit, 8 exponent bits with bias 127, 7 fraction
 * bits -- the upper half of an IEEE binary32) is the element type of the
 * SM120 walk-through's kernel ("TensorCore_GEMM_with_TMA": nv_bfloat16 A, B
 * and C at §2.2 entrance, FP32 accumulators rounded with
 * __float22bfloat162_rn in the §2.3 kernel's epilogue).  The bf16 GEMM and
 * GEMV are the same definitions with bf16 in and out; their conversions are
 * written here from that format's definition, in the same way.
 *
 * GEMM with a bias and an activation (not defined on the pages, which end
 * their epilogue at the rounded store; this is the plain definition of the
 * usual fused epilogue):
 *
 *          D[m,n] = RNE( act( sum_{k<K} A[m,k] * B[n,k] + bias[n] ) )
 *
 *          bias [N] in the element format, added to every row; act is the
 *          identity (0) or ReLU (1): act(v) = +0 for v < 0, else v (a NaN
 *          stays NaN).  Still one rounding, after the activation.
 *
 * Parallel over output rows with OpenMP; nothing else is reordered, blocked
 * or fused.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---- fp16 decode: binary16 bits -> exact double ------------------------- */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int exp = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (exp == 0) {
        /* zero or subnormal: frac * 2^-24 */
        mag = ldexp((double)frac, -24);
    } else if (exp == 31) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (1024 + frac) * 2^(exp - 15 - 10) */
        mag = ldexp((double)(1024 + frac), exp - 25);
    }
    return sign ? -mag : mag;
}

/* Round a non-negative double that is an exact multiple of 1/2^60 or so to
 * the nearest integer, ties to even.  q is exact here because the callers
 * only scale by powers of two. */
static double round_half_even(double q)
{
    double fl = floor(q);
    double diff = q - fl;
    if (diff > 0.5) return fl + 1.0;
    if (diff < 0.5) return fl;
    /* exactly halfway: pick the even neighbour */
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* ---- fp16 encode: double -> binary16 bits, round to nearest even ------- */
uint16_t oracle_f64_to_f16_rne(double v)
{
    if (isnan(v)) return (uint16_t)0x7e00; /* a quiet NaN */
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    /* Largest finite fp16 is 65504 = (2 - 2^-10) * 2^15.  The next step of
     * the grid would be 65536; the halfway point 65520 rounds to the even
     * neighbour, which is 65536, i.e. overflows to infinity. */
    if (a >= 65520.0) return (uint16_t)(sign | 0x7c00);
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: integer multiple of 2^-24; a count of 1024
         * becomes the smallest normal, which is exactly bit pattern 0x0400 */
        double q = round_half_even(ldexp(a, 24));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;      /* a in [2^E, 2^(E+1)) */
    double q = round_half_even(ldexp(a, 10 - E)); /* in [1024, 2048] */
    if (q >= 2048.0) { /* rounding carried into the next binade */
        q = 1024.0;
        E += 1;
    }
    if (E + 15 >= 31) return (uint16_t)(sign | 0x7c00);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | (uint16_t)((int)q - 1024));
}

/* ---- bf16 decode: bfloat16 bits -> exact double ------------------------ */
double oracle_bf16_to_f64(uint16_t b)
{
    const int sign = (b >> 15) & 1;
    const int exp = (b >> 7) & 0xff;
    const int frac = b & 0x7f;
    double mag;
    if (exp == 0) {
        /* zero or subnormal: frac * 2^(1 - 127 - 7) */
        mag = ldexp((double)frac, -133);
    } else if (exp == 255) {
        mag = frac ? NAN : INFINITY;
    } else {
        /* normal: (128 + frac) * 2^(exp - 127 - 7) */
        mag = ldexp((double)(128 + frac), exp - 134);
    }
    return sign ? -mag : mag;
}

/* ---- bf16 encode: double -> bfloat16 bits, round to nearest even ------- */
uint16_t oracle_f64_to_bf16_rne(double v)
{
    if (isnan(v)) return (uint16_t)0x7fc0; /* a quiet NaN */
    const uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    /* Largest finite bf16 is (2 - 2^-7) * 2^127; halfway to the next grid
     * point 2^128 is (2 - 2^-8) * 2^127, and that tie rounds to the even
     * neighbour 2^128, i.e. to infinity. */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127)) return (uint16_t)(sign | 0x7f80);
    if (a < ldexp(1.0, -126)) {
        /* subnormal range: integer multiple of 2^-133; a count of 128 is
         * the smallest normal, bit pattern 0x0080 */
        double q = round_half_even(ldexp(a, 133));
        return (uint16_t)(sign | (uint16_t)q);
    }
    int e2;
    (void)frexp(a, &e2); /* a = f * 2^e2, f in [0.5, 1) */
    int E = e2 - 1;      /* a in [2^E, 2^(E+1)) */
    double q = round_half_even(ldexp(a, 7 - E)); /* in [128, 256] */
    if (q >= 256.0) { /* rounding carried into the next binade */
        q = 128.0;
        E += 1;
    }
    if (E + 127 >= 255) return (uint16_t)(sign | 0x7f80);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | (uint16_t)((int)q - 128));
}

void oracle_bf16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_bf16_to_f64(h[i]);
}

void oracle_f64_to_bf16_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_bf16_rne(v[i]);
}

/* The element formats: 0 = fp16, 1 = bf16. */
static double decode(int fmt, uint16_t bits)
{
    return fmt ? oracle_bf16_to_f64(bits) : oracle_f16_to_f64(bits);
}

static uint16_t encode(int fmt, double v)
{
    return fmt ? oracle_f64_to_bf16_rne(v) : oracle_f64_to_f16_rne(v);
}

/* Bulk conversions so the Python side can sweep every bit pattern. */
void oracle_f16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_f64_to_f16_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16_rne(v[i]);
}

static double *decode_matrix(int fmt, const uint16_t *src, int64_t count)
{
    double *dst = (double *)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
    if (!dst) return NULL;
    for (int64_t i = 0; i < count; ++i) dst[i] = decode(fmt, src[i]);
    return dst;
}

/*
 * GEMM on a chosen set of output rows, elements in format fmt.
 *   A     [M,K] bits, row-major
 *   B     [N,K] bits, row-major
 *   bias  [N] bits added to every output row before the activation, or NULL
 *   act   0: identity, 1: ReLU
 *   rows  nrows row indices into [0,M); NULL means all rows 0..M-1
 *   D     [nrows, N] bits, row-major (row r of D is output row rows[r])
 * Returns 0 on success, -1 on a bad argument or out of memory.
 */
static int gemm_fmt(int fmt, const uint16_t *A, const uint16_t *B, const uint16_t *bias, int act, uint16_t *D,
                    int64_t M, int64_t N, int64_t K,
                    const int64_t *rows, int64_t nrows, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || act < 0 || act > 1) return -1;
    if (!rows) nrows = M;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;

    double *Bd = decode_matrix(fmt, B, N * K);
    if (!Bd) return -1;
    int status = 0;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel
    {
        double *arow = (double *)malloc((size_t)(K > 0 ? K : 1) * sizeof(double));
        if (!arow) {
#pragma omp atomic write
            status = -1;
        }
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            if (!arow) continue;
            const int64_t m = rows ? rows[r] : r;
            for (int64_t k = 0; k < K; ++k) arow[k] = decode(fmt, A[m * K + k]);
            for (int64_t n = 0; n < N; ++n) {
                const double *brow = Bd + n * K;
                double sum = 0.0;
                for (int64_t k = 0; k < K; ++k) sum += arow[k] * brow[k];
                if (bias) sum += decode(fmt, bias[n]);
                if (act == 1 && sum < 0.0) sum = 0.0;
                D[r * N + n] = encode(fmt, sum);
            }
        }
        free(arow);
    }
    free(Bd);
    return status;
}

int oracle_gemm_f16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                    int64_t M, int64_t N, int64_t K,
                    const int64_t *rows, int64_t nrows, int nthreads)
{
    return gemm_fmt(0, A, B, NULL, 0, D, M, N, K, rows, nrows, nthreads);
}

int oracle_gemm_bf16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                     int64_t M, int64_t N, int64_t K,
                     const int64_t *rows, int64_t nrows, int nthreads)
{
    return gemm_fmt(1, A, B, NULL, 0, D, M, N, K, rows, nrows, nthreads);
}

int oracle_gemm_bias_f16(const uint16_t *A, const uint16_t *B, const uint16_t *bias, int act, uint16_t *D,
                         int64_t M, int64_t N, int64_t K,
                         const int64_t *rows, int64_t nrows, int nthreads)
{
    return gemm_fmt(0, A, B, bias, act, D, M, N, K, rows, nrows, nthreads);
}

int oracle_gemm_bias_bf16(const uint16_t *A, const uint16_t *B, const uint16_t *bias, int act, uint16_t *D,
                          int64_t M, int64_t N, int64_t K,
                          const int64_t *rows, int64_t nrows, int nthreads)
{
    return gemm_fmt(1, A, B, bias, act, D, M, N, K, rows, nrows, nthreads);
}

/*
 * GEMV y = x . W^T, elements in format fmt.
 *   x [K], W [N,K] row-major, y [N]; bits.
 */
static int gemv_fmt(int fmt, const uint16_t *x, const uint16_t *W, uint16_t *y,
                    int64_t N, int64_t K, int nthreads)
{
    if (N < 0 || K < 0) return -1;
    if (N == 0) return 0;
    double *xd = decode_matrix(fmt, x, K);
    if (!xd) return -1;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) sum += xd[k] * decode(fmt, W[n * K + k]);
        y[n] = encode(fmt, sum);
    }
    free(xd);
    return 0;
}

int oracle_gemv_f16(const uint16_t *x, const uint16_t *W, uint16_t *y,
                    int64_t N, int64_t K, int nthreads)
{
    return gemv_fmt(0, x, W, y, N, K, nthreads);
}

int oracle_gemv_bf16(const uint16_t *x, const uint16_t *W, uint16_t *y,
                     int64_t N, int64_t K, int nthreads)
{
    return gemv_fmt(1, x, W, y, N, K, nthreads);
}

/* Threads OpenMP will use by default (for reporting). */
int oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
