/*
 * oracle.c -- the plain, slow CPU oracle for the FP16 GEMM and GEMV.
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

/* Bulk conversions so the Python side can sweep every bit pattern. */
void oracle_f16_to_f64_array(const uint16_t *h, double *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f16_to_f64(h[i]);
}

void oracle_f64_to_f16_array(const double *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_f16_rne(v[i]);
}

static double *decode_matrix(const uint16_t *src, int64_t count)
{
    double *dst = (double *)malloc((size_t)(count > 0 ? count : 1) * sizeof(double));
    if (!dst) return NULL;
    for (int64_t i = 0; i < count; ++i) dst[i] = oracle_f16_to_f64(src[i]);
    return dst;
}

/*
 * GEMM on a chosen set of output rows.
 *   A     [M,K] fp16 bits, row-major
 *   B     [N,K] fp16 bits, row-major
 *   rows  nrows row indices into [0,M); NULL means all rows 0..M-1
 *   D     [nrows, N] fp16 bits, row-major (row r of D is output row rows[r])
 * Returns 0 on success, -1 on a bad argument or out of memory.
 */
int oracle_gemm_f16(const uint16_t *A, const uint16_t *B, uint16_t *D,
                    int64_t M, int64_t N, int64_t K,
                    const int64_t *rows, int64_t nrows, int nthreads)
{
    if (M < 0 || N < 0 || K < 0 || nrows < 0) return -1;
    if (!rows) nrows = M;
    for (int64_t r = 0; rows && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;

    double *Bd = decode_matrix(B, N * K);
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
            for (int64_t k = 0; k < K; ++k) arow[k] = oracle_f16_to_f64(A[m * K + k]);
            for (int64_t n = 0; n < N; ++n) {
                const double *brow = Bd + n * K;
                double sum = 0.0;
                for (int64_t k = 0; k < K; ++k) sum += arow[k] * brow[k];
                D[r * N + n] = oracle_f64_to_f16_rne(sum);
            }
        }
        free(arow);
    }
    free(Bd);
    return status;
}

/*
 * GEMV y = x . W^T.
 *   x [K], W [N,K] row-major, y [N]; fp16 bits.
 */
int oracle_gemv_f16(const uint16_t *x, const uint16_t *W, uint16_t *y,
                    int64_t N, int64_t K, int nthreads)
{
    if (N < 0 || K < 0) return -1;
    if (N == 0) return 0;
    double *xd = decode_matrix(x, K);
    if (!xd) return -1;

#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif

#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        double sum = 0.0;
        for (int64_t k = 0; k < K; ++k) sum += xd[k] * oracle_f16_to_f64(W[n * K + k]);
        y[n] = oracle_f64_to_f16_rne(sum);
    }
    free(xd);
    return 0;
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
