/*
 * CPU oracle for the skinny BF16 decode projection -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg may
 * call this code.  It shares nothing with the HIP library: its own BF16
 * decoding, its own loops, no GPU headers.
 *
 * What it computes (definition on the pages):
 *   out[m][n] = sum_k x[m][k] * W[n][k]       for m < M, n < N
 * i.e. out[M, N] = x[M, K] @ weight[N, K]^T -- the docstring of class
 * PreparedWarpSplitK on the page "vllm.models.kimi_k3.nvidia.specialized_decode.
 * cutedsl.gemm.warp_splitk", and "x @ weight.T" in class Projection on the page
 * "vllm.models.glm5next.nvidia.specialized_decode.gemm".  No bias is added: the
 * warp split-K wrapper's run() notes that the kernel never reads its bias
 * argument.  x and W are packed row-major BF16 (same docstring: "packed
 * row-major").
 *
 * Besides O it returns S[m][n] = sum_k |x[m][k] * W[n][k]|, which scales the
 * parity tolerance (|gpu - O| <= 1e-3 * S + 1e-6 for fp32 output).
 *
 * The _t entry points take the input type: BF16 (f16 = 0) or FP16 (f16 = 1),
 * the two weight types class PreparedProjection accepts on the page
 * "vllm.models.kimi_k3.nvidia.specialized_decode.cutedsl.gemm.projection".
 * Every FP16 value is also exactly a double, and a product of two has at most
 * 22 significant bits, so the same precision argument holds.
 *
 * Precision: every BF16 value is exactly a double; every product of two BF16
 * values has at most 16 significant bits and is exact in double; the sums are
 * taken in double with k ascending.  For K <= 2^20 and the value ranges used,
 * the rounding error is below K * 2^-53 * S, far under the tolerance.
 *
 * Parity pins for this file live in tests/test_oracle.py (brute force against
 * Python integers, one-hot closed forms, linearity, NumPy float64).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* BF16 is the upper half of an IEEE binary32: widen by a 16-bit shift. */
static double bf16_to_double(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/*
 * IEEE 754 binary16: sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent 0 is zero or subnormal (fraction * 2^-24); exponent 31 is
 * infinity (fraction 0) or NaN; otherwise (1024 + fraction) * 2^(e - 25).
 */
static double f16_to_double(uint16_t bits)
{
    const int sign = bits >> 15, e = (bits >> 10) & 0x1F, f = bits & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

static double to_double(uint16_t bits, int f16) { return f16 ? f16_to_double(bits) : bf16_to_double(bits); }

/* Decode a BF16 or FP16 matrix into doubles (rows * cols values). */
static double *decode(const uint16_t *src, long rows, long cols, int f16)
{
    double *dst = (double *)malloc(sizeof(double) * (size_t)(rows * cols));
    if (!dst)
        return NULL;
    for (long i = 0; i < rows * cols; ++i)
        dst[i] = to_double(src[i], f16);
    return dst;
}

/*
 * Full product.  x: [M][K] bits, w: [N][K] bits, row-major, BF16 (f16 = 0)
 * or FP16 (f16 = 1).  o, s: [M][N] doubles (s may be NULL).  Returns 0, or -1
 * on bad sizes or allocation failure.
 */
int oracle_gemm_t(const uint16_t *x, const uint16_t *w, int M, int N, int K, int f16,
                  double *o, double *s)
{
    if (M < 0 || N < 0 || K < 0 || (M > 0 && N > 0 && (!x || !w || !o)))
        return -1;
    if (M == 0 || N == 0)
        return 0;
    double *xd = decode(x, M, K, f16);
    if (!xd)
        return -1;
    int failed = 0;
#pragma omp parallel
    {
        double *wrow = (double *)malloc(sizeof(double) * (size_t)(K > 0 ? K : 1));
        if (!wrow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int n = 0; n < N; ++n) {
                for (int k = 0; k < K; ++k)
                    wrow[k] = to_double(w[(long)n * K + k], f16);
                for (int m = 0; m < M; ++m) {
                    const double *xr = xd + (long)m * K;
                    double acc = 0.0, mag = 0.0;
                    for (int k = 0; k < K; ++k) {
                        double p = xr[k] * wrow[k];
                        acc += p;
                        mag += fabs(p);
                    }
                    o[(long)m * N + n] = acc;
                    if (s)
                        s[(long)m * N + n] = mag;
                }
            }
            free(wrow);
        }
    }
    free(xd);
    return failed ? -1 : 0;
}

/* BF16 inputs. */
int oracle_gemm(const uint16_t *x, const uint16_t *w, int M, int N, int K,
                double *o, double *s)
{
    return oracle_gemm_t(x, w, M, N, K, 0, o, s);
}

/*
 * Selected elements only: for i < count, element (mi[i], ni[i]) of the same
 * product.  Lets large shapes be checked on a sample.
 */
int oracle_gemm_sampled_t(const uint16_t *x, const uint16_t *w, int M, int N, int K, int f16,
                          const int *mi, const int *ni, long count,
                          double *o, double *s)
{
    if (M < 0 || N < 0 || K < 0 || count < 0)
        return -1;
    for (long i = 0; i < count; ++i)
        if (mi[i] < 0 || mi[i] >= M || ni[i] < 0 || ni[i] >= N)
            return -1;
#pragma omp parallel for schedule(static)
    for (long i = 0; i < count; ++i) {
        const uint16_t *xr = x + (long)mi[i] * K;
        const uint16_t *wr = w + (long)ni[i] * K;
        double acc = 0.0, mag = 0.0;
        for (int k = 0; k < K; ++k) {
            double p = to_double(xr[k], f16) * to_double(wr[k], f16);
            acc += p;
            mag += fabs(p);
        }
        o[i] = acc;
        if (s)
            s[i] = mag;
    }
    return 0;
}

int oracle_gemm_sampled(const uint16_t *x, const uint16_t *w, int M, int N, int K,
                        const int *mi, const int *ni, long count,
                        double *o, double *s)
{
    return oracle_gemm_sampled_t(x, w, M, N, K, 0, mi, ni, count, o, s);
}

/*
 * Round doubles to BF16 bit patterns, to nearest with ties to even, in one
 * step from the double (no intermediate binary32 rounding).  Used to state the
 * expected BF16 output where the exact value is known.  NaN maps to a quiet
 * NaN; values past the largest finite BF16 go to infinity.
 */
void oracle_round_bf16(const double *v, long count, uint16_t *out)
{
    for (long i = 0; i < count; ++i) {
        double a = v[i];
        uint16_t sign = signbit(a) ? 0x8000u : 0u;
        if (isnan(a)) {
            out[i] = 0x7FC0u;
            continue;
        }
        a = fabs(a);
        if (isinf(a)) {
            out[i] = sign | 0x7F80u;
            continue;
        }
        if (a == 0.0) {
            out[i] = sign;
            continue;
        }
        /* BF16: 8 significant bits for normals (exponent >= -126), a fixed
         * quantum of 2^-133 for subnormals. */
        int e;
        frexp(a, &e);                 /* a = f * 2^e, f in [0.5, 1) */
        int q_exp = e - 8;            /* quantum 2^(e-8) keeps 8 bits */
        if (q_exp < -133)
            q_exp = -133;
        double scaled = ldexp(a, -q_exp);   /* exact: a power-of-two scale */
        double fl = floor(scaled);
        double rem = scaled - fl;
        double r = fl;
        if (rem > 0.5 || (rem == 0.5 && fmod(fl, 2.0) != 0.0))
            r = fl + 1.0;
        double rounded = ldexp(r, q_exp);
        if (rounded >= 0x1p128) {          /* beyond the BF16 range */
            out[i] = sign | 0x7F80u;
            continue;
        }
        /* Re-encode: rounded is exactly representable in binary32. */
        float f = (float)rounded;
        uint32_t u;
        memcpy(&u, &f, sizeof u);
        out[i] = sign | (uint16_t)(u >> 16);
    }
}

/* Widen BF16 bit patterns to doubles (exact). */
void oracle_decode_bf16(const uint16_t *bits, long count, double *out)
{
    for (long i = 0; i < count; ++i)
        out[i] = bf16_to_double(bits[i]);
}

/* Widen FP16 bit patterns to doubles (exact). */
void oracle_decode_f16(const uint16_t *bits, long count, double *out)
{
    for (long i = 0; i < count; ++i)
        out[i] = f16_to_double(bits[i]);
}

/* Threads later parallel regions use (n >= 1), for timing the oracle on one
 * core next to all of them; without OpenMP there is only one. */
void oracle_set_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* Threads an OpenMP parallel region uses here (for reporting). */
int oracle_threads(void)
{
    int t = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            t = omp_get_num_threads();
#endif
        }
    }
    return t;
}
