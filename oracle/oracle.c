/*
 * Oracle for C = A * B with bf16 inputs (CPU, float64).
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may call, link or load this file: only
 * the tests, the package smoke check and the benchmark's CPU-baseline leg use it. It shares no
 * code, header, table or helper with the GPU library.
 *
 * What it computes (the plain definition, run in higher precision):
 *   ref[i][j]  = sum over k = 0 .. K-1 of a[i][k] * b[k][j]        in float64
 *   sabs[i][j] = sum over k = 0 .. K-1 of |a[i][k] * b[k][j]|      in float64
 * A is M x K and B is K x N, both row-major bf16 bit patterns with leading dimensions lda, ldb.
 * Each bf16 value widens exactly (bits << 16 is its float32 pattern, and float32 widens exactly to
 * float64); every product of two bf16 values (8 significant bits each) is exact in float64, so the
 * only rounding is the float64 summation, relatively at most about (K-1) * 2^-53 of sabs.
 * Sources: the fp64 reference rule ("Kernel development on sm_120", section 6, "Numerics
 * rules"); checking against a CPU double-precision version (spark-kernels post, "how things are
 * measured"); a full-output comparison with a relative L2 error ("Benchmarks" page of gemm3,
 * "Correctness").
 *
 * Loop order: rows i are split over threads; inside a row the loops run k then j, so each
 * ref[i][j] still receives its K products in ascending k, exactly as the i-j-k triple loop of the
 * definition would add them (bit-identical results; only the order in which different elements
 * are updated changes). No blocking, reassociation or fusion beyond that.
 *
 * The acceptance check (oracle_check) applied to a bf16 result c, widened exactly:
 *   |c - ref| <= 2^-8 * |ref| + 2^-16 * sabs      for every element (NaN or Inf fails), and
 *   ||c - ref||_F / ||ref||_F <= 4e-3             over the whole matrix,
 * with ref the unrounded float64 value. 2^-8 is bf16's unit roundoff (the output rounding) and
 * 2^-16 * sabs covers float32 accumulation in any order.
 *
 * oracle_bf16_rne rounds a float64 to bf16, nearest with ties to even, for the bit-exact pins
 * (integer-valued inputs whose float32 sums are exact).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_VERSION 1

int oracle_version(void) { return ORACLE_VERSION; }

/* Exact bf16 -> float64. */
static double widen(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

double oracle_bf16_to_f64(uint16_t h) { return widen(h); }

/* float64 -> bf16 bits, round to nearest, ties to even, in one step (no float32 double rounding).
 * bf16 has 8 significant bits and float32's exponent range. NaN -> 0x7FC0 (sign kept),
 * overflow -> Inf, results below the smallest normal bf16 are rounded on the subnormal grid
 * (spacing 2^-133). */
uint16_t oracle_bf16_rne(double x) {
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    double a = fabs(x);
    if (isnan(x)) return (uint16_t)(sign | 0x7FC0u);
    if (a == 0.0) return sign;
    if (isinf(x)) return (uint16_t)(sign | 0x7F80u);
    int e;
    (void)frexp(a, &e);               /* a = f * 2^e, f in [0.5, 1) */
    int exp_unbiased = e - 1;         /* a = 1.m * 2^(e-1) */
    int q;                            /* quantum exponent: representable values are n * 2^q */
    if (exp_unbiased >= -126) q = exp_unbiased - 7;   /* normal: 8 significant bits */
    else q = -133;                                    /* subnormal grid */
    double n = ldexp(a, -q);          /* exact: scaling by a power of two */
    double r = nearbyint(n);          /* current rounding mode is nearest-even */
    double v = ldexp(r, q);
    /* re-encode v (exactly representable) as bf16 */
    if (v == 0.0) return sign;
    int e2;
    double f2 = frexp(v, &e2);        /* v = f2 * 2^e2 */
    int be = e2 - 1 + 127;            /* biased exponent */
    if (be >= 255) return (uint16_t)(sign | 0x7F80u);
    uint32_t mant;
    if (be <= 0) {                    /* subnormal: v = mant * 2^-133 */
        mant = (uint32_t)ldexp(v, 133);
        return (uint16_t)(sign | mant);
    }
    mant = (uint32_t)(ldexp(f2, 8)) - 128u;  /* f2 in [0.5,1) -> 8-bit significand 128..255 */
    return (uint16_t)(sign | ((uint32_t)be << 7) | mant);
}

/* Element-wise oracle_bf16_rne over n values. */
void oracle_bf16_rne_array(const double *x, uint16_t *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = oracle_bf16_rne(x[t]);
}

/* Element-wise exact bf16 -> float64 over n values. */
void oracle_bf16_to_f64_array(const uint16_t *h, double *out, int64_t n) {
    for (int64_t t = 0; t < n; ++t) out[t] = widen(h[t]);
}

typedef struct {
    int64_t row0, row1, N, K;
    const uint16_t *A; int64_t lda;
    const uint16_t *B; int64_t ldb;
    double *ref, *sabs; int64_t ldr;
    int64_t out_row0;  /* row of ref/sabs that receives row row0 */
} rows_job;

static void *rows_worker(void *p) {
    const rows_job *j = (const rows_job *)p;
    for (int64_t i = j->row0; i < j->row1; ++i) {
        double *r = j->ref + (i - j->out_row0) * j->ldr;
        double *s = j->sabs ? j->sabs + (i - j->out_row0) * j->ldr : NULL;
        for (int64_t c = 0; c < j->N; ++c) r[c] = 0.0;
        if (s) for (int64_t c = 0; c < j->N; ++c) s[c] = 0.0;
        for (int64_t k = 0; k < j->K; ++k) {
            const double a = widen(j->A[i * j->lda + k]);
            const uint16_t *brow = j->B + k * j->ldb;
            if (s) {
                for (int64_t c = 0; c < j->N; ++c) {
                    const double p = a * widen(brow[c]);
                    r[c] += p;
                    s[c] += fabs(p);
                }
            } else {
                for (int64_t c = 0; c < j->N; ++c) r[c] += a * widen(brow[c]);
            }
        }
    }
    return NULL;
}

/* Rows [row0, row0 + nrows) of ref and sabs (sabs may be NULL). Output row r of ref/sabs holds
 * matrix row row0 + r, with leading dimension ldr. Returns 0, or -1 on a bad argument. */
int oracle_gemm_rows(int64_t row0, int64_t nrows, int64_t N, int64_t K,
                     const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                     double *ref, double *sabs, int64_t ldr, int nthreads) {
    if (row0 < 0 || nrows < 0 || N < 0 || K < 0 || ldr < N) return -1;
    if (K > 0 && (lda < K || ldb < N)) return -1;
    if (nrows == 0 || N == 0) return 0;
    if (!ref || (K > 0 && (!A || !B))) return -1;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    pthread_t *th = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    rows_job *jobs = (rows_job *)calloc((size_t)nthreads, sizeof(rows_job));
    if (!th || !jobs) { free(th); free(jobs); return -1; }
    int64_t per = nrows / nthreads, extra = nrows % nthreads, at = row0;
    for (int t = 0; t < nthreads; ++t) {
        int64_t cnt = per + (t < extra ? 1 : 0);
        jobs[t] = (rows_job){at, at + cnt, N, K, A, lda, B, ldb, ref, sabs, ldr, row0};
        at += cnt;
    }
    for (int t = 1; t < nthreads; ++t) pthread_create(&th[t], NULL, rows_worker, &jobs[t]);
    rows_worker(&jobs[0]);
    for (int t = 1; t < nthreads; ++t) pthread_join(th[t], NULL);
    free(th);
    free(jobs);
    return 0;
}

/* Whole product: ref and sabs are M x N with leading dimension ldr. */
int oracle_gemm(int64_t M, int64_t N, int64_t K,
                const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                double *ref, double *sabs, int64_t ldr, int nthreads) {
    return oracle_gemm_rows(0, M, N, K, A, lda, B, ldb, ref, sabs, ldr, nthreads);
}

/* Individual entries (rows[t], cols[t]) for t < n, one at a time. */
int oracle_gemm_entries(int64_t K, const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb,
                        const int64_t *rows, const int64_t *cols, int64_t n,
                        double *ref, double *sabs) {
    if (K < 0 || n < 0) return -1;
    for (int64_t t = 0; t < n; ++t) {
        double r = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const double p = widen(A[rows[t] * lda + k]) * widen(B[k * ldb + cols[t]]);
            r += p;
            s += fabs(p);
        }
        ref[t] = r;
        if (sabs) sabs[t] = s;
    }
    return 0;
}

typedef struct {
    int64_t checked;        /* elements compared */
    int64_t failures;       /* elements outside the element-wise bound (NaN/Inf included) */
    int64_t nonfinite;      /* NaN or Inf in c */
    int64_t worst_row, worst_col;
    double worst_ratio;     /* max |c-ref| / bound (bound > 0), or +Inf for a failure at bound 0 */
    double err_sq;          /* sum (c - ref)^2 over finite c */
    double ref_sq;          /* sum ref^2 */
} oracle_check_result;

/* Compare a bf16 result c (M x N, ldc) with ref and sabs (M x N, ldr). */
int oracle_check(int64_t M, int64_t N, const uint16_t *C, int64_t ldc,
                 const double *ref, const double *sabs, int64_t ldr,
                 oracle_check_result *out) {
    if (!out || M < 0 || N < 0) return -1;
    memset(out, 0, sizeof *out);
    out->worst_row = out->worst_col = -1;
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            const double c = widen(C[i * ldc + j]);
            const double r = ref[i * ldr + j];
            const double s = sabs[i * ldr + j];
            const double bound = ldexp(fabs(r), -8) + ldexp(s, -16);
            out->checked++;
            out->ref_sq += r * r;
            if (!isfinite(c)) {
                out->nonfinite++;
                out->failures++;
                out->worst_ratio = INFINITY;
                out->worst_row = i; out->worst_col = j;
                continue;
            }
            const double d = fabs(c - r);
            out->err_sq += d * d;
            double ratio;
            if (bound > 0) ratio = d / bound;
            else ratio = (d == 0.0) ? 0.0 : INFINITY;
            if (!(d <= bound)) out->failures++;
            if (ratio > out->worst_ratio || out->worst_row < 0) {
                out->worst_ratio = ratio;
                out->worst_row = i; out->worst_col = j;
            }
        }
    }
    return 0;
}
