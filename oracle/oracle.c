/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the row-wise
 * reduction-reuse operators: softmax, LayerNorm and RMSNorm.
 *
 * TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load this code.  It shares no source, header, table or helper
 * with the HIP library, and the HIP library never calls it.
 *
 * Everything is computed in IEEE double, sequentially along a row, in the order
 * the definitions are written; rows are independent and spread over OpenMP
 * threads (the row loop is the only parallel loop, so each row's arithmetic is
 * identical to a single-threaded run).  Build with -O2 and without fast-math.
 *
 * Source of the operator shapes: the CREDIT paper ("CREDIT: Cost-guided
 * Reduction-reuse with Efficient DSMEM Inter-CTA Tiling"), Sec. III-B, Eq. 1:
 * L sequential reduction stages produce per-row statistics r_1..r_L, and an
 * elementwise function h(x_i, r_1..L) then writes a full-size output.  The
 * three operator bodies are the textbook definitions (the paper cites
 * LayerNorm to Ba et al. and names softmax and RMSNorm without writing them
 * out); the readings taken where the page is silent are:
 *   softmax   : over the last dimension, max-subtracted, no scale or mask;
 *   LayerNorm : biased variance (divide by N), eps inside the square root;
 *   RMSNorm   : mean of squares over N, eps inside the square root, gamma only.
 *
 * Eq. 2 of the same section splits a row into P disjoint slices, reduces each
 * slice to a partial, and combines the partials into the full-row statistic.
 * The oracle_*_partials / oracle_*_merge functions below write that identity
 * out in double so the tests can check it for arbitrary partitions; they are
 * independent of the plain definitions above them.
 */
#include <math.h>
#include <stdint.h>

/* ---------------------------------------------------------------------------
 * Plain definitions (Eq. 1 instances).
 * ------------------------------------------------------------------------- */

/* Softmax: stage 1 r1 = max_i x_i; stage 2 r2 = sum_i exp(x_i - r1);
 * output y_i = exp(x_i - r1) / r2. */
void oracle_softmax(const double *x, double *y, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double m = xr[0];
        for (int64_t i = 1; i < cols; ++i)
            if (xr[i] > m)
                m = xr[i];
        double s = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            s += exp(xr[i] - m);
        for (int64_t i = 0; i < cols; ++i)
            yr[i] = exp(xr[i] - m) / s;
    }
}

/* LayerNorm: stage 1 mu = (1/N) sum_i x_i; stage 2 v = (1/N) sum_i (x_i - mu)^2;
 * output y_i = (x_i - mu) / sqrt(v + eps) * gamma_i + beta_i. */
void oracle_layernorm(const double *x, const double *gamma, const double *beta,
                      double eps, double *y, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            sum += xr[i];
        double mu = sum / (double)cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            ss += (xr[i] - mu) * (xr[i] - mu);
        double v = ss / (double)cols;
        double denom = sqrt(v + eps);
        for (int64_t i = 0; i < cols; ++i)
            yr[i] = (xr[i] - mu) / denom * gamma[i] + beta[i];
    }
}

/* RMSNorm: stage 1 ms = (1/N) sum_i x_i^2; output y_i = x_i / sqrt(ms + eps) * gamma_i. */
void oracle_rmsnorm(const double *x, const double *gamma, double eps, double *y,
                    int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double *yr = y + r * cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            ss += xr[i] * xr[i];
        double ms = ss / (double)cols;
        double denom = sqrt(ms + eps);
        for (int64_t i = 0; i < cols; ++i)
            yr[i] = xr[i] / denom * gamma[i];
    }
}

/* ---------------------------------------------------------------------------
 * Row statistics by the plain definition (used by the partition tests).
 * ------------------------------------------------------------------------- */

/* Per row: max and sum_i exp(x_i - max). */
void oracle_softmax_stats(const double *x, int64_t rows, int64_t cols,
                          double *m_out, double *s_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double m = xr[0];
        for (int64_t i = 1; i < cols; ++i)
            if (xr[i] > m)
                m = xr[i];
        double s = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            s += exp(xr[i] - m);
        m_out[r] = m;
        s_out[r] = s;
    }
}

/* Per row: mean and sum of squared deviations from the mean (N * biased variance). */
void oracle_layernorm_stats(const double *x, int64_t rows, int64_t cols,
                            double *mean_out, double *m2_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            sum += xr[i];
        double mu = sum / (double)cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            ss += (xr[i] - mu) * (xr[i] - mu);
        mean_out[r] = mu;
        m2_out[r] = ss;
    }
}

/* ---------------------------------------------------------------------------
 * Eq. 2: slice partials and their combination, written out in double.
 *
 * A partition of one row of length N into P slices is given by P+1 bounds
 * b_0 = 0 <= b_1 <= ... <= b_P = N; slice c holds columns [b_c, b_{c+1}).
 * Empty slices are allowed and contribute the identity element.
 * ------------------------------------------------------------------------- */

/* Softmax partial of one slice: (m_c, s_c) with m_c = max over the slice and
 * s_c = sum over the slice of exp(x_i - m_c).  Identity: (-inf, 0). */
void oracle_softmax_partials(const double *xrow, const int64_t *bounds, int p,
                             double *m_c, double *s_c)
{
    for (int c = 0; c < p; ++c) {
        double m = -INFINITY;
        for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
            if (xrow[i] > m)
                m = xrow[i];
        double s = 0.0;
        if (bounds[c + 1] > bounds[c])
            for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
                s += exp(xrow[i] - m);
        m_c[c] = m;
        s_c[c] = s;
    }
}

/* Combine softmax partials in the order c = 0..P-1:
 * m = max_c m_c;  s = sum_c s_c * exp(m_c - m)  (empty slices skipped). */
void oracle_softmax_merge(const double *m_c, const double *s_c, int p,
                          double *m_out, double *s_out)
{
    double m = -INFINITY;
    for (int c = 0; c < p; ++c)
        if (m_c[c] > m)
            m = m_c[c];
    double s = 0.0;
    for (int c = 0; c < p; ++c)
        if (s_c[c] > 0.0)
            s += s_c[c] * exp(m_c[c] - m);
    *m_out = m;
    *s_out = s;
}

/* LayerNorm partial of one slice: count n_c, slice mean mu_c and the slice's
 * sum of squared deviations from its own mean, M2_c.  Identity: n = 0. */
void oracle_layernorm_partials(const double *xrow, const int64_t *bounds, int p,
                               double *n_c, double *mu_c, double *m2_c)
{
    for (int c = 0; c < p; ++c) {
        int64_t n = bounds[c + 1] - bounds[c];
        double mu = 0.0, m2 = 0.0;
        if (n > 0) {
            double sum = 0.0;
            for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
                sum += xrow[i];
            mu = sum / (double)n;
            for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
                m2 += (xrow[i] - mu) * (xrow[i] - mu);
        }
        n_c[c] = (double)n;
        mu_c[c] = mu;
        m2_c[c] = m2;
    }
}

/* Combine LayerNorm partials by the pairwise update of Chan, Golub and LeVeque,
 * folding c = 0..P-1 into a running (n, mu, M2):
 *   n' = n + n_c,  d = mu_c - mu,  mu' = mu + d * n_c / n',
 *   M2' = M2 + M2_c + d^2 * n * n_c / n'. */
void oracle_layernorm_merge(const double *n_c, const double *mu_c, const double *m2_c,
                            int p, double *n_out, double *mu_out, double *m2_out)
{
    double n = 0.0, mu = 0.0, m2 = 0.0;
    for (int c = 0; c < p; ++c) {
        if (n_c[c] == 0.0)
            continue;
        double n2 = n + n_c[c];
        double d = mu_c[c] - mu;
        mu = mu + d * n_c[c] / n2;
        m2 = m2 + m2_c[c] + d * d * n * n_c[c] / n2;
        n = n2;
    }
    *n_out = n;
    *mu_out = mu;
    *m2_out = m2;
}

/* RMSNorm partial: sum of squares over the slice; combination is a plain sum. */
void oracle_rmsnorm_partials(const double *xrow, const int64_t *bounds, int p, double *ss_c)
{
    for (int c = 0; c < p; ++c) {
        double ss = 0.0;
        for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
            ss += xrow[i] * xrow[i];
        ss_c[c] = ss;
    }
}

/* ---------------------------------------------------------------------------
 * Output rounding: double -> bfloat16, round to nearest, ties to even, taken
 * directly from the double value (no intermediate float rounding).
 *
 * bfloat16 keeps float's 8-bit exponent and 7 explicit fraction bits, so a
 * normal value carries 8 significant bits and the subnormal spacing is 2^-133.
 * The rounded value is exactly representable in float, so its bit pattern is
 * the top 16 bits of that float.
 * ------------------------------------------------------------------------- */
static uint16_t bf16_from_double(double d)
{
    union { float f; uint32_t u; } cvt;
    if (isnan(d))
        return (uint16_t)(signbit(d) ? 0xFFC0u : 0x7FC0u);
    if (isinf(d) || d == 0.0) {
        cvt.f = (float)d; /* exact for 0 and inf */
        return (uint16_t)(cvt.u >> 16);
    }
    double a = fabs(d);
    int e;
    (void)frexp(a, &e); /* a = f * 2^e, f in [0.5, 1) */
    /* weight of the last kept bit: 2^(e-8) for normals, 2^-133 below 2^-126 */
    int lsb_exp = e - 8;
    if (lsb_exp < -133)
        lsb_exp = -133;
    double q = ldexp(a, -lsb_exp);    /* exact: scaling by a power of two */
    double qr = nearbyint(q);         /* default rounding mode: nearest, ties to even */
    double v = ldexp(qr, lsb_exp);    /* exact */
    const double bf16_max = ldexp(255.0, 120); /* (2 - 2^-7) * 2^127 */
    if (v > bf16_max)
        v = INFINITY;
    cvt.f = (float)(signbit(d) ? -v : v);
    return (uint16_t)(cvt.u >> 16);
}

void oracle_round_bf16(const double *y, uint16_t *out, int64_t n)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_from_double(y[i]);
}

/* Number of OpenMP threads the parallel loops above use (1 without OpenMP). */
#ifdef _OPENMP
#include <omp.h>
int oracle_num_threads(void) { return omp_get_max_threads(); }
void oracle_set_num_threads(int n) { omp_set_num_threads(n); }
#else
int oracle_num_threads(void) { return 1; }
void oracle_set_num_threads(int n) { (void)n; }
#endif
