/*
 * oracle.c -- plain, slow, obviously correct CPU reference for the row-wise
 * reduction-reuse operators: softmax, LayerNorm and RMSNorm, and the
 * softmax-logits backward, LayerNorm backward (row part) and int8
 * quantization workloads.
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
 *
 * Three further reduction-reuse workloads of the paper's evaluation (Sec. IV-A:
 * softmax-logits backward, LayerNorm backward and row-wise int8 quantization,
 * whose traffic Sec. IV-D and Fig. 5 report) are defined at the end of the
 * file.  The paper names them without writing them out; the readings are:
 *   softmax-logits backward : the gradient of softmax with respect to its
 *       logits x given the gradient dy of its output, recomputing the
 *       probabilities from x: dx_i = p_i (dy_i - sum_j dy_j p_j);
 *   LayerNorm backward      : the gradient with respect to x of the
 *       LayerNorm above given dy, recomputing mean and variance from x (the
 *       row part), and the gradients with respect to gamma and beta, sums
 *       over the rows (the parameter part, a separate column reduction);
 *   int8 quantization       : symmetric per-row absmax, 127 levels each side,
 *       computed in IEEE single precision because an integer code is decided
 *       by floating-point rounding (see oracle_quantize_int8).
 */
#include <float.h>
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

/* ---------------------------------------------------------------------------
 * Softmax-logits backward.  Stages: r1 = max_i x_i, r2 = sum_i exp(x_i - r1),
 * r3 = sum_i dy_i exp(x_i - r1) / r2 (the dot product of dy with the
 * probabilities p_i = exp(x_i - r1) / r2); output dx_i = p_i (dy_i - r3).
 * ------------------------------------------------------------------------- */
void oracle_softmax_backward(const double *x, const double *dy, double *dx, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        const double *gr = dy + r * cols;
        double *out = dx + r * cols;
        double m = xr[0];
        for (int64_t i = 1; i < cols; ++i)
            if (xr[i] > m)
                m = xr[i];
        double s = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            s += exp(xr[i] - m);
        double dot = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            dot += gr[i] * (exp(xr[i] - m) / s);
        for (int64_t i = 0; i < cols; ++i)
            out[i] = exp(xr[i] - m) / s * (gr[i] - dot);
    }
}

/* ---------------------------------------------------------------------------
 * LayerNorm backward, row part.  With mu and v the mean and biased variance of
 * the row, rstd = 1 / sqrt(v + eps), xhat_i = (x_i - mu) rstd and
 * g_i = gamma_i dy_i (the gradient reaching xhat), the gradient of
 * y_i = xhat_i gamma_i + beta_i with respect to x_i is
 *   dx_i = rstd (g_i - mean_j g_j - xhat_i mean_j (g_j xhat_j)).
 * Stages: mu; v; the two means of g and g * xhat; then the output.
 * ------------------------------------------------------------------------- */
void oracle_layernorm_backward(const double *x, const double *dy, const double *gamma, double eps,
                               double *dx, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        const double *gr = dy + r * cols;
        double *out = dx + r * cols;
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            sum += xr[i];
        double mu = sum / (double)cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            ss += (xr[i] - mu) * (xr[i] - mu);
        double v = ss / (double)cols;
        double rstd = 1.0 / sqrt(v + eps);
        double sg = 0.0, sgx = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            double g = gamma[i] * gr[i];
            sg += g;
            sgx += g * ((xr[i] - mu) * rstd);
        }
        double mean_g = sg / (double)cols;
        double mean_gx = sgx / (double)cols;
        for (int64_t i = 0; i < cols; ++i) {
            double xhat = (xr[i] - mu) * rstd;
            out[i] = rstd * (gamma[i] * gr[i] - mean_g - xhat * mean_gx);
        }
    }
}

/* ---------------------------------------------------------------------------
 * LayerNorm backward, the parameter part.  For y_ij = xhat_ij gamma_j +
 * beta_j (row i, column j) and an upstream gradient dy, the gradients with
 * respect to the parameter vectors are sums over the rows:
 *   dgamma_j = sum_i dy_ij xhat_ij,    dbeta_j = sum_i dy_ij,
 * where xhat_ij = (x_ij - mu_i) rstd_i uses row i's own mean and variance
 * (as in the LayerNorm above: biased variance, eps inside the root).
 * oracle_layernorm_row_stats gives mu_i and rstd_i; the sums then run over
 * the rows in order, one column at a time (columns are independent and
 * spread over threads).
 * ------------------------------------------------------------------------- */
void oracle_layernorm_row_stats(const double *x, double eps, double *mu, double *rstd, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            sum += xr[i];
        double m = sum / (double)cols;
        double ss = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            ss += (xr[i] - m) * (xr[i] - m);
        mu[r] = m;
        rstd[r] = 1.0 / sqrt(ss / (double)cols + eps);
    }
}

void oracle_layernorm_backward_params(const double *x, const double *dy, const double *mu, const double *rstd,
                                      double *dgamma, double *dbeta, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < cols; ++j) {
        double sg = 0.0, sb = 0.0;
        for (int64_t r = 0; r < rows; ++r) {
            double d = dy[r * cols + j];
            sg += d * ((x[r * cols + j] - mu[r]) * rstd[r]);
            sb += d;
        }
        dgamma[j] = sg;
        dbeta[j] = sb;
    }
}

/* ---------------------------------------------------------------------------
 * Row-wise symmetric int8 quantization, in IEEE single precision:
 *   a     = max_i |x_i|                      (exact)
 *   inv   = 127 / a, capped at FLT_MAX       (a > 0; 0 when a == 0)
 *   q_i   = clamp(round_half_even(x_i * inv), -127, 127)
 *   scale = a / 127                          (so x_i ~ q_i * scale)
 * Each of /, * is one correctly rounded float operation.  The cap only
 * matters for rows whose absmax is below 127 / FLT_MAX (about 3.7e-37): it
 * keeps 0 * inv at 0 instead of 0 * inf.  Inputs are finite.
 * ------------------------------------------------------------------------- */
void oracle_quantize_int8(const float *x, int8_t *q, float *scale, int64_t rows, int64_t cols)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        const float *xr = x + r * cols;
        int8_t *qr = q + r * cols;
        float a = 0.0f;
        for (int64_t i = 0; i < cols; ++i) {
            float v = fabsf(xr[i]);
            if (v > a)
                a = v;
        }
        float inv = 0.0f;
        if (a > 0.0f) {
            inv = 127.0f / a;
            if (inv > FLT_MAX)
                inv = FLT_MAX;
        }
        for (int64_t i = 0; i < cols; ++i) {
            float t = xr[i] * inv;
            float k = rintf(t); /* default rounding mode: nearest, ties to even */
            if (k > 127.0f)
                k = 127.0f;
            if (k < -127.0f)
                k = -127.0f;
            qr[i] = (int8_t)k;
        }
        scale[r] = a / 127.0f;
    }
}

/* ---------------------------------------------------------------------------
 * Eq. 2 for the two backward operators: slice partials and their combination.
 * ------------------------------------------------------------------------- */

/* Per row, by the plain definition: m = max x, s = sum exp(x - m) and
 * u = sum dy exp(x - m). */
void oracle_softmax_backward_stats(const double *x, const double *dy, int64_t rows, int64_t cols,
                                   double *m_out, double *s_out, double *u_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        const double *gr = dy + r * cols;
        double m = xr[0];
        for (int64_t i = 1; i < cols; ++i)
            if (xr[i] > m)
                m = xr[i];
        double s = 0.0, u = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            s += exp(xr[i] - m);
            u += gr[i] * exp(xr[i] - m);
        }
        m_out[r] = m;
        s_out[r] = s;
        u_out[r] = u;
    }
}

/* Slice partial (m_c, s_c, u_c): the same three sums over the slice, taken
 * relative to the slice's own maximum.  Identity: (-inf, 0, 0). */
void oracle_softmax_backward_partials(const double *xrow, const double *dyrow, const int64_t *bounds, int p,
                                      double *m_c, double *s_c, double *u_c)
{
    for (int c = 0; c < p; ++c) {
        double m = -INFINITY;
        for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
            if (xrow[i] > m)
                m = xrow[i];
        double s = 0.0, u = 0.0;
        for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i) {
            s += exp(xrow[i] - m);
            u += dyrow[i] * exp(xrow[i] - m);
        }
        m_c[c] = m;
        s_c[c] = s;
        u_c[c] = u;
    }
}

/* m = max_c m_c; both sums are rescaled to the common maximum:
 * s = sum_c s_c exp(m_c - m), u = sum_c u_c exp(m_c - m) (empty slices skipped). */
void oracle_softmax_backward_merge(const double *m_c, const double *s_c, const double *u_c, int p,
                                   double *m_out, double *s_out, double *u_out)
{
    double m = -INFINITY;
    for (int c = 0; c < p; ++c)
        if (m_c[c] > m)
            m = m_c[c];
    double s = 0.0, u = 0.0;
    for (int c = 0; c < p; ++c)
        if (s_c[c] > 0.0) {
            s += s_c[c] * exp(m_c[c] - m);
            u += u_c[c] * exp(m_c[c] - m);
        }
    *m_out = m;
    *s_out = s;
    *u_out = u;
}

/* Per row, by the plain definition, for g = gamma * dy given directly:
 * mean, M2 = sum (x - mean)^2, a = sum g, b = sum g (x - mean). */
void oracle_layernorm_backward_stats(const double *x, const double *g, int64_t rows, int64_t cols,
                                     double *mean_out, double *m2_out, double *a_out, double *b_out)
{
    for (int64_t r = 0; r < rows; ++r) {
        const double *xr = x + r * cols;
        const double *gr = g + r * cols;
        double sum = 0.0;
        for (int64_t i = 0; i < cols; ++i)
            sum += xr[i];
        double mu = sum / (double)cols;
        double m2 = 0.0, a = 0.0, b = 0.0;
        for (int64_t i = 0; i < cols; ++i) {
            m2 += (xr[i] - mu) * (xr[i] - mu);
            a += gr[i];
            b += gr[i] * (xr[i] - mu);
        }
        mean_out[r] = mu;
        m2_out[r] = m2;
        a_out[r] = a;
        b_out[r] = b;
    }
}

/* Slice partial (n_c, mu_c, M2_c, a_c, b_c): count, slice mean, squared
 * deviations from the slice mean, sum of g, and sum of g times the deviation
 * from the slice mean.  Identity: n = 0 (and zero sums). */
void oracle_layernorm_backward_partials(const double *xrow, const double *grow, const int64_t *bounds, int p,
                                        double *n_c, double *mu_c, double *m2_c, double *a_c, double *b_c)
{
    for (int c = 0; c < p; ++c) {
        int64_t n = bounds[c + 1] - bounds[c];
        double mu = 0.0, m2 = 0.0, a = 0.0, b = 0.0;
        if (n > 0) {
            double sum = 0.0;
            for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i)
                sum += xrow[i];
            mu = sum / (double)n;
            for (int64_t i = bounds[c]; i < bounds[c + 1]; ++i) {
                m2 += (xrow[i] - mu) * (xrow[i] - mu);
                a += grow[i];
                b += grow[i] * (xrow[i] - mu);
            }
        }
        n_c[c] = (double)n;
        mu_c[c] = mu;
        m2_c[c] = m2;
        a_c[c] = a;
        b_c[c] = b;
    }
}

/* Fold c = 0..P-1 into a running (n, mu, M2, a, b).  n, mu and M2 follow the
 * Chan-Golub-LeVeque update; a adds; b is re-centred on the new mean mu':
 * sum g (x - mu') = b + a (mu - mu') for the running part and
 * b_c + a_c (mu_c - mu') for slice c. */
void oracle_layernorm_backward_merge(const double *n_c, const double *mu_c, const double *m2_c,
                                     const double *a_c, const double *b_c, int p, double *n_out,
                                     double *mu_out, double *m2_out, double *a_out, double *b_out)
{
    double n = 0.0, mu = 0.0, m2 = 0.0, a = 0.0, b = 0.0;
    for (int c = 0; c < p; ++c) {
        if (n_c[c] == 0.0)
            continue;
        double n2 = n + n_c[c];
        double d = mu_c[c] - mu;
        double mu2 = mu + d * n_c[c] / n2;
        m2 = m2 + m2_c[c] + d * d * n * n_c[c] / n2;
        b = (b + a * (mu - mu2)) + (b_c[c] + a_c[c] * (mu_c[c] - mu2));
        a = a + a_c[c];
        mu = mu2;
        n = n2;
    }
    *n_out = n;
    *mu_out = mu;
    *m2_out = m2;
    *a_out = a;
    *b_out = b;
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
