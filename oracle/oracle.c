/*
 * CPU oracle for the fused fp32 linear layer with an elementwise tail.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * Everything is computed in IEEE binary64 from fp32 inputs widened exactly,
 * unfused, in the order the pages state the model:
 *
 *   y      = x @ W^T + b                      (nn.Linear, W is [out, in])
 *   tail a = GELU(hardtanh(y * s, lo, hi))    page "Kimi-K2.6 l2_p53", problem
 *                                             statement (GEMM, scale,
 *                                             Hardtanh clamp, GELU)
 *   tail b = max_j s * GELU(avgpool_k(y)[j])  page "Kimi-K2.6 l2_p98", the
 *                                             step-by-step reading of the
 *                                             reference model (Linear,
 *                                             AvgPool1d, GELU, scale, max)
 *   tail c = (y * sigmoid(y)) * s             page "Kimi-K2.6 l2_p59", problem
 *                                             analysis (swish, then scaling)
 *
 * GELU is the exact-erf form 0.5*x*(1+erf(x/sqrt(2))), which is PyTorch's
 * default (approximate='none'); page l2_p53 settles on it after first
 * drafting the tanh approximation.
 *
 * Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp -shared -fPIC.
 * No blocking, tiling or reordering of the reduction: every dot product runs
 * k = 0 .. K-1 in order into one double accumulator.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>

/* Linear layer over a subset of rows.
 * X is [M,K] row-major, W is [N,K] row-major (each output feature's weights
 * are K-contiguous), b is [N].  rows[0..nrows) are the row indices m to
 * compute; Y receives [nrows, N] in binary64.
 * Loop order: output column n outermost (so each W row is read once), then
 * the requested rows, then k in increasing order. */
void oracle_linear_rows(int64_t M, int64_t N, int64_t K,
                        const float *X, const float *W, const float *b,
                        const int64_t *rows, int64_t nrows, double *Y)
{
    (void)M;
#pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n) {
        const float *w = W + n * K;
        for (int64_t r = 0; r < nrows; ++r) {
            const float *x = X + rows[r] * K;
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)x[k] * (double)w[k];
            Y[r * N + n] = acc + (double)b[n];
        }
    }
}

/* GELU, exact form: x * Phi(x) with Phi the standard normal CDF,
 * Phi(x) = 0.5 * (1 + erf(x / sqrt(2))). */
static double gelu_erf(double x)
{
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/* Hardtanh: the inclusive clamp min(max(t, lo), hi). */
static double hardtanh(double t, double lo, double hi)
{
    if (t < lo) return lo;
    if (t > hi) return hi;
    return t;
}

/* Logistic sigmoid 1 / (1 + e^-y). */
static double sigmoid(double y)
{
    return 1.0 / (1.0 + exp(-y));
}

void oracle_gelu(const double *in, int64_t count, double *out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = gelu_erf(in[i]);
}

/* Tail (a), elementwise: scale, then Hardtanh, then GELU. */
void oracle_tail_scale_hardtanh_gelu(const double *y, int64_t count, double s,
                                     double lo, double hi, double *out)
{
    for (int64_t i = 0; i < count; ++i) {
        double t = y[i] * s;
        t = hardtanh(t, lo, hi);
        out[i] = gelu_erf(t);
    }
}

/* AvgPool1d over the last axis of a [rows, N] array with kernel k, stride st,
 * no padding, floor mode: L_out = floor((N - k) / st) + 1 windows, each the sum
 * of its k inputs divided by k (count_include_pad is moot without padding).
 * Returns L_out; writes [rows, L_out] to out.  N < k gives 0 windows. */
int64_t oracle_avgpool1d(const double *y, int64_t rows, int64_t N, int64_t k,
                         int64_t st, double *out)
{
    if (k <= 0 || st <= 0 || N < k) return 0;
    int64_t L = (N - k) / st + 1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t j = 0; j < L; ++j) {
            double acc = 0.0;
            for (int64_t t = 0; t < k; ++t) acc += y[r * N + j * st + t];
            out[r * L + j] = acc / (double)k;
        }
    return L;
}

/* Tail (b): pooled [rows, L] -> g = GELU(p) * s (kept in g, the materialised
 * vector) -> out[r] = max_j g[r, j]. */
void oracle_tail_gelu_scale_rowmax(const double *pooled, int64_t rows, int64_t L,
                                   double s, double *g, double *out)
{
    for (int64_t r = 0; r < rows; ++r) {
        double best = -INFINITY;
        for (int64_t j = 0; j < L; ++j) {
            double v = gelu_erf(pooled[r * L + j]) * s;
            g[r * L + j] = v;
            if (v > best) best = v;
        }
        out[r] = best;
    }
}

/* Tail (c), elementwise: swish y * sigmoid(y), then scale. */
void oracle_tail_swish_scale(const double *y, int64_t count, double s, double *out)
{
    for (int64_t i = 0; i < count; ++i) out[i] = (y[i] * sigmoid(y[i])) * s;
}

/* Number of OpenMP threads the linear layer above runs on. */
int oracle_num_threads(void)
{
    return omp_get_max_threads();
}
