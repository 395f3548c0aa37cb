/* End-to-end use of the C ABI from plain C on the GPU: device buffers from
 * the HIP runtime, lin_epi_run on the default stream and on a stream of its
 * own, results checked against the CPU oracle (oracle/liboracle.so, linked
 * as a test dependency).  Prints "ok" and exits 0 when every check passes.
 *
 * Cases: integer-valued inputs with no tail, bit-exact (every partial sum is
 * an integer below 2^24); tail (a) with a forced 3-way K split on its own
 * stream; tail (b) with a width that leaves 5 trailing columns unpooled.
 * Floating-point cases use |gpu - ref| <= 1e-3 * (1 + |ref|). */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "lin_epi.h"

/* oracle/oracle.c (binary64 reference; no header of its own) */
void oracle_linear_rows(int64_t M, int64_t N, int64_t K, const float *X, const float *W, const float *b,
                        const int64_t *rows, int64_t nrows, double *Y);
void oracle_tail_scale_hardtanh_gelu(const double *y, int64_t count, double s, double lo, double hi, double *out);
int64_t oracle_avgpool1d(const double *y, int64_t rows, int64_t N, int64_t k, int64_t st, double *out);
void oracle_tail_gelu_scale_rowmax(const double *pooled, int64_t rows, int64_t L, double s, double *g,
                                   double *out);

static int failures = 0;
#define CHECK(c)                                                       \
    do {                                                               \
        if (!(c)) {                                                    \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                \
        }                                                              \
    } while (0)
#define HIP_OK(c) CHECK((c) == hipSuccess)

/* 64-bit LCG (Knuth's MMIX constants); the top bits drive the draws */
static uint64_t lcg_state = 12345;
static uint32_t lcg_next(void)
{
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(lcg_state >> 33);
}
static float draw_int(void) { return (float)((int)(lcg_next() % 5u) - 2); }            /* {-2..2} */
static float draw_unit(void) { return (float)(lcg_next() & 0xFFFFFF) / 8388608.0f - 1.0f; } /* [-1, 1) */

typedef struct {
    float *X, *W, *b;     /* host */
    float *dX, *dW, *db;  /* device */
} inputs;

static inputs make_inputs(int64_t M, int64_t N, int64_t K, int integer, float wscale)
{
    inputs in;
    int64_t i;
    in.X = malloc(sizeof(float) * (size_t)(M * K));
    in.W = malloc(sizeof(float) * (size_t)(N * K));
    in.b = malloc(sizeof(float) * (size_t)N);
    for (i = 0; i < M * K; ++i) in.X[i] = integer ? draw_int() : draw_unit() * 1.7f;
    for (i = 0; i < N * K; ++i) in.W[i] = integer ? draw_int() : draw_unit() * wscale;
    for (i = 0; i < N; ++i) in.b[i] = integer ? draw_int() : draw_unit() * wscale;
    HIP_OK(hipMalloc((void **)&in.dX, sizeof(float) * (size_t)(M * K)));
    HIP_OK(hipMalloc((void **)&in.dW, sizeof(float) * (size_t)(N * K)));
    HIP_OK(hipMalloc((void **)&in.db, sizeof(float) * (size_t)N));
    HIP_OK(hipMemcpy(in.dX, in.X, sizeof(float) * (size_t)(M * K), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(in.dW, in.W, sizeof(float) * (size_t)(N * K), hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(in.db, in.b, sizeof(float) * (size_t)N, hipMemcpyHostToDevice));
    return in;
}

static void free_inputs(inputs *in)
{
    free(in->X);
    free(in->W);
    free(in->b);
    HIP_OK(hipFree(in->dX));
    HIP_OK(hipFree(in->dW));
    HIP_OK(hipFree(in->db));
}

/* y = X W^T + b in binary64 for every row, from the oracle */
static double *reference_linear(const inputs *in, int64_t M, int64_t N, int64_t K)
{
    int64_t m;
    int64_t *rows = malloc(sizeof(int64_t) * (size_t)M);
    double *y = malloc(sizeof(double) * (size_t)(M * N));
    for (m = 0; m < M; ++m) rows[m] = m;
    oracle_linear_rows(M, N, K, in->X, in->W, in->b, rows, M, y);
    free(rows);
    return y;
}

static int close_enough(float got, double ref) { return fabs((double)got - ref) <= 1e-3 * (1.0 + fabs(ref)); }

int main(void)
{
    lin_epi_handle h = NULL, hs = NULL;
    lin_epi_desc d;
    lin_epi_plan plan;
    lin_epi_profile prof;
    hipStream_t stream;
    int64_t i;

    CHECK(lin_epi_create(&h, NULL) == LIN_EPI_OK);
    HIP_OK(hipStreamCreate(&stream));
    CHECK(lin_epi_create(&hs, (void *)stream) == LIN_EPI_OK);

    /* 1. integer inputs, no tail, default stream: bit-exact */
    {
        const int64_t M = 300, N = 520, K = 260;
        inputs in = make_inputs(M, N, K, 1, 1.0f);
        float *dY, *Y = malloc(sizeof(float) * (size_t)(M * N));
        double *ref = reference_linear(&in, M, N, K);
        int64_t bad = 0;
        HIP_OK(hipMalloc((void **)&dY, sizeof(float) * (size_t)(M * N)));
        d.kind = LIN_EPI_NONE;
        d.scale = 1.0f;
        d.ht_min = -1.0f;
        d.ht_max = 1.0f;
        d.pool_kernel = 16;
        d.pool_stride = 16;
        CHECK(lin_epi_set_option(h, LIN_EPI_OPT_PROFILE, 1) == LIN_EPI_OK);
        CHECK(lin_epi_run(h, M, N, K, in.dX, in.dW, in.db, &d, dY) == LIN_EPI_OK);
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(Y, dY, sizeof(float) * (size_t)(M * N), hipMemcpyDeviceToHost));
        for (i = 0; i < M * N; ++i) bad += (double)Y[i] != ref[i];
        CHECK(bad == 0);
        CHECK(lin_epi_profile_read(h, &prof) == LIN_EPI_OK && prof.launches[0] == 1 && prof.total_ms[0] > 0.0);
        HIP_OK(hipFree(dY));
        free(Y);
        free(ref);
        free_inputs(&in);
    }

    /* 2. tail (a), forced split into 3 K slices, on the handle's own stream */
    {
        const int64_t M = 200, N = 390, K = 1000;
        inputs in = make_inputs(M, N, K, 0, 1.0f / 32.0f);
        float *dY, *Y = malloc(sizeof(float) * (size_t)(M * N));
        double *y = reference_linear(&in, M, N, K);
        double *ref = malloc(sizeof(double) * (size_t)(M * N));
        int64_t bad = 0;
        HIP_OK(hipMalloc((void **)&dY, sizeof(float) * (size_t)(M * N)));
        d.kind = LIN_EPI_SCALE_HARDTANH_GELU;
        d.scale = 0.5f;
        d.ht_min = -2.0f;
        d.ht_max = 2.0f;
        CHECK(lin_epi_set_option(hs, LIN_EPI_OPT_SPLIT_K, 3) == LIN_EPI_OK);
        CHECK(lin_epi_run(hs, M, N, K, in.dX, in.dW, in.db, &d, dY) == LIN_EPI_OK);
        HIP_OK(hipStreamSynchronize(stream));
        CHECK(lin_epi_last_plan(hs, &plan) == LIN_EPI_OK && plan.split_k == 3 && plan.kernels == 1 &&
              plan.schedule == 1);
        HIP_OK(hipMemcpy(Y, dY, sizeof(float) * (size_t)(M * N), hipMemcpyDeviceToHost));
        oracle_tail_scale_hardtanh_gelu(y, M * N, 0.5, -2.0, 2.0, ref);
        for (i = 0; i < M * N; ++i) bad += !close_enough(Y[i], ref[i]);
        CHECK(bad == 0);
        HIP_OK(hipFree(dY));
        free(Y);
        free(y);
        free(ref);
        free_inputs(&in);
    }

    /* 3. tail (b): AvgPool1d(16) -> GELU -> x2 -> row max, 5 columns unpooled */
    {
        const int64_t M = 130, N = 16 * 33 + 5, K = 520, L = 33;
        inputs in = make_inputs(M, N, K, 0, 1.0f / 16.0f);
        float *dY, Y[130];
        double *y = reference_linear(&in, M, N, K);
        double *pooled = malloc(sizeof(double) * (size_t)(M * L));
        double *g = malloc(sizeof(double) * (size_t)(M * L));
        double ref[130];
        int64_t bad = 0;
        HIP_OK(hipMalloc((void **)&dY, sizeof(float) * (size_t)M));
        d.kind = LIN_EPI_POOL_GELU_SCALE_ROWMAX;
        d.scale = 2.0f;
        d.pool_kernel = 16;
        d.pool_stride = 16;
        CHECK(lin_epi_run(h, M, N, K, in.dX, in.dW, in.db, &d, dY) == LIN_EPI_OK);
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(Y, dY, sizeof(float) * (size_t)M, hipMemcpyDeviceToHost));
        CHECK(oracle_avgpool1d(y, M, N, 16, 16, pooled) == L);
        oracle_tail_gelu_scale_rowmax(pooled, M, L, 2.0, g, ref);
        for (i = 0; i < M; ++i) bad += !close_enough(Y[i], ref[i]);
        CHECK(bad == 0);
        HIP_OK(hipFree(dY));
        free(y);
        free(pooled);
        free(g);
        free_inputs(&in);
    }

    CHECK(lin_epi_destroy(hs) == LIN_EPI_OK);
    CHECK(lin_epi_destroy(h) == LIN_EPI_OK);
    HIP_OK(hipStreamDestroy(stream));
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
