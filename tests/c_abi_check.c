/* Plain C99 user of include/lin_epi.h: compiled and run by tests/test_c_abi.py.
 * Exercises only the host-side paths (argument validation, options, the
 * planner as a pure host call), so it needs no GPU.  Prints "ok" and exits 0
 * when every check passes, else names the first failing check. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lin_epi.h"

#define CHECK(cond)                                              \
    do {                                                         \
        if (!(cond)) {                                           \
            printf("FAIL line %d: %s\n", __LINE__, #cond);       \
            return 1;                                            \
        }                                                        \
    } while (0)

int main(void)
{
    lin_epi_handle h = NULL;
    const float *fake = (const float *)(uintptr_t)0x10000; /* never dereferenced */
    float *fake_out = (float *)(uintptr_t)0x10000;
    lin_epi_desc d;
    lin_epi_plan p;
    lin_epi_profile prof;

    CHECK(lin_epi_create(NULL, NULL) == LIN_EPI_EINVAL);
    CHECK(lin_epi_create(&h, NULL) == LIN_EPI_OK && h != NULL);

    memset(&d, 0, sizeof d);
    d.kind = LIN_EPI_SCALE_HARDTANH_GELU;
    d.scale = 0.5f;
    d.ht_min = -2.0f;
    d.ht_max = 2.0f;
    d.pool_kernel = 16;
    d.pool_stride = 16;

    /* validation happens before any HIP call */
    CHECK(lin_epi_run(NULL, 8, 8, 8, fake, fake, fake, &d, fake_out) == LIN_EPI_EINVAL);
    CHECK(lin_epi_run(h, -1, 8, 8, fake, fake, fake, &d, fake_out) == LIN_EPI_EINVAL);
    CHECK(lin_epi_run(h, 8, 8, 6, fake, fake, fake, &d, fake_out) == LIN_EPI_EALIGN);
    CHECK(lin_epi_run(h, 8, 8, 8, fake, fake, NULL, &d, fake_out) == LIN_EPI_EINVAL);
    CHECK(lin_epi_run(h, 0, 8, 8, NULL, NULL, NULL, &d, NULL) == LIN_EPI_OK);
    d.ht_min = 3.0f;
    CHECK(lin_epi_run(h, 8, 8, 8, fake, fake, fake, &d, fake_out) == LIN_EPI_EINVAL);
    d.ht_min = -2.0f;
    d.kind = LIN_EPI_POOL_GELU_SCALE_ROWMAX;
    d.pool_kernel = 8;
    CHECK(lin_epi_run(h, 8, 64, 8, fake, fake, fake, &d, fake_out) == LIN_EPI_ENOTSUP);
    d.pool_kernel = 16;
    CHECK(lin_epi_pool_weights(h, 64, 8, fake, fake, 0, fake_out, fake_out) == LIN_EPI_EINVAL);
    CHECK(lin_epi_scale_weights(h, 64, 6, fake, fake, 0.5f, fake_out, fake_out) == LIN_EPI_EALIGN);

    /* options and the host-only planner */
    CHECK(lin_epi_set_option(h, LIN_EPI_OPT_SPLIT_K, -1) == LIN_EPI_EINVAL);
    CHECK(lin_epi_set_option(h, LIN_EPI_OPT_TILE, 1) == LIN_EPI_OK);
    d.kind = LIN_EPI_SCALE_HARDTANH_GELU;
    CHECK(lin_epi_query_plan(h, 2048, 8192, 8192, &d, 256, &p) == LIN_EPI_OK);
    CHECK(p.tile_m == 256 && p.tile_n == 256 && p.split_k == 1 && p.grid_main == 256 && p.kernels == 1);
    CHECK(lin_epi_set_option(h, LIN_EPI_OPT_TILE, 0) == LIN_EPI_OK);
    CHECK(lin_epi_query_plan(h, 128, 32768, 32768, &d, 256, &p) == LIN_EPI_OK);
    /* 128 tiles of 128x256 split over 256 workgroups: one partial-sum slot
     * of 128x256 floats per workgroup after the per-tile counters */
    CHECK(p.tile_m == 128 && p.split_k >= 2 && p.schedule == 1 && p.kernels == 1);
    CHECK(p.workspace_bytes >= p.grid_main * 128 * 256 * 4);
    CHECK(lin_epi_set_option(h, LIN_EPI_OPT_GRID, 300) == LIN_EPI_OK);
    CHECK(lin_epi_query_plan(h, 128, 32768, 32768, &d, 256, &p) == LIN_EPI_OK);
    CHECK(p.grid_main == 300 && p.schedule == 2);
    CHECK(lin_epi_set_option(h, LIN_EPI_OPT_GRID, -1) == LIN_EPI_EINVAL);
    CHECK(lin_epi_set_option(h, LIN_EPI_OPT_GRID, 0) == LIN_EPI_OK);
    CHECK(lin_epi_last_plan(h, &p) == LIN_EPI_EINVAL); /* nothing has run */
    CHECK(lin_epi_profile_read(h, &prof) == LIN_EPI_OK && prof.launches[0] == 0);

    CHECK(strcmp(lin_epi_status_string(LIN_EPI_OK), "ok") == 0);
    CHECK(lin_epi_destroy(h) == LIN_EPI_OK);
    CHECK(lin_epi_destroy(NULL) == LIN_EPI_OK);
    printf("ok\n");
    return 0;
}
