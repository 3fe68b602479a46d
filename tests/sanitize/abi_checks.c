/*
 * Sanitized run of libfhd.so's host-side argument handling, built by
 * tests/test_sanitize_cpu.py with the host code of the library compiled
 * under -fsanitize=address,undefined. Every call here is refused (or
 * returns) before the library touches a device, so it runs on a host
 * without a GPU; the sanitizers check the argument checks, overlap tests,
 * error messages and status strings. Exit status 0 when every check holds.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fhd.h"

static int failures = 0;
static void expect(int ok, const char *what)
{
    if (!ok) {
        fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

int main(void)
{
    float *fake[10];
    for (int i = 0; i < 10; ++i) fake[i] = (float *)(uintptr_t)(0x10000000u * (unsigned)(i + 1));
    const float *const *c = (const float *const *)fake;
    /* negative sizes, NULL pointers, misalignment, overlap, unknown paths */
    expect(fhd_compute(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[9], -1, 4, NULL) == FHD_ERR_INVALID_ARG, "M < 0");
    expect(fhd_compute(NULL, NULL, NULL, NULL, NULL, c[5], c[6], c[7], fake[8], fake[9], 3, 4, NULL) == FHD_ERR_INVALID_ARG, "NULL k");
    expect(strstr(fhd_last_error(), "NULL") != NULL, "NULL message");
    expect(fhd_compute(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], (float *)((char *)fake[8] + 2), fake[9], 3, 4, NULL) == FHD_ERR_INVALID_ARG, "misaligned output");
    expect(fhd_compute(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[8], 3, 4, NULL) == FHD_ERR_INVALID_ARG, "outputs overlap");
    expect(fhd_compute_paths(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[9], 3, 4, 9, NULL) == FHD_ERR_INVALID_ARG, "unknown paths");
    expect(fhd_compute(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, 0, NULL) == FHD_OK, "empty call");
    expect(fhd_forward_paths(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[9], 3, -2, 0, NULL) == FHD_ERR_INVALID_ARG, "forward N < 0");
    expect(fhd_normal_paths(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[9], 3, 4, 5, NULL) == FHD_ERR_INVALID_ARG, "normal paths");
    int iters = 7;
    expect(fhd_cg_paths(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[9], 3, 4, 2, -1.0f, &iters, NULL, 0, NULL) == FHD_ERR_INVALID_ARG, "cg tol < 0");
    expect(fhd_pack(c[0], c[1], c[2], c[3], c[4], 10, fake[5], 8, NULL) == FHD_ERR_INVALID_ARG, "short pack buffer");
    expect(strstr(fhd_last_error(), "packed_bytes") != NULL, "pack message");
    expect(fhd_packed_bytes(-1) == -1 && fhd_packed_bytes(9) == 2 * 160, "packed bytes");
    expect(fhd_compute_noalloc(c[0], c[1], c[2], c[3], c[4], c[5], c[6], c[7], fake[8], fake[9], 8000000, 4096, 0, NULL) == FHD_ERR_INVALID_ARG, "noalloc beyond scratch");
    expect(strstr(fhd_last_error(), "needs") != NULL, "noalloc message");
    float axis[6] = {0.0f, 1.0f, 0.0f, 1.0f, 0.0f, 1.0f};
    expect(fhd_compute_grid(c[0], c[1], c[2], c[3], c[4], 3, 2, 2, -1, axis, FHD_GRID_FP32, fake[8], fake[9], NULL) == FHD_ERR_INVALID_ARG, "grid size < 0");
    expect(fhd_time_kernel("fhd_gather_kernel<16, true>", NULL, 1) == FHD_ERR_INVALID_ARG, "timing hook NULL events");
    expect(fhd_time_kernel(NULL, NULL, 0) == FHD_OK && fhd_timed_launches() == 0, "timing hook disarm");
    expect(fhd_release_workspaces() == FHD_OK, "release with nothing kept");
    for (int s = 0; s >= -4; --s) expect(strlen(fhd_status_string(s)) > 0, "status string");
    if (failures) return 1;
    printf("ABI argument checks passed under the sanitizers\n");
    return 0;
}
