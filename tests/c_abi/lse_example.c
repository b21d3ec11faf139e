/*
 * A plain C11 caller of the library's C ABI (include/lse.h): no Python, no
 * torch. It fills device rows with constants, whose log-sum-exp has the
 * closed form c + ln(cols), runs lse_forward for fp32 and bf16 input on its
 * own stream, checks the results and a few error returns, and prints "ok".
 * Exit status 0 on success, 1 on a wrong result, 2 on a HIP or library error.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "lse.h"

#define ROWS 6
#define COLS 5000

static int hip_ok(hipError_t e, const char *what) {
    if (e != hipSuccess) {
        fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
        return 0;
    }
    return 1;
}

static int lse_ok(lse_status_t s, const char *what) {
    if (s != LSE_OK) {
        fprintf(stderr, "%s: %s\n", what, lse_status_string(s));
        return 0;
    }
    return 1;
}

/* bf16 bits of a float that bf16 holds exactly (the high half of its word) */
static uint16_t bf16_of(float v) {
    uint32_t u;
    memcpy(&u, &v, sizeof u);
    return (uint16_t)(u >> 16);
}

int main(void) {
    /* row r holds the constant c[r]; bf16 holds every one of them exactly */
    const float c[ROWS] = {0.0f, 1.5f, -3.25f, 20.0f, -87.5f, 1024.0f};
    float *hx = (float *)malloc(sizeof(float) * ROWS * COLS);
    uint16_t *hb = (uint16_t *)malloc(sizeof(uint16_t) * ROWS * COLS);
    float got[ROWS];
    if (!hx || !hb) return 2;
    for (int r = 0; r < ROWS; ++r)
        for (int j = 0; j < COLS; ++j) {
            hx[r * COLS + j] = c[r];
            hb[r * COLS + j] = bf16_of(c[r]);
        }

    lse_handle_t h = NULL;
    hipStream_t stream;
    void *dx = NULL, *db = NULL;
    float *dout = NULL;
    if (!lse_ok(lse_create(&h, 0), "lse_create")) return 2;
    if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate") ||
        !hip_ok(hipMalloc(&dx, sizeof(float) * ROWS * COLS), "hipMalloc") ||
        !hip_ok(hipMalloc(&db, sizeof(uint16_t) * ROWS * COLS), "hipMalloc") ||
        !hip_ok(hipMalloc((void **)&dout, sizeof(float) * ROWS), "hipMalloc") ||
        !hip_ok(hipMemcpy(dx, hx, sizeof(float) * ROWS * COLS, hipMemcpyHostToDevice), "copy") ||
        !hip_ok(hipMemcpy(db, hb, sizeof(uint16_t) * ROWS * COLS, hipMemcpyHostToDevice), "copy"))
        return 2;

    int bad = 0;
    const lse_dtype_t types[2] = {LSE_DTYPE_F32, LSE_DTYPE_BF16};
    for (int t = 0; t < 2; ++t) {
        const void *src = t == 0 ? dx : db;
        const double tol = t == 0 ? 2e-6 : 1e-5;
        if (!lse_ok(lse_forward(h, src, types[t], ROWS, COLS, COLS, dout, stream), "lse_forward") ||
            !hip_ok(hipStreamSynchronize(stream), "sync") ||
            !hip_ok(hipMemcpy(got, dout, sizeof got, hipMemcpyDeviceToHost), "copy back"))
            return 2;
        for (int r = 0; r < ROWS; ++r) {
            const double want = (double)c[r] + log((double)COLS);
            const double scale = fabs(want) > 1.0 ? fabs(want) : 1.0;
            if (!(fabs((double)got[r] - want) <= tol * scale)) {
                fprintf(stderr, "dtype %d row %d: got %.9g want %.9g\n", (int)types[t], r, got[r], want);
                bad = 1;
            }
        }
    }

    /* argument errors come back as status codes, before any device work */
    if (lse_forward(h, dx, (lse_dtype_t)7, ROWS, COLS, COLS, dout, stream) != LSE_ERR_UNSUPPORTED_DTYPE ||
        lse_forward(h, dx, LSE_DTYPE_F32, ROWS, COLS, COLS - 1, dout, stream) != LSE_ERR_INVALID_ARG ||
        lse_forward(NULL, dx, LSE_DTYPE_F32, ROWS, COLS, COLS, dout, stream) != LSE_ERR_INVALID_ARG ||
        lse_forward(h, NULL, LSE_DTYPE_F32, 0, COLS, COLS, NULL, stream) != LSE_OK) {
        fprintf(stderr, "unexpected status from an invalid call\n");
        bad = 1;
    }
    /* an empty row gives -inf; a row of -inf gives -inf */
    if (!lse_ok(lse_forward(h, dx, LSE_DTYPE_F32, ROWS, 0, COLS, dout, stream), "lse_forward cols=0") ||
        !hip_ok(hipStreamSynchronize(stream), "sync") ||
        !hip_ok(hipMemcpy(got, dout, sizeof got, hipMemcpyDeviceToHost), "copy back"))
        return 2;
    for (int r = 0; r < ROWS; ++r)
        if (!(isinf(got[r]) && got[r] < 0)) {
            fprintf(stderr, "cols=0 row %d: got %g\n", r, got[r]);
            bad = 1;
        }
    for (int j = 0; j < COLS; ++j) hx[j] = -INFINITY;
    if (!hip_ok(hipMemcpy(dx, hx, sizeof(float) * COLS, hipMemcpyHostToDevice), "copy") ||
        !lse_ok(lse_forward(h, dx, LSE_DTYPE_F32, 1, COLS, COLS, dout, stream), "lse_forward -inf") ||
        !hip_ok(hipStreamSynchronize(stream), "sync") ||
        !hip_ok(hipMemcpy(got, dout, sizeof(float), hipMemcpyDeviceToHost), "copy back"))
        return 2;
    if (!(isinf(got[0]) && got[0] < 0)) {
        fprintf(stderr, "row of -inf: got %g\n", got[0]);
        bad = 1;
    }

    (void)hipFree(dx);
    (void)hipFree(db);
    (void)hipFree(dout);
    (void)hipStreamDestroy(stream);
    if (!lse_ok(lse_destroy(h), "lse_destroy")) return 2;
    free(hx);
    free(hb);
    if (bad) return 1;
    printf("ok\n");
    return 0;
}
