/*
 * End-to-end check of the activation's C ABI from plain C (test infrastructure, not
 * part of the library). Inputs come from a fixed linear congruential generator. The
 * HIP library's forward and backward run on a stream. The same two calls are then
 * captured into a HIP graph, and two replays must reproduce the eager run bit for
 * bit. The CPU oracle's C functions give the expected values: bf16 outputs within
 * 1 ulp, grad_probs within 1e-6 + 1e-5 S (S = the row's sum of |terms|), padding
 * rows exactly +0, and slots of rows that are not live left as they were.
 *
 * Cases: a ragged width on whole-row walks and a width whose backward rows are
 * shared by a workgroup's four waves, each with a device n_used, a permutation
 * holding dummy entries, and zero padding on.
 *
 * Exit status 0 when every check passes; the first failure is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "swiglu_probs.h"

int oracle_swiglu_fwd(const uint16_t *x, const float *probs, uint16_t *y, int64_t rows, int64_t inter,
                      float limit, const int32_t *n_used, const int32_t *permutation_map,
                      int zero_padding, int threads);
int oracle_swiglu_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y, uint16_t *grad_x,
                      float *grad_probs, double *grad_probs_f64, double *row_scale, int64_t rows,
                      int64_t inter, float limit, const int32_t *n_used,
                      const int32_t *permutation_map, int zero_padding, int threads);

#define CHECK_HIP(call)                                                                   \
    do {                                                                                  \
        hipError_t err_ = (call);                                                         \
        if (err_ != hipSuccess) {                                                         \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)err_, __FILE__, __LINE__);     \
            exit(2);                                                                      \
        }                                                                                 \
    } while (0)

#define CHECK(cond, ...)                                                                  \
    do {                                                                                  \
        if (!(cond)) {                                                                    \
            fprintf(stderr, __VA_ARGS__);                                                 \
            fprintf(stderr, "\n");                                                        \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

static uint64_t lcg_state;
static uint32_t lcg(void)
{
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(lcg_state >> 33);
}
static float uniform(void) { return (float)(lcg() + 0.5) / 2147483648.0f; }
/* approximately normal: the sum of four uniforms, centred and scaled */
static float normalish(float sd) { return (uniform() + uniform() + uniform() + uniform() - 2.0f) * 1.7320508f * sd; }

static uint16_t to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

static int64_t ordinal(uint16_t h) { return (h & 0x8000) ? -(int64_t)(h & 0x7FFF) : (int64_t)(h & 0x7FFF); }
static int is_nan_bf16(uint16_t h) { return (h & 0x7F80) == 0x7F80 && (h & 0x7F); }

static void check_ulp(const uint16_t *got, const uint16_t *want, size_t n, const char *what)
{
    for (size_t i = 0; i < n; ++i) {
        if (is_nan_bf16(got[i]) && is_nan_bf16(want[i]))
            continue;
        int64_t d = ordinal(got[i]) - ordinal(want[i]);
        CHECK(d <= 1 && d >= -1, "%s: element %zu got 0x%04x want 0x%04x", what, i, got[i], want[i]);
    }
}

static int run_case(int64_t rows, int64_t inter, int32_t n_used, int zero_padding, uint64_t seed)
{
    const float limit = 7.0f;
    const size_t nx = (size_t)rows * 2 * inter, ny = (size_t)rows * inter;
    uint16_t *x = malloc(nx * 2), *gy = malloc(ny * 2), *y = malloc(ny * 2), *gx = malloc(nx * 2);
    uint16_t *ry = malloc(ny * 2), *rgx = malloc(nx * 2), *y2 = malloc(ny * 2), *gx2 = malloc(nx * 2);
    float *p = malloc(rows * 4), *gp = malloc(rows * 4), *rgp = malloc(rows * 4), *gp2 = malloc(rows * 4);
    double *gp64 = malloc(rows * 8), *scale = malloc(rows * 8);
    int32_t *perm = malloc(rows * 4);
    lcg_state = seed;
    for (size_t i = 0; i < nx; ++i)
        x[i] = to_bf16(normalish(3.0f));
    for (size_t i = 0; i < ny; ++i)
        gy[i] = to_bf16(normalish(1.0f));
    for (int64_t r = 0; r < rows; ++r) {
        p[r] = uniform();
        perm[r] = (int32_t)r;
    }
    for (int64_t r = rows - 1; r > 0; --r) { /* Fisher-Yates */
        int64_t j = lcg() % (uint32_t)(r + 1);
        int32_t t = perm[r];
        perm[r] = perm[j];
        perm[j] = t;
    }
    for (int k = 0; k < 16; ++k) /* interior dummy rows */
        perm[lcg() % (uint32_t)n_used] = (k & 1) ? -1 : (int32_t)(rows + k);

    /* the oracle; sentinels mark what must stay untouched */
    for (size_t i = 0; i < ny; ++i) ry[i] = 0xFFFF;
    for (size_t i = 0; i < nx; ++i) rgx[i] = 0xFFFF;
    for (int64_t r = 0; r < rows; ++r) { rgp[r] = -12345.5f; gp64[r] = NAN; scale[r] = NAN; }
    CHECK(oracle_swiglu_fwd(x, p, ry, rows, inter, limit, &n_used, perm, zero_padding, 8) == 0, "oracle fwd");
    CHECK(oracle_swiglu_bwd(x, p, gy, rgx, rgp, gp64, scale, rows, inter, limit, &n_used, perm,
                            zero_padding, 8) == 0, "oracle bwd");

    /* device buffers */
    uint16_t *dx, *dgy, *dy, *dgx;
    float *dp, *dgp;
    int32_t *dnu, *dperm;
    CHECK_HIP(hipMalloc((void **)&dx, nx * 2));
    CHECK_HIP(hipMalloc((void **)&dgy, ny * 2));
    CHECK_HIP(hipMalloc((void **)&dy, ny * 2));
    CHECK_HIP(hipMalloc((void **)&dgx, nx * 2));
    CHECK_HIP(hipMalloc((void **)&dp, rows * 4));
    CHECK_HIP(hipMalloc((void **)&dgp, rows * 4));
    CHECK_HIP(hipMalloc((void **)&dnu, 4));
    CHECK_HIP(hipMalloc((void **)&dperm, rows * 4));
    CHECK_HIP(hipMemcpy(dx, x, nx * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dgy, gy, ny * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dp, p, rows * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dnu, &n_used, 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dperm, perm, rows * 4, hipMemcpyHostToDevice));
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));

    /* eager run, outputs pre-filled with the oracle's sentinels */
    for (size_t i = 0; i < ny; ++i) y[i] = 0xFFFF;
    for (size_t i = 0; i < nx; ++i) gx[i] = 0xFFFF;
    for (int64_t r = 0; r < rows; ++r) gp[r] = -12345.5f;
    CHECK_HIP(hipMemcpy(dy, y, ny * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dgx, gx, nx * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dgp, gp, rows * 4, hipMemcpyHostToDevice));
    CHECK(swiglu_probs_fwd(dx, dp, dy, rows, inter, limit, dnu, dperm, zero_padding, st) == SWIGLU_OK, "fwd");
    CHECK(swiglu_probs_bwd(dx, dp, dgy, dgx, dgp, rows, inter, limit, dnu, dperm, zero_padding, st) == SWIGLU_OK,
          "bwd");
    CHECK_HIP(hipStreamSynchronize(st));
    CHECK_HIP(hipMemcpy(y, dy, ny * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gx, dgx, nx * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(gp, dgp, rows * 4, hipMemcpyDeviceToHost));

    check_ulp(y, ry, ny, "y");
    check_ulp(gx, rgx, nx, "grad_x");
    for (int64_t r = 0; r < rows; ++r) {
        if (rgp[r] == -12345.5f) {
            CHECK(gp[r] == -12345.5f, "grad_probs slot %lld of a row that is not live was written", (long long)r);
            continue;
        }
        CHECK(fabs((double)gp[r] - gp64[r]) <= 1e-6 + 1e-5 * scale[r], "grad_probs slot %lld: %.9g vs %.9g",
              (long long)r, (double)gp[r], gp64[r]);
    }
    for (int64_t r = n_used; zero_padding && r < rows; ++r) /* padding rows are +0 */
        for (int64_t j = 0; j < inter; ++j)
            CHECK(y[r * inter + j] == 0 && gx[r * 2 * inter + j] == 0 && gx[r * 2 * inter + inter + j] == 0,
                  "padding row %lld not +0", (long long)r);

    /* the same calls in a HIP graph, replayed twice with other work in between */
    hipGraph_t graph;
    hipGraphExec_t exec;
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    CHECK(swiglu_probs_fwd(dx, dp, dy, rows, inter, limit, dnu, dperm, zero_padding, st) == SWIGLU_OK, "fwd (capture)");
    CHECK(swiglu_probs_bwd(dx, dp, dgy, dgx, dgp, rows, inter, limit, dnu, dperm, zero_padding, st) == SWIGLU_OK,
          "bwd (capture)");
    CHECK_HIP(hipStreamEndCapture(st, &graph));
    CHECK_HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
    for (int rep = 0; rep < 2; ++rep) {
        for (size_t i = 0; i < ny; ++i) y2[i] = 0xFFFF;
        for (size_t i = 0; i < nx; ++i) gx2[i] = 0xFFFF;
        for (int64_t r = 0; r < rows; ++r) gp2[r] = -12345.5f;
        CHECK_HIP(hipMemcpy(dy, y2, ny * 2, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(dgx, gx2, nx * 2, hipMemcpyHostToDevice));
        CHECK_HIP(hipMemcpy(dgp, gp2, rows * 4, hipMemcpyHostToDevice));
        CHECK_HIP(hipGraphLaunch(exec, st));
        CHECK_HIP(hipStreamSynchronize(st));
        CHECK_HIP(hipMemcpy(y2, dy, ny * 2, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(gx2, dgx, nx * 2, hipMemcpyDeviceToHost));
        CHECK_HIP(hipMemcpy(gp2, dgp, rows * 4, hipMemcpyDeviceToHost));
        CHECK(memcmp(y2, y, ny * 2) == 0 && memcmp(gx2, gx, nx * 2) == 0 && memcmp(gp2, gp, rows * 4) == 0,
              "graph replay %d differs from the eager run", rep);
    }
    CHECK_HIP(hipGraphExecDestroy(exec));
    CHECK_HIP(hipGraphDestroy(graph));
    CHECK_HIP(hipStreamDestroy(st));
    CHECK_HIP(hipFree(dx));
    CHECK_HIP(hipFree(dgy));
    CHECK_HIP(hipFree(dy));
    CHECK_HIP(hipFree(dgx));
    CHECK_HIP(hipFree(dp));
    CHECK_HIP(hipFree(dgp));
    CHECK_HIP(hipFree(dnu));
    CHECK_HIP(hipFree(dperm));
    free(x); free(gy); free(y); free(gx); free(ry); free(rgx); free(y2); free(gx2);
    free(p); free(gp); free(rgp); free(gp2); free(gp64); free(scale); free(perm);
    printf("rows %lld inter %lld n_used %d zero_padding %d: ok\n", (long long)rows, (long long)inter, n_used,
           zero_padding);
    fflush(stdout);
    return 0;
}

int main(void)
{
    CHECK(swiglu_probs_abi_version() == 1, "ABI version");
    run_case(3001, 2056, 2700, 1, 1);   /* ragged width: whole rows per wave */
    run_case(3001, 4096, 2999, 1, 2);   /* the backward shares each row among four waves */
    run_case(1000, 4096, 1000, 0, 3);   /* every row live */
    printf("C ABI check: ok\n");
    return 0;
}
