/*
 * End-to-end check of the MoE elementwise operations' C ABI from plain C (test
 * infrastructure, not part of the library). Inputs come from a fixed linear
 * congruential generator. Every operation runs on a stream; then the whole sequence
 * is captured into a HIP graph, and two replays must reproduce the eager run bit for
 * bit. The MoE oracle's C functions give the expected values:
 *   - residual add (bf16, an odd length): bitwise;
 *   - router weight, bf16 x and fp32 out, 7168-column rows shared by four waves:
 *     forward and grad_x bitwise, grad_probs within 1e-6 + 1e-5 S;
 *   - soft-clamped squared ReLU with a device n_used, a permutation holding dummy
 *     entries and zero padding: y and grad_x within 1 bf16 ulp, grad_probs within
 *     1e-6 + 1e-5 S, padding rows +0, slots of rows that are not live untouched;
 *   - unpermute in expert order, 8 local experts, expert-major rows, fp32 out, a
 *     device valid_tokens bound: bitwise, tokens past the bound untouched.
 *
 * Exit status 0 when every check passes; the first failure is printed.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "moe_elementwise.h"

int oracle_residual_add(const void *expert, const void *shared, const void *residual, void *out,
                        int64_t n, int dt);
int oracle_router_weight_fwd(const void *x, int x_dt, const float *probs, void *out, int out_dt,
                             int64_t tokens, int64_t hidden);
int oracle_router_weight_bwd(const void *grad_out, int out_dt, const void *x, int x_dt,
                             const float *probs, void *grad_x, float *grad_probs,
                             double *grad_probs_f64, double *row_scale, int64_t tokens,
                             int64_t hidden);
int oracle_squared_relu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y, int64_t rows,
                                  int64_t hidden, int clamp, float clamp_scale,
                                  const int32_t *n_used, const int32_t *perm, int zero_padding);
int oracle_squared_relu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                  uint16_t *grad_x, float *grad_probs, double *grad_probs_f64,
                                  double *row_scale, int64_t rows, int64_t hidden, int clamp,
                                  float clamp_scale, const int32_t *n_used, const int32_t *perm,
                                  int zero_padding);
int oracle_unpermute_expert_order(const uint16_t *expert_output, int64_t expert_rows,
                                  const int32_t *inverse_map, const int32_t *valid_tokens,
                                  void *out, int out_dt, int64_t tokens, int64_t hidden,
                                  int64_t num_local_experts);

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

static uint64_t lcg_state = 42;
static uint32_t lcg(void)
{
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(lcg_state >> 33);
}
static float uniform(void) { return (float)(lcg() + 0.5) / 2147483648.0f; }
static float normalish(float sd) { return (uniform() + uniform() + uniform() + uniform() - 2.0f) * 1.7320508f * sd; }

static uint16_t to_bf16(float f)
{
    uint32_t b;
    memcpy(&b, &f, 4);
    return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}
static void fill_bf16(uint16_t *a, size_t n, float sd)
{
    for (size_t i = 0; i < n; ++i)
        a[i] = to_bf16(normalish(sd));
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

static void check_bits(const void *got, const void *want, size_t bytes, const char *what)
{
    CHECK(memcmp(got, want, bytes) == 0, "%s: not bit-identical to the oracle", what);
}

static void check_sums(const float *got, const float *want_f32, const double *want, const double *scale,
                       int64_t n, const char *what)
{
    for (int64_t r = 0; r < n; ++r) {
        if (want_f32[r] == -12345.5f) { /* a slot the oracle left alone */
            CHECK(got[r] == -12345.5f, "%s: slot %lld of a row that is not live was written", what, (long long)r);
            continue;
        }
        CHECK(fabs((double)got[r] - want[r]) <= 1e-6 + 1e-5 * scale[r], "%s: slot %lld: %.9g vs %.9g", what,
              (long long)r, (double)got[r], want[r]);
    }
}

static void *dalloc(size_t bytes)
{
    void *p = NULL;
    CHECK_HIP(hipMalloc(&p, bytes));
    return p;
}
static void *upload(const void *h, size_t bytes)
{
    void *d = dalloc(bytes);
    CHECK_HIP(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice));
    return d;
}
static void download(void *h, const void *d, size_t bytes) { CHECK_HIP(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost)); }

/* sizes */
enum { RA_N = 1000003, RW_T = 777, RW_H = 7168, SQ_R = 2001, SQ_H = 2056, SQ_USED = 1900, UP_T = 1500, UP_E = 8,
       UP_H = 1032, UP_VALID = 1400 };
static const float kScale = 4.0f;

/* device buffers of every operation, and their host copies of the outputs */
static uint16_t *ra_e, *ra_s, *ra_r, *ra_o;
static uint16_t *rw_x;
static float *rw_p, *rw_out, *rw_gout, *rw_gp;
static uint16_t *rw_gx;
static uint16_t *sq_x, *sq_gy, *sq_y, *sq_gx;
static float *sq_p, *sq_gp;
static int32_t *sq_nu, *sq_perm;
static uint16_t *up_eo;
static int32_t *up_map, *up_valid;
static float *up_out;
static int64_t up_rows;

/* fills every output with its sentinel (outputs the operations must leave alone keep it) */
static void reset_outputs(void)
{
    static uint16_t *h16;
    static float *hf;
    const size_t big = (size_t)SQ_R * SQ_H > (size_t)RA_N ? (size_t)SQ_R * SQ_H : (size_t)RA_N;
    const size_t bigf = (size_t)UP_T * UP_H > (size_t)RW_T * RW_H ? (size_t)UP_T * UP_H : (size_t)RW_T * RW_H;
    if (!h16) {
        h16 = malloc(big * 2);
        hf = malloc(bigf * 4);
        for (size_t i = 0; i < big; ++i) h16[i] = 0xFFFF;
        for (size_t i = 0; i < bigf; ++i) hf[i] = NAN;
    }
    CHECK_HIP(hipMemcpy(ra_o, h16, (size_t)RA_N * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(rw_out, hf, (size_t)RW_T * RW_H * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(rw_gx, h16, (size_t)RW_T * RW_H * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(sq_y, h16, (size_t)SQ_R * SQ_H * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(sq_gx, h16, (size_t)SQ_R * SQ_H * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(up_out, hf, (size_t)UP_T * UP_H * 4, hipMemcpyHostToDevice));
    float s[SQ_R > RW_T ? SQ_R : RW_T];
    for (int i = 0; i < (SQ_R > RW_T ? SQ_R : RW_T); ++i) s[i] = -12345.5f;
    CHECK_HIP(hipMemcpy(rw_gp, s, RW_T * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(sq_gp, s, SQ_R * 4, hipMemcpyHostToDevice));
}

/* every operation once, in order, on stream st */
static void run_all(hipStream_t st)
{
    CHECK(moe_residual_add(ra_e, ra_s, ra_r, ra_o, RA_N, MOE_BF16, st, 0) == MOE_OK, "residual add");
    CHECK(moe_router_weight_fwd(rw_x, MOE_BF16, rw_p, rw_out, MOE_FP32, RW_T, RW_H, st, 0) == MOE_OK, "router fwd");
    CHECK(moe_router_weight_bwd(rw_gout, MOE_FP32, rw_x, MOE_BF16, rw_p, rw_gx, rw_gp, RW_T, RW_H, st, 0) == MOE_OK,
          "router bwd");
    CHECK(moe_squared_relu_probs_fwd(sq_x, sq_p, sq_y, SQ_R, SQ_H, 1, kScale, sq_nu, sq_perm, 1, st, 0) == MOE_OK,
          "squared relu fwd");
    CHECK(moe_squared_relu_probs_bwd(sq_x, sq_p, sq_gy, sq_gx, sq_gp, SQ_R, SQ_H, 1, kScale, sq_nu, sq_perm, 1, st,
                                     0) == MOE_OK,
          "squared relu bwd");
    CHECK(moe_unpermute_expert_order(up_eo, up_rows, up_map, up_valid, up_out, MOE_FP32, UP_T, UP_H, UP_E, st, 0) ==
              MOE_OK,
          "unpermute");
}

/* all outputs, downloaded, in one block of host memory */
typedef struct {
    uint16_t *ra, *rw_gx, *sq_y, *sq_gx;
    float *rw_out, *rw_gp, *sq_gp, *up;
} Outputs;

static Outputs download_all(void)
{
    Outputs o;
    o.ra = malloc((size_t)RA_N * 2);
    o.rw_out = malloc((size_t)RW_T * RW_H * 4);
    o.rw_gx = malloc((size_t)RW_T * RW_H * 2);
    o.rw_gp = malloc(RW_T * 4);
    o.sq_y = malloc((size_t)SQ_R * SQ_H * 2);
    o.sq_gx = malloc((size_t)SQ_R * SQ_H * 2);
    o.sq_gp = malloc(SQ_R * 4);
    o.up = malloc((size_t)UP_T * UP_H * 4);
    download(o.ra, ra_o, (size_t)RA_N * 2);
    download(o.rw_out, rw_out, (size_t)RW_T * RW_H * 4);
    download(o.rw_gx, rw_gx, (size_t)RW_T * RW_H * 2);
    download(o.rw_gp, rw_gp, RW_T * 4);
    download(o.sq_y, sq_y, (size_t)SQ_R * SQ_H * 2);
    download(o.sq_gx, sq_gx, (size_t)SQ_R * SQ_H * 2);
    download(o.sq_gp, sq_gp, SQ_R * 4);
    download(o.up, up_out, (size_t)UP_T * UP_H * 4);
    return o;
}

static void same_outputs(const Outputs *a, const Outputs *b, int rep)
{
    CHECK(memcmp(a->ra, b->ra, (size_t)RA_N * 2) == 0 && memcmp(a->rw_out, b->rw_out, (size_t)RW_T * RW_H * 4) == 0 &&
              memcmp(a->rw_gx, b->rw_gx, (size_t)RW_T * RW_H * 2) == 0 && memcmp(a->rw_gp, b->rw_gp, RW_T * 4) == 0 &&
              memcmp(a->sq_y, b->sq_y, (size_t)SQ_R * SQ_H * 2) == 0 &&
              memcmp(a->sq_gx, b->sq_gx, (size_t)SQ_R * SQ_H * 2) == 0 && memcmp(a->sq_gp, b->sq_gp, SQ_R * 4) == 0 &&
              memcmp(a->up, b->up, (size_t)UP_T * UP_H * 4) == 0,
          "graph replay %d differs from the eager run", rep);
}

int main(void)
{
    CHECK(moe_elementwise_abi_version() == 1, "ABI version");

    /* inputs */
    uint16_t *h_ra_e = malloc((size_t)RA_N * 2), *h_ra_s = malloc((size_t)RA_N * 2), *h_ra_r = malloc((size_t)RA_N * 2);
    fill_bf16(h_ra_e, RA_N, 1.0f);
    fill_bf16(h_ra_s, RA_N, 1.0f);
    fill_bf16(h_ra_r, RA_N, 4.0f);
    uint16_t *h_rw_x = malloc((size_t)RW_T * RW_H * 2);
    float *h_rw_p = malloc(RW_T * 4), *h_rw_gout = malloc((size_t)RW_T * RW_H * 4);
    fill_bf16(h_rw_x, (size_t)RW_T * RW_H, 3.0f);
    for (int t = 0; t < RW_T; ++t) h_rw_p[t] = uniform();
    for (size_t i = 0; i < (size_t)RW_T * RW_H; ++i) h_rw_gout[i] = normalish(1.0f);
    uint16_t *h_sq_x = malloc((size_t)SQ_R * SQ_H * 2), *h_sq_gy = malloc((size_t)SQ_R * SQ_H * 2);
    float *h_sq_p = malloc(SQ_R * 4);
    int32_t *h_sq_perm = malloc(SQ_R * 4), h_sq_nu = SQ_USED;
    fill_bf16(h_sq_x, (size_t)SQ_R * SQ_H, 6.0f);
    fill_bf16(h_sq_gy, (size_t)SQ_R * SQ_H, 1.0f);
    for (int r = 0; r < SQ_R; ++r) { h_sq_p[r] = uniform(); h_sq_perm[r] = r; }
    for (int r = SQ_R - 1; r > 0; --r) { /* Fisher-Yates */
        int j = (int)(lcg() % (uint32_t)(r + 1));
        int32_t t = h_sq_perm[r]; h_sq_perm[r] = h_sq_perm[j]; h_sq_perm[j] = t;
    }
    for (int k = 0; k < 16; ++k) /* interior dummy rows */
        h_sq_perm[lcg() % (uint32_t)SQ_USED] = (k & 1) ? -1 : SQ_R + k;
    int32_t *h_up_map = malloc((size_t)UP_T * UP_E * 4), h_up_valid = UP_VALID;
    up_rows = 0;
    for (int e = 0; e < UP_E; ++e) /* expert-major rows, each (token, expert) routed with probability 1/2 */
        for (int t = 0; t < UP_T; ++t)
            h_up_map[(size_t)t * UP_E + e] = (lcg() & 1) ? (int32_t)up_rows++ : -1;
    uint16_t *h_up_eo = malloc((size_t)up_rows * UP_H * 2);
    fill_bf16(h_up_eo, (size_t)up_rows * UP_H, 1.0f);

    /* the oracle */
    uint16_t *w_ra = malloc((size_t)RA_N * 2), *w_rw_gx = malloc((size_t)RW_T * RW_H * 2);
    float *w_rw_out = malloc((size_t)RW_T * RW_H * 4), *w_rw_gp = malloc(RW_T * 4);
    double *w_rw_gp64 = malloc(RW_T * 8), *w_rw_scale = malloc(RW_T * 8);
    CHECK(oracle_residual_add(h_ra_e, h_ra_s, h_ra_r, w_ra, RA_N, MOE_BF16) == 0, "oracle residual add");
    CHECK(oracle_router_weight_fwd(h_rw_x, MOE_BF16, h_rw_p, w_rw_out, MOE_FP32, RW_T, RW_H) == 0, "oracle router fwd");
    CHECK(oracle_router_weight_bwd(h_rw_gout, MOE_FP32, h_rw_x, MOE_BF16, h_rw_p, w_rw_gx, w_rw_gp, w_rw_gp64,
                                   w_rw_scale, RW_T, RW_H) == 0,
          "oracle router bwd");
    uint16_t *w_sq_y = malloc((size_t)SQ_R * SQ_H * 2), *w_sq_gx = malloc((size_t)SQ_R * SQ_H * 2);
    float *w_sq_gp = malloc(SQ_R * 4);
    double *w_sq_gp64 = malloc(SQ_R * 8), *w_sq_scale = malloc(SQ_R * 8);
    for (size_t i = 0; i < (size_t)SQ_R * SQ_H; ++i) { w_sq_y[i] = 0xFFFF; w_sq_gx[i] = 0xFFFF; }
    for (int r = 0; r < SQ_R; ++r) { w_sq_gp[r] = -12345.5f; w_sq_gp64[r] = NAN; w_sq_scale[r] = NAN; }
    CHECK(oracle_squared_relu_probs_fwd(h_sq_x, h_sq_p, w_sq_y, SQ_R, SQ_H, 1, kScale, &h_sq_nu, h_sq_perm, 1) == 0,
          "oracle squared relu fwd");
    CHECK(oracle_squared_relu_probs_bwd(h_sq_x, h_sq_p, h_sq_gy, w_sq_gx, w_sq_gp, w_sq_gp64, w_sq_scale, SQ_R, SQ_H, 1,
                                        kScale, &h_sq_nu, h_sq_perm, 1) == 0,
          "oracle squared relu bwd");
    float *w_up = malloc((size_t)UP_T * UP_H * 4);
    for (size_t i = 0; i < (size_t)UP_T * UP_H; ++i) w_up[i] = NAN;
    CHECK(oracle_unpermute_expert_order(h_up_eo, up_rows, h_up_map, &h_up_valid, w_up, MOE_FP32, UP_T, UP_H, UP_E) == 0,
          "oracle unpermute");

    /* device buffers */
    ra_e = upload(h_ra_e, (size_t)RA_N * 2);
    ra_s = upload(h_ra_s, (size_t)RA_N * 2);
    ra_r = upload(h_ra_r, (size_t)RA_N * 2);
    ra_o = dalloc((size_t)RA_N * 2);
    rw_x = upload(h_rw_x, (size_t)RW_T * RW_H * 2);
    rw_p = upload(h_rw_p, RW_T * 4);
    rw_gout = upload(h_rw_gout, (size_t)RW_T * RW_H * 4);
    rw_out = dalloc((size_t)RW_T * RW_H * 4);
    rw_gx = dalloc((size_t)RW_T * RW_H * 2);
    rw_gp = dalloc(RW_T * 4);
    sq_x = upload(h_sq_x, (size_t)SQ_R * SQ_H * 2);
    sq_gy = upload(h_sq_gy, (size_t)SQ_R * SQ_H * 2);
    sq_p = upload(h_sq_p, SQ_R * 4);
    sq_nu = upload(&h_sq_nu, 4);
    sq_perm = upload(h_sq_perm, SQ_R * 4);
    sq_y = dalloc((size_t)SQ_R * SQ_H * 2);
    sq_gx = dalloc((size_t)SQ_R * SQ_H * 2);
    sq_gp = dalloc(SQ_R * 4);
    up_eo = upload(h_up_eo, (size_t)up_rows * UP_H * 2);
    up_map = upload(h_up_map, (size_t)UP_T * UP_E * 4);
    up_valid = upload(&h_up_valid, 4);
    up_out = dalloc((size_t)UP_T * UP_H * 4);
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));

    /* eager run against the oracle */
    reset_outputs();
    run_all(st);
    CHECK_HIP(hipStreamSynchronize(st));
    Outputs eager = download_all();
    check_bits(eager.ra, w_ra, (size_t)RA_N * 2, "residual add");
    check_bits(eager.rw_out, w_rw_out, (size_t)RW_T * RW_H * 4, "router fwd");
    check_bits(eager.rw_gx, w_rw_gx, (size_t)RW_T * RW_H * 2, "router grad_x");
    check_sums(eager.rw_gp, w_rw_gp, w_rw_gp64, w_rw_scale, RW_T, "router grad_probs");
    check_ulp(eager.sq_y, w_sq_y, (size_t)SQ_R * SQ_H, "squared relu y");
    check_ulp(eager.sq_gx, w_sq_gx, (size_t)SQ_R * SQ_H, "squared relu grad_x");
    check_sums(eager.sq_gp, w_sq_gp, w_sq_gp64, w_sq_scale, SQ_R, "squared relu grad_probs");
    for (int64_t r = SQ_USED; r < SQ_R; ++r) /* padding rows are +0 */
        for (int64_t j = 0; j < SQ_H; ++j)
            CHECK(eager.sq_y[r * SQ_H + j] == 0 && eager.sq_gx[r * SQ_H + j] == 0, "padding row %lld not +0",
                  (long long)r);
    for (size_t i = 0; i < (size_t)UP_T * UP_H; ++i) { /* bitwise, with NaN (untouched tokens) matching NaN */
        uint32_t g, w;
        memcpy(&g, &eager.up[i], 4);
        memcpy(&w, &w_up[i], 4);
        CHECK(g == w || (isnan(eager.up[i]) && isnan(w_up[i])), "unpermute: element %zu got %08x want %08x", i, g, w);
    }
    for (size_t i = (size_t)UP_VALID * UP_H; i < (size_t)UP_T * UP_H; ++i)
        CHECK(isnan(eager.up[i]), "unpermute: a token past valid_tokens was written");
    printf("eager run: ok (residual add %d, router %dx%d, squared relu %dx%d, unpermute %dx%dx%d)\n", RA_N, RW_T,
           RW_H, SQ_R, SQ_H, UP_T, UP_E, UP_H);
    fflush(stdout);

    /* the whole sequence in a HIP graph, replayed twice with other work in between */
    hipGraph_t graph;
    hipGraphExec_t exec;
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    run_all(st);
    CHECK_HIP(hipStreamEndCapture(st, &graph));
    CHECK_HIP(hipGraphInstantiate(&exec, graph, NULL, NULL, 0));
    for (int rep = 0; rep < 2; ++rep) {
        reset_outputs();
        CHECK_HIP(hipGraphLaunch(exec, st));
        CHECK_HIP(hipStreamSynchronize(st));
        Outputs replay = download_all();
        same_outputs(&replay, &eager, rep);
    }
    CHECK_HIP(hipGraphExecDestroy(exec));
    CHECK_HIP(hipGraphDestroy(graph));
    CHECK_HIP(hipStreamDestroy(st));
    printf("MoE C ABI check: ok\n");
    return 0;
}
