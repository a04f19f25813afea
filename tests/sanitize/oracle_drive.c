/*
 * Drives every function of the CPU oracle (oracle/swiglu_oracle.c, oracle/moe_oracle.c)
 * over small inputs and edge cases, for a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer (test infrastructure). Inputs hold every kind of bf16 /
 * fp16 / fp32 value (NaN, +-inf, subnormals, +-0) and every row rule: a device-style
 * n_used (negative, inside, past the end), permutations with dummy entries (-1, rows,
 * INT_MIN), zero padding on and off, several thread counts, zero-size and rejected
 * arguments. It checks what the oracle documents about rows it must not touch and
 * rows it must zero; any sanitizer report ends the run with a non-zero status.
 */
#include <limits.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

uint16_t oracle_bf16_rne(float f);
void oracle_bf16_rne_array(const float *src, uint16_t *dst, int64_t n);
int oracle_swiglu_fwd(const uint16_t *x, const float *probs, uint16_t *y, int64_t rows, int64_t inter,
                      float limit, const int32_t *n_used, const int32_t *permutation_map, int zero_padding,
                      int threads);
int oracle_swiglu_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y, uint16_t *grad_x,
                      float *grad_probs, double *grad_probs_f64, double *row_scale, int64_t rows, int64_t inter,
                      float limit, const int32_t *n_used, const int32_t *permutation_map, int zero_padding,
                      int threads);
int oracle_swiglu_fwd_f64(const double *x, const double *probs, double *y, int64_t rows, int64_t inter,
                          double limit);
int oracle_swiglu_bwd_f64(const double *x, const double *probs, const double *grad_y, double *grad_x,
                          double *grad_probs, int64_t rows, int64_t inter, double limit);

void oracle_f16_from_f32(const float *src, uint16_t *dst, int64_t n);
void oracle_f32_from_f16(const uint16_t *src, float *dst, int64_t n);
int oracle_residual_add(const void *expert, const void *shared, const void *residual, void *out, int64_t n,
                        int dt, int threads);
int oracle_router_weight_fwd(const void *x, int x_dt, const float *probs, void *out, int out_dt, int64_t tokens,
                             int64_t hidden, int threads);
int oracle_router_weight_bwd(const void *grad_out, int out_dt, const void *x, int x_dt, const float *probs,
                             void *grad_x, float *grad_probs, double *grad_probs_f64, double *row_scale,
                             int64_t tokens, int64_t hidden, int threads);
int oracle_squared_relu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y, int64_t rows,
                                  int64_t hidden, int clamp, float clamp_scale, const int32_t *n_used,
                                  const int32_t *perm, int zero_padding, int threads);
int oracle_squared_relu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                  uint16_t *grad_x, float *grad_probs, double *grad_probs_f64,
                                  double *row_scale, int64_t rows, int64_t hidden, int clamp,
                                  float clamp_scale, const int32_t *n_used, const int32_t *perm,
                                  int zero_padding, int threads);
int oracle_unpermute_expert_order(const uint16_t *expert_output, int64_t expert_rows,
                                  const int32_t *inverse_map, const int32_t *valid_tokens, void *out,
                                  int out_dt, int64_t tokens, int64_t hidden, int64_t num_local_experts,
                                  int threads);

#define CHECK(cond, ...)                                                                  \
    do {                                                                                  \
        if (!(cond)) {                                                                    \
            fprintf(stderr, __VA_ARGS__);                                                 \
            fprintf(stderr, "\n");                                                        \
            exit(1);                                                                      \
        }                                                                                 \
    } while (0)

static uint64_t state = 7;
static uint32_t next(void)
{
    state = state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (uint32_t)(state >> 32);
}

/* 16-bit patterns: mostly ordinary bf16 values, with every special kind mixed in */
static void fill16(uint16_t *a, size_t n)
{
    static const uint16_t specials[] = {0x0000, 0x8000, 0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0001, 0x8001,
                                        0x007F, 0x40E0, 0xC0E0, 0x40E1, 0x7F7F, 0xFF7F};
    for (size_t i = 0; i < n; ++i) {
        const uint32_t r = next();
        a[i] = (r & 15) == 0 ? specials[(r >> 4) % (sizeof specials / sizeof specials[0])]
                             : (uint16_t)(0x3C00 + ((r >> 8) & 0x0FFF) - 0x0800 + ((r >> 20) & 1 ? 0x8000 : 0));
    }
}

static void fill32(float *a, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        const uint32_t r = next();
        a[i] = (r & 31) == 0 ? ((r >> 5) & 1 ? INFINITY : NAN) : (float)(r >> 8) / 16777216.0f * 4.0f - 2.0f;
    }
}

static void probs01(float *p, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        p[i] = (float)(next() >> 8) / 16777216.0f;
}

static int all16(const uint16_t *a, size_t n, uint16_t v)
{
    for (size_t i = 0; i < n; ++i)
        if (a[i] != v)
            return 0;
    return 1;
}

/* row bookkeeping variants shared by the activation and the squared ReLU */
enum { ROWS = 37 };
static const int32_t kNUsed[] = {-5, 0, 1, 20, ROWS, ROWS + 9};

static void make_perm(int32_t *perm, int dummies)
{
    for (int r = 0; r < ROWS; ++r)
        perm[r] = r;
    for (int r = ROWS - 1; r > 0; --r) {
        const int j = (int)(next() % (uint32_t)(r + 1));
        const int32_t t = perm[r];
        perm[r] = perm[j];
        perm[j] = t;
    }
    if (dummies) {
        perm[3] = -1;
        perm[11] = ROWS;
        perm[19] = INT_MIN;
    }
}

/* a row is live iff r < clamp(n_used) and its slot is in range; mirrors the oracle's rule */
static int live(int r, const int32_t *nu, const int32_t *perm)
{
    int bound = ROWS;
    if (nu)
        bound = *nu < 0 ? 0 : (*nu > ROWS ? ROWS : *nu);
    if (r >= bound)
        return 0;
    const int64_t slot = perm ? perm[r] : r;
    return slot >= 0 && slot < ROWS;
}

static void drive_swiglu(void)
{
    const int64_t inter = 24, W = 2 * inter;
    uint16_t *x = malloc(ROWS * W * 2), *gy = malloc(ROWS * inter * 2), *y = malloc(ROWS * inter * 2),
             *gx = malloc(ROWS * W * 2);
    float *p = malloc(ROWS * 4), *gp = malloc(ROWS * 4);
    double *gp64 = malloc(ROWS * 8), *scale = malloc(ROWS * 8);
    int32_t perm[ROWS];
    fill16(x, ROWS * W);
    fill16(gy, ROWS * inter);
    probs01(p, ROWS);
    const float limits[] = {7.0f, INFINITY, 0.5f};
    for (int li = 0; li < 3; ++li)
        for (int nui = -1; nui < (int)(sizeof kNUsed / sizeof kNUsed[0]); ++nui)
            for (int pm = 0; pm < 3; ++pm)
                for (int zp = 0; zp < 2; ++zp) {
                    const int32_t *nu = nui < 0 ? NULL : &kNUsed[nui];
                    if (pm)
                        make_perm(perm, pm == 2);
                    const int32_t *mp = pm ? perm : NULL;
                    const int threads = 1 + (int)(next() % 4);
                    memset(y, 0xAB, ROWS * inter * 2);
                    memset(gx, 0xAB, ROWS * W * 2);
                    for (int r = 0; r < ROWS; ++r)
                        gp[r] = -3.0f;
                    CHECK(oracle_swiglu_fwd(x, p, y, ROWS, inter, limits[li], nu, mp, zp, threads) == 0, "fwd");
                    CHECK(oracle_swiglu_bwd(x, p, gy, gx, gp, gp64, scale, ROWS, inter, limits[li], nu, mp, zp,
                                            threads) == 0,
                          "bwd");
                    for (int r = 0; r < ROWS; ++r)
                        if (!live(r, nu, mp)) {
                            const uint16_t want = zp ? 0x0000 : 0xABAB;
                            CHECK(all16(y + r * inter, inter, want) && all16(gx + r * W, W, want),
                                  "swiglu row %d not live: wrong contents", r);
                        }
                    if (!mp)  /* unmapped: slot r is written exactly for the live rows */
                        for (int r = 0; r < ROWS; ++r)
                            CHECK(live(r, nu, mp) == (gp[r] != -3.0f), "swiglu grad_probs slot %d", r);
                }
    /* fp64 path, a NULL grad_probs, and the rejected / empty calls */
    double *xd = malloc(ROWS * W * 8), *pd = malloc(ROWS * 8), *gyd = malloc(ROWS * inter * 8),
           *yd = malloc(ROWS * inter * 8), *gxd = malloc(ROWS * W * 8), *gpd = malloc(ROWS * 8);
    for (int64_t i = 0; i < ROWS * W; ++i)
        xd[i] = (double)(next() >> 8) / 1048576.0 - 8.0;
    for (int64_t i = 0; i < ROWS * inter; ++i)
        gyd[i] = (double)(next() >> 8) / 8388608.0 - 1.0;
    for (int r = 0; r < ROWS; ++r)
        pd[r] = (double)p[r];
    CHECK(oracle_swiglu_fwd_f64(xd, pd, yd, ROWS, inter, 7.0) == 0, "fwd f64");
    CHECK(oracle_swiglu_bwd_f64(xd, pd, gyd, gxd, gpd, ROWS, inter, 7.0) == 0, "bwd f64");
    CHECK(oracle_swiglu_bwd(x, p, gy, gx, NULL, NULL, NULL, ROWS, inter, 7.0f, NULL, NULL, 0, 2) == 0, "bwd, no sums");
    CHECK(oracle_swiglu_fwd(x, p, y, 0, inter, 7.0f, NULL, NULL, 0, 1) == 0, "rows 0");
    CHECK(oracle_swiglu_bwd(x, p, gy, gx, gp, gp64, scale, 0, inter, 7.0f, NULL, NULL, 0, 1) == 0, "rows 0 bwd");
    CHECK(oracle_swiglu_fwd(x, p, y, -1, inter, 7.0f, NULL, NULL, 0, 1) != 0, "rows < 0 accepted");
    CHECK(oracle_swiglu_fwd(x, p, y, ROWS, 0, 7.0f, NULL, NULL, 0, 1) != 0, "inter 0 accepted");
    CHECK(oracle_swiglu_fwd(x, p, y, ROWS, inter, NAN, NULL, NULL, 0, 1) != 0, "NaN limit accepted");
    CHECK(oracle_swiglu_fwd(x, p, y, ROWS, inter, -1.0f, NULL, NULL, 0, 1) != 0, "negative limit accepted");
    CHECK(oracle_swiglu_fwd_f64(xd, pd, yd, ROWS, inter, 0.0) != 0, "f64 limit 0 accepted");
    /* the rounding helpers on every special */
    float f[8] = {0.0f, -0.0f, INFINITY, -INFINITY, NAN, 1e-45f, 3.4028235e38f, 1.0039062f};
    uint16_t h[8];
    oracle_bf16_rne_array(f, h, 8);
    CHECK(h[0] == 0x0000 && h[1] == 0x8000 && h[2] == 0x7F80 && h[3] == 0xFF80 && (h[4] & 0x7F80) == 0x7F80 &&
              (h[4] & 0x7F) && h[6] == 0x7F80 && h[7] == oracle_bf16_rne(f[7]),
          "bf16 rounding specials");
    free(x), free(gy), free(y), free(gx), free(p), free(gp), free(gp64), free(scale);
    free(xd), free(pd), free(gyd), free(yd), free(gxd), free(gpd);
}

static void drive_moe(void)
{
    /* fp16 conversions both ways over every pattern */
    uint16_t *h = malloc(65536 * 2), *h2 = malloc(65536 * 2);
    float *f = malloc(65536 * 4);
    for (int i = 0; i < 65536; ++i)
        h[i] = (uint16_t)i;
    oracle_f32_from_f16(h, f, 65536);
    oracle_f16_from_f32(f, h2, 65536);
    for (int i = 0; i < 65536; ++i)
        CHECK(h2[i] == h[i] || ((h[i] & 0x7C00) == 0x7C00 && (h[i] & 0x3FF)), "fp16 round trip %04x", i);
    free(h), free(h2), free(f);

    /* residual add and router weight in every dtype (0 bf16, 1 fp16, 2 fp32) */
    const int64_t T = 29, H = 40;
    uint16_t *a16 = malloc(T * H * 2), *b16 = malloc(T * H * 2), *c16 = malloc(T * H * 2), *o16 = malloc(T * H * 2);
    float *a32 = malloc(T * H * 4), *b32 = malloc(T * H * 4), *c32 = malloc(T * H * 4), *o32 = malloc(T * H * 4);
    float *p = malloc(T * 4), *gp = malloc(T * 4);
    double *gp64 = malloc(T * 8), *scale = malloc(T * 8);
    fill16(a16, T * H), fill16(b16, T * H), fill16(c16, T * H);
    fill32(a32, T * H), fill32(b32, T * H), fill32(c32, T * H);
    probs01(p, T);
    for (int dt = 0; dt < 3; ++dt) {
        const void *a = dt == 2 ? (const void *)a32 : a16, *b = dt == 2 ? (const void *)b32 : b16,
                   *c = dt == 2 ? (const void *)c32 : c16;
        void *o = dt == 2 ? (void *)o32 : o16;
        CHECK(oracle_residual_add(a, b, c, o, T * H - 3, dt, 3) == 0, "residual add dt %d", dt);
        CHECK(oracle_residual_add(a, b, c, o, 0, dt, 3) == 0, "residual add n 0");
        for (int odt = 0; odt < 3; ++odt) {
            if (!(odt == dt || odt == 2))
                continue;
            const void *g = odt == 2 ? (const void *)b32 : b16;
            void *out = odt == 2 ? (void *)o32 : o16;
            void *gx = dt == 2 ? (void *)c32 : c16;
            CHECK(oracle_router_weight_fwd(a, dt, p, out, odt, T, H, 3) == 0, "router fwd");
            CHECK(oracle_router_weight_bwd(g, odt, a, dt, p, gx, gp, gp64, scale, T, H, 3) == 0, "router bwd");
            CHECK(oracle_router_weight_bwd(g, odt, NULL, dt, p, gx, NULL, NULL, NULL, T, H, 2) == 0, "router bwd gx only");
        }
    }
    CHECK(oracle_residual_add(a16, b16, c16, o16, -1, 0, 1) != 0 && oracle_residual_add(a16, b16, c16, o16, 4, 3, 1) != 0,
          "bad residual add accepted");
    CHECK(oracle_router_weight_fwd(a16, 0, p, o16, 0, -1, H, 1) != 0, "bad router accepted");

    /* squared ReLU forward and backward over the row rules, with and without the clamp */
    const int64_t SH = 16;
    uint16_t *x = malloc(ROWS * SH * 2), *gy = malloc(ROWS * SH * 2), *y = malloc(ROWS * SH * 2),
             *gx = malloc(ROWS * SH * 2);
    float *sp = malloc(ROWS * 4), *sgp = malloc(ROWS * 4);
    double *sgp64 = malloc(ROWS * 8), *sscale = malloc(ROWS * 8);
    int32_t perm[ROWS];
    fill16(x, ROWS * SH), fill16(gy, ROWS * SH);
    probs01(sp, ROWS);
    const float scales[] = {4.0f, 1e-30f, 3.0e38f};
    for (int clamp = 0; clamp < 2; ++clamp)
        for (int si = 0; si < (clamp ? 3 : 1); ++si)
            for (int nui = -1; nui < (int)(sizeof kNUsed / sizeof kNUsed[0]); ++nui)
                for (int pm = 0; pm < 3; ++pm)
                    for (int zp = 0; zp < 2; ++zp) {
                        const int32_t *nu = nui < 0 ? NULL : &kNUsed[nui];
                        if (pm)
                            make_perm(perm, pm == 2);
                        const int32_t *mp = pm ? perm : NULL;
                        memset(y, 0xAB, ROWS * SH * 2);
                        memset(gx, 0xAB, ROWS * SH * 2);
                        CHECK(oracle_squared_relu_probs_fwd(x, sp, y, ROWS, SH, clamp, scales[si], nu, mp, zp, 3) == 0,
                              "sqrelu fwd");
                        CHECK(oracle_squared_relu_probs_bwd(x, sp, gy, gx, sgp, sgp64, sscale, ROWS, SH, clamp,
                                                            scales[si], nu, mp, zp, 3) == 0,
                              "sqrelu bwd");
                        for (int r = 0; r < ROWS; ++r)
                            if (!live(r, nu, mp)) {
                                const uint16_t want = zp ? 0x0000 : 0xABAB;
                                CHECK(all16(y + r * SH, SH, want) && all16(gx + r * SH, SH, want),
                                      "sqrelu row %d not live: wrong contents", r);
                            }
                    }
    CHECK(oracle_squared_relu_probs_fwd(x, sp, y, ROWS, SH, 1, 0.0f, NULL, NULL, 0, 1) != 0, "clamp scale 0 accepted");
    CHECK(oracle_squared_relu_probs_bwd(x, sp, gy, gx, sgp, NULL, NULL, ROWS, SH, 1, INFINITY, NULL, NULL, 0, 1) != 0,
          "infinite clamp scale accepted");

    /* unpermute: 1 to 8 experts, maps with invalid entries, a valid_tokens bound, both outputs */
    const int64_t UT = 23, UH = 24, ER = 50;
    uint16_t *eo = malloc(ER * UH * 2), *u16 = malloc(UT * UH * 2);
    float *u32 = malloc(UT * UH * 4);
    int32_t *map = malloc(UT * 8 * 4);
    fill16(eo, ER * UH);
    const int32_t valid[] = {-2, 0, 11, (int32_t)UT, (int32_t)UT + 5};
    for (int E = 1; E <= 8; ++E)
        for (int vi = -1; vi < 5; ++vi) {
            for (int64_t i = 0; i < UT * E; ++i) {
                const uint32_t r = next() % 8;
                map[i] = r < 4 ? (int32_t)(next() % ER) : (r == 4 ? -1 : (r == 5 ? (int32_t)ER : (r == 6 ? INT_MIN : -7)));
            }
            const int32_t *vt = vi < 0 ? NULL : &valid[vi];
            memset(u32, 0xAB, UT * UH * 4);
            memset(u16, 0xAB, UT * UH * 2);
            CHECK(oracle_unpermute_expert_order(eo, ER, map, vt, u32, 2, UT, UH, E, 3) == 0, "unpermute f32");
            CHECK(oracle_unpermute_expert_order(eo, ER, map, vt, u16, 0, UT, UH, E, 3) == 0, "unpermute bf16");
            int bound = (int)UT;
            if (vt)
                bound = *vt < 0 ? 0 : (*vt > UT ? (int)UT : *vt);
            for (int64_t t = bound; t < UT; ++t)
                CHECK(all16(u16 + t * UH, UH, 0xABAB), "unpermute wrote past valid_tokens");
        }
    CHECK(oracle_unpermute_expert_order(eo, ER, map, NULL, u32, 2, UT, UH, 0, 1) != 0, "zero experts accepted");
    CHECK(oracle_unpermute_expert_order(eo, 0, map, NULL, u32, 2, UT, UH, 2, 2) == 0, "no expert rows");

    free(a16), free(b16), free(c16), free(o16), free(a32), free(b32), free(c32), free(o32), free(p), free(gp);
    free(gp64), free(scale), free(x), free(gy), free(y), free(gx), free(sp), free(sgp), free(sgp64), free(sscale);
    free(eo), free(u16), free(u32), free(map);
}

int main(void)
{
    drive_swiglu();
    drive_moe();
    printf("oracle sanitizer drive: ok\n");
    return 0;
}
