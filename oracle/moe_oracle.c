/*
 * CPU oracle for the MoE elementwise operations next to the routed-expert
 * activation. TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
 * bench's CPU-baseline leg use it. It shares no code with the HIP libraries.
 *
 *   residual add      Megatron-Core "core.fusions.fused_moe_residual_add" page:
 *                     out = residual + (expert_output + shared_expert_output). Each
 *                     of the two additions is done in fp32 and rounded to the element
 *                     type on its own, inner one first: the bits two separate
 *                     elementwise additions would give.
 *   router weight     NeMo AutoModel "moe/optimized_ops" page, _RouterWeightMulFunction:
 *                     forward: out = x * p per row, one fp32 product rounded to the
 *                     output type; backward: grad_x = g * p, one fp32 product rounded
 *                     to x's type, and grad_p = the row sum of g * x in fp32.
 *   squared ReLU      Megatron-Core "core.inference.moe.batch_invariant" page,
 *                     _squared_relu_with_probs_kernel / squared_relu_with_probs:
 *                     with the soft clamp, c = s * tanh(x / s), relu(c)^2 * p all in
 *                     fp32 with one final bf16 rounding; without it the square of the
 *                     bf16 ReLU output is rounded to bf16 first, then multiplied by
 *                     the fp32 probability and rounded again. Rows follow the same
 *                     n_used / permutation_map / zero_padding rules as the SwiGLU
 *                     activation (see swiglu_oracle.c). The backward, which the page
 *                     does not give, is the chain rule through that forward (see
 *                     oracle_squared_relu_probs_bwd).
 *   unpermute         same page, _unpermute_tokens_in_expert_order_kernel /
 *                     unpermute_tokens_in_expert_order: each output token sums its
 *                     local experts' contributions in fp32 in increasing expert id.
 *
 * Every elementwise operation is written in the order the pages state it, with
 * separately rounded fp32 operations (built without fast-math or FMA contraction).
 * Rows (tokens, or blocks of elements for the residual add) are split in static
 * contiguous blocks over `threads` POSIX threads; every row's arithmetic is the same
 * whichever thread runs it, so the results are bit-identical for any thread count.
 *
 * Element types: 0 = bf16, 1 = fp16, 2 = fp32 (16-bit types passed as bit patterns).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

enum { DT_BF16 = 0, DT_F16 = 1, DT_F32 = 2 };

/* ---------------------------------------------------------------------------
 * Conversions. bf16 and fp16 narrowings round to nearest, ties to even; NaN
 * stays NaN; values past the largest finite value become infinities.
 * ------------------------------------------------------------------------- */
static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, 4);
    return f;
}

static uint32_t bits_from_f32(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bf16_to_f32(uint16_t h) { return f32_from_bits((uint32_t)h << 16); }

static uint16_t f32_to_bf16(float f)
{
    uint32_t u = bits_from_f32(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16, drop = u & 0xffffu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u;
    return (uint16_t)keep;
}

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static float f16_to_f32(uint16_t h)
{
    uint32_t sign = (uint32_t)(h >> 15) & 1u, e = (h >> 10) & 0x1fu, m = h & 0x3ffu;
    float mag;
    if (e == 0)
        mag = ldexpf((float)m, -24);                 /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        mag = m ? NAN : INFINITY;
    else
        mag = ldexpf((float)(m | 0x400u), (int)e - 25); /* (1024 + m) * 2^(e - 25) */
    return sign ? -mag : mag;
}

static uint16_t f32_to_f16(float f)
{
    uint32_t u = bits_from_f32(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    float a = fabsf(f);
    if (isnan(f))
        return (uint16_t)(sign | 0x7e00u);
    if (a >= 65520.0f) /* at or past the midpoint between 65504 and 2^16: overflow */
        return (uint16_t)(sign | 0x7c00u);
    if (a < ldexpf(1.0f, -14)) {
        /* subnormal range: value = n * 2^-24, n rounded to nearest even */
        float n = a * 16777216.0f; /* exact: scales by 2^24 */
        float r = nearbyintf(n);   /* default rounding mode: ties to even */
        return (uint16_t)(sign | (uint16_t)r); /* r == 1024 carries into the exponent */
    }
    int ex;
    float fr = frexpf(a, &ex);           /* a = fr * 2^ex, fr in [0.5, 1) */
    float n = ldexpf(fr, 11);            /* 11 significant bits: [1024, 2048) */
    float r = nearbyintf(n);
    if (r == 2048.0f) {
        r = 1024.0f;
        ex += 1;
    }
    int e16 = ex - 1 + 15;               /* a = (r / 1024) * 2^(ex - 1) */
    if (e16 >= 31)
        return (uint16_t)(sign | 0x7c00u);
    return (uint16_t)(sign | (uint16_t)(e16 << 10) | ((uint16_t)r - 1024u));
}

static float load_elem(const void *p, int64_t i, int dt)
{
    if (dt == DT_BF16)
        return bf16_to_f32(((const uint16_t *)p)[i]);
    if (dt == DT_F16)
        return f16_to_f32(((const uint16_t *)p)[i]);
    return ((const float *)p)[i];
}

static void store_elem(void *p, int64_t i, int dt, float v)
{
    if (dt == DT_BF16)
        ((uint16_t *)p)[i] = f32_to_bf16(v);
    else if (dt == DT_F16)
        ((uint16_t *)p)[i] = f32_to_f16(v);
    else
        ((float *)p)[i] = v;
}

/* rounding of an fp32 value to the element type and back */
static float round_to(float v, int dt)
{
    if (dt == DT_BF16)
        return bf16_to_f32(f32_to_bf16(v));
    if (dt == DT_F16)
        return f16_to_f32(f32_to_f16(v));
    return v;
}

void oracle_f16_from_f32(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = f32_to_f16(src[i]);
}

void oracle_f32_from_f16(const uint16_t *src, float *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = f16_to_f32(src[i]);
}

/* ---------------------------------------------------------------------------
 * Static row blocks over POSIX threads
 * ------------------------------------------------------------------------- */
#define MOE_ORACLE_MAX_THREADS 256

typedef struct {
    const void *args;
    int64_t r0, r1;
    void (*body)(const void *, int64_t, int64_t);
} row_block_t;

static void *run_row_block(void *p)
{
    const row_block_t *b = (const row_block_t *)p;
    b->body(b->args, b->r0, b->r1);
    return NULL;
}

/* body(args, r0, r1) over [0, rows) in `threads` contiguous blocks (at most one per row). */
static void over_rows(int64_t rows, int threads, const void *args, void (*body)(const void *, int64_t, int64_t))
{
    if (threads < 1)
        threads = 1;
    if (threads > MOE_ORACLE_MAX_THREADS)
        threads = MOE_ORACLE_MAX_THREADS;
    if ((int64_t)threads > rows)
        threads = rows > 0 ? (int)rows : 1;
    if (threads == 1) {
        body(args, 0, rows);
        return;
    }
    pthread_t tid[MOE_ORACLE_MAX_THREADS];
    row_block_t blk[MOE_ORACLE_MAX_THREADS];
    int started[MOE_ORACLE_MAX_THREADS];
    int64_t per = rows / threads, extra = rows % threads, r = 0;
    for (int t = 0; t < threads; ++t) {
        const int64_t n = per + (t < extra ? 1 : 0);
        blk[t] = (row_block_t){args, r, r + n, body};
        r += n;
        started[t] = pthread_create(&tid[t], NULL, run_row_block, &blk[t]) == 0;
        if (!started[t])
            run_row_block(&blk[t]); /* fall back to the calling thread */
    }
    for (int t = 0; t < threads; ++t)
        if (started[t])
            pthread_join(tid[t], NULL);
}

/* ---------------------------------------------------------------------------
 * Fused MoE residual add
 * ------------------------------------------------------------------------- */
typedef struct {
    const void *expert, *shared, *residual;
    void *out;
    int64_t n;
    int dt;
} residual_args_t;

#define RESIDUAL_BLOCK 65536 /* elements per row block of the thread split */

static void residual_rows(const void *p, int64_t b0, int64_t b1)
{
    const residual_args_t *A = (const residual_args_t *)p;
    const int64_t i1 = b1 * RESIDUAL_BLOCK < A->n ? b1 * RESIDUAL_BLOCK : A->n;
    for (int64_t i = b0 * RESIDUAL_BLOCK; i < i1; ++i) {
        /* first add, rounded to the activation dtype; then the residual add */
        float t = round_to(load_elem(A->expert, i, A->dt) + load_elem(A->shared, i, A->dt), A->dt);
        store_elem(A->out, i, A->dt, load_elem(A->residual, i, A->dt) + t);
    }
}

int oracle_residual_add(const void *expert, const void *shared, const void *residual, void *out,
                        int64_t n, int dt, int threads)
{
    if (n < 0 || dt < 0 || dt > 2)
        return 1;
    const residual_args_t a = {expert, shared, residual, out, n, dt};
    over_rows((n + RESIDUAL_BLOCK - 1) / RESIDUAL_BLOCK, threads, &a, residual_rows);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Router-weight multiply
 * ------------------------------------------------------------------------- */
typedef struct {
    const void *x;
    int x_dt;
    const float *probs;
    void *out;
    int out_dt;
    int64_t hidden;
} router_fwd_args_t;

static void router_fwd_rows(const void *p, int64_t t0, int64_t t1)
{
    const router_fwd_args_t *A = (const router_fwd_args_t *)p;
    const int64_t hidden = A->hidden;
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t h = 0; h < hidden; ++h)
            store_elem(A->out, t * hidden + h, A->out_dt, load_elem(A->x, t * hidden + h, A->x_dt) * A->probs[t]);
}

int oracle_router_weight_fwd(const void *x, int x_dt, const float *probs, void *out, int out_dt,
                             int64_t tokens, int64_t hidden, int threads)
{
    if (tokens < 0 || hidden < 0)
        return 1;
    const router_fwd_args_t a = {x, x_dt, probs, out, out_dt, hidden};
    over_rows(tokens, threads, &a, router_fwd_rows);
    return 0;
}

/* grad_probs accumulated in fp64 in column order (and returned rounded to fp32),
 * beside the row scale S = sum |g * x|; grad_x / grad_probs may be NULL. */
typedef struct {
    const void *grad_out;
    int out_dt;
    const void *x;
    int x_dt;
    const float *probs;
    void *grad_x;
    float *grad_probs;
    double *grad_probs_f64, *row_scale;
    int64_t hidden;
} router_bwd_args_t;

static void router_bwd_rows(const void *p, int64_t t0, int64_t t1)
{
    const router_bwd_args_t *A = (const router_bwd_args_t *)p;
    const int64_t hidden = A->hidden;
    for (int64_t t = t0; t < t1; ++t) {
        double acc = 0.0, scale = 0.0;
        for (int64_t h = 0; h < hidden; ++h) {
            float g = load_elem(A->grad_out, t * hidden + h, A->out_dt);
            if (A->grad_x)
                store_elem(A->grad_x, t * hidden + h, A->x_dt, g * A->probs[t]);
            if (A->grad_probs || A->grad_probs_f64 || A->row_scale) {
                float term = g * load_elem(A->x, t * hidden + h, A->x_dt);
                acc += (double)term;
                scale += fabs((double)term);
            }
        }
        if (A->grad_probs)
            A->grad_probs[t] = (float)acc;
        if (A->grad_probs_f64)
            A->grad_probs_f64[t] = acc;
        if (A->row_scale)
            A->row_scale[t] = scale;
    }
}

/* grad_probs accumulated in fp64 in column order (and returned rounded to fp32),
 * beside the row scale S = sum |g * x|; grad_x / grad_probs may be NULL. */
int oracle_router_weight_bwd(const void *grad_out, int out_dt, const void *x, int x_dt,
                             const float *probs, void *grad_x, float *grad_probs,
                             double *grad_probs_f64, double *row_scale, int64_t tokens,
                             int64_t hidden, int threads)
{
    if (tokens < 0 || hidden < 0)
        return 1;
    const router_bwd_args_t a = {grad_out, out_dt, x, x_dt, probs, grad_x, grad_probs, grad_probs_f64,
                                 row_scale, hidden};
    over_rows(tokens, threads, &a, router_bwd_rows);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Squared ReLU x probs (forward), with the SwiGLU rows' bookkeeping
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *x;
    const float *probs;
    uint16_t *y;
    int64_t rows, hidden, bound;
    int clamp;
    float clamp_scale;
    const int32_t *perm;
    int zero_padding;
} sqrelu_fwd_args_t;

/* the slot of row r (-1 when not live): the SwiGLU rows' rules */
static int64_t row_slot(int64_t r, int64_t rows, int64_t bound, const int32_t *perm)
{
    if (r >= bound)
        return -1;
    const int64_t slot = perm ? (int64_t)perm[r] : r;
    return (slot < 0 || slot >= rows) ? -1 : slot;
}

static void sqrelu_fwd_rows(const void *p, int64_t r0, int64_t r1)
{
    const sqrelu_fwd_args_t *A = (const sqrelu_fwd_args_t *)p;
    const int64_t hidden = A->hidden;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t slot = row_slot(r, A->rows, A->bound, A->perm);
        uint16_t *yr = A->y + r * hidden;
        if (slot < 0) {
            if (A->zero_padding)
                memset(yr, 0, (size_t)hidden * sizeof(uint16_t));
            continue;
        }
        const float p = A->probs[slot];
        for (int64_t h = 0; h < hidden; ++h) {
            float v = bf16_to_f32(A->x[r * hidden + h]);
            if (A->clamp) {
                float c = A->clamp_scale * tanhf(v / A->clamp_scale); /* soft clamp, fp32 */
                float a = c < 0.0f ? 0.0f : c;                       /* relu; NaN passes, as torch.relu */
                yr[h] = f32_to_bf16((a * a) * p);                     /* one rounding */
            } else {
                float a = v < 0.0f ? 0.0f : v;                        /* relu of bf16: bf16 */
                float sq = bf16_to_f32(f32_to_bf16(a * a));           /* square materialised in bf16 */
                yr[h] = f32_to_bf16(sq * p);
            }
        }
    }
}

int oracle_squared_relu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y, int64_t rows,
                                  int64_t hidden, int clamp, float clamp_scale,
                                  const int32_t *n_used, const int32_t *perm, int zero_padding, int threads)
{
    if (rows < 0 || hidden <= 0)
        return 1;
    if (clamp && !(clamp_scale > 0.0f && isfinite(clamp_scale)))
        return 1;
    int64_t bound = rows;
    if (n_used) {
        bound = *n_used < 0 ? 0 : *n_used;
        if (bound > rows)
            bound = rows;
    }
    const sqrelu_fwd_args_t a = {x, probs, y, rows, hidden, bound, clamp, clamp_scale, perm, zero_padding};
    over_rows(rows, threads, &a, sqrelu_fwd_rows);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Squared ReLU x probs, backward: the chain rule through the forward above.
 * With y_pre the fp32 value the forward multiplies by p (a^2 with the soft clamp,
 * the bf16-rounded square without it) and g = grad_y widened to fp32:
 *   grad_x     = bf16( ((g * p) * (2 a)) * d )  where x > 0, else +0
 *                d = dc/dx = sech^2(x / s) with the clamp, 1 without it
 *   grad_probs = sum over the row of g * y_pre  (fp64 here, returned as fp32)
 * The bf16 rounding of the square passes the gradient through unchanged, as a
 * dtype cast does under autograd. The ReLU mask is x > 0 (for s > 0 the sign of
 * s * tanh(x / s) is the sign of x), false for NaN, so a NaN input gets a zero
 * gradient. sech^2 is written as 4 e / (1 + e)^2, e = e^(-2|z|): it equals
 * 1 - tanh^2(z) but keeps its relative accuracy where tanh(z) rounds to 1.
 * Rows follow the forward's rules; with zero_padding, grad_x of a row that is
 * not live is +0; grad_probs is written only for live slots.
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *x;
    const float *probs;
    const uint16_t *grad_y;
    uint16_t *grad_x;
    float *grad_probs;
    double *grad_probs_f64, *row_scale;
    int64_t rows, hidden, bound;
    int clamp;
    float clamp_scale;
    const int32_t *perm;
    int zero_padding;
} sqrelu_bwd_args_t;

static void sqrelu_bwd_rows(const void *p, int64_t r0, int64_t r1)
{
    const sqrelu_bwd_args_t *A = (const sqrelu_bwd_args_t *)p;
    const int64_t hidden = A->hidden;
    const float clamp_scale = A->clamp_scale;
    for (int64_t r = r0; r < r1; ++r) {
        const int64_t slot = row_slot(r, A->rows, A->bound, A->perm);
        if (slot < 0) {
            if (A->zero_padding && A->grad_x)
                memset(A->grad_x + r * hidden, 0, (size_t)hidden * sizeof(uint16_t));
            continue;
        }
        const float prob = A->probs[slot]; /* gathered through the map */
        double acc = 0.0, scale = 0.0;
        for (int64_t h = 0; h < hidden; ++h) {
            const float v = bf16_to_f32(A->x[r * hidden + h]);
            const float g = bf16_to_f32(A->grad_y[r * hidden + h]);
            float ypre, gx;
            if (A->clamp) {
                float z = v / clamp_scale;
                float c = clamp_scale * tanhf(z);
                float a = (c < 0.0f) ? 0.0f : c; /* relu; NaN passes */
                ypre = a * a;
                float e = expf(-2.0f * fabsf(z));
                float sech2 = (4.0f * e) / ((1.0f + e) * (1.0f + e));
                gx = v > 0.0f ? ((g * prob) * (2.0f * a)) * sech2 : 0.0f;
            } else {
                float a = (v < 0.0f) ? 0.0f : v;
                ypre = bf16_to_f32(f32_to_bf16(a * a));
                gx = v > 0.0f ? (g * prob) * (2.0f * a) : 0.0f;
            }
            if (A->grad_x)
                A->grad_x[r * hidden + h] = f32_to_bf16(gx);
            const float term = g * ypre;
            acc += (double)term;
            scale += fabs((double)term);
        }
        if (A->grad_probs)
            A->grad_probs[slot] = (float)acc;
        if (A->grad_probs_f64)
            A->grad_probs_f64[slot] = acc;
        if (A->row_scale)
            A->row_scale[slot] = scale;
    }
}

int oracle_squared_relu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                  uint16_t *grad_x, float *grad_probs, double *grad_probs_f64,
                                  double *row_scale, int64_t rows, int64_t hidden, int clamp,
                                  float clamp_scale, const int32_t *n_used, const int32_t *perm,
                                  int zero_padding, int threads)
{
    if (rows < 0 || hidden <= 0)
        return 1;
    if (clamp && !(clamp_scale > 0.0f && isfinite(clamp_scale)))
        return 1;
    int64_t bound = rows;
    if (n_used) {
        bound = *n_used < 0 ? 0 : *n_used;
        if (bound > rows)
            bound = rows;
    }
    const sqrelu_bwd_args_t a = {x, probs, grad_y, grad_x, grad_probs, grad_probs_f64, row_scale,
                                 rows, hidden, bound, clamp, clamp_scale, perm, zero_padding};
    over_rows(rows, threads, &a, sqrelu_bwd_rows);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Token-local unpermute in fixed expert order
 * out[t, :] = sum over local experts e = 0, 1, ..., E-1 with map[t, e] a valid row
 * of expert_output[map[t, e], :], accumulated in fp32 in that order from +0, then
 * stored as fp32 or rounded once to bf16. Tokens t >= valid_tokens are neither read
 * nor written.
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *expert_output;
    int64_t expert_rows;
    const int32_t *inverse_map;
    void *out;
    int out_dt;
    int64_t hidden, num_local_experts;
} unpermute_args_t;

static void unpermute_rows(const void *p, int64_t t0, int64_t t1)
{
    const unpermute_args_t *A = (const unpermute_args_t *)p;
    const int64_t hidden = A->hidden, E = A->num_local_experts;
    for (int64_t t = t0; t < t1; ++t)
        for (int64_t h = 0; h < hidden; ++h) {
            float acc = 0.0f;
            for (int64_t e = 0; e < E; ++e) {
                int64_t row = A->inverse_map[t * E + e];
                if (row >= 0 && row < A->expert_rows)
                    acc = acc + bf16_to_f32(A->expert_output[row * hidden + h]);
            }
            store_elem(A->out, t * hidden + h, A->out_dt, acc);
        }
}

int oracle_unpermute_expert_order(const uint16_t *expert_output, int64_t expert_rows,
                                  const int32_t *inverse_map, const int32_t *valid_tokens,
                                  void *out, int out_dt, int64_t tokens, int64_t hidden,
                                  int64_t num_local_experts, int threads)
{
    if (tokens < 0 || hidden <= 0 || num_local_experts <= 0 || expert_rows < 0)
        return 1;
    int64_t bound = tokens;
    if (valid_tokens) {
        bound = *valid_tokens < 0 ? 0 : *valid_tokens;
        if (bound > tokens)
            bound = tokens;
    }
    const unpermute_args_t a = {expert_output, expert_rows, inverse_map, out, out_dt, hidden, num_local_experts};
    over_rows(bound, threads, &a, unpermute_rows);
    return 0;
}
