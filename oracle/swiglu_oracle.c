/*
 * CPU oracle for the clamped SwiGLU x routing-probability expert activation.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may link, load or call
 * this file: only the tests, the smoke check and the bench's CPU-baseline leg
 * use it. It shares no code, header, table or helper with the HIP library.
 *
 * What it computes (NeMo AutoModel "moe/swiglu_triton" page, module docstring
 * and the SwigluClampedTriton class entry):
 *   x = [gate | up], bf16, [rows, 2*inter], gate is the first half;
 *   y = silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs
 * with every step in fp32 and a single rounding of y to bf16 (same page, the
 * forward kernel description; Megatron-Core "core.inference.moe.batch_invariant"
 * page, _swiglu_with_probs_kernel: fp32 SiLU(gate)*up*prob, one BF16 round).
 *
 * Backward (swiglu_triton page, backward kernel description; clamp gradients
 * follow torch.clamp, i.e. inclusive range masks on the input values):
 *   gp      = grad_y * p
 *   d_gate  = [gate <= L]        * ((gp * cu) * silu'(cg))
 *   d_up    = [-L <= up <= L]    * (gp * s)
 *   grad_p  = sum_j grad_y * (s * cu)
 * where cg = clamp(gate, max=L), cu = clamp(up, -L, L), sig = 1/(1+exp(-cg)),
 * s = cg*sig and silu'(cg) = sig*(1 + cg*(1 - sig)). d_gate and d_up are each
 * rounded once to bf16 and stored into the gate and up halves of grad_x. The
 * association order follows autograd's chain for y = (s*cu)*p, the same chain
 * the NeMo AutoModel "moe/optimized_ops" page spells out for a probs multiply
 * (_RouterWeightMulFunction: grad_x = g*probs, grad_probs = sum(g*x) in fp32).
 * The per-row sum is accumulated here in fp64, in column order; the row's
 * condition scale S = sum_j |grad_y * s * cu| is returned beside it.
 *
 * Row bookkeeping (Megatron-Core batch_invariant page: _swiglu_with_probs_kernel,
 * swiglu_with_probs, _weighted_silu_mul_bounded_kernel):
 *   live bound = n_used ? clamp(*n_used, 0, rows) : rows;
 *   row r is live iff r < bound and (no permutation_map, or 0 <= map[r] < rows);
 *   slot(r) = map ? map[r] : r; the probability is probs[slot(r)] and the
 *   probability gradient goes to grad_probs[slot(r)];
 *   rows that are not live are not read; with zero_padding their output rows
 *   are set to +0, without it they are left untouched; grad_probs is written
 *   only for live rows.
 *
 * Rows are split in static contiguous blocks over `threads` POSIX threads.
 * Every output element is computed by one thread from its own row only, so the
 * bits do not depend on the thread count.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared (no fast-math, no FMA
 * contraction: every fp32 operation is rounded as written).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <string.h>

/* ---------------------------------------------------------------------------
 * bf16 <-> fp32
 * bf16 is the upper half of an IEEE-754 binary32, so widening is exact.
 * Narrowing rounds to nearest, ties to even; NaN stays a quiet NaN with its
 * sign; values past the largest finite bf16 round to +-inf.
 * ------------------------------------------------------------------------- */
static float widen(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

uint16_t oracle_bf16_rne(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7fffffffu) > 0x7f800000u) /* NaN */
        return (uint16_t)((u >> 16) | 0x0040u);
    /* keep = upper 16 bits, drop = lower 16 bits. Round up when the dropped
     * part is above one half, or exactly one half and keep is odd. */
    uint32_t keep = u >> 16;
    uint32_t drop = u & 0xffffu;
    if (drop > 0x8000u || (drop == 0x8000u && (keep & 1u)))
        keep += 1u; /* a carry into the exponent is the correct result */
    return (uint16_t)keep;
}

void oracle_bf16_rne_array(const float *src, uint16_t *dst, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        dst[i] = oracle_bf16_rne(src[i]);
}

/* ---------------------------------------------------------------------------
 * Row bookkeeping
 * ------------------------------------------------------------------------- */
static int64_t live_bound(int64_t rows, const int32_t *n_used)
{
    if (!n_used)
        return rows;
    int64_t n = *n_used;
    if (n < 0)
        n = 0;
    if (n > rows)
        n = rows;
    return n;
}

/* slot of row r, or -1 when the row is not live */
static int64_t row_slot(int64_t r, int64_t bound, int64_t rows, const int32_t *perm)
{
    if (r >= bound)
        return -1;
    if (!perm)
        return r;
    int64_t s = perm[r];
    if (s < 0 || s >= rows)
        return -1;
    return s;
}

/* ---------------------------------------------------------------------------
 * fp32 elementwise pieces, in the order the formula is written
 * ------------------------------------------------------------------------- */
static float clamp_gate(float a, float L)
{
    return (a > L) ? L : a; /* upper clamp only; NaN passes through */
}

static float clamp_up(float b, float L)
{
    if (b > L)
        return L;
    if (b < -L)
        return -L;
    return b; /* NaN passes through */
}

static float sigmoid_f32(float z)
{
    return 1.0f / (1.0f + expf(-z));
}

/* ---------------------------------------------------------------------------
 * Threading helper
 * ------------------------------------------------------------------------- */
typedef struct {
    int64_t r0, r1;
    const void *args;
    void (*body)(const void *args, int64_t r0, int64_t r1);
} block_t;

static void *run_block(void *p)
{
    block_t *b = (block_t *)p;
    b->body(b->args, b->r0, b->r1);
    return NULL;
}

#define ORACLE_MAX_THREADS 256

static void parallel_rows(int64_t rows, int threads, const void *args,
                          void (*body)(const void *, int64_t, int64_t))
{
    if (threads < 1)
        threads = 1;
    if (threads > ORACLE_MAX_THREADS)
        threads = ORACLE_MAX_THREADS;
    if ((int64_t)threads > rows)
        threads = rows > 0 ? (int)rows : 1;
    if (threads == 1) {
        body(args, 0, rows);
        return;
    }
    pthread_t tid[ORACLE_MAX_THREADS];
    block_t blk[ORACLE_MAX_THREADS];
    int started[ORACLE_MAX_THREADS];
    int64_t per = rows / threads, extra = rows % threads, r = 0;
    for (int t = 0; t < threads; ++t) {
        int64_t n = per + (t < extra ? 1 : 0);
        blk[t].r0 = r;
        blk[t].r1 = r + n;
        blk[t].args = args;
        blk[t].body = body;
        r += n;
        started[t] = (pthread_create(&tid[t], NULL, run_block, &blk[t]) == 0);
        if (!started[t])
            run_block(&blk[t]); /* fall back to the calling thread */
    }
    for (int t = 0; t < threads; ++t)
        if (started[t])
            pthread_join(tid[t], NULL);
}

/* ---------------------------------------------------------------------------
 * Forward, fp32 math, one bf16 rounding
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *x;
    const float *probs;
    uint16_t *y;
    int64_t rows, inter, bound;
    float L;
    const int32_t *perm;
    int zero_padding;
} fwd_args_t;

static void fwd_rows(const void *vp, int64_t r0, int64_t r1)
{
    const fwd_args_t *A = (const fwd_args_t *)vp;
    const int64_t inter = A->inter;
    for (int64_t r = r0; r < r1; ++r) {
        uint16_t *yr = A->y + r * inter;
        int64_t slot = row_slot(r, A->bound, A->rows, A->perm);
        if (slot < 0) {
            if (A->zero_padding)
                memset(yr, 0, (size_t)inter * sizeof(uint16_t));
            continue;
        }
        const uint16_t *gate = A->x + r * 2 * inter;
        const uint16_t *up = gate + inter;
        const float p = A->probs[slot];
        for (int64_t j = 0; j < inter; ++j) {
            float cg = clamp_gate(widen(gate[j]), A->L);
            float cu = clamp_up(widen(up[j]), A->L);
            float s = cg * sigmoid_f32(cg);
            yr[j] = oracle_bf16_rne((s * cu) * p);
        }
    }
}

int oracle_swiglu_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                      int64_t rows, int64_t inter, float limit,
                      const int32_t *n_used, const int32_t *permutation_map,
                      int zero_padding, int threads)
{
    if (rows < 0 || inter <= 0 || !(limit > 0.0f))
        return 1;
    if (rows == 0)
        return 0;
    if (!x || !probs || !y)
        return 1;
    fwd_args_t A = {x, probs, y, rows, inter, live_bound(rows, n_used),
                    limit, permutation_map, zero_padding};
    parallel_rows(rows, threads, &A, fwd_rows);
    return 0;
}

/* ---------------------------------------------------------------------------
 * Backward, fp32 elementwise math, fp64 row accumulation
 * ------------------------------------------------------------------------- */
typedef struct {
    const uint16_t *x;
    const float *probs;
    const uint16_t *grad_y;
    uint16_t *grad_x;
    float *grad_probs;
    double *grad_probs_f64;
    double *row_scale;
    int64_t rows, inter, bound;
    float L;
    const int32_t *perm;
    int zero_padding;
} bwd_args_t;

static void bwd_rows(const void *vp, int64_t r0, int64_t r1)
{
    const bwd_args_t *A = (const bwd_args_t *)vp;
    const int64_t inter = A->inter;
    const float L = A->L;
    for (int64_t r = r0; r < r1; ++r) {
        uint16_t *dgate = A->grad_x + r * 2 * inter;
        uint16_t *dup = dgate + inter;
        int64_t slot = row_slot(r, A->bound, A->rows, A->perm);
        if (slot < 0) {
            if (A->zero_padding)
                memset(dgate, 0, (size_t)(2 * inter) * sizeof(uint16_t));
            continue;
        }
        const uint16_t *gate = A->x + r * 2 * inter;
        const uint16_t *up = gate + inter;
        const uint16_t *gy = A->grad_y + r * inter;
        const float p = A->probs[slot];
        double acc = 0.0, scale = 0.0;
        for (int64_t j = 0; j < inter; ++j) {
            float a = widen(gate[j]);
            float b = widen(up[j]);
            float g = widen(gy[j]);
            float cg = clamp_gate(a, L);
            float cu = clamp_up(b, L);
            float sig = sigmoid_f32(cg);
            float s = cg * sig;
            float gp = g * p;
            /* inclusive masks on the input values, as torch.clamp's gradient */
            int in_gate = (a <= L);
            int in_up = (b >= -L) && (b <= L);
            float dsilu = sig * (1.0f + cg * (1.0f - sig));
            float dg = in_gate ? (gp * cu) * dsilu : 0.0f;
            float du = in_up ? gp * s : 0.0f;
            dgate[j] = oracle_bf16_rne(dg);
            dup[j] = oracle_bf16_rne(du);
            float term = g * (s * cu);
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

int oracle_swiglu_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                      uint16_t *grad_x, float *grad_probs, double *grad_probs_f64,
                      double *row_scale, int64_t rows, int64_t inter, float limit,
                      const int32_t *n_used, const int32_t *permutation_map,
                      int zero_padding, int threads)
{
    if (rows < 0 || inter <= 0 || !(limit > 0.0f))
        return 1;
    if (rows == 0)
        return 0;
    if (!x || !probs || !grad_y || !grad_x)
        return 1;
    bwd_args_t A = {x, probs, grad_y, grad_x, grad_probs, grad_probs_f64, row_scale,
                    rows, inter, live_bound(rows, n_used), limit, permutation_map,
                    zero_padding};
    parallel_rows(rows, threads, &A, bwd_rows);
    return 0;
}

/* ---------------------------------------------------------------------------
 * fp64 instantiation: the same formula with no rounding anywhere, on real
 * numbers given as doubles. Used by the finite-difference and brute-force
 * checks. Every row is live; gate/up are the two halves of x [rows, 2*inter].
 * ------------------------------------------------------------------------- */
int oracle_swiglu_fwd_f64(const double *x, const double *probs, double *y,
                          int64_t rows, int64_t inter, double limit)
{
    if (rows < 0 || inter <= 0 || !(limit > 0.0))
        return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *gate = x + r * 2 * inter, *up = gate + inter;
        for (int64_t j = 0; j < inter; ++j) {
            double a = gate[j], b = up[j];
            double cg = (a > limit) ? limit : a;
            double cu = (b > limit) ? limit : ((b < -limit) ? -limit : b);
            double sig = 1.0 / (1.0 + exp(-cg));
            y[r * inter + j] = ((cg * sig) * cu) * probs[r];
        }
    }
    return 0;
}

int oracle_swiglu_bwd_f64(const double *x, const double *probs, const double *grad_y,
                          double *grad_x, double *grad_probs, int64_t rows,
                          int64_t inter, double limit)
{
    if (rows < 0 || inter <= 0 || !(limit > 0.0))
        return 1;
    for (int64_t r = 0; r < rows; ++r) {
        const double *gate = x + r * 2 * inter, *up = gate + inter;
        const double *gy = grad_y + r * inter;
        double *dgate = grad_x + r * 2 * inter, *dup = dgate + inter;
        const double p = probs[r];
        double acc = 0.0;
        for (int64_t j = 0; j < inter; ++j) {
            double a = gate[j], b = up[j], g = gy[j];
            double cg = (a > limit) ? limit : a;
            double cu = (b > limit) ? limit : ((b < -limit) ? -limit : b);
            double sig = 1.0 / (1.0 + exp(-cg));
            double s = cg * sig;
            double gp = g * p;
            dgate[j] = (a <= limit) ? (gp * cu) * (sig * (1.0 + cg * (1.0 - sig))) : 0.0;
            dup[j] = (b >= -limit && b <= limit) ? gp * s : 0.0;
            acc += g * (s * cu);
        }
        grad_probs[r] = acc;
    }
    return 0;
}
