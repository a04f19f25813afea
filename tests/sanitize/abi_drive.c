/*
 * Drives the host-side argument checks of the three C-ABI libraries (activation, MoE
 * elementwise operations, streaming probe), for a host-only build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (test infrastructure). Every call
 * either fails validation or has nothing to do, so it returns before the first HIP
 * runtime call: no device is needed and no kernel is launched. Pointers are fake,
 * suitably aligned addresses that these paths compare but never dereference. Sizes
 * run up to the extremes (2^40 rows, negative counts, 2^31 - 1 workgroups), where an
 * unchecked product of sizes would overflow. Exit status 0 when every call returns
 * the documented status; any sanitizer report ends the run with a non-zero status.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "hbm_probe.h"
#include "moe_elementwise.h"
#include "swiglu_probs.h"

#define A16 ((uintptr_t)1 << 20)
#define P(off) ((void *)(A16 + (uintptr_t)(off)))
#define MB16(k) ((uintptr_t)(k) << 24)

static int failures = 0;
#define EXPECT(call, want)                                                                   \
    do {                                                                                     \
        const int got_ = (int)(call);                                                        \
        if (got_ != (want)) {                                                                \
            fprintf(stderr, "%s:%d: %s returned %d, expected %d\n", __FILE__, __LINE__, #call, \
                    got_, (want));                                                           \
            ++failures;                                                                      \
        }                                                                                    \
    } while (0)

static int fwd(uintptr_t x, uintptr_t p, uintptr_t y, int64_t rows, int64_t inter, float limit, uintptr_t nu,
               uintptr_t perm, int nwg)
{
    return swiglu_probs_fwd_ex((const uint16_t *)P(x), (const float *)P(p), (uint16_t *)P(y), rows, inter, limit,
                               nu ? (const int32_t *)P(nu) : NULL, perm ? (const int32_t *)P(perm) : NULL, 0, NULL,
                               nwg);
}

static int bwd(uintptr_t x, uintptr_t p, uintptr_t gy, uintptr_t gx, uintptr_t gp, int64_t rows, int64_t inter,
               float limit, uintptr_t perm, int nwg)
{
    return swiglu_probs_bwd_ex((const uint16_t *)P(x), (const float *)P(p), (const uint16_t *)P(gy),
                               (uint16_t *)P(gx), gp == UINTPTR_MAX ? NULL : (float *)P(gp), rows, inter, limit, NULL,
                               perm ? (const int32_t *)P(perm) : NULL, 0, NULL, nwg);
}

static void activation(void)
{
    const uintptr_t x = 0, p = MB16(1), y = MB16(2), gy = MB16(2), gx = MB16(3), gp = MB16(4);
    EXPECT(fwd(x, p, y, 0, 8, 7.0f, 0, 0, 0), SWIGLU_OK);
    EXPECT(swiglu_probs_fwd(NULL, NULL, NULL, 0, 8, 7.0f, NULL, NULL, 0, NULL), SWIGLU_OK);
    EXPECT(fwd(x, p, y, -1, 8, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 0, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, -8, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 12, 7.0f, 0, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(fwd(x, p, y, 4, 8, NAN, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 8, 0.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 8, -INFINITY, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 8, 7.0f, 0, 0, -1), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 8, 7.0f, 0, 0, 1 << 24), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, 8, 7.0f, 0, 0, INT32_MAX), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x + 8, p, y, 4, 8, 7.0f, 0, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(fwd(x, p + 2, y, 4, 8, 7.0f, 0, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(fwd(x, p, y, 4, 8, 7.0f, MB16(5) + 1, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(fwd(x, p, y, 4, 8, 7.0f, 0, MB16(6) + 3, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(fwd(x, p, x + 16, 4, 8, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);  /* y over x */
    EXPECT(fwd(x, p, p, 4, 8, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);       /* y over probs */
    EXPECT(fwd(x, p, y, (int64_t)1 << 40, 8, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, 4, (int64_t)1 << 40, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(fwd(x, p, y, INT64_MAX, INT64_MAX - 7, 7.0f, 0, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(bwd(x, p, gy, gx, gp, 0, 8, 7.0f, 0, 0), SWIGLU_OK);
    EXPECT(bwd(x, p, gy, gx, gp, -3, 8, 7.0f, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(bwd(x, p, gy, gx, gp, 4, 20, 7.0f, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(bwd(x, p, gy, gx, gp, 4, 8, 7.0f, 0, 1 << 24), SWIGLU_ERR_INVALID_ARG);
    EXPECT(bwd(x, p, gy, gx, gp + 1, 4, 8, 7.0f, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(bwd(x, p, gy, gx + 4, gp, 4, 8, 7.0f, 0, 0), SWIGLU_ERR_ALIGNMENT);
    EXPECT(bwd(x, p, gy, x, gp, 4, 8, 7.0f, 0, 0), SWIGLU_ERR_INVALID_ARG);        /* grad_x over x */
    EXPECT(bwd(x, p, gy, gy, gp, 4, 8, 7.0f, 0, 0), SWIGLU_ERR_INVALID_ARG);       /* grad_x over grad_y */
    EXPECT(bwd(x, p, gy, gx, p, 4, 8, 7.0f, 0, 0), SWIGLU_ERR_INVALID_ARG);        /* grad_probs over probs */
    EXPECT(bwd(x, p, gy, gx, gx + 16, 4, 8, 7.0f, 0, 0), SWIGLU_ERR_INVALID_ARG);  /* grad_probs in grad_x */
    EXPECT(bwd(x, p, gy, gx, gp, 4, 8, 7.0f, gx, 0), SWIGLU_ERR_INVALID_ARG);      /* map under an output */
    EXPECT(bwd(x, p, gy, gx, UINTPTR_MAX, (int64_t)1 << 40, 8, 7.0f, 0, 0), SWIGLU_ERR_INVALID_ARG);
    EXPECT(swiglu_probs_abi_version(), 1);
    for (int st = 0; st < 4; ++st)
        if (!swiglu_probs_status_string((swiglu_status_t)st))
            ++failures;
    if (!swiglu_probs_status_string((swiglu_status_t)99))
        ++failures;
    EXPECT(swiglu_probs_last_hip_error(), 0);
    EXPECT(swiglu_probs_default_workgroups(2, 4, 8), -1);
    EXPECT(swiglu_probs_default_workgroups(0, -1, 8), -1);
    EXPECT(swiglu_probs_default_workgroups(1, 4, 12), -1);
}

static void moe(void)
{
    const uintptr_t a = 0, b = MB16(1), c = MB16(2), d = MB16(3), e = MB16(4), f = MB16(5);
#define Q(o) P(o)
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), 0, MOE_BF16, NULL, 0), MOE_OK);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), -1, MOE_BF16, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), 8, (moe_dtype_t)7, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(Q(a + 2), Q(b), Q(c), Q(d), 8, MOE_BF16, NULL, 0), MOE_ERR_ALIGNMENT);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(a + 16), 64, MOE_BF16, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(NULL, Q(b), Q(c), Q(d), 8, MOE_BF16, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), 8, MOE_BF16, NULL, -1), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), 8, MOE_BF16, NULL, 1 << 24), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), INT64_MAX, MOE_FP32, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_residual_add(Q(a), Q(b), Q(c), Q(d), ((int64_t)1 << 48) + 8, MOE_BF16, NULL, 0),
           MOE_ERR_INVALID_ARG);

    EXPECT(moe_router_weight_fwd(Q(a), MOE_BF16, Q(b), Q(c), MOE_BF16, 0, 8, NULL, 0), MOE_OK);
    EXPECT(moe_router_weight_fwd(Q(a), MOE_BF16, Q(b), Q(c), MOE_FP16, 4, 8, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_fwd(Q(a), MOE_BF16, Q(b), Q(c), MOE_FP32, 4, 12, NULL, 0), MOE_ERR_ALIGNMENT);
    EXPECT(moe_router_weight_fwd(Q(a), MOE_BF16, Q(b + 2), Q(c), MOE_FP32, 4, 8, NULL, 0), MOE_ERR_ALIGNMENT);
    EXPECT(moe_router_weight_fwd(Q(a), MOE_BF16, Q(b), Q(a), MOE_BF16, 4, 8, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_fwd(Q(a), MOE_BF16, Q(b), Q(c), MOE_BF16, 4, 8, NULL, 1 << 24), MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_fwd(Q(a), MOE_FP32, Q(b), Q(c), MOE_FP32, (int64_t)1 << 40, (int64_t)1 << 40, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_bwd(Q(a), MOE_BF16, NULL, MOE_BF16, Q(b), Q(c), Q(d), 4, 8, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_bwd(Q(a), MOE_BF16, Q(f), MOE_BF16, Q(b), Q(c), Q(d), 4, 8, NULL, 1 << 24),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_bwd(Q(a), MOE_BF16, Q(f), MOE_BF16, Q(b), Q(c), Q(c + 16), 4, 8, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_router_weight_bwd(Q(a), MOE_BF16, Q(f), MOE_BF16, Q(b), NULL, NULL, 0, 8, NULL, 0), MOE_OK);

    const uint16_t *x = Q(a);
    const float *pr = Q(b);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(c), 4, 8, 1, 0.0f, NULL, NULL, 0, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(c), 4, 8, 1, INFINITY, NULL, NULL, 0, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(c), 4, 8, 1, NAN, NULL, NULL, 0, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(c), 0, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0), MOE_OK);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(a), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(c), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 1 << 24), MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_fwd(x, pr, Q(c), (int64_t)1 << 40, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(d), Q(e), 0, 8, 1, 2.0f, NULL, NULL, 0, NULL, 0), MOE_OK);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(d), Q(e), 4, 8, 1, -2.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(d), Q(e), 4, 12, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_ALIGNMENT);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c + 8), Q(d), Q(e), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_ALIGNMENT);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(d), Q(e + 2), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_ALIGNMENT);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, NULL, Q(d), Q(e), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(c), Q(e), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(d), Q(d + 16), 4, 8, 0, 0.0f, NULL, NULL, 0, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_squared_relu_probs_bwd(x, pr, Q(c), Q(d), Q(e), 4, 8, 0, 0.0f, Q(d), NULL, 0, NULL, 0),
           MOE_ERR_INVALID_ARG);

    EXPECT(moe_unpermute_expert_order(x, 10, Q(b), NULL, Q(c), MOE_FP32, 0, 8, 4, NULL, 0), MOE_OK);
    EXPECT(moe_unpermute_expert_order(x, 10, Q(b), NULL, Q(c), MOE_FP16, 4, 8, 4, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_unpermute_expert_order(x, 10, Q(b), NULL, Q(c), MOE_FP32, 4, 8, 0, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_unpermute_expert_order(x, 10, Q(b), NULL, Q(c), MOE_FP32, 4, 8, 2000, NULL, 0), MOE_ERR_INVALID_ARG);
    EXPECT(moe_unpermute_expert_order(x, 10, Q(b + 1), NULL, Q(c), MOE_FP32, 4, 8, 4, NULL, 0), MOE_ERR_ALIGNMENT);
    EXPECT(moe_unpermute_expert_order(x, 10, Q(b), NULL, Q(c), MOE_FP32, 4, 8, 4, NULL, 1 << 24),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_unpermute_expert_order(x, INT64_MAX, Q(b), NULL, Q(c), MOE_FP32, 4, 8, 4, NULL, 0),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_elementwise_abi_version(), 1);
    for (int st = 0; st < 4; ++st)
        if (!moe_elementwise_status_string((moe_status_t)st))
            ++failures;
    EXPECT(moe_elementwise_last_hip_error(), 0);
#undef Q
}

static void probe(void)
{
    const void *s[1] = {P(0)};
    void *d[1] = {P(MB16(1))}, *d2[1] = {P(16)};
    EXPECT(hbm_probe_stream(s, 1, d, 1, 0, 0, NULL), 0);
    EXPECT(hbm_probe_stream(s, 0, d, 1, 4, 0, NULL), 1);
    EXPECT(hbm_probe_stream(s, 1, d, 3, 4, 0, NULL), 1);
    EXPECT(hbm_probe_stream(s, 1, d2, 1, 4, 0, NULL), 1);
    EXPECT(hbm_probe_stream(s, 1, d, 1, 4, 1 << 24, NULL), 1);
    EXPECT(hbm_probe_stream(s, 1, d, 1, -4, 0, NULL), 1);
    EXPECT(hbm_probe_stream(s, 1, d, 1, ((int64_t)1 << 44) + 1, 0, NULL), 1);
    EXPECT(hbm_probe_stream(s, 1, d, 1, INT64_MAX, 0, NULL), 1);
}

int main(void)
{
    activation();
    moe();
    probe();
    if (failures) {
        fprintf(stderr, "%d unexpected statuses\n", failures);
        return 1;
    }
    printf("ABI sanitizer drive: ok\n");
    return 0;
}
