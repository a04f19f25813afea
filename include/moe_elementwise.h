/*
 * moe_elementwise.h - C ABI of the MoE elementwise operations next to the routed-
 * expert activation, for AMD Instinct MI355X (gfx950).
 *
 *   moe_residual_add            fused MoE output residual add (Megatron-Core
 *                               "core.fusions.fused_moe_residual_add" page)
 *   moe_router_weight_fwd/_bwd  router-weight multiply applied after the down
 *                               projection (NeMo AutoModel "moe/optimized_ops" page,
 *                               _RouterWeightMulFunction)
 *   moe_squared_relu_probs_fwd  squared ReLU x probs with and without the tanh soft
 *                               clamp (Megatron-Core "core.inference.moe.batch_invariant"
 *                               page, squared_relu_with_probs)
 *   moe_unpermute_expert_order  token-local unpermute summing local experts in fixed
 *                               expert order (same page, unpermute_tokens_in_expert_order)
 *
 * Conventions shared by every call:
 *   - Pointers are caller-owned DEVICE memory on the calling thread's current HIP
 *     device, contiguous, row-major. 16-bit element types are passed as their bit
 *     patterns. Unless stated otherwise every tensor pointer must be 16-byte aligned.
 *   - Work is enqueued on `stream` (0 = the null stream); no host synchronisation, no
 *     allocation, no host read of device data: calls are hipGraph-capturable.
 *   - Arguments are checked on the host before anything is launched; on error nothing
 *     is written.
 *   - num_workgroups: 0 = the library's choice: one wave per row or block when a row
 *     is at most two column chunks (and always for the soft-clamped squared ReLU);
 *     one workgroup per row, its four waves sharing the row, for router-weight rows
 *     of four or more chunks; one wave per (token, column chunk) for the unpermute
 *     with at most 8 local experts; else persistent workgroups (one per CU) with the
 *     rows balanced over the waves. Never more than 16,777,215 workgroups (a dispatch
 *     holds its work-item count in 32 bits); the waves then take several rows each.
 *     An explicit count must lie in 1 .. 16,777,215; any count gives the same
 *     result bits.
 *   - The library keeps no pointer after a call returns; calls are thread-safe.
 */
#ifndef MOE_ELEMENTWISE_H
#define MOE_ELEMENTWISE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ELEMENTWISE_ABI_VERSION 1

/* The enums are int-sized. Compiled as C++ they take int as their fixed underlying
 * type, so every int a C caller passes is a value of the type; the library rejects
 * the ones it does not know (an enum without a fixed type would make loading such a
 * value undefined in C++). */
#ifdef __cplusplus
#define MOE_ENUM_BASE : int
#else
#define MOE_ENUM_BASE
#endif

typedef enum moe_dtype MOE_ENUM_BASE { MOE_BF16 = 0, MOE_FP16 = 1, MOE_FP32 = 2 } moe_dtype_t;

typedef enum moe_status MOE_ENUM_BASE {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* NULL required pointer, bad size (negative; rows or
                                 tokens above 2,143,289,343; hidden above 2^26; more
                                 than 2^48 residual-add elements), dtype, scale or
                                 workgroup count, overlap */
    MOE_ERR_ALIGNMENT = 2,    /* misaligned pointer, or a row width not a multiple of 8 */
    MOE_ERR_HIP = 3           /* launch failed; see moe_elementwise_last_hip_error */
} moe_status_t;

/*
 * Fused MoE residual add (Megatron-Core "core.fusions.fused_moe_residual_add" page,
 * fused_moe_residual_add and its kernel entry). Per element, in fp32:
 *     s      = dtype(expert_output + shared_expert_output)
 *     output = dtype(residual + s)
 * where dtype() is one round-to-nearest-even to the tensors' dtype. These are the two
 * roundings, in the same order, that two separate elementwise adds in that dtype make,
 * so each output element equals theirs bit for bit. Its gradient reaches each of the
 * three inputs unchanged; the backward launches nothing.
 *   num_elements: elements of each tensor, 0 <= num_elements <= 2^48.
 *   dtype: MOE_BF16, MOE_FP16 or MOE_FP32, the same for all four tensors.
 *   output may be the same pointer as one of the inputs (in place); any other
 *   overlap is an error.
 */
moe_status_t moe_residual_add(const void *expert_output, const void *shared_expert_output,
                              const void *residual, void *output, int64_t num_elements,
                              moe_dtype_t dtype, hipStream_t stream, int num_workgroups);

/*
 * out = (x.float() * probs.float()).to(out_dtype), bitwise.
 *   x: [tokens, hidden] of x_dtype; probs: fp32 [tokens] (= [tokens, 1], 4-byte aligned);
 *   out: [tokens, hidden] of out_dtype, which is x_dtype or MOE_FP32.
 *   hidden % 8 == 0.
 */
moe_status_t moe_router_weight_fwd(const void *x, moe_dtype_t x_dtype, const float *probs,
                                   void *out, moe_dtype_t out_dtype, int64_t tokens,
                                   int64_t hidden, hipStream_t stream, int num_workgroups);

/*
 * grad_x = (grad_out.float() * probs).to(x_dtype)            (bitwise)
 * grad_probs[t] = sum_h grad_out[t, h] * x[t, h], fp32, a fixed order per row
 *   grad_out: [tokens, hidden] of out_dtype; x: [tokens, hidden] of x_dtype, may be
 *   NULL when grad_probs is NULL (x is read only for the probability gradient);
 *   grad_x: [tokens, hidden] of x_dtype or NULL (skip); grad_probs: fp32 [tokens]
 *   (4-byte aligned) or NULL (skip).
 */
moe_status_t moe_router_weight_bwd(const void *grad_out, moe_dtype_t out_dtype, const void *x,
                                   moe_dtype_t x_dtype, const float *probs, void *grad_x,
                                   float *grad_probs, int64_t tokens, int64_t hidden,
                                   hipStream_t stream, int num_workgroups);

/*
 * Squared ReLU x routing probability, forward, bf16 in and out.
 *   clamp != 0: c = clamp_scale * tanh(x / clamp_scale); y = bf16(relu(c)^2 * p), all
 *               in fp32 with one final rounding; clamp_scale must be finite and > 0.
 *               relu(c) is evaluated to 6.5e-5 relative (a rational form of tanh, under
 *               2^-11), so y is within 1 bf16 ulp of the exactly rounded value.
 *   clamp == 0: y = bf16(bf16(relu(x)^2) * p): the square is rounded to bf16 first.
 *   x, y: [rows, hidden] bf16, hidden % 8 == 0; probs: fp32 [rows] indexed by slot.
 *   n_used, permutation_map, zero_padding: exactly as for swiglu_probs_fwd (device
 *   row bound, gather of probs[map[r]], dummy rows, +0 padding rows).
 */
moe_status_t moe_squared_relu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                                        int64_t rows, int64_t hidden, int clamp,
                                        float clamp_scale, const int32_t *n_used,
                                        const int32_t *permutation_map, int zero_padding,
                                        hipStream_t stream, int num_workgroups);

/*
 * Squared ReLU x routing probability, backward: the chain rule through the forward
 * above (Megatron-Core "core.inference.moe.batch_invariant" page gives the forward
 * only). With g = grad_y, y_pre the fp32 value the forward multiplies by p (relu(c)^2
 * with the clamp, the bf16-rounded square without it) and a = relu(c) (c = x without
 * the clamp):
 *   grad_x[r, j]     = bf16(((g * p) * (2 a)) * d) where x > 0, else +0 (also for NaN),
 *                      d = sech^2(x / clamp_scale) with the clamp, 1 without it; the
 *                      bf16 rounding of the square passes the gradient through.
 *   grad_probs[slot] = sum over j of g * y_pre, in fp32 in a fixed order that does not
 *                      depend on the grid.
 *   x, grad_y, grad_x: [rows, hidden] bf16, 16-byte aligned, hidden % 8 == 0.
 *   probs: fp32 [rows] indexed by slot; grad_probs: fp32 [rows] or NULL (skip).
 *   n_used, permutation_map, zero_padding: as for the forward. Rows that are not live
 *   read nothing; their grad_x is +0 with zero_padding and untouched without it; their
 *   grad_probs slots are never written.
 *   The clamp path is within 1 bf16 ulp of the exactly rounded gradient (its tanh and
 *   sech^2 are evaluated to about 1e-6 relative); the unclamped grad_x is the fp32
 *   expression above, rounded once.
 *   Errors: INVALID_ARG (null x / probs / grad_y / grad_x, rows < 0, hidden <= 0, a bad
 *   clamp_scale, an output overlapping an input or the other output), ALIGNMENT.
 */
moe_status_t moe_squared_relu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                        uint16_t *grad_x, float *grad_probs, int64_t rows,
                                        int64_t hidden, int clamp, float clamp_scale,
                                        const int32_t *n_used, const int32_t *permutation_map,
                                        int zero_padding, hipStream_t stream, int num_workgroups);

/*
 * out[t, :] = sum over e = 0, 1, ..., num_local_experts-1 with 0 <= inverse_map[t, e] <
 *             expert_rows of expert_output[inverse_map[t, e], :], accumulated in fp32 in
 *             that order from +0; stored as fp32 or rounded once to bf16 (out_dtype).
 *   expert_output: bf16 [expert_rows, hidden]; inverse_map: int32 [tokens,
 *   num_local_experts] (4-byte aligned; other entries mean "no contribution");
 *   valid_tokens: device int32 scalar or NULL (= tokens); tokens at or past it are
 *   neither read nor written; out: [tokens, hidden] of MOE_FP32 or MOE_BF16.
 *   hidden % 8 == 0; 1 <= num_local_experts <= 1024.
 */
moe_status_t moe_unpermute_expert_order(const uint16_t *expert_output, int64_t expert_rows,
                                        const int32_t *inverse_map, const int32_t *valid_tokens,
                                        void *out, moe_dtype_t out_dtype, int64_t tokens,
                                        int64_t hidden, int num_local_experts, hipStream_t stream,
                                        int num_workgroups);

/* Static text for a status code. Never NULL. */
const char *moe_elementwise_status_string(moe_status_t status);

/* hipError_t of the last MOE_ERR_HIP returned on the calling thread (0 if none). */
int moe_elementwise_last_hip_error(void);

/* MOE_ELEMENTWISE_ABI_VERSION of the loaded library. */
int moe_elementwise_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ELEMENTWISE_H */
