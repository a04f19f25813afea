/*
 * swiglu_probs.h - C ABI of the fused clamped-SwiGLU x routing-probability
 * expert activation for AMD Instinct MI355X (gfx950).
 *
 * The operation (NeMo AutoModel "moe/swiglu_triton" page, module docstring and
 * the SwigluClampedTriton class entry): with x = [gate | up], the bf16 result of the
 * routed experts' grouped GEMM ([rows, 2*inter], gate in the first half), and one fp32
 * routing probability per row,
 *
 *     y = silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs
 *
 * computed in fp32 and rounded once to bf16 (round to nearest, ties to even).
 * The backward stores d_gate in the first half of grad_x and d_up in the second (no
 * separate concatenation) and reduces the per-row probability gradient
 * grad_probs = sum_j grad_y * silu(cg) * cu in fp32. Clamp gradients follow
 * torch.clamp: the masks gate <= L and -L <= up <= L are inclusive on the input
 * values.
 *
 * Row bookkeeping (Megatron-Core "core.inference.moe.batch_invariant" page,
 * _swiglu_with_probs_kernel / swiglu_with_probs / _weighted_silu_mul_bounded_kernel):
 *   - n_used: optional DEVICE int32 scalar. Rows r >= clamp(*n_used, 0, rows) are
 *     padding. It is read on the device, never by the host, so a call can be
 *     captured in a HIP graph and replayed after the count changes.
 *   - permutation_map: optional DEVICE int32 [rows]. Row r takes its probability
 *     from probs[map[r]] and writes its probability gradient to grad_probs[map[r]];
 *     an entry outside [0, rows) marks row r as a dummy (padding) row. Without a
 *     map, slot(r) = r. Live rows must map to distinct slots (a permutation);
 *     otherwise which row's gradient a shared slot keeps is unspecified.
 *   - zero_padding: nonzero -> every padding/dummy row of y (forward) or grad_x
 *     (backward) is written with +0.0 (0x0000) without reading its inputs; zero ->
 *     those rows are neither read nor written. grad_probs is never written for
 *     padding or dummy rows.
 *
 * Memory layout and ownership: every pointer is caller-owned DEVICE memory on the
 * calling thread's current HIP device, row-major and contiguous. bf16 tensors are
 * passed as their 16-bit patterns (uint16_t). Base pointers of x, y, grad_y and
 * grad_x must be 16-byte aligned and inter a multiple of 8 (each lane moves 8 bf16
 * = 128 bits per access); probs, grad_probs, n_used and permutation_map must be
 * 4-byte aligned. Inputs and outputs must not overlap. The library allocates no
 * memory and keeps no pointer after a call returns.
 *
 * Execution: work is enqueued on `stream` (0 = the null stream) and the call
 * returns without synchronising. No host read of device data, no allocation:
 * calls are hipGraph-capturable. The launch grid depends only on rows and inter
 * (host sizes, never device data), as swiglu_probs_default_workgroups describes:
 * one wave per row for rows of up to two column chunks, one workgroup per row for
 * rows the four waves of a workgroup share, one workgroup per compute unit for
 * rows of three chunks; never more than 16,777,215 workgroups, the waves then
 * striding over the rows the grid does not cover. The grid never changes the
 * result bits. Calls are re-entrant and thread-safe.
 *
 * Errors: arguments are checked on the host before anything is launched; on any
 * error nothing is written. Device data cannot raise errors (out-of-range
 * n_used is clamped, out-of-range map entries mark dummy rows).
 */
#ifndef SWIGLU_PROBS_H
#define SWIGLU_PROBS_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SWIGLU_PROBS_ABI_VERSION 1

/* The status enum is int-sized. Compiled as C++ it takes int as its fixed underlying
 * type, so any int a C caller passes (say to swiglu_probs_status_string) is a value
 * of the type (an enum without a fixed type would make loading an unknown value
 * undefined in C++). */
#ifdef __cplusplus
#define SWIGLU_ENUM_BASE : int
#else
#define SWIGLU_ENUM_BASE
#endif

typedef enum swiglu_status SWIGLU_ENUM_BASE {
    SWIGLU_OK = 0,
    /* a required pointer is NULL, rows < 0, inter <= 0, rows > 2,143,289,343,
     * inter > 2^28 (268,435,456), limit is NaN or <= 0, num_workgroups < 0 or
     * > 16,777,215, or an output overlaps an input */
    SWIGLU_ERR_INVALID_ARG = 1,
    /* inter % 8 != 0, or a base pointer misses its alignment (16 B for bf16
     * tensors, 4 B for fp32/int32) */
    SWIGLU_ERR_ALIGNMENT = 2,
    /* a HIP runtime call or the kernel launch failed; see swiglu_probs_last_hip_error */
    SWIGLU_ERR_HIP = 3
} swiglu_status_t;

/*
 * Forward (swiglu_triton page: forward kernel, one pass, fp32 math, one rounding;
 * batch_invariant page: swiglu_with_probs for n_used / permutation_map / zero_padding).
 *
 *   x       [rows, 2*inter] bf16 bits, gate = columns [0, inter), up = [inter, 2*inter)
 *   probs   [rows] fp32 (the [rows, 1] routing probabilities)
 *   y       [rows, inter] bf16 bits, output
 *   limit   L > 0; +inf means no clamp (plain SwiGLU x probs)
 *   n_used, permutation_map: optional device pointers (NULL = absent), see above
 *   zero_padding: 0 or 1
 *   rows == 0 returns SWIGLU_OK without launching.
 */
swiglu_status_t swiglu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                                 int64_t rows, int64_t inter, float limit,
                                 const int32_t *n_used, const int32_t *permutation_map,
                                 int zero_padding, hipStream_t stream);

/*
 * Backward (swiglu_triton page: the one-pass backward kernel, gate and up gradients
 * stored in place in grad_x, the per-row probability gradient summed as it goes).
 *
 *   x, probs     as in the forward (the forward's saved inputs; nothing else is saved)
 *   grad_y       [rows, inter] bf16 bits, gradient of y
 *   grad_x       [rows, 2*inter] bf16 bits, output: d_gate in [0, inter), d_up in [inter, 2*inter)
 *   grad_probs   [rows] fp32 output indexed by slot, or NULL to skip the reduction
 *   other arguments as in the forward
 */
swiglu_status_t swiglu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                 uint16_t *grad_x, float *grad_probs,
                                 int64_t rows, int64_t inter, float limit,
                                 const int32_t *n_used, const int32_t *permutation_map,
                                 int zero_padding, hipStream_t stream);

/*
 * The same two calls with an explicit workgroup count (0 = the library's choice).
 * For tests of grid invariance and for launch sweeps; the result bits do not
 * depend on num_workgroups (Megatron-Core batch_invariant page,
 * weighted_silu_mul_bounded: grid size is an occupancy knob only).
 */
swiglu_status_t swiglu_probs_fwd_ex(const uint16_t *x, const float *probs, uint16_t *y,
                                    int64_t rows, int64_t inter, float limit,
                                    const int32_t *n_used, const int32_t *permutation_map,
                                    int zero_padding, hipStream_t stream, int num_workgroups);

swiglu_status_t swiglu_probs_bwd_ex(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                    uint16_t *grad_x, float *grad_probs,
                                    int64_t rows, int64_t inter, float limit,
                                    const int32_t *n_used, const int32_t *permutation_map,
                                    int zero_padding, hipStream_t stream, int num_workgroups);

/*
 * The _ex calls with the kernel's own start and end recorded into `start` and `stop`
 * (HIP events the caller created; either may be NULL) as part of the launch, with no
 * separate event command on the stream (hipExtLaunchKernel). For benchmarks:
 * hipEventElapsedTime(start, stop) is then the kernel's duration alone. The events
 * must belong to the current device; otherwise as the _ex calls.
 */
swiglu_status_t swiglu_probs_fwd_timed(const uint16_t *x, const float *probs, uint16_t *y,
                                       int64_t rows, int64_t inter, float limit,
                                       const int32_t *n_used, const int32_t *permutation_map,
                                       int zero_padding, hipStream_t stream, int num_workgroups,
                                       hipEvent_t start, hipEvent_t stop);

swiglu_status_t swiglu_probs_bwd_timed(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                       uint16_t *grad_x, float *grad_probs,
                                       int64_t rows, int64_t inter, float limit,
                                       const int32_t *n_used, const int32_t *permutation_map,
                                       int zero_padding, hipStream_t stream, int num_workgroups,
                                       hipEvent_t start, hipEvent_t stop);

/* Workgroup count the library would launch for this call shape on the current
 * device (direction 0 = forward, 1 = backward), or -1 on error. Host only.
 * A row is cut into column chunks of U 16-byte vectors per lane (64 lanes): the
 * forward takes the U in 1..4 that leaves the fewest idle lanes (U = 2 for rows of
 * exactly 4 vectors per lane), the backward cuts rows of 4 or more vectors per lane
 * into 4 or more chunks. Rows of one or two chunks get one wave per row,
 * ceil(rows / 4) workgroups (a forward row of at most 4 vectors per lane is then
 * loaded whole); rows of three chunks one workgroup per CU, balanced; rows of four
 * or more one workgroup per row, its four waves sharing the row. Never more than
 * 16,777,215 workgroups (a dispatch holds its work-item count in 32 bits); the
 * waves then take several rows each. */
int swiglu_probs_default_workgroups(int direction, int64_t rows, int64_t inter);

/* Static text for a status code. Never NULL. */
const char *swiglu_probs_status_string(swiglu_status_t status);

/* hipError_t of the last SWIGLU_ERR_HIP returned on the calling thread (0 if none). */
int swiglu_probs_last_hip_error(void);

/* SWIGLU_PROBS_ABI_VERSION of the loaded library. */
int swiglu_probs_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SWIGLU_PROBS_H */
