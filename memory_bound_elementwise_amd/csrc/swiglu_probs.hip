// Fused clamped-SwiGLU x routing-probability activation, forward and backward,
// for AMD Instinct MI355X (gfx950, CDNA4). C ABI declared in swiglu_probs.h.
//
// What is computed (NeMo AutoModel "moe/swiglu_triton" page, module docstring):
//   y = silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs, fp32 math, one bf16
//   rounding; the backward writes d_gate / d_up into the two halves of grad_x and
//   reduces the per-row probability gradient in fp32. Clamp gradients follow
//   torch.clamp (inclusive masks). Row bookkeeping (n_used, permutation_map,
//   zero_padding, fixed grid striding over rows) follows the Megatron-Core
//   "core.inference.moe.batch_invariant" page (_swiglu_with_probs_kernel,
//   _weighted_silu_mul_bounded_kernel).
//
// Design (HBM-bound; no MFMA):
//   * Lane l of a wave handles the 16-byte vectors l, l+64, l+128, ... of the gate
//     half, the up half and (backward) grad_y: every access is 128 bits wide and one
//     wave instruction covers 1 KiB of contiguous memory. A row is processed in
//     chunks of U vectors per lane: the forward takes the U that leaves the fewest
//     idle lanes (two chunks of 2 for rows of exactly 4 vectors per lane), the backward
//     cuts rows of 4 or more vectors per lane into 4 or more chunks. Rows of 4 or more chunks are shared by a workgroup's four waves, a
//     quarter of the chunks each (walk_row_split); shorter rows go one per wave
//     (walk_rows).
//   * Every load and store is a buffer instruction on a per-row buffer resource
//     whose size is the row's byte length, or 0 for a row that is not live. The
//     hardware range check then does all masking: lanes past the row end and rows
//     that are not live read zeros without touching memory, and their stores are
//     dropped (or, for zero-padded rows, write the +0 that zero inputs produce).
//     No branch guards a memory instruction, so the compiler's wait counts stay
//     exact across the software pipeline below.
//   * Software pipeline: each wave holds two register buffers and issues the loads
//     of its next chunk (usually its next row) before computing the current one,
//     so its own memory traffic overlaps its arithmetic.
//   * Waves (or workgroups, for shared rows) stride over rows with a fixed grid
//     (row r, r + W, r + 2W, ...), so the launch never depends on device data and
//     is graph-safe. By default the grid has one wave (or workgroup) per row, up to
//     the dispatch limit of 16,777,215 workgroups; rows of exactly three chunks get
//     one persistent workgroup per CU instead, sized so every wave gets the same
//     number of rows (walk_workgroups in cdna4_stream.h).
//   * Per-row metadata (permutation slot and probability) for a wave's next 64
//     rows is gathered with one vector load, one row per lane, and broadcast with
//     v_readlane when the row is processed: no per-row dependent scalar loads.
//   * The probability gradient: each lane sums its own columns in a fixed order,
//     then a butterfly over the wave (DPP quad/row permutes, then two lane
//     exchanges) combines the 64 partials; on shared rows the four waves' totals
//     are then added in wave order through LDS. The order depends only on the row
//     width, never on the grid, so the bits are grid-invariant.
//   * fp32 -> bf16 uses v_cvt_pk_bf16_f32 (round to nearest even, two values per
//     instruction); the clamps use v_minimum3/v_maximum3 (NaN-propagating, as
//     torch.clamp); the inclusive masks are "the clamp left the value unchanged".
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cmath>
#include <mutex>

#include "cdna4_stream.h"
#include "swiglu_probs.h"

namespace {

using namespace cdna4;

#ifndef SWIGLU_MAX_U
#define SWIGLU_MAX_U 4
#endif
constexpr int kMaxU = SWIGLU_MAX_U;  // 16-byte vectors per lane per stream per chunk
#ifndef SWIGLU_WALK
#define SWIGLU_WALK walk_row_split
#endif
constexpr float kNegLog2e = -1.4426950408889634f;

// ---------------------------------------------------------------------------
// Element math
// ---------------------------------------------------------------------------
// clamp(gate, max=L) and clamp(up, -L, L); NaN propagates like torch.clamp.
__device__ __forceinline__ float clamp_gate(float a, float L)
{
    return __builtin_elementwise_minimum(a, L);
}
__device__ __forceinline__ float clamp_up(float b, float L)
{
    return __builtin_elementwise_maximum(__builtin_elementwise_minimum(b, L), -L);
}

// logistic sigmoid 1 / (1 + e^-z) from v_exp_f32 (2^x) and v_rcp_f32.
// v_rcp_f32 flushes subnormal results to zero, and 1 / (1 + e^-z) is subnormal once
// 1 + e^-z exceeds 2^126 (z < -87.3), where silu(z) = z * sigmoid(z) is still a normal
// number. The reciprocal is therefore taken of 2^-64 * (1 + e^-z) (one fma, exact: a
// power-of-two scale of a value >= 1), which keeps it normal, and the result is scaled
// back by 2^-64 in a multiply, which does produce subnormals. For e^-z = inf (z < -88.7)
// the sigmoid is 0, as 1 / (1 + inf) is in fp32.
__device__ __forceinline__ float sigmoid(float z)
{
    constexpr float kTwoM64 = 0x1p-64f;
    float e = __builtin_amdgcn_exp2f(z * kNegLog2e);
    return __builtin_amdgcn_rcpf(__builtin_fmaf(e, kTwoM64, kTwoM64)) * kTwoM64;
}

__device__ __forceinline__ float fwd_elem(float a, float b, float p, float L)
{
    float cg = clamp_gate(a, L);
    float cu = clamp_up(b, L);
    float s = cg * sigmoid(cg);
    return (s * cu) * p;
}

// Autograd chain of y = (silu(cg) * cu) * p with inclusive clamp masks.
__device__ __forceinline__ void bwd_elem(float a, float b, float g, float p, float L,
                                         float &dg, float &du, float &acc)
{
    float cg = clamp_gate(a, L);
    float cu = clamp_up(b, L);
    float sig = sigmoid(cg);
    float s = cg * sig;
    float gp = g * p;
    float dsilu = sig * (1.0f + cg * (1.0f - sig));
    // a <= L  <=>  min(a, L) == a ;  -L <= b <= L  <=>  clamp(b) == b  (false for NaN)
    dg = (cg == a) ? (gp * cu) * dsilu : 0.0f;
    du = (cu == b) ? gp * s : 0.0f;
    acc += g * (s * cu);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
template <int U>
struct FwdOp {
    static constexpr bool kRowSum = false;
    struct Buf {
        u32x4 g[U], u[U];
    };
    const uint16_t *__restrict__ x;
    uint16_t *__restrict__ y;
    int inter;
    float L;
    int zero_padding;
    uint32_t voff;  // this lane's byte offset within a chunk

    __device__ __forceinline__ void load(Buf &b, int64_t r, int c, bool live) const
    {
        const uint16_t *gate = x + r * 2 * inter;
        const uint32_t n = live ? (uint32_t)inter * 2u : 0u;
        const uint32_t off = (uint32_t)c * U * kWave * kVecBytes;
        const rsrc_t rg = chunk_rsrc(gate, n, off), ru = chunk_rsrc(gate + inter, n, off);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b.g[u] = load_vec(rg, voff + u * kWave * kVecBytes);
            b.u[u] = load_vec(ru, voff + u * kWave * kVecBytes);
        }
    }

    __device__ __forceinline__ void process(const Buf &b, int64_t r, int c, int slot, float p) const
    {
        const uint32_t n = (slot >= 0 || zero_padding) ? (uint32_t)inter * 2u : 0u;
        const rsrc_t ry = chunk_rsrc(y + r * inter, n, (uint32_t)c * U * kWave * kVecBytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float y0 = fwd_elem(bf16_lo(b.g[u][q]), bf16_lo(b.u[u][q]), p, L);
                float y1 = fwd_elem(bf16_hi(b.g[u][q]), bf16_hi(b.u[u][q]), p, L);
                o[q] = pack_bf16x2(y0, y1);
            }
            store_vec(ry, o, voff + u * kWave * kVecBytes);
        }
    }
};

template <int U>
__global__ __launch_bounds__(kBlock) void swiglu_probs_fwd_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ probs, uint16_t *__restrict__ y,
    int rows, int inter, float L, const int *__restrict__ n_used, const int *__restrict__ perm,
    int zero_padding)
{
    const RowSchedule sched = make_schedule(rows, n_used, zero_padding);
    const int vpr = inter / 8;
    const int nch = (vpr + U * kWave - 1) / (U * kWave);
    FwdOp<U> op{x, y, inter, L, zero_padding, (uint32_t)(threadIdx.x & (kWave - 1)) * kVecBytes};
    SWIGLU_WALK(op, sched, perm, probs, nch);
}

// ---------------------------------------------------------------------------
// Backward
// ---------------------------------------------------------------------------
template <int U>
struct BwdOp {
    static constexpr bool kRowSum = true;
    struct Buf {
        u32x4 g[U], u[U], d[U];
    };
    const uint16_t *__restrict__ x;
    const uint16_t *__restrict__ gy;
    uint16_t *__restrict__ gx;
    float *__restrict__ gprobs;
    int inter;
    float L;
    int zero_padding;
    uint32_t voff;
    float acc;  // this lane's partial of the current row's probability gradient

    __device__ __forceinline__ void load(Buf &b, int64_t r, int c, bool live) const
    {
        const uint16_t *gate = x + r * 2 * inter;
        const uint32_t n = live ? (uint32_t)inter * 2u : 0u;
        const uint32_t off = (uint32_t)c * U * kWave * kVecBytes;
        const rsrc_t rg = chunk_rsrc(gate, n, off), ru = chunk_rsrc(gate + inter, n, off);
        const rsrc_t rd = chunk_rsrc(gy + r * inter, n, off);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b.g[u] = load_vec(rg, voff + u * kWave * kVecBytes);
            b.u[u] = load_vec(ru, voff + u * kWave * kVecBytes);
            b.d[u] = load_vec(rd, voff + u * kWave * kVecBytes);
        }
    }

    __device__ __forceinline__ void process(const Buf &b, int64_t r, int c, int slot, float p)
    {
        const uint32_t n = (slot >= 0 || zero_padding) ? (uint32_t)inter * 2u : 0u;
        uint16_t *dgate = gx + r * 2 * inter;
        const uint32_t off = (uint32_t)c * U * kWave * kVecBytes;
        const rsrc_t rdg = chunk_rsrc(dgate, n, off), rdu = chunk_rsrc(dgate + inter, n, off);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 og, ou;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float dg0, du0, dg1, du1;
                bwd_elem(bf16_lo(b.g[u][q]), bf16_lo(b.u[u][q]), bf16_lo(b.d[u][q]), p, L, dg0, du0, acc);
                bwd_elem(bf16_hi(b.g[u][q]), bf16_hi(b.u[u][q]), bf16_hi(b.d[u][q]), p, L, dg1, du1, acc);
                og[q] = pack_bf16x2(dg0, dg1);
                ou[q] = pack_bf16x2(du0, du1);
            }
            store_vec(rdg, og, voff + u * kWave * kVecBytes);
            store_vec(rdu, ou, voff + u * kWave * kVecBytes);
        }
    }

    __device__ __forceinline__ bool row_sum_wanted() const { return gprobs != nullptr; }
    __device__ __forceinline__ void store_row_sum(int slot, float total) const
    {
        if (lane_id() == 0)
            gprobs[slot] = total;
    }
};

template <int U>
__global__ __launch_bounds__(kBlock) void swiglu_probs_bwd_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ probs, const uint16_t *__restrict__ gy,
    uint16_t *__restrict__ gx, float *__restrict__ gprobs, int rows, int inter, float L,
    const int *__restrict__ n_used, const int *__restrict__ perm, int zero_padding)
{
    const RowSchedule sched = make_schedule(rows, n_used, zero_padding);
    const int vpr = inter / 8;
    const int nch = (vpr + U * kWave - 1) / (U * kWave);
    BwdOp<U> op{x, gy, gx, gprobs, inter, L, zero_padding,
                (uint32_t)(threadIdx.x & (kWave - 1)) * kVecBytes, 0.0f};
    SWIGLU_WALK(op, sched, perm, probs, nch);
}

// ---------------------------------------------------------------------------
// Host side: validation, launch configuration
// ---------------------------------------------------------------------------
thread_local int t_last_hip_error = 0;

constexpr int kMaxDevices = 64;

struct DeviceLaunchInfo {
    std::once_flag once;
    hipError_t err = hipSuccess;
    int cus = 0;
    int fwd_blocks_per_cu[5] = {};  // indexed by U (1..4)
    int bwd_blocks_per_cu[5] = {};
};
DeviceLaunchInfo g_devices[kMaxDevices];

template <int U>
hipError_t occupancy(int *fwd, int *bwd)
{
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
        fwd, reinterpret_cast<const void *>(swiglu_probs_fwd_kernel<U>), kBlock, 0);
    if (e != hipSuccess)
        return e;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(
        bwd, reinterpret_cast<const void *>(swiglu_probs_bwd_kernel<U>), kBlock, 0);
}

void init_device(int dev, DeviceLaunchInfo &info)
{
    hipDeviceProp_t prop;
    info.err = hipGetDeviceProperties(&prop, dev);
    if (info.err != hipSuccess)
        return;
    info.cus = prop.multiProcessorCount;
    hipError_t e = hipSuccess;
    if (e == hipSuccess) e = occupancy<1>(&info.fwd_blocks_per_cu[1], &info.bwd_blocks_per_cu[1]);
    if (e == hipSuccess) e = occupancy<2>(&info.fwd_blocks_per_cu[2], &info.bwd_blocks_per_cu[2]);
    if (e == hipSuccess) e = occupancy<3>(&info.fwd_blocks_per_cu[3], &info.bwd_blocks_per_cu[3]);
    if (e == hipSuccess) e = occupancy<4>(&info.fwd_blocks_per_cu[4], &info.bwd_blocks_per_cu[4]);
    info.err = e;
}

hipError_t device_info(DeviceLaunchInfo **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    DeviceLaunchInfo &info = g_devices[dev];
    std::call_once(info.once, init_device, dev, std::ref(info));
    *out = &info;
    return info.err;
}

// Vectors per lane per chunk: the U in 1..kMaxU that leaves the fewest idle lane slots
// in a row's last chunk, ties to the larger U. A lane's vectors are lane + 64 k in
// increasing k for every U, so the probability gradient does not depend on the choice.
int pick_u(int64_t vpr)
{
    const int64_t u = (vpr + kWave - 1) / kWave;
    int best = 1;
    int64_t best_waste = INT64_MAX;
    for (int c = kMaxU; c >= 1; --c) {
        const int64_t waste = (u + c - 1) / c * c - u;
        if (waste < best_waste)
            best = c, best_waste = waste;
    }
    return best;
}

// Column chunks of a row: U vectors per lane, 64 lanes.
int64_t chunks_per_row(int64_t vpr, int U) { return (vpr + (int64_t)U * kWave - 1) / ((int64_t)U * kWave); }

// The backward's chunk width: with at least 4 vectors per lane per row, the width that
// gives 4 or more chunks, so the workgroup's four waves share each row; else pick_u.
// Measured against pick_u's width at 53760 x 2048: 171 against 176 us; 26880 x 4096:
// 172 against 186 us; narrower rows are unaffected. (The forward measured faster with
// whole rows per wave, 103 against 111 us at 2048 columns, so it does not split rows.)
int pick_u_bwd(int64_t vpr)
{
    const int64_t u = (vpr + kWave - 1) / kWave;
    if (u >= kWavesPerBlock)
        return (int)(u / kWavesPerBlock > kMaxU ? kMaxU : u / kWavesPerBlock);
    return pick_u(vpr);
}

// The forward's chunk width: pick_u, except that a row of exactly 4 vectors per lane
// (2,048 columns) is read as two chunks of 2, which the wave pipelines. 2 KiB per wave
// per stream is what the plain streaming probe moves fastest at every read:write mix
// on MI355X (2:1: 6,657 GB/s against 6,610 at 4 KiB); interleaved at 53760 x 2048 the
// forward took 104.0 against 104.6 us. Other widths keep pick_u, whose chunks fit them
// with fewer idle lanes.
int pick_u_fwd(int64_t vpr)
{
    const int64_t u = (vpr + kWave - 1) / kWave;
    return u == 4 && kMaxU >= 2 ? 2 : pick_u(vpr);
}

// Address ranges, for the check that no output overlaps an input.
struct Range {
    uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(Range a, Range b)
{
    if (a.lo == a.hi || b.lo == b.hi)
        return false;
    return a.lo < b.hi && b.lo < a.hi;
}

Range range_of(const void *p, uint64_t bytes)
{
    uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Range{lo, p ? lo + (uintptr_t)bytes : lo};
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

constexpr int64_t kMaxRows = 0x7fffffffLL - 64LL * 65536LL;  // row indices stay in int32
constexpr int64_t kMaxInter = 1LL << 28;

swiglu_status_t check_shape(int64_t rows, int64_t inter, float limit, int num_workgroups)
{
    if (rows < 0 || inter <= 0 || rows > kMaxRows || inter > kMaxInter)
        return SWIGLU_ERR_INVALID_ARG;
    if ((uint64_t)rows * (uint64_t)inter > (1ULL << 60))
        return SWIGLU_ERR_INVALID_ARG;
    if (!(limit > 0.0f))  // NaN or <= 0; +inf is allowed (no clamp)
        return SWIGLU_ERR_INVALID_ARG;
    if (num_workgroups < 0 || num_workgroups > kMaxWorkgroups)
        return SWIGLU_ERR_INVALID_ARG;
    if (inter % 8 != 0)
        return SWIGLU_ERR_ALIGNMENT;
    return SWIGLU_OK;
}

swiglu_status_t fail_hip(hipError_t e)
{
    t_last_hip_error = (int)e;
    return SWIGLU_ERR_HIP;
}

template <int U>
void launch_fwd(int blocks, hipStream_t stream, const uint16_t *x, const float *probs, uint16_t *y,
                int rows, int inter, float limit, const int32_t *n_used, const int32_t *perm, int zp)
{
    hipLaunchKernelGGL(swiglu_probs_fwd_kernel<U>, dim3(blocks), dim3(kBlock), 0, stream, x, probs, y,
                       rows, inter, limit, n_used, perm, zp);
}

template <int U>
void launch_bwd(int blocks, hipStream_t stream, const uint16_t *x, const float *probs,
                const uint16_t *gy, uint16_t *gx, float *gp, int rows, int inter, float limit,
                const int32_t *n_used, const int32_t *perm, int zp)
{
    hipLaunchKernelGGL(swiglu_probs_bwd_kernel<U>, dim3(blocks), dim3(kBlock), 0, stream, x, probs, gy,
                       gx, gp, rows, inter, limit, n_used, perm, zp);
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

swiglu_status_t swiglu_probs_fwd_ex(const uint16_t *x, const float *probs, uint16_t *y,
                                    int64_t rows, int64_t inter, float limit,
                                    const int32_t *n_used, const int32_t *permutation_map,
                                    int zero_padding, hipStream_t stream, int num_workgroups)
{
    swiglu_status_t st = check_shape(rows, inter, limit, num_workgroups);
    if (st != SWIGLU_OK)
        return st;
    if (rows == 0)
        return SWIGLU_OK;
    if (!x || !probs || !y)
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(probs, 4) || !aligned(n_used, 4) ||
        !aligned(permutation_map, 4))
        return SWIGLU_ERR_ALIGNMENT;
    const uint64_t R = (uint64_t)rows, I = (uint64_t)inter;
    const Range out = range_of(y, R * I * 2);
    const Range ins[] = {range_of(x, R * I * 4), range_of(probs, R * 4), range_of(n_used, 4),
                         range_of(permutation_map, R * 4)};
    for (const Range &in : ins)
        if (overlaps(out, in))
            return SWIGLU_ERR_INVALID_ARG;

    DeviceLaunchInfo *info = nullptr;
    hipError_t e = device_info(&info);
    if (e != hipSuccess)
        return fail_hip(e);
    const int vpr = (int)(inter / 8);
    const int U = pick_u_fwd(vpr);
    const int blocks = num_workgroups > 0 ? num_workgroups
                                          : split_walk_workgroups(rows, chunks_per_row(vpr, U), info->cus,
                                                                  info->fwd_blocks_per_cu[U]);
    const int zp = zero_padding ? 1 : 0;
    switch (U) {
    case 1: launch_fwd<1>(blocks, stream, x, probs, y, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    case 2: launch_fwd<2>(blocks, stream, x, probs, y, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    case 3: launch_fwd<3>(blocks, stream, x, probs, y, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    default: launch_fwd<4>(blocks, stream, x, probs, y, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess)
        return fail_hip(e);
    return SWIGLU_OK;
}

swiglu_status_t swiglu_probs_bwd_ex(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                    uint16_t *grad_x, float *grad_probs,
                                    int64_t rows, int64_t inter, float limit,
                                    const int32_t *n_used, const int32_t *permutation_map,
                                    int zero_padding, hipStream_t stream, int num_workgroups)
{
    swiglu_status_t st = check_shape(rows, inter, limit, num_workgroups);
    if (st != SWIGLU_OK)
        return st;
    if (rows == 0)
        return SWIGLU_OK;
    if (!x || !probs || !grad_y || !grad_x)
        return SWIGLU_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(grad_y, 16) || !aligned(grad_x, 16) || !aligned(probs, 4) ||
        !aligned(grad_probs, 4) || !aligned(n_used, 4) || !aligned(permutation_map, 4))
        return SWIGLU_ERR_ALIGNMENT;
    const uint64_t R = (uint64_t)rows, I = (uint64_t)inter;
    const Range outs[] = {range_of(grad_x, R * I * 4), range_of(grad_probs, R * 4)};
    const Range ins[] = {range_of(x, R * I * 4), range_of(probs, R * 4), range_of(grad_y, R * I * 2),
                         range_of(n_used, 4), range_of(permutation_map, R * 4)};
    for (const Range &o : outs)
        for (const Range &in : ins)
            if (overlaps(o, in))
                return SWIGLU_ERR_INVALID_ARG;
    if (overlaps(outs[0], outs[1]))
        return SWIGLU_ERR_INVALID_ARG;

    DeviceLaunchInfo *info = nullptr;
    hipError_t e = device_info(&info);
    if (e != hipSuccess)
        return fail_hip(e);
    const int vpr = (int)(inter / 8);
    const int U = pick_u_bwd(vpr);
    const int blocks = num_workgroups > 0 ? num_workgroups
                                          : split_walk_workgroups(rows, chunks_per_row(vpr, U), info->cus,
                                                                  info->bwd_blocks_per_cu[U]);
    const int zp = zero_padding ? 1 : 0;
    switch (U) {
    case 1: launch_bwd<1>(blocks, stream, x, probs, grad_y, grad_x, grad_probs, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    case 2: launch_bwd<2>(blocks, stream, x, probs, grad_y, grad_x, grad_probs, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    case 3: launch_bwd<3>(blocks, stream, x, probs, grad_y, grad_x, grad_probs, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    default: launch_bwd<4>(blocks, stream, x, probs, grad_y, grad_x, grad_probs, (int)rows, (int)inter, limit, n_used, permutation_map, zp); break;
    }
    e = hipGetLastError();
    if (e != hipSuccess)
        return fail_hip(e);
    return SWIGLU_OK;
}

swiglu_status_t swiglu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                                 int64_t rows, int64_t inter, float limit,
                                 const int32_t *n_used, const int32_t *permutation_map,
                                 int zero_padding, hipStream_t stream)
{
    return swiglu_probs_fwd_ex(x, probs, y, rows, inter, limit, n_used, permutation_map,
                               zero_padding, stream, 0);
}

swiglu_status_t swiglu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                 uint16_t *grad_x, float *grad_probs,
                                 int64_t rows, int64_t inter, float limit,
                                 const int32_t *n_used, const int32_t *permutation_map,
                                 int zero_padding, hipStream_t stream)
{
    return swiglu_probs_bwd_ex(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, n_used,
                               permutation_map, zero_padding, stream, 0);
}

int swiglu_probs_default_workgroups(int direction, int64_t rows, int64_t inter)
{
    if (rows < 0 || inter <= 0 || inter % 8 != 0 || (direction != 0 && direction != 1))
        return -1;
    DeviceLaunchInfo *info = nullptr;
    if (device_info(&info) != hipSuccess)
        return -1;
    const int U = direction == 0 ? pick_u_fwd(inter / 8) : pick_u_bwd(inter / 8);
    const int bpc = direction == 0 ? info->fwd_blocks_per_cu[U] : info->bwd_blocks_per_cu[U];
    return split_walk_workgroups(rows, chunks_per_row(inter / 8, U), info->cus, bpc);
}

const char *swiglu_probs_status_string(swiglu_status_t status)
{
    switch (status) {
    case SWIGLU_OK: return "ok";
    case SWIGLU_ERR_INVALID_ARG: return "invalid argument";
    case SWIGLU_ERR_ALIGNMENT: return "misaligned pointer or inter not a multiple of 8";
    case SWIGLU_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int swiglu_probs_last_hip_error(void) { return t_last_hip_error; }

int swiglu_probs_abi_version(void) { return SWIGLU_PROBS_ABI_VERSION; }

}  // extern "C"
