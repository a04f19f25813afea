// Fused clamped-SwiGLU x routing-probability activation, forward and backward,
// for AMD Instinct MI355X (gfx950, CDNA4). C ABI declared in swiglu_probs.h.
//
// What is computed (NeMo AutoModel "moe/swiglu_triton" page, module docstring):
//   y = silu(clamp(gate, max=L)) * clamp(up, -L, L) * probs, fp32 math, one bf16
//   rounding; the backward stores d_gate / d_up in the gate / up halves of grad_x and
//   reduces the per-row probability gradient in fp32. Clamp gradients follow
//   torch.clamp (inclusive masks). Row bookkeeping (n_used, permutation_map,
//   zero_padding, fixed grid striding over rows) follows the Megatron-Core
//   "core.inference.moe.batch_invariant" page (_swiglu_with_probs_kernel,
//   _weighted_silu_mul_bounded_kernel).
//
// Design (HBM-bound; no MFMA):
//   * Lane l of a wave handles the 16-byte vectors l, l+64, l+128, ... of the gate
//     half, the up half and (backward) grad_y: every access is 128 bits wide and one
//     wave instruction covers 1 KiB of contiguous memory.
//   * Every load and store is a buffer instruction on a per-row buffer resource
//     whose size is the row's byte length, or 0 for a row that is not live. The
//     hardware range check then does all masking: lanes past the row end and rows
//     that are not live read zeros without touching memory, and their stores are
//     dropped (or, for zero-padded rows, write the +0 that zero inputs produce).
//     No branch guards a memory instruction, so the compiler's wait counts are exact.
//   * Default launches are straight-line kernels with one unit of work per wave:
//     the forward gives each wave one whole row (up to 4 vectors per lane per stream,
//     all loads issued at once); the backward gives each wave one whole row of up to
//     3 vectors per lane, and splits rows of exactly 4 chunks among the four waves of
//     a workgroup, one chunk each (the 2,048- and 4,096-column rows). The row's slot
//     comes from scalar loads (n_used, the map entry) and its probability from a
//     one-dword buffer load issued with the row's streaming loads, so a wave carries no
//     per-row bookkeeping beyond its own row.
//   * Other shapes, and launches with an explicit workgroup count, run the fixed-grid
//     walks of cdna4_stream.h: waves (or workgroups, for shared rows) stride over
//     rows (row r, r + W, r + 2W, ...), each wave pipelining the loads of its next
//     chunk ahead of the current one's arithmetic. The launch never depends on device
//     data and is graph-safe; both forms give the same bits, because the element
//     arithmetic, each lane's column order and the reduction order are the same.
//   * The probability gradient: each lane sums its own columns in a fixed order, then
//     a fixed DPP butterfly over the wave combines the 64 partials; on shared rows the
//     four waves first add their lane partials in wave order through LDS. The order
//     depends only on the row width, never on the grid, so the bits are grid-invariant.
//   * fp32 -> bf16 uses v_cvt_pk_bf16_f32 (round to nearest even, two values per
//     instruction); the clamps use v_minimum3/v_maximum3 (NaN-propagating, as
//     torch.clamp); the inclusive masks are "the clamp left the value unchanged".
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cmath>
#include <mutex>

#include "cdna4_stream.h"
#include "swiglu_probs.h"

namespace {

using namespace cdna4;

constexpr int kMaxU = 4;  // 16-byte vectors per lane per stream per chunk
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

// logistic sigmoid sig = 1 / (1 + e^-z) and 1 - sig, from v_exp_f32 (2^x) and v_rcp_f32.
// v_rcp_f32 flushes subnormal results to zero, and 1 / (1 + e^-z) is subnormal once
// 1 + e^-z exceeds 2^126 (z < -87.3), where silu(z) = z * sigmoid(z) is still a normal
// number. The reciprocal is therefore taken of 2^-64 * (1 + e^-z) (one fma, exact: a
// power-of-two scale of a value >= 1), which keeps it normal, and the result is scaled
// back by 2^-64 in a multiply, which does produce subnormals. For e^-z = inf (z < -88.7)
// the sigmoid is 0, as 1 / (1 + inf) is in fp32. 1 - sig is one fma of the scaled
// reciprocal.
__device__ __forceinline__ void sigmoid(float z, float &sig, float &one_minus_sig)
{
    constexpr float kTwoM64 = 0x1p-64f;
    const float e = __builtin_amdgcn_exp2f(z * kNegLog2e);
    const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(e, kTwoM64, kTwoM64));  // 2^64 sig
    sig = r * kTwoM64;
    one_minus_sig = __builtin_fmaf(r, -kTwoM64, 1.0f);
}

__device__ __forceinline__ float fwd_elem(float a, float b, float p, float L)
{
    float cg = clamp_gate(a, L);
    float cu = clamp_up(b, L);
    float sig, oms;
    sigmoid(cg, sig, oms);
    float s = cg * sig;
    return (s * cu) * p;
}

// Autograd chain of y = (silu(cg) * cu) * p with inclusive clamp masks. The silu
// derivative sig * (1 + cg * (1 - sig)) is taken as sig + s * (1 - sig), one fma: the
// same value (s = cg * sig), one rounding instead of two. Near silu's minimum
// (cg = -1.2785, where the derivative crosses 0) both forms cancel alike; a bf16 gate
// stays at least 0.0027 away from it, and over every bf16 gate the relative error of
// either form in fp32 stays under 1e-5 (an fp64 check), far inside half a bf16 ulp.
__device__ __forceinline__ void bwd_elem(float a, float b, float g, float p, float L,
                                         float &dg, float &du, float &acc)
{
    float cg = clamp_gate(a, L);
    float cu = clamp_up(b, L);
    float sig, oms;
    sigmoid(cg, sig, oms);
    float s = cg * sig;
    float gp = g * p;
    float dsilu = __builtin_fmaf(s, oms, sig);
    // a <= L  <=>  min(a, L) == a ;  -L <= b <= L  <=>  clamp(b) == b  (false for NaN)
    dg = (cg == a) ? (gp * cu) * dsilu : 0.0f;
    du = (cu == b) ? gp * s : 0.0f;
    acc += g * (s * cu);
}

// Eight elements of a 16-byte vector (four packed bf16 pairs): forward.
__device__ __forceinline__ u32x4 fwd_vec(const u32x4 &g, const u32x4 &u, float p, float L)
{
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float y0 = fwd_elem(bf16_lo(g[q]), bf16_lo(u[q]), p, L);
        const float y1 = fwd_elem(bf16_hi(g[q]), bf16_hi(u[q]), p, L);
        o[q] = pack_bf16x2(y0, y1);
    }
    return o;
}

// Eight elements of a 16-byte vector: backward, in column order (lo then hi of each
// pair), adding to the lane's row-sum partial in that order.
__device__ __forceinline__ void bwd_vec(const u32x4 &g, const u32x4 &u, const u32x4 &d, float p, float L,
                                        u32x4 &og, u32x4 &ou, float &acc)
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float dg0, du0, dg1, du1;
        bwd_elem(bf16_lo(g[q]), bf16_lo(u[q]), bf16_lo(d[q]), p, L, dg0, du0, acc);
        bwd_elem(bf16_hi(g[q]), bf16_hi(u[q]), bf16_hi(d[q]), p, L, dg1, du1, acc);
        og[q] = pack_bf16x2(dg0, dg1);
        ou[q] = pack_bf16x2(du0, du1);
    }
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
        for (int u = 0; u < U; ++u)
            store_vec(ry, fwd_vec(b.g[u], b.u[u], p, L), voff + u * kWave * kVecBytes);
    }
};

template <int U>
__global__ __launch_bounds__(kBlock) void swiglu_probs_fwd_kernel(
    const uint16_t *__restrict__ x, const float *__restrict__ probs, uint16_t *__restrict__ y,
    const int *__restrict__ n_used, const int *__restrict__ perm, int rows, int inter, float L,
    int zero_padding)
{
    const RowSchedule sched = make_schedule(rows, n_used, zero_padding);
    const int vpr = inter / 8;
    const int nch = (vpr + U * kWave - 1) / (U * kWave);
    FwdOp<U> op{x, y, inter, L, zero_padding, (uint32_t)(threadIdx.x & (kWave - 1)) * kVecBytes};
    walk_row_split(op, sched, perm, probs, nch);
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
            bwd_vec(b.g[u], b.u[u], b.d[u], p, L, og, ou, acc);
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
    int rows, int inter, float L, int zero_padding, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ gy, uint16_t *__restrict__ gx, const int *__restrict__ n_used,
    const int *__restrict__ perm, const float *__restrict__ probs, float *__restrict__ gprobs)
{
    const RowSchedule sched = make_schedule(rows, n_used, zero_padding);
    const int vpr = inter / 8;
    const int nch = (vpr + U * kWave - 1) / (U * kWave);
    BwdOp<U> op{x, gy, gx, gprobs, inter, L, zero_padding,
                (uint32_t)(threadIdx.x & (kWave - 1)) * kVecBytes, 0.0f};
    walk_row_split(op, sched, perm, probs, nch);
}

// ---------------------------------------------------------------------------
// Straight-line kernels of the default launches: one unit of work per wave
// ---------------------------------------------------------------------------
// Forward, one wave per row (row = the wave's index in the grid), every vector of the
// row at once: V = ceil(inter / 512) <= 4 vectors per lane per stream.
template <int V>
__global__ __launch_bounds__(kBlock) void swiglu_probs_fwd_row_kernel(
    int rows, int inter, float L, int flags, const uint16_t *__restrict__ x,
    const float *__restrict__ probs, uint16_t *__restrict__ y, const int *__restrict__ n_used,
    const int *__restrict__ perm)
{
    const int r = wave_id();
    if (r >= rows)
        return;
    const int slot = row_slot(r, rows, flags, n_used, perm);
    if (slot < 0 && !(flags & kZeroPadding))
        return;
    const uint32_t row_bytes = (uint32_t)inter * 2u;
    const uint32_t n_in = slot >= 0 ? row_bytes : 0u;
    const uint16_t *gate = x + (int64_t)r * 2 * inter;
    const rsrc_t rg = make_rsrc(gate, n_in), ru = make_rsrc(gate + inter, n_in);
    const uint32_t voff = (uint32_t)lane_id() * kVecBytes;
    const float p = load_row_prob(probs, slot);
    u32x4 g[V], u[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        g[v] = load_vec(rg, voff + v * kWave * kVecBytes);
        u[v] = load_vec(ru, voff + v * kWave * kVecBytes);
    }
    const rsrc_t ry = make_rsrc(y + (int64_t)r * inter, row_bytes);
#pragma unroll
    for (int v = 0; v < V; ++v)
        store_vec(ry, fwd_vec(g[v], u[v], p, L), voff + v * kWave * kVecBytes);
}

// Backward, one wave per row, every vector of the row at once (V <= 3 vectors per lane
// per stream: rows of one chunk). The row sum is the lane partials in column order,
// then wave_sum: walk_rows' order for a one-chunk row.
template <int V>
__global__ __launch_bounds__(kBlock) void swiglu_probs_bwd_row_kernel(
    int rows, int inter, float L, int flags, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ gy, uint16_t *__restrict__ gx, const float *__restrict__ probs,
    float *__restrict__ gprobs, const int *__restrict__ n_used, const int *__restrict__ perm)
{
    const int r = wave_id();
    if (r >= rows)
        return;
    const int slot = row_slot(r, rows, flags, n_used, perm);
    if (slot < 0 && !(flags & kZeroPadding))
        return;
    const uint32_t row_bytes = (uint32_t)inter * 2u;
    const uint32_t n_in = slot >= 0 ? row_bytes : 0u;
    const uint16_t *gate = x + (int64_t)r * 2 * inter;
    const rsrc_t rg = make_rsrc(gate, n_in), ru = make_rsrc(gate + inter, n_in);
    const rsrc_t rd = make_rsrc(gy + (int64_t)r * inter, n_in);
    const uint32_t voff = (uint32_t)lane_id() * kVecBytes;
    const float p = load_row_prob(probs, slot);
    u32x4 g[V], u[V], d[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        g[v] = load_vec(rg, voff + v * kWave * kVecBytes);
        u[v] = load_vec(ru, voff + v * kWave * kVecBytes);
        d[v] = load_vec(rd, voff + v * kWave * kVecBytes);
    }
    uint16_t *dgate = gx + (int64_t)r * 2 * inter;
    const rsrc_t rdg = make_rsrc(dgate, row_bytes), rdu = make_rsrc(dgate + inter, row_bytes);
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < V; ++v) {
        u32x4 og, ou;
        bwd_vec(g[v], u[v], d[v], p, L, og, ou, acc);
        store_vec(rdg, og, voff + v * kWave * kVecBytes);
        store_vec(rdu, ou, voff + v * kWave * kVecBytes);
    }
    if (slot >= 0 && gprobs) {
        const float total = wave_sum(acc);
        if (lane_id() == 0)
            gprobs[slot] = total;
    }
}

// Backward, one workgroup per row (row = workgroup index) cut into exactly four chunks
// of U vectors per lane, wave w taking chunk w. The row sum goes through row_sum_last:
// walk_row_split's order for a row of four chunks, with no barrier at the end (the
// slowest wave of the row does the sum; the others leave). At 53760 x 2048 (medians of
// twelve interleaved rounds): 172.0 against 172.7 us with row_sum_split's end-of-row
// barrier; with no row sum at all (grad_probs NULL) the backward takes about 0.9% less.
template <int U>
__global__ __launch_bounds__(kBlock) void swiglu_probs_bwd_quarter_kernel(
    int rows, int inter, float L, int flags, const uint16_t *__restrict__ x,
    const uint16_t *__restrict__ gy, uint16_t *__restrict__ gx, const float *__restrict__ probs,
    float *__restrict__ gprobs, const int *__restrict__ n_used, const int *__restrict__ perm)
{
    __shared__ float part[kWavesPerBlock][kWave];
    __shared__ unsigned arrived;
    const int r = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
    const int w = wave_in_block();
    if (r >= rows)
        return;
    // the same for all four waves: either all return here or all reach the barrier below
    const int slot = row_slot(r, rows, flags, n_used, perm);
    if (slot < 0 && !(flags & kZeroPadding))
        return;
    const uint32_t row_bytes = (uint32_t)inter * 2u;
    const uint32_t n_in = slot >= 0 ? row_bytes : 0u;
    const uint32_t off = (uint32_t)w * U * kWave * kVecBytes;
    const uint16_t *gate = x + (int64_t)r * 2 * inter;
    const rsrc_t rg = chunk_rsrc(gate, n_in, off), ru = chunk_rsrc(gate + inter, n_in, off);
    const rsrc_t rd = chunk_rsrc(gy + (int64_t)r * inter, n_in, off);
    const uint32_t voff = (uint32_t)lane_id() * kVecBytes;
    const float p = load_row_prob(probs, slot);
    u32x4 g[U], u[U], d[U];
#pragma unroll
    for (int v = 0; v < U; ++v) {
        g[v] = load_vec(rg, voff + v * kWave * kVecBytes);
        u[v] = load_vec(ru, voff + v * kWave * kVecBytes);
        d[v] = load_vec(rd, voff + v * kWave * kVecBytes);
    }
    // the same for all four waves, like slot: all or none take the barrier
    const bool row_sum = slot >= 0 && gprobs;
    if (row_sum)
        row_sum_last_init(&arrived, w, lane_id());
    uint16_t *dgate = gx + (int64_t)r * 2 * inter;
    const rsrc_t rdg = chunk_rsrc(dgate, row_bytes, off), rdu = chunk_rsrc(dgate + inter, row_bytes, off);
    float acc = 0.0f;
#pragma unroll
    for (int v = 0; v < U; ++v) {
        u32x4 og, ou;
        bwd_vec(g[v], u[v], d[v], p, L, og, ou, acc);
        store_vec(rdg, og, voff + v * kWave * kVecBytes);
        store_vec(rdu, ou, voff + v * kWave * kVecBytes);
    }
    float total;
    if (row_sum && row_sum_last(part, &arrived, acc, w, lane_id(), total) && lane_id() == 0)
        gprobs[slot] = total;
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

// Default launches take the straight-line kernels where one unit of work per wave
// fits: the forward for rows of at most 4 vectors per lane per stream (inter <= 2048,
// one wave per row), the backward for rows of at most 3 (inter <= 1536, one wave per
// row) and for rows that pick_u_bwd cuts into exactly four chunks (one per wave of a
// workgroup: 2,048 and 4,096 columns among others). Their grids are the walks' default
// grids for those shapes. Where one unit per wave would need more than 16,777,215
// workgroups the walks take over, with the same bits. Each returns the kernel's vector
// count (V, or U for the quarters), 0 when the shape takes a walk.
int lean_fwd_vectors(int64_t rows, int64_t vpr)
{
    const int64_t u = (vpr + kWave - 1) / kWave;
    return u <= 4 && (rows + kWavesPerBlock - 1) / kWavesPerBlock <= kMaxWorkgroups ? (int)u : 0;
}

int lean_bwd_row_vectors(int64_t rows, int64_t vpr)
{
    const int64_t u = (vpr + kWave - 1) / kWave;
    return u <= 3 && (rows + kWavesPerBlock - 1) / kWavesPerBlock <= kMaxWorkgroups ? (int)u : 0;
}

int lean_bwd_quarter_u(int64_t rows, int64_t vpr)
{
    const int64_t u = (vpr + kWave - 1) / kWave;
    const int U = pick_u_bwd(vpr);
    return u >= kWavesPerBlock && chunks_per_row(vpr, U) == kWavesPerBlock && rows <= kMaxWorkgroups ? U : 0;
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

// Every launch goes through hipExtLaunchKernel: with events (the timed entry points) the
// kernel's own start and end are recorded into them, with no separate command on the
// stream; with null events it is a plain launch.
struct Launch {
    hipStream_t stream;
    hipEvent_t start, stop;
};

template <int U>
void launch_fwd(const Launch &l, int blocks, const uint16_t *x, const float *probs, uint16_t *y,
                int rows, int inter, float limit, const int32_t *n_used, const int32_t *perm, int zp)
{
    hipExtLaunchKernelGGL(swiglu_probs_fwd_kernel<U>, dim3(blocks), dim3(kBlock), 0, l.stream, l.start, l.stop, 0,
                          x, probs, y, n_used, perm, rows, inter, limit, zp);
}

template <int U>
void launch_bwd(const Launch &l, int blocks, const uint16_t *x, const float *probs,
                const uint16_t *gy, uint16_t *gx, float *gp, int rows, int inter, float limit,
                const int32_t *n_used, const int32_t *perm, int zp)
{
    hipExtLaunchKernelGGL(swiglu_probs_bwd_kernel<U>, dim3(blocks), dim3(kBlock), 0, l.stream, l.start, l.stop, 0,
                          rows, inter, limit, zp, x, gy, gx, n_used, perm, probs, gp);
}

// The flags argument of the one-row-per-wave kernels.
int row_flags(int zp, const int32_t *n_used, const int32_t *perm)
{
    return (zp ? kZeroPadding : 0) | (n_used ? kHasNUsed : 0) | (perm ? kHasPerm : 0);
}

template <int V>
void launch_fwd_row_v(const Launch &l, const uint16_t *x, const float *probs, uint16_t *y, int rows,
                      int inter, float limit, const int32_t *n_used, const int32_t *perm, int zp)
{
    const int blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    hipExtLaunchKernelGGL(swiglu_probs_fwd_row_kernel<V>, dim3(blocks), dim3(kBlock), 0, l.stream, l.start, l.stop,
                          0, rows, inter, limit, row_flags(zp, n_used, perm), x, probs, y, n_used, perm);
}

// The straight-line forward of a default launch; false (nothing launched) when the
// shape takes a walk.
bool launch_fwd_row(const Launch &l, const uint16_t *x, const float *probs, uint16_t *y, int64_t rows,
                    int64_t inter, float limit, const int32_t *n_used, const int32_t *perm, int zp)
{
    const int r = (int)rows, n = (int)inter;
    switch (lean_fwd_vectors(rows, inter / 8)) {
    case 1: launch_fwd_row_v<1>(l, x, probs, y, r, n, limit, n_used, perm, zp); return true;
    case 2: launch_fwd_row_v<2>(l, x, probs, y, r, n, limit, n_used, perm, zp); return true;
    case 3: launch_fwd_row_v<3>(l, x, probs, y, r, n, limit, n_used, perm, zp); return true;
    case 4: launch_fwd_row_v<4>(l, x, probs, y, r, n, limit, n_used, perm, zp); return true;
    default: return false;
    }
}

template <int V>
void launch_bwd_row_v(const Launch &l, const uint16_t *x, const float *probs, const uint16_t *gy,
                      uint16_t *gx, float *gp, int rows, int inter, float limit, const int32_t *n_used,
                      const int32_t *perm, int zp)
{
    const int blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    hipExtLaunchKernelGGL(swiglu_probs_bwd_row_kernel<V>, dim3(blocks), dim3(kBlock), 0, l.stream, l.start, l.stop,
                          0, rows, inter, limit, row_flags(zp, n_used, perm), x, gy, gx, probs, gp, n_used, perm);
}

template <int U>
void launch_bwd_quarter_u(const Launch &l, const uint16_t *x, const float *probs, const uint16_t *gy,
                          uint16_t *gx, float *gp, int rows, int inter, float limit, const int32_t *n_used,
                          const int32_t *perm, int zp)
{
    hipExtLaunchKernelGGL(swiglu_probs_bwd_quarter_kernel<U>, dim3(rows), dim3(kBlock), 0, l.stream, l.start,
                          l.stop, 0, rows, inter, limit, row_flags(zp, n_used, perm), x, gy, gx, probs, gp, n_used,
                          perm);
}

// The straight-line backward of a default launch; false (nothing launched) when the
// shape takes a walk.
bool launch_bwd_lean(const Launch &l, const uint16_t *x, const float *probs, const uint16_t *gy,
                     uint16_t *gx, float *gp, int64_t rows, int64_t inter, float limit,
                     const int32_t *n_used, const int32_t *perm, int zp)
{
    const int r = (int)rows, n = (int)inter;
    switch (lean_bwd_row_vectors(rows, inter / 8)) {
    case 1: launch_bwd_row_v<1>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    case 2: launch_bwd_row_v<2>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    case 3: launch_bwd_row_v<3>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    default: break;
    }
    switch (lean_bwd_quarter_u(rows, inter / 8)) {
    case 1: launch_bwd_quarter_u<1>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    case 2: launch_bwd_quarter_u<2>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    case 3: launch_bwd_quarter_u<3>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    case 4: launch_bwd_quarter_u<4>(l, x, probs, gy, gx, gp, r, n, limit, n_used, perm, zp); return true;
    default: return false;
    }
}

// Validation, then the launch. Arguments are checked on the host before anything is
// launched; on any error nothing is written.
swiglu_status_t fwd_impl(const uint16_t *x, const float *probs, uint16_t *y, int64_t rows, int64_t inter,
                         float limit, const int32_t *n_used, const int32_t *permutation_map, int zero_padding,
                         int num_workgroups, const Launch &l)
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

    const int vpr = (int)(inter / 8);
    const int zp = zero_padding ? 1 : 0;
    if (num_workgroups != 0 || !launch_fwd_row(l, x, probs, y, rows, inter, limit, n_used, permutation_map, zp)) {
        DeviceLaunchInfo *info = nullptr;
        const hipError_t e = device_info(&info);
        if (e != hipSuccess)
            return fail_hip(e);
        const int U = pick_u_fwd(vpr);
        const int blocks = num_workgroups > 0 ? num_workgroups
                                              : split_walk_workgroups(rows, chunks_per_row(vpr, U), info->cus,
                                                                      info->fwd_blocks_per_cu[U]);
        const int r = (int)rows, n = (int)inter;
        switch (U) {
        case 1: launch_fwd<1>(l, blocks, x, probs, y, r, n, limit, n_used, permutation_map, zp); break;
        case 2: launch_fwd<2>(l, blocks, x, probs, y, r, n, limit, n_used, permutation_map, zp); break;
        case 3: launch_fwd<3>(l, blocks, x, probs, y, r, n, limit, n_used, permutation_map, zp); break;
        default: launch_fwd<4>(l, blocks, x, probs, y, r, n, limit, n_used, permutation_map, zp); break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail_hip(e);
    return SWIGLU_OK;
}

swiglu_status_t bwd_impl(const uint16_t *x, const float *probs, const uint16_t *grad_y, uint16_t *grad_x,
                         float *grad_probs, int64_t rows, int64_t inter, float limit, const int32_t *n_used,
                         const int32_t *permutation_map, int zero_padding, int num_workgroups, const Launch &l)
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

    const int vpr = (int)(inter / 8);
    const int zp = zero_padding ? 1 : 0;
    if (num_workgroups != 0 || !launch_bwd_lean(l, x, probs, grad_y, grad_x, grad_probs, rows, inter, limit,
                                                n_used, permutation_map, zp)) {
        DeviceLaunchInfo *info = nullptr;
        const hipError_t e = device_info(&info);
        if (e != hipSuccess)
            return fail_hip(e);
        const int U = pick_u_bwd(vpr);
        const int blocks = num_workgroups > 0 ? num_workgroups
                                              : split_walk_workgroups(rows, chunks_per_row(vpr, U), info->cus,
                                                                      info->bwd_blocks_per_cu[U]);
        const int r = (int)rows, n = (int)inter;
        switch (U) {
        case 1: launch_bwd<1>(l, blocks, x, probs, grad_y, grad_x, grad_probs, r, n, limit, n_used, permutation_map, zp); break;
        case 2: launch_bwd<2>(l, blocks, x, probs, grad_y, grad_x, grad_probs, r, n, limit, n_used, permutation_map, zp); break;
        case 3: launch_bwd<3>(l, blocks, x, probs, grad_y, grad_x, grad_probs, r, n, limit, n_used, permutation_map, zp); break;
        default: launch_bwd<4>(l, blocks, x, probs, grad_y, grad_x, grad_probs, r, n, limit, n_used, permutation_map, zp); break;
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return fail_hip(e);
    return SWIGLU_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

swiglu_status_t swiglu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                                 int64_t rows, int64_t inter, float limit,
                                 const int32_t *n_used, const int32_t *permutation_map,
                                 int zero_padding, hipStream_t stream)
{
    return fwd_impl(x, probs, y, rows, inter, limit, n_used, permutation_map, zero_padding, 0,
                    Launch{stream, nullptr, nullptr});
}

swiglu_status_t swiglu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                 uint16_t *grad_x, float *grad_probs,
                                 int64_t rows, int64_t inter, float limit,
                                 const int32_t *n_used, const int32_t *permutation_map,
                                 int zero_padding, hipStream_t stream)
{
    return bwd_impl(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, n_used, permutation_map,
                    zero_padding, 0, Launch{stream, nullptr, nullptr});
}

swiglu_status_t swiglu_probs_fwd_ex(const uint16_t *x, const float *probs, uint16_t *y,
                                    int64_t rows, int64_t inter, float limit,
                                    const int32_t *n_used, const int32_t *permutation_map,
                                    int zero_padding, hipStream_t stream, int num_workgroups)
{
    return fwd_impl(x, probs, y, rows, inter, limit, n_used, permutation_map, zero_padding, num_workgroups,
                    Launch{stream, nullptr, nullptr});
}

swiglu_status_t swiglu_probs_bwd_ex(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                    uint16_t *grad_x, float *grad_probs,
                                    int64_t rows, int64_t inter, float limit,
                                    const int32_t *n_used, const int32_t *permutation_map,
                                    int zero_padding, hipStream_t stream, int num_workgroups)
{
    return bwd_impl(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, n_used, permutation_map,
                    zero_padding, num_workgroups, Launch{stream, nullptr, nullptr});
}

swiglu_status_t swiglu_probs_fwd_timed(const uint16_t *x, const float *probs, uint16_t *y,
                                       int64_t rows, int64_t inter, float limit,
                                       const int32_t *n_used, const int32_t *permutation_map,
                                       int zero_padding, hipStream_t stream, int num_workgroups,
                                       hipEvent_t start, hipEvent_t stop)
{
    return fwd_impl(x, probs, y, rows, inter, limit, n_used, permutation_map, zero_padding, num_workgroups,
                    Launch{stream, start, stop});
}

swiglu_status_t swiglu_probs_bwd_timed(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                       uint16_t *grad_x, float *grad_probs,
                                       int64_t rows, int64_t inter, float limit,
                                       const int32_t *n_used, const int32_t *permutation_map,
                                       int zero_padding, hipStream_t stream, int num_workgroups,
                                       hipEvent_t start, hipEvent_t stop)
{
    return bwd_impl(x, probs, grad_y, grad_x, grad_probs, rows, inter, limit, n_used, permutation_map,
                    zero_padding, num_workgroups, Launch{stream, start, stop});
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
