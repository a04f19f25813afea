// MoE elementwise operations next to the routed-expert activation, for AMD Instinct
// MI355X (gfx950). C ABI declared in moe_elementwise.h.
//
//   residual add   Megatron-Core "core.fusions.fused_moe_residual_add" page
//   router weight  NeMo AutoModel "moe/optimized_ops" page (_RouterWeightMulFunction)
//   squared ReLU   Megatron-Core "core.inference.moe.batch_invariant" page
//                  (_squared_relu_with_probs_kernel, squared_relu_with_probs);
//                  the backward is the chain rule through it (the page gives none)
//   unpermute      same page (_unpermute_tokens_in_expert_order_kernel)
//
// All are streams built on cdna4_stream.h: 128-bit buffer accesses on per-row (or
// per-block) resources whose hardware range check masks ragged ends and rows that
// are not live, nontemporal hints, and the two-buffer software pipeline per wave.
// Default grids: one wave per 2 KiB block (residual add), rows of 4 or more chunks
// shared by a workgroup's four waves (router weight), one wave per row of at most two
// chunks, loaded whole (squared ReLU, both directions), and one wave per (token,
// column chunk) gathering only the contributing experts' rows (unpermute, up to 8
// local experts). Other shapes, and launches with an explicit workgroup count, take
// the fixed-grid walks (walk_workgroups / split_walk_workgroups; a persistent
// pipelined walk for the unpermute), with the same bits. Values are handled in groups
// of eight elements per lane ("octs": one 16-byte access for 16-bit types, two for
// fp32).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <cmath>
#include <mutex>

#include "cdna4_stream.h"
#include "moe_elementwise.h"

namespace {

using namespace cdna4;

enum : int { DT_BF16 = 0, DT_F16 = 1, DT_F32 = 2 };

template <int DT>
constexpr int kElemBytes = DT == DT_F32 ? 4 : 2;
template <int DT>
constexpr int kOctBytes = 8 * kElemBytes<DT>;

struct Oct {
    u32x4 v[2];  // v[1] used only for fp32
};

template <int DT>
__device__ __forceinline__ Oct load_oct(rsrc_t r, uint32_t off)
{
    Oct o;
    o.v[0] = load_vec(r, off);
    if constexpr (DT == DT_F32)
        o.v[1] = load_vec(r, off + kVecBytes);
    return o;
}

template <int DT>
__device__ __forceinline__ void store_oct(rsrc_t r, const Oct &o, uint32_t off)
{
    store_vec(r, o.v[0], off);
    if constexpr (DT == DT_F32)
        store_vec(r, o.v[1], off + kVecBytes);
}

template <int DT>
__device__ __forceinline__ void widen(const Oct &o, float (&f)[8])
{
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (DT == DT_BF16) {
            f[2 * q] = bf16_lo(o.v[0][q]);
            f[2 * q + 1] = bf16_hi(o.v[0][q]);
        } else if constexpr (DT == DT_F16) {
            const f32x2 t = unpack_f16x2(o.v[0][q]);
            f[2 * q] = t.x;
            f[2 * q + 1] = t.y;
        } else {
            f[q] = __uint_as_float(o.v[0][q]);
            f[4 + q] = __uint_as_float(o.v[1][q]);
        }
    }
}

template <int DT>
__device__ __forceinline__ Oct narrow(const float (&f)[8])
{
    Oct o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if constexpr (DT == DT_BF16) {
            o.v[0][q] = pack_bf16x2(f[2 * q], f[2 * q + 1]);
        } else if constexpr (DT == DT_F16) {
            o.v[0][q] = pack_f16x2(f[2 * q], f[2 * q + 1]);
        } else {
            o.v[0][q] = __float_as_uint(f[q]);
            o.v[1][q] = __float_as_uint(f[4 + q]);
        }
    }
    return o;
}

// Rounds eight fp32 values to DT and back (the activation-dtype rounding of a sum).
template <int DT>
__device__ __forceinline__ void round_to(float (&f)[8])
{
    if constexpr (DT != DT_F32)
        widen<DT>(narrow<DT>(f), f);
}

// ---------------------------------------------------------------------------
// Fused MoE residual add: out = residual + round_to_dtype(expert + shared)
// ---------------------------------------------------------------------------
template <int DT, int U>
struct ResidualAddOp {
    static constexpr uint32_t kBlockBytes = U * kWave * kOctBytes<DT>;
    struct Buf {
        Oct e[U], s[U], r[U];
    };
    const char *e, *s, *r;
    char *out;
    int64_t full_bytes;  // bytes of the whole octs of each tensor
    uint32_t voff;       // this lane's offset within a block

    __device__ __forceinline__ uint32_t valid(int64_t b) const
    {
        const int64_t left = full_bytes - b * kBlockBytes;
        return left <= 0 ? 0u : (left < kBlockBytes ? (uint32_t)left : kBlockBytes);
    }

    __device__ __forceinline__ void load(Buf &buf, int64_t b, bool live) const
    {
        const int64_t off = b * kBlockBytes;
        const uint32_t n = live ? valid(b) : 0u;
        const rsrc_t re = make_rsrc(e + off, n), rs = make_rsrc(s + off, n), rr = make_rsrc(r + off, n);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t o = voff + u * kWave * kOctBytes<DT>;
            buf.e[u] = load_oct<DT>(re, o);
            buf.s[u] = load_oct<DT>(rs, o);
            buf.r[u] = load_oct<DT>(rr, o);
        }
    }

    __device__ __forceinline__ void process(const Buf &buf, int64_t b) const
    {
        const rsrc_t ro = make_rsrc(out + b * kBlockBytes, valid(b));
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float fe[8], fs[8], fr[8], t[8];
            widen<DT>(buf.e[u], fe);
            widen<DT>(buf.s[u], fs);
            widen<DT>(buf.r[u], fr);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t[i] = fe[i] + fs[i];
            round_to<DT>(t);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                t[i] = fr[i] + t[i];
            store_oct<DT>(ro, narrow<DT>(t), voff + u * kWave * kOctBytes<DT>);
        }
    }
};

template <int DT>
__device__ __forceinline__ float load_scalar(const char *p, int64_t i)
{
    if constexpr (DT == DT_BF16)
        return __uint_as_float((uint32_t)reinterpret_cast<const uint16_t *>(p)[i] << 16);
    else if constexpr (DT == DT_F16)
        return (float)reinterpret_cast<const _Float16 *>(p)[i];
    else
        return reinterpret_cast<const float *>(p)[i];
}

template <int DT>
__device__ __forceinline__ void store_scalar(char *p, int64_t i, float v)
{
    if constexpr (DT == DT_BF16)
        reinterpret_cast<uint16_t *>(p)[i] = (uint16_t)(pack_bf16x2(v, 0.0f) & 0xffffu);
    else if constexpr (DT == DT_F16)
        reinterpret_cast<_Float16 *>(p)[i] = (_Float16)v;
    else
        reinterpret_cast<float *>(p)[i] = v;
}

template <int DT>
__device__ __forceinline__ float round_scalar(float v)
{
    if constexpr (DT == DT_BF16)
        return __uint_as_float(pack_bf16x2(v, 0.0f) << 16);
    else if constexpr (DT == DT_F16)
        return (float)(_Float16)v;
    else
        return v;
}

template <int DT, int U>
__global__ __launch_bounds__(kBlock) void residual_add_kernel(const char *e, const char *s,
                                                              const char *r, char *out,
                                                              int64_t num_elements)
{
    const int64_t full_octs = num_elements / 8;
    ResidualAddOp<DT, U> op{e, s, r, out, full_octs * kOctBytes<DT>,
                            (uint32_t)lane_id() * kOctBytes<DT>};
    const int64_t n_blocks = (full_octs + U * kWave - 1) / (U * kWave);
    walk_blocks(op, n_blocks);
    // the last num_elements % 8 elements: one lane each of the first wave
    const int64_t tail = num_elements - full_octs * 8;
    if (wave_id() == 0 && lane_id() < tail) {
        const int64_t i = full_octs * 8 + lane_id();
        const float t = round_scalar<DT>(load_scalar<DT>(e, i) + load_scalar<DT>(s, i));
        store_scalar<DT>(out, i, load_scalar<DT>(r, i) + t);
    }
}

// ---------------------------------------------------------------------------
// Router-weight multiply
// ---------------------------------------------------------------------------
// A wave covers octs [oct0, oct0 + octs) of each row it visits: the whole row, or its
// quarter of the row when the four waves of a workgroup split rows into equal spans.
template <int XDT, int ODT, int U>
struct RouterFwdOp {
    static constexpr bool kRowSum = false;
    struct Buf {
        Oct x[U];
    };
    const char *x;
    char *out;
    int hidden;
    uint32_t oct0, octs;
    uint32_t lane;

    __device__ __forceinline__ void load(Buf &b, int64_t r, int c, bool live) const
    {
        const uint32_t row = (uint32_t)hidden * kElemBytes<XDT>;
        const rsrc_t rx = chunk_rsrc(x + r * row + oct0 * kOctBytes<XDT>, live ? octs * kOctBytes<XDT> : 0u,
                                     (uint32_t)c * U * kWave * kOctBytes<XDT>);
#pragma unroll
        for (int u = 0; u < U; ++u)
            b.x[u] = load_oct<XDT>(rx, (lane + u * kWave) * kOctBytes<XDT>);
    }

    __device__ __forceinline__ void process(const Buf &b, int64_t r, int c, int slot, float p) const
    {
        const uint32_t row = (uint32_t)hidden * kElemBytes<ODT>;
        const rsrc_t ro = chunk_rsrc(out + r * row + oct0 * kOctBytes<ODT>, slot >= 0 ? octs * kOctBytes<ODT> : 0u,
                                     (uint32_t)c * U * kWave * kOctBytes<ODT>);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float f[8];
            widen<XDT>(b.x[u], f);
#pragma unroll
            for (int i = 0; i < 8; ++i)
                f[i] = f[i] * p;
            store_oct<ODT>(ro, narrow<ODT>(f), (lane + u * kWave) * kOctBytes<ODT>);
        }
    }
};

// The wave's span of each row: the whole row, or with `spans` the wave's quarter.
struct RowSpan {
    uint32_t oct0, octs;
    int nch;  // chunks of U * 64 octs in the span
};

template <int U>
__device__ __forceinline__ RowSpan row_span(int hidden, int spans)
{
    const uint32_t row_octs = (uint32_t)hidden / 8;
    RowSpan sp;
    sp.octs = spans ? row_octs / kWavesPerBlock : row_octs;
    sp.oct0 = spans ? (uint32_t)wave_in_block() * sp.octs : 0u;
    sp.nch = (int)((sp.octs + U * kWave - 1) / (U * kWave));
    return sp;
}

template <int XDT, int ODT, int U>
__global__ __launch_bounds__(kBlock) void router_weight_fwd_kernel(const char *x, const float *probs,
                                                                   char *out, int tokens, int hidden, int spans)
{
    const RowSchedule sched = make_schedule(tokens, nullptr, 0);
    const RowSpan sp = row_span<U>(hidden, spans);
    RouterFwdOp<XDT, ODT, U> op{x, out, hidden, sp.oct0, sp.octs, (uint32_t)lane_id()};
    walk_row_split(op, sched, nullptr, probs, sp.nch, spans != 0);
}

template <int XDT, int ODT, int U>
struct RouterBwdOp {
    static constexpr bool kRowSum = true;
    struct Buf {
        Oct g[U], x[U];
    };
    const char *g;
    const char *x;
    char *gx;
    float *gp;
    int hidden;
    uint32_t oct0, octs;
    uint32_t lane;
    float acc;  // this lane's partial of the current row's probability gradient

    __device__ __forceinline__ void load(Buf &b, int64_t r, int c, bool live) const
    {
        const uint32_t grow = (uint32_t)hidden * kElemBytes<ODT>, xrow = (uint32_t)hidden * kElemBytes<XDT>;
        const rsrc_t rg = chunk_rsrc(g + r * grow + oct0 * kOctBytes<ODT>, live ? octs * kOctBytes<ODT> : 0u,
                                     (uint32_t)c * U * kWave * kOctBytes<ODT>);
        // x is read only for the probability gradient
        const rsrc_t rx = chunk_rsrc(x + r * xrow + oct0 * kOctBytes<XDT>, live && gp ? octs * kOctBytes<XDT> : 0u,
                                     (uint32_t)c * U * kWave * kOctBytes<XDT>);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b.g[u] = load_oct<ODT>(rg, (lane + u * kWave) * kOctBytes<ODT>);
            b.x[u] = load_oct<XDT>(rx, (lane + u * kWave) * kOctBytes<XDT>);
        }
    }

    __device__ __forceinline__ void process(const Buf &b, int64_t r, int c, int slot, float p)
    {
        const uint32_t xrow = (uint32_t)hidden * kElemBytes<XDT>;
        const rsrc_t rgx = chunk_rsrc(gx + r * xrow + oct0 * kOctBytes<XDT>, slot >= 0 && gx ? octs * kOctBytes<XDT> : 0u,
                                      (uint32_t)c * U * kWave * kOctBytes<XDT>);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float fg[8], fx[8], d[8];
            widen<ODT>(b.g[u], fg);
            widen<XDT>(b.x[u], fx);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                d[i] = fg[i] * p;
                acc += fg[i] * fx[i];
            }
            store_oct<XDT>(rgx, narrow<XDT>(d), (lane + u * kWave) * kOctBytes<XDT>);
        }
    }

    __device__ __forceinline__ bool row_sum_wanted() const { return gp != nullptr; }
    __device__ __forceinline__ void store_row_sum(int slot, float total) const
    {
        if (lane == 0)
            gp[slot] = total;
    }
};

template <int XDT, int ODT, int U>
__global__ __launch_bounds__(kBlock) void router_weight_bwd_kernel(const char *g, const char *x,
                                                                   const float *probs, char *gx,
                                                                   float *gp, int tokens, int hidden, int spans)
{
    const RowSchedule sched = make_schedule(tokens, nullptr, 0);
    const RowSpan sp = row_span<U>(hidden, spans);
    RouterBwdOp<XDT, ODT, U> op{g, x, gx, gp, hidden, sp.oct0, sp.octs, (uint32_t)lane_id(), 0.0f};
    walk_row_split(op, sched, nullptr, probs, sp.nch, spans != 0);
}

// ---------------------------------------------------------------------------
// Squared ReLU x probs
// ---------------------------------------------------------------------------
// The soft clamp c = s * tanh(x / s) as x * R(u), u = (x / s)^2, with
// R(u) = P(u) / Q(u) a (2,2) rational fitted minimax in relative error to tanh(z) / z
// over 0 <= z <= 5.2 (coefficients from fit_tanh_rational.py beside this file).
// Beyond z = 5.2, u is held at 5.2^2, so x * R grows past s and the clamp to s below
// takes over; 1 - tanh(5.2) is 6.1e-5. Evaluated in fp32 this gives c to 6.5e-5
// relative for every x (so about 1.3e-4 on c^2), against 2^-8 for the one rounding
// the result goes through: it moves no result by more than one bf16 ulp. Two fmas
// fewer than a (3,3) fit to 1.5e-6, on the op whose pace the vector ALU sets; one
// reciprocal is its only quarter-rate operation.
constexpr float kTanhP0 = 0.9999353885650635f, kTanhP1 = 0.10179443657398224f,
                kTanhP2 = 0.0006515600252896547f;
constexpr float kTanhQ1 = 0.4347437024116516f, kTanhQ2 = 0.01262988243252039f;
constexpr float kTanhUMax = 27.040000915527344f;

// relu(s * tanh(x / s)) for s > 0. u stays finite (so no inf * 0 at x = +-inf: the
// clamps give s and 0), and the NaN-propagating min / max keep a NaN input NaN, as
// the ReLU does.
__device__ __forceinline__ float soft_clamp_relu(float x, float s, float inv_s)
{
    const float z = x * inv_s;
    const float u = __builtin_fminf(z * z, kTanhUMax);
    const float pn = __builtin_fmaf(__builtin_fmaf(kTanhP2, u, kTanhP1), u, kTanhP0);
    const float qd = __builtin_fmaf(__builtin_fmaf(kTanhQ2, u, kTanhQ1), u, 1.0f);
    const float c = x * (pn * __builtin_amdgcn_rcpf(qd));
    return __builtin_elementwise_maximum(__builtin_elementwise_minimum(c, s), 0.0f);
}

template <int U, bool kClamp>
struct SquaredReluOp {
    static constexpr bool kRowSum = false;
    struct Buf {
        u32x4 x[U];
    };
    const uint16_t *x;
    uint16_t *y;
    int hidden;
    float s, inv_s;
    int zero_padding;
    uint32_t voff;

    __device__ __forceinline__ void load(Buf &b, int64_t r, int c, bool live) const
    {
        const uint32_t row = (uint32_t)hidden * 2u;
        const rsrc_t rx = chunk_rsrc(x + r * hidden, live ? row : 0u, (uint32_t)c * U * kWave * kVecBytes);
#pragma unroll
        for (int u = 0; u < U; ++u)
            b.x[u] = load_vec(rx, voff + u * kWave * kVecBytes);
    }

    __device__ __forceinline__ float act(float v) const
    {
        if constexpr (kClamp) {
            const float a = soft_clamp_relu(v, s, inv_s);
            return a * a;
        } else {
            const float a = __builtin_elementwise_maximum(v, 0.0f);
            return a * a;
        }
    }

    __device__ __forceinline__ void process(const Buf &b, int64_t r, int c, int slot, float p) const
    {
        const uint32_t row = (uint32_t)hidden * 2u;
        const rsrc_t ry = chunk_rsrc(y + r * hidden, (slot >= 0 || zero_padding) ? row : 0u,
                                     (uint32_t)c * U * kWave * kVecBytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                float a0 = act(bf16_lo(b.x[u][q])), a1 = act(bf16_hi(b.x[u][q]));
                if constexpr (!kClamp) {
                    // the square is materialised in bf16 before the probability multiply
                    const unsigned sq = pack_bf16x2(a0, a1);
                    a0 = bf16_lo(sq);
                    a1 = bf16_hi(sq);
                }
                o[q] = pack_bf16x2(a0 * p, a1 * p);
            }
            store_vec(ry, o, voff + u * kWave * kVecBytes);
        }
    }
};

template <int U, bool kClamp>
__global__ __launch_bounds__(kBlock) void squared_relu_probs_kernel(
    const uint16_t *x, const float *probs, uint16_t *y, int rows, int hidden, float s, float inv_s,
    const int *n_used, const int *perm, int zero_padding)
{
    const RowSchedule sched = make_schedule(rows, n_used, zero_padding);
    const int nch = (hidden / 8 + U * kWave - 1) / (U * kWave);
    SquaredReluOp<U, kClamp> op{x, y, hidden, s, inv_s, zero_padding, (uint32_t)lane_id() * kVecBytes};
    walk_rows(op, sched, perm, probs, nch);
}

// Squared ReLU x probs, backward: grad_x = ((g p) (2a)) d where x > 0, else +0, with
// d = sech^2(x / s) under the soft clamp and 1 without it, and the row sum of
// g * y_pre (y_pre = a^2, or the bf16-rounded square without the clamp) as the
// probability gradient.
//
// Under the clamp, E = e^(-2z) and r = 1 / (1 + E) give both factors with two
// quarter-rate operations: tanh z = (1 - E) r (for z >= 1/8; below, the odd series
// z - z^3/3 + 2z^5/15, whose first omitted term is under 2.2e-7 of z there) and
// sech^2 z = 4 E r^2, which stays accurate where tanh rounds to 1. The ReLU is taken
// first (z = max(x / s, 0), NaN kept), so only z >= 0 is ever evaluated.
template <int U, bool kClamp>
struct SquaredReluBwdOp {
    static constexpr bool kRowSum = true;
    struct Buf {
        u32x4 x[U], g[U];
    };
    const uint16_t *x;
    const uint16_t *g;
    uint16_t *gx;
    float *gp;
    int hidden;
    float s, inv_s;
    int zero_padding;
    uint32_t voff;
    float acc;  // this lane's partial of the current row's probability gradient

    __device__ __forceinline__ void load(Buf &b, int64_t r, int c, bool live) const
    {
        const uint32_t row = (uint32_t)hidden * 2u, off = (uint32_t)c * U * kWave * kVecBytes;
        const rsrc_t rx = chunk_rsrc(x + r * hidden, live ? row : 0u, off);
        const rsrc_t rg = chunk_rsrc(g + r * hidden, live ? row : 0u, off);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            b.x[u] = load_vec(rx, voff + u * kWave * kVecBytes);
            b.g[u] = load_vec(rg, voff + u * kWave * kVecBytes);
        }
    }

    // two elements (one packed word of x and of g): the packed bf16 gradients; the
    // terms g * y_pre go into acc in element order
    __device__ __forceinline__ unsigned pair(unsigned xw, unsigned gw, float p)
    {
        const float v[2] = {bf16_lo(xw), bf16_hi(xw)}, gv[2] = {bf16_lo(gw), bf16_hi(gw)};
        float grad[2], ypre[2];
        if constexpr (kClamp) {
            constexpr float kNeg2Log2e = -2.8853900817779268f;
            constexpr float kThird = -1.0f / 3.0f, kTwoFifteenths = 2.0f / 15.0f;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const float z = __builtin_elementwise_maximum(v[i] * inv_s, 0.0f);
                // v_exp_f32 flushes subnormal results, so E * 2^64 is formed instead and
                // the 2^-64 goes into the fmas and the multiply that use it: sech^2
                // keeps its value down to the smallest subnormal, as the fp32 chain has it
                const float e64 = __builtin_amdgcn_exp2f(__builtin_fmaf(z, kNeg2Log2e, 64.0f));
                const float r = __builtin_amdgcn_rcpf(__builtin_fmaf(e64, 0x1p-64f, 1.0f));
                const float u = z * z;
                const float small = z * __builtin_fmaf(u, __builtin_fmaf(u, kTwoFifteenths, kThird), 1.0f);
                const float t = z < 0.125f ? small : __builtin_fmaf(-e64, 0x1p-64f, 1.0f) * r;
                const float a = s * t;
                const float sech2 = ((e64 * 0x1p-62f) * r) * r;  // 4 E r^2
                ypre[i] = a * a;
                grad[i] = ((gv[i] * p) * (2.0f * a)) * sech2;
            }
        } else {
            const float a[2] = {__builtin_elementwise_maximum(v[0], 0.0f),
                                __builtin_elementwise_maximum(v[1], 0.0f)};
            const unsigned sq = pack_bf16x2(a[0] * a[0], a[1] * a[1]);  // the square in bf16
            ypre[0] = bf16_lo(sq);
            ypre[1] = bf16_hi(sq);
#pragma unroll
            for (int i = 0; i < 2; ++i)
                grad[i] = (gv[i] * p) * (2.0f * a[i]);
        }
        acc += gv[0] * ypre[0];
        acc += gv[1] * ypre[1];
        return pack_bf16x2(v[0] > 0.0f ? grad[0] : 0.0f, v[1] > 0.0f ? grad[1] : 0.0f);
    }

    __device__ __forceinline__ void process(const Buf &b, int64_t r, int c, int slot, float p)
    {
        const uint32_t row = (uint32_t)hidden * 2u;
        const rsrc_t rgx = chunk_rsrc(gx + r * hidden, (slot >= 0 || zero_padding) ? row : 0u,
                                      (uint32_t)c * U * kWave * kVecBytes);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pair(b.x[u][q], b.g[u][q], p);
            store_vec(rgx, o, voff + u * kWave * kVecBytes);
        }
    }

    __device__ __forceinline__ bool row_sum_wanted() const { return gp != nullptr; }
    __device__ __forceinline__ void store_row_sum(int slot, float total) const
    {
        if (lane_id() == 0)
            gp[slot] = total;
    }
};

template <int U, bool kClamp>
__global__ __launch_bounds__(kBlock) void squared_relu_probs_bwd_kernel(
    const uint16_t *x, const float *probs, const uint16_t *g, uint16_t *gx, float *gp, int rows,
    int hidden, float s, float inv_s, const int *n_used, const int *perm, int zero_padding)
{
    const RowSchedule sched = make_schedule(rows, n_used, zero_padding);
    const int nch = (hidden / 8 + U * kWave - 1) / (U * kWave);
    SquaredReluBwdOp<U, kClamp> op{x, g, gx, gp, hidden, s, inv_s, zero_padding,
                                   (uint32_t)lane_id() * kVecBytes, 0.0f};
    walk_rows(op, sched, perm, probs, nch);
}

// The default launches for rows of at most two chunks: one wave per row, the row's
// chunks loaded at once (row_per_wave). Arguments ordered so the ones every wave needs
// arrive preloaded; `flags` says which optional row arguments exist.
template <int U, int NCH, bool kClamp>
__global__ __launch_bounds__(kBlock) void squared_relu_probs_row_kernel(
    int rows, int hidden, float s, float inv_s, int flags, const uint16_t *x, const float *probs, uint16_t *y,
    const int *n_used, const int *perm)
{
    SquaredReluOp<U, kClamp> op{x, y, hidden, s, inv_s, flags & kZeroPadding, (uint32_t)lane_id() * kVecBytes};
    row_per_wave<NCH>(op, rows, flags, n_used, perm, probs);
}

template <int U, int NCH, bool kClamp>
__global__ __launch_bounds__(kBlock) void squared_relu_probs_bwd_row_kernel(
    int rows, int hidden, float s, float inv_s, int flags, const uint16_t *x, const uint16_t *g, uint16_t *gx,
    const float *probs, float *gp, const int *n_used, const int *perm)
{
    SquaredReluBwdOp<U, kClamp> op{x, g, gx, gp, hidden, s, inv_s, flags & kZeroPadding,
                                   (uint32_t)lane_id() * kVecBytes, 0.0f};
    row_per_wave<NCH>(op, rows, flags, n_used, perm, probs);
}

// ---------------------------------------------------------------------------
// Token-local unpermute in fixed expert order
// ---------------------------------------------------------------------------
// One wave per output token (a fixed grid striding over tokens), lanes over the
// hidden dimension in chunks of U octs. The token's map entries sit one per lane and
// are broadcast with v_readlane. Contributions are loaded G experts at a time, all G
// issued before any is added; an expert with no contribution gets an empty buffer
// resource, which reads +0 without touching memory, and adding +0 to the running
// sum changes no bit (the sum starts at +0 and can never be -0). The adds then run
// in increasing expert id.
template <int ODT, int U, int G>
__global__ __launch_bounds__(kBlock) void unpermute_kernel(const uint16_t *eo, int64_t erows,
                                                           const int *map, const int *valid_tokens,
                                                           char *out, int tokens, int hidden, int E)
{
    const int lane = lane_id();
    const int64_t W = (int64_t)gridDim.x * kWavesPerBlock;
    int bound = tokens;
    if (valid_tokens) {
        const int v = *valid_tokens;
        bound = v < 0 ? 0 : (v > tokens ? tokens : v);
    }
    const uint32_t row = (uint32_t)hidden * 2u;
    const uint32_t orow = (uint32_t)hidden * kElemBytes<ODT>;
    const int nch = (hidden / 8 + U * kWave - 1) / (U * kWave);
    for (int64_t t = wave_id(); t < bound; t += W) {
        for (int c = 0; c < nch; ++c) {
            float acc[U][8];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[u][i] = 0.0f;
            for (int e0 = 0; e0 < E; e0 += kWave) {
                const int ne = E - e0 < kWave ? E - e0 : kWave;
                const int mv = lane < ne ? map[t * E + e0 + lane] : -1;
                for (int g0 = 0; g0 < ne; g0 += G) {
                    u32x4 buf[G][U];
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const int m = g0 + g < ne ? __builtin_amdgcn_readlane(mv, g0 + g) : -1;
                        const bool ok = m >= 0 && m < erows;
                        const rsrc_t rs = chunk_rsrc(eo + (int64_t)(ok ? m : 0) * hidden, ok ? row : 0u,
                                                     (uint32_t)c * U * kWave * kVecBytes);
#pragma unroll
                        for (int u = 0; u < U; ++u)
                            buf[g][u] = load_vec(rs, (lane + u * kWave) * kVecBytes);
                    }
#pragma unroll
                    for (int g = 0; g < G; ++g)
#pragma unroll
                        for (int u = 0; u < U; ++u)
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                acc[u][2 * q] = acc[u][2 * q] + bf16_lo(buf[g][u][q]);
                                acc[u][2 * q + 1] = acc[u][2 * q + 1] + bf16_hi(buf[g][u][q]);
                            }
                }
            }
            const rsrc_t ro = chunk_rsrc(out + t * orow, orow, (uint32_t)c * U * kWave * kOctBytes<ODT>);
#pragma unroll
            for (int u = 0; u < U; ++u)
                store_oct<ODT>(ro, narrow<ODT>(acc[u]), (lane + u * kWave) * kOctBytes<ODT>);
        }
    }
}

// The same reduction for up to G local experts, pipelined. A wave walks its units
// (token, chunk) in order. All G gathers of the next unit are issued before the
// current unit is added and stored, so one memory latency is exposed per wave, not
// one per chunk, also across token boundaries. One load fetches the map rows of the
// wave's next 64 / G tokens (lane l holds entry l % G of token l / G), so the
// pipeline waits on the map once per 64 / G tokens.
//
// With fp32 output, a lane's eight elements are two groups of four, elements
// 4l .. 4l+3 of two adjacent 256-element blocks (two 8-byte loads), so each of the
// two 16-byte fp32 stores writes 1 KiB contiguous across the wave. The plain layout
// (eight consecutive elements, one 16-byte load) would give each store instruction
// every other 16 bytes of a 2 KiB span: half-written lines, which measured about
// twice the write cost. The adds run in the same order either way.
template <int U, int G>
struct UnpermuteBuf {
    u32x4 v[G][U];
};

template <int ODT, int U, int G>
__global__ __launch_bounds__(kBlock) void unpermute_pipelined_kernel(const uint16_t *eo, int64_t erows,
                                                                     const int *map, const int *valid_tokens,
                                                                     char *out, int tokens, int hidden, int E)
{
    constexpr int kTokensPerMap = kWave / G;
    constexpr bool kSplit = ODT == DT_F32;
    const int lane = lane_id();
    const int64_t W = (int64_t)gridDim.x * kWavesPerBlock;
    int bound = tokens;
    if (valid_tokens) {
        const int v = *valid_tokens;
        bound = v < 0 ? 0 : (v > tokens ? tokens : v);
    }
    const uint32_t row = (uint32_t)hidden * 2u;
    const uint32_t orow = (uint32_t)hidden * kElemBytes<ODT>;
    const int nch = (hidden / 8 + U * kWave - 1) / (U * kWave);
    const uint32_t chunk = (uint32_t)U * kWave * kVecBytes;
    const int erows32 = (int)erows;  // below 2^31 (checked on the host): a scalar compare

    // map entries of tokens t0 + j W, j < kTokensPerMap; -1 past E or past the bound
    auto load_maps = [&](int64_t t0) -> int {
        const int64_t tok = t0 + (int64_t)(lane / G) * W;
        const int e = lane % G;
        const bool ok = e < E && tok < bound;
        const int v = map[ok ? tok * E + e : 0];
        return ok ? v : -1;
    };
    auto issue = [&](UnpermuteBuf<U, G> &b, int c, int mvs, int j) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int m = __builtin_amdgcn_readlane(mvs, j * G + g);
            const bool ok = m >= 0 && m < erows32;
            const rsrc_t rs = chunk_rsrc(eo + (int64_t)(ok ? m : 0) * hidden, ok ? row : 0u, (uint32_t)c * chunk);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (kSplit) {
                    const uint32_t o = (uint32_t)u * kWave * kVecBytes + (uint32_t)lane * 8u;
                    const auto lo = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, kLoadAux);
                    const auto hi = __builtin_amdgcn_raw_buffer_load_b64(rs, o + kWave * 8u, 0, kLoadAux);
                    b.v[g][u] = u32x4{lo[0], lo[1], hi[0], hi[1]};
                } else {
                    b.v[g][u] = load_vec(rs, (uint32_t)(lane + u * kWave) * kVecBytes);
                }
            }
        }
    };
    auto finish = [&](const UnpermuteBuf<U, G> &b, int64_t tok, int c) {
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i)
                acc[u][i] = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc[u][2 * q] = acc[u][2 * q] + bf16_lo(b.v[g][u][q]);
                    acc[u][2 * q + 1] = acc[u][2 * q + 1] + bf16_hi(b.v[g][u][q]);
                }
        const rsrc_t ro = chunk_rsrc(out + tok * orow, orow, (uint32_t)c * U * kWave * kOctBytes<ODT>);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (kSplit) {
                const uint32_t o = (uint32_t)u * kWave * 32u + (uint32_t)lane * 16u;
                store_vec(ro, u32x4{__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]),
                                    __float_as_uint(acc[u][2]), __float_as_uint(acc[u][3])}, o);
                store_vec(ro, u32x4{__float_as_uint(acc[u][4]), __float_as_uint(acc[u][5]),
                                    __float_as_uint(acc[u][6]), __float_as_uint(acc[u][7])}, o + kWave * 16u);
            } else {
                store_oct<ODT>(ro, narrow<ODT>(acc[u]), (lane + u * kWave) * kOctBytes<ODT>);
            }
        }
    };

    // current unit (t, c), token t being entry j of its map group
    int64_t t = wave_id();
    if (t >= bound)
        return;
    // map group of the next unit to issue. Only issue() reads it, and the current
    // unit's gathers are already out, so a new group replaces it in place: one
    // register, never copied (a copy through a register that a pending gather fills
    // makes the compiler drain that gather first).
    int mvs = load_maps(t);
    int j = 0, c = 0;
    // the unit after (c, j): the next chunk, else the next token of the map group,
    // else the first token of a new group (whose map the gathers need at once)
    struct Next {
        int c, j;
        bool group;
    };
    auto next = [nch](int c0, int j0) -> Next {
        if (c0 + 1 < nch)
            return {c0 + 1, j0, false};
        if (j0 + 1 < kTokensPerMap)
            return {0, j0 + 1, false};
        return {0, 0, true};
    };
    // The scheduling barriers keep each unit's gathers ahead of the previous unit's
    // adds: the two are independent, and the scheduler would otherwise sink the loads.
    UnpermuteBuf<U, G> A, B;
    issue(A, 0, mvs, 0);
    for (;;) {
        Next n = next(c, j);
        if (n.group)
            mvs = load_maps(t + W);
        issue(B, n.c, mvs, n.j);
        __builtin_amdgcn_sched_barrier(0);
        finish(A, t, c);
        t = n.c == 0 ? t + W : t;
        c = n.c, j = n.j;
        if (t >= bound)
            break;
        n = next(c, j);
        if (n.group)
            mvs = load_maps(t + W);
        issue(A, n.c, mvs, n.j);
        __builtin_amdgcn_sched_barrier(0);
        finish(B, t, c);
        t = n.c == 0 ? t + W : t;
        c = n.c, j = n.j;
        if (t >= bound)
            break;
    }
}

// The same reduction for up to 8 local experts with one wave per unit (token t, chunk
// c), unit = t * nch + c, a grid of one wave per unit. The token's map row comes by
// scalar loads; the contributing experts are compacted, in increasing expert id, into
// the first K gather slots, and exactly those K gathers are issued (the kernel takes
// a straight-line path per K, so every wait count is exact and no slot is empty); the
// adds then run over the K slots in order. Skipping an absent expert is adding +0,
// which changes no bit of the fp32 sum (it starts at +0 and is never -0), so the
// result is the pipelined kernel's. With fp32 output the lanes hold the split layout
// of the pipelined kernel.
template <int ODT, int U, int K>
__device__ __forceinline__ void unpermute_unit(const uint16_t *eo, const int (&rows)[8], char *out, int64_t t,
                                               int c, int hidden)
{
    constexpr bool kSplit = ODT == DT_F32;
    const int lane = lane_id();
    const uint32_t row = (uint32_t)hidden * 2u;
    const uint32_t chunk = (uint32_t)U * kWave * kVecBytes;
    u32x4 b[K > 0 ? K : 1][U];
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const rsrc_t rs = chunk_rsrc(eo + (int64_t)rows[k] * hidden, row, (uint32_t)c * chunk);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if constexpr (kSplit) {
                const uint32_t o = (uint32_t)u * kWave * kVecBytes + (uint32_t)lane * 8u;
                const auto lo = __builtin_amdgcn_raw_buffer_load_b64(rs, o, 0, kLoadAux);
                const auto hi = __builtin_amdgcn_raw_buffer_load_b64(rs, o + kWave * 8u, 0, kLoadAux);
                b[k][u] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
                b[k][u] = load_vec(rs, (uint32_t)(lane + u * kWave) * kVecBytes);
            }
        }
    }
    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            acc[u][i] = 0.0f;
#pragma unroll
    for (int k = 0; k < K; ++k)
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[u][2 * q] = acc[u][2 * q] + bf16_lo(b[k][u][q]);
                acc[u][2 * q + 1] = acc[u][2 * q + 1] + bf16_hi(b[k][u][q]);
            }
    const uint32_t orow = (uint32_t)hidden * kElemBytes<ODT>;
    const rsrc_t ro = chunk_rsrc(out + t * orow, orow, (uint32_t)c * U * kWave * kOctBytes<ODT>);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if constexpr (kSplit) {
            const uint32_t o = (uint32_t)u * kWave * 32u + (uint32_t)lane * 16u;
            store_vec(ro, u32x4{__float_as_uint(acc[u][0]), __float_as_uint(acc[u][1]),
                                __float_as_uint(acc[u][2]), __float_as_uint(acc[u][3])}, o);
            store_vec(ro, u32x4{__float_as_uint(acc[u][4]), __float_as_uint(acc[u][5]),
                                __float_as_uint(acc[u][6]), __float_as_uint(acc[u][7])}, o + kWave * 16u);
        } else {
            store_oct<ODT>(ro, narrow<ODT>(acc[u]), (lane + u * kWave) * kOctBytes<ODT>);
        }
    }
}

template <int ODT, int U>
__global__ __launch_bounds__(kBlock) void unpermute_unit_kernel(int tokens, int hidden, int E, int nch, int erows,
                                                                const uint16_t *eo, const int *map, char *out,
                                                                const int *valid_tokens)
{
    const int unit = wave_id();
    const int t = unit / nch;
    const int c = unit - t * nch;
    if (t >= tokens)
        return;
    if (valid_tokens) {
        const int v = *valid_tokens;
        if (t >= v)  // also every token when v <= 0
            return;
    }
    int rows[8];
    int K = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        rows[e] = 0;
        if (e < E) {
            const int m = map[(int64_t)t * E + e];
            if (m >= 0 && m < erows)
                rows[K++] = m;
        }
    }
    switch (K) {
    case 0: unpermute_unit<ODT, U, 0>(eo, rows, out, t, c, hidden); break;
    case 1: unpermute_unit<ODT, U, 1>(eo, rows, out, t, c, hidden); break;
    case 2: unpermute_unit<ODT, U, 2>(eo, rows, out, t, c, hidden); break;
    case 3: unpermute_unit<ODT, U, 3>(eo, rows, out, t, c, hidden); break;
    case 4: unpermute_unit<ODT, U, 4>(eo, rows, out, t, c, hidden); break;
    case 5: unpermute_unit<ODT, U, 5>(eo, rows, out, t, c, hidden); break;
    case 6: unpermute_unit<ODT, U, 6>(eo, rows, out, t, c, hidden); break;
    case 7: unpermute_unit<ODT, U, 7>(eo, rows, out, t, c, hidden); break;
    default: unpermute_unit<ODT, U, 8>(eo, rows, out, t, c, hidden); break;
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
thread_local int t_last_hip_error = 0;

constexpr int kMaxDevices = 64;
struct DeviceInfo {
    std::once_flag once;
    hipError_t err = hipSuccess;
    int cus = 0;
};
DeviceInfo g_devices[kMaxDevices];

hipError_t device_cus(int *cus)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    DeviceInfo &d = g_devices[dev];
    std::call_once(d.once, [&d, dev] {
        hipDeviceProp_t prop;
        d.err = hipGetDeviceProperties(&prop, dev);
        if (d.err == hipSuccess)
            d.cus = prop.multiProcessorCount;
    });
    *cus = d.cus;
    return d.err;
}

moe_status_t fail_hip(hipError_t e)
{
    t_last_hip_error = (int)e;
    return MOE_ERR_HIP;
}

struct Range {
    uintptr_t lo, hi;
};
Range span(const void *p, uint64_t bytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return Range{a, p ? a + (uintptr_t)bytes : a};
}
bool overlap(Range a, Range b) { return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi; }
bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
int elem_bytes(moe_dtype_t d) { return d == MOE_FP32 ? 4 : 2; }
bool dtype_ok(moe_dtype_t d) { return d == MOE_BF16 || d == MOE_FP16 || d == MOE_FP32; }

constexpr int64_t kMaxRows = 0x7fffffffLL - 64LL * 65536LL;
constexpr int64_t kMaxHidden = 1LL << 26;  // a row stays under 2^32 bytes in fp32
// Elements of one residual-add tensor: far past any device's memory, and small enough
// that its byte count and every byte offset fit in 64-bit arithmetic.
constexpr int64_t kMaxElements = 1LL << 48;

// Octs per lane per chunk: the U in 1..4 that leaves the fewest idle lane slots in a
// row's last chunk, ties to the larger U (7168 columns: U = 2, seven full chunks, not
// four chunks of which the last is half empty). A lane's octs are lane + 64 k in
// increasing k for every U, so row sums do not depend on the choice.
int pick_u(int64_t octs)
{
    const int64_t u = (octs + kWave - 1) / kWave;
    int best = 1;
    int64_t best_waste = INT64_MAX;
    for (int c = 4; c >= 1; --c) {
        const int64_t waste = (u + c - 1) / c * c - u;
        if (waste < best_waste)
            best = c, best_waste = waste;
    }
    return best;
}

// Column chunks of a row of `octs` octs at U octs per lane.
int64_t row_chunks(int64_t octs, int U) { return (octs + (int64_t)U * kWave - 1) / ((int64_t)U * kWave); }

// How the router-weight kernels cover their rows.
//   * Rows of 4 or more chunks are shared by a workgroup's four waves, which take
//     consecutive runs of whole chunks (7168 columns: 7 chunks of 128 octs, taken 1, 2,
//     2, 2).
//   * The backward meets its four waves at a barrier at the end of every row (for the row
//     sum), so there the wave with one chunk waits for the others. When the chunks do not
//     divide evenly over four, each of its waves instead takes an equal quarter of the
//     row (224 octs: one chunk of U = 4 whose last 32 lane slots the range check masks),
//     provided its slowest wave covers no more lane slots than the chunk split's. The row
//     sum still combines the four quarters in order. At 53760 x 7168 (bf16) that took
//     the backward from 377 to 372 us; quarters of two U = 2 chunks, or U = 1, were no
//     faster than the split. The forward, with no barrier, stays on the split (quarters
//     measured 0.3-1% slower).
//   * Shorter rows go one per wave (walk_row_split falls back to walk_rows).

struct RouterPlan {
    int U;
    int spans;
    int blocks;
};

RouterPlan plan_router(int64_t tokens, int64_t hidden, int cus, int num_workgroups, bool backward)
{
    const int64_t octs = hidden / 8;
    RouterPlan pl{pick_u(octs), 0, 0};
    const int64_t nch = row_chunks(octs, pl.U);
    if (backward && octs % kWavesPerBlock == 0 && nch >= kWavesPerBlock) {
        const int64_t q = octs / kWavesPerBlock;
        const int Uq = pick_u(q);
        const int64_t span_slots = row_chunks(q, Uq) * Uq;                      // per lane
        const int64_t split_slots = (nch + kWavesPerBlock - 1) / kWavesPerBlock * pl.U;
        if (nch % kWavesPerBlock != 0 && span_slots <= split_slots) {
            pl.U = Uq;
            pl.spans = 1;
        }
    }
    pl.blocks = num_workgroups > 0 ? num_workgroups
                                   : split_walk_workgroups(tokens, pl.spans ? kWavesPerBlock : nch, cus, 1);
    return pl;
}

moe_status_t launched()
{
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOE_OK : fail_hip(e);
}

// residual add dispatch ------------------------------------------------------
// residual add: octs per lane per block (U) of the flat walk. U = 2 moves 2 KiB per wave
// per stream (bf16), the block the plain streaming probe moves fastest on MI355X; at
// 6720 x 7168 bf16 it measured 61.3 against 61.7 us for 4 KiB blocks, interleaved.
constexpr int kResidualU = 2;

template <int DT>
void launch_residual(int blocks, hipStream_t st, const void *e, const void *s, const void *r, void *o,
                     int64_t n)
{
    hipLaunchKernelGGL((residual_add_kernel<DT, kResidualU>), dim3(blocks), dim3(kBlock), 0, st,
                       static_cast<const char *>(e), static_cast<const char *>(s),
                       static_cast<const char *>(r), static_cast<char *>(o), n);
}

// router weight dispatch -----------------------------------------------------
template <int XDT, int ODT, int U>
void launch_router_fwd_u(int blocks, hipStream_t st, const void *x, const float *p, void *o, int t, int h,
                         int spans)
{
    hipLaunchKernelGGL((router_weight_fwd_kernel<XDT, ODT, U>), dim3(blocks), dim3(kBlock), 0, st,
                       static_cast<const char *>(x), p, static_cast<char *>(o), t, h, spans);
}

template <int XDT, int ODT>
void launch_router_fwd(const RouterPlan &pl, hipStream_t st, const void *x, const float *p, void *o, int t, int h)
{
    switch (pl.U) {
    case 1: launch_router_fwd_u<XDT, ODT, 1>(pl.blocks, st, x, p, o, t, h, pl.spans); break;
    case 2: launch_router_fwd_u<XDT, ODT, 2>(pl.blocks, st, x, p, o, t, h, pl.spans); break;
    case 3: launch_router_fwd_u<XDT, ODT, 3>(pl.blocks, st, x, p, o, t, h, pl.spans); break;
    default: launch_router_fwd_u<XDT, ODT, 4>(pl.blocks, st, x, p, o, t, h, pl.spans); break;
    }
}

template <int XDT, int ODT, int U>
void launch_router_bwd_u(int blocks, hipStream_t st, const void *g, const void *x, const float *p, void *gx,
                         float *gp, int t, int h, int spans)
{
    hipLaunchKernelGGL((router_weight_bwd_kernel<XDT, ODT, U>), dim3(blocks), dim3(kBlock), 0, st,
                       static_cast<const char *>(g), static_cast<const char *>(x), p,
                       static_cast<char *>(gx), gp, t, h, spans);
}

template <int XDT, int ODT>
void launch_router_bwd(const RouterPlan &pl, hipStream_t st, const void *g, const void *x, const float *p,
                       void *gx, float *gp, int t, int h)
{
    switch (pl.U) {
    case 1: launch_router_bwd_u<XDT, ODT, 1>(pl.blocks, st, g, x, p, gx, gp, t, h, pl.spans); break;
    case 2: launch_router_bwd_u<XDT, ODT, 2>(pl.blocks, st, g, x, p, gx, gp, t, h, pl.spans); break;
    case 3: launch_router_bwd_u<XDT, ODT, 3>(pl.blocks, st, g, x, p, gx, gp, t, h, pl.spans); break;
    default: launch_router_bwd_u<XDT, ODT, 4>(pl.blocks, st, g, x, p, gx, gp, t, h, pl.spans); break;
    }
}

// squared relu dispatch ------------------------------------------------------
template <int U, bool C>
void launch_sqrelu_u(int blocks, hipStream_t st, const uint16_t *x, const float *p, uint16_t *y, int rows,
                     int hidden, float s, float inv_s, const int *nu, const int *pm, int zp)
{
    hipLaunchKernelGGL((squared_relu_probs_kernel<U, C>), dim3(blocks), dim3(kBlock), 0, st, x, p, y, rows,
                       hidden, s, inv_s, nu, pm, zp);
}

template <bool C>
void launch_sqrelu(int U, int blocks, hipStream_t st, const uint16_t *x, const float *p, uint16_t *y,
                   int rows, int hidden, float s, float inv_s, const int *nu, const int *pm, int zp)
{
    switch (U) {
    case 1: launch_sqrelu_u<1, C>(blocks, st, x, p, y, rows, hidden, s, inv_s, nu, pm, zp); break;
    case 2: launch_sqrelu_u<2, C>(blocks, st, x, p, y, rows, hidden, s, inv_s, nu, pm, zp); break;
    case 3: launch_sqrelu_u<3, C>(blocks, st, x, p, y, rows, hidden, s, inv_s, nu, pm, zp); break;
    default: launch_sqrelu_u<4, C>(blocks, st, x, p, y, rows, hidden, s, inv_s, nu, pm, zp); break;
    }
}

template <int U, bool C>
void launch_sqrelu_bwd_u(int blocks, hipStream_t st, const uint16_t *x, const float *p, const uint16_t *g,
                         uint16_t *gx, float *gp, int rows, int hidden, float s, float inv_s, const int *nu,
                         const int *pm, int zp)
{
    hipLaunchKernelGGL((squared_relu_probs_bwd_kernel<U, C>), dim3(blocks), dim3(kBlock), 0, st, x, p, g,
                       gx, gp, rows, hidden, s, inv_s, nu, pm, zp);
}

template <bool C>
void launch_sqrelu_bwd(int U, int blocks, hipStream_t st, const uint16_t *x, const float *p,
                       const uint16_t *g, uint16_t *gx, float *gp, int rows, int hidden, float s,
                       float inv_s, const int *nu, const int *pm, int zp)
{
    switch (U) {
    case 1: launch_sqrelu_bwd_u<1, C>(blocks, st, x, p, g, gx, gp, rows, hidden, s, inv_s, nu, pm, zp); break;
    case 2: launch_sqrelu_bwd_u<2, C>(blocks, st, x, p, g, gx, gp, rows, hidden, s, inv_s, nu, pm, zp); break;
    case 3: launch_sqrelu_bwd_u<3, C>(blocks, st, x, p, g, gx, gp, rows, hidden, s, inv_s, nu, pm, zp); break;
    default: launch_sqrelu_bwd_u<4, C>(blocks, st, x, p, g, gx, gp, rows, hidden, s, inv_s, nu, pm, zp); break;
    }
}

// unpermute: G experts per batch of loads, U octs per lane per chunk
constexpr int kUnpermuteU = 4;
constexpr int kUnpermuteG = 4;
// The unpermute waits on each group of gathers before adding it, so it keeps more
// waves resident than the pure streams do.
constexpr int kUnpermuteBlocksPerCU = 2;
// Up to this many local experts take the pipelined unpermute, one workgroup per CU
// (measured best: 110 us against 113 us at two, for 6720 tokens x 8 experts).
constexpr int kUnpermutePipelinedMaxExperts = 8;
constexpr int kUnpermutePipeU = 2;
constexpr int kUnpermutePipeBlocksPerCU = 1;
// Octs per lane per chunk of the one-unit-per-wave unpermute, by output type. At 6,720
// tokens x 8 experts x 7,168 (medians of five windows, interleaved builds): fp32 out
// 91.4 us at 1, 94.5 at 2, 97.8 at 4; bf16 out 80.4, 79.5, 81.8. The bits do not
// depend on it.
template <int ODT>
constexpr int kUnpermuteUnitU = ODT == DT_F32 ? 1 : 2;
// The soft-clamped squared ReLU (forward ~16, backward ~31 vector instructions per
// element) keeps the VALU 61% / 84% busy. It runs with 2 octs per lane per chunk
// (83 registers, up to 6 waves per SIMD) and one wave per row whatever the row length.
// Measured at 53760 x 2048: forward 72.6 us and backward 103.8 us, level with the
// unclamped kernels, against 81.9 / 118.9 us with a balanced grid of 1920
// resident-sized workgroups, whose last dispatch round ran half empty. Without the
// clamp the kernel is a plain stream and follows the default grid rule.
constexpr int kSquaredReluClampMaxU = 2;

// An explicit workgroup count: 0 (the default grid) up to the dispatch limit.
bool bad_grid(int num_workgroups) { return num_workgroups < 0 || num_workgroups > kMaxWorkgroups; }

// Under the clamp: at most 2 octs per lane per chunk (fewer registers, more waves).
int squared_relu_u(int64_t octs, int clamp)
{
    const int u = pick_u(octs);
    return clamp && u > kSquaredReluClampMaxU ? kSquaredReluClampMaxU : u;
}

// Under the clamp one wave per row whatever the row length (the arithmetic needs the
// waves); without it the grid rule of plain streams.
int squared_relu_workgroups(int64_t rows, int64_t hidden, int cus, int clamp)
{
    if (clamp)
        return walk_workgroups(rows, 1, cus, 1);
    return walk_workgroups(rows, row_chunks(hidden / 8, squared_relu_u(hidden / 8, 0)), cus, 1);
}

int row_flags(int zp, const int32_t *n_used, const int32_t *perm)
{
    return (zp ? kZeroPadding : 0) | (n_used ? kHasNUsed : 0) | (perm ? kHasPerm : 0);
}

// The default launch of the squared ReLU when a row is one or two chunks and one wave
// per row fits in a dispatch: the row kernels. Returns false (nothing launched) when
// the shape takes the walk.
template <bool C, int U, int NCH>
void launch_sqrelu_row_un(bool bwd, hipStream_t st, int rows, int hidden, float s, float inv_s, int flags,
                          const uint16_t *x, const uint16_t *g, uint16_t *out, const float *p, float *gp,
                          const int *nu, const int *pm)
{
    const int blocks = (rows + kWavesPerBlock - 1) / kWavesPerBlock;
    if (bwd)
        hipLaunchKernelGGL((squared_relu_probs_bwd_row_kernel<U, NCH, C>), dim3(blocks), dim3(kBlock), 0, st, rows,
                           hidden, s, inv_s, flags, x, g, out, p, gp, nu, pm);
    else
        hipLaunchKernelGGL((squared_relu_probs_row_kernel<U, NCH, C>), dim3(blocks), dim3(kBlock), 0, st, rows,
                           hidden, s, inv_s, flags, x, p, out, nu, pm);
}

template <bool C>
bool launch_sqrelu_row(bool bwd, int U, hipStream_t st, int64_t rows, int64_t hidden, float s, float inv_s,
                       int flags, const uint16_t *x, const uint16_t *g, uint16_t *out, const float *p, float *gp,
                       const int *nu, const int *pm)
{
    const int64_t nch = row_chunks(hidden / 8, U);
    if (nch > 2 || (rows + kWavesPerBlock - 1) / kWavesPerBlock > kMaxWorkgroups)
        return false;
    const int r = (int)rows, h = (int)hidden;
    const int key = U * 10 + (int)nch;
    switch (key) {
    case 11: launch_sqrelu_row_un<C, 1, 1>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 12: launch_sqrelu_row_un<C, 1, 2>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 21: launch_sqrelu_row_un<C, 2, 1>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 22: launch_sqrelu_row_un<C, 2, 2>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 31: launch_sqrelu_row_un<C, 3, 1>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 32: launch_sqrelu_row_un<C, 3, 2>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 41: launch_sqrelu_row_un<C, 4, 1>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    case 42: launch_sqrelu_row_un<C, 4, 2>(bwd, st, r, h, s, inv_s, flags, x, g, out, p, gp, nu, pm); return true;
    default: return false;
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------
extern "C" {

moe_status_t moe_residual_add(const void *expert_output, const void *shared_expert_output,
                              const void *residual, void *output, int64_t num_elements,
                              moe_dtype_t dtype, hipStream_t stream, int num_workgroups)
{
    if (num_elements < 0 || num_elements > kMaxElements || !dtype_ok(dtype) || bad_grid(num_workgroups))
        return MOE_ERR_INVALID_ARG;
    if (num_elements == 0)
        return MOE_OK;
    if (!expert_output || !shared_expert_output || !residual || !output)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(expert_output, 16) || !aligned(shared_expert_output, 16) || !aligned(residual, 16) ||
        !aligned(output, 16))
        return MOE_ERR_ALIGNMENT;
    const uint64_t bytes = (uint64_t)num_elements * elem_bytes(dtype);
    const Range o = span(output, bytes);
    for (const void *in : {expert_output, shared_expert_output, residual})
        if (in != output && overlap(o, span(in, bytes)))
            return MOE_ERR_INVALID_ARG;
    int cus = 0;
    hipError_t he = device_cus(&cus);
    if (he != hipSuccess)
        return fail_hip(he);
    const int64_t octs = num_elements / 8;
    const int64_t n_blocks = (octs + kResidualU * kWave - 1) / (kResidualU * kWave);
    const int blocks = num_workgroups > 0 ? num_workgroups : walk_workgroups(n_blocks, 1, cus, 1);
    switch (dtype) {
    case MOE_BF16: launch_residual<DT_BF16>(blocks, stream, expert_output, shared_expert_output, residual, output, num_elements); break;
    case MOE_FP16: launch_residual<DT_F16>(blocks, stream, expert_output, shared_expert_output, residual, output, num_elements); break;
    default: launch_residual<DT_F32>(blocks, stream, expert_output, shared_expert_output, residual, output, num_elements); break;
    }
    return launched();
}

moe_status_t moe_router_weight_fwd(const void *x, moe_dtype_t x_dtype, const float *probs,
                                   void *out, moe_dtype_t out_dtype, int64_t tokens,
                                   int64_t hidden, hipStream_t stream, int num_workgroups)
{
    if (tokens < 0 || hidden <= 0 || tokens > kMaxRows || hidden > kMaxHidden || bad_grid(num_workgroups) ||
        !dtype_ok(x_dtype) || !(out_dtype == x_dtype || out_dtype == MOE_FP32))
        return MOE_ERR_INVALID_ARG;
    if (hidden % 8 != 0)
        return MOE_ERR_ALIGNMENT;
    if (tokens == 0)
        return MOE_OK;
    if (!x || !probs || !out)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(out, 16) || !aligned(probs, 4))
        return MOE_ERR_ALIGNMENT;
    const uint64_t T = (uint64_t)tokens, H = (uint64_t)hidden;
    const Range o = span(out, T * H * elem_bytes(out_dtype));
    if (overlap(o, span(x, T * H * elem_bytes(x_dtype))) || overlap(o, span(probs, T * 4)))
        return MOE_ERR_INVALID_ARG;
    int cus = 0;
    hipError_t he = device_cus(&cus);
    if (he != hipSuccess)
        return fail_hip(he);
    const RouterPlan pl = plan_router(tokens, hidden, cus, num_workgroups, false);
    const int t = (int)tokens, h = (int)hidden;
    if (x_dtype == MOE_BF16 && out_dtype == MOE_BF16) launch_router_fwd<DT_BF16, DT_BF16>(pl, stream, x, probs, out, t, h);
    else if (x_dtype == MOE_BF16) launch_router_fwd<DT_BF16, DT_F32>(pl, stream, x, probs, out, t, h);
    else if (x_dtype == MOE_FP16 && out_dtype == MOE_FP16) launch_router_fwd<DT_F16, DT_F16>(pl, stream, x, probs, out, t, h);
    else if (x_dtype == MOE_FP16) launch_router_fwd<DT_F16, DT_F32>(pl, stream, x, probs, out, t, h);
    else launch_router_fwd<DT_F32, DT_F32>(pl, stream, x, probs, out, t, h);
    return launched();
}

moe_status_t moe_router_weight_bwd(const void *grad_out, moe_dtype_t out_dtype, const void *x,
                                   moe_dtype_t x_dtype, const float *probs, void *grad_x,
                                   float *grad_probs, int64_t tokens, int64_t hidden,
                                   hipStream_t stream, int num_workgroups)
{
    if (tokens < 0 || hidden <= 0 || tokens > kMaxRows || hidden > kMaxHidden || bad_grid(num_workgroups) ||
        !dtype_ok(x_dtype) || !(out_dtype == x_dtype || out_dtype == MOE_FP32))
        return MOE_ERR_INVALID_ARG;
    if (hidden % 8 != 0)
        return MOE_ERR_ALIGNMENT;
    if (tokens == 0)
        return MOE_OK;
    if (!grad_out || !probs || (grad_probs && !x))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(grad_out, 16) || !aligned(x, 16) || !aligned(grad_x, 16) || !aligned(probs, 4) ||
        !aligned(grad_probs, 4))
        return MOE_ERR_ALIGNMENT;
    const uint64_t T = (uint64_t)tokens, H = (uint64_t)hidden;
    const Range ins[] = {span(grad_out, T * H * elem_bytes(out_dtype)), span(x, T * H * elem_bytes(x_dtype)),
                         span(probs, T * 4)};
    const Range outs[] = {span(grad_x, T * H * elem_bytes(x_dtype)), span(grad_probs, T * 4)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i))
                return MOE_ERR_INVALID_ARG;
    if (overlap(outs[0], outs[1]))
        return MOE_ERR_INVALID_ARG;
    if (!grad_x && !grad_probs)
        return MOE_OK;
    int cus = 0;
    hipError_t he = device_cus(&cus);
    if (he != hipSuccess)
        return fail_hip(he);
    const RouterPlan pl = plan_router(tokens, hidden, cus, num_workgroups, true);
    const int t = (int)tokens, h = (int)hidden;
    if (x_dtype == MOE_BF16 && out_dtype == MOE_BF16) launch_router_bwd<DT_BF16, DT_BF16>(pl, stream, grad_out, x, probs, grad_x, grad_probs, t, h);
    else if (x_dtype == MOE_BF16) launch_router_bwd<DT_BF16, DT_F32>(pl, stream, grad_out, x, probs, grad_x, grad_probs, t, h);
    else if (x_dtype == MOE_FP16 && out_dtype == MOE_FP16) launch_router_bwd<DT_F16, DT_F16>(pl, stream, grad_out, x, probs, grad_x, grad_probs, t, h);
    else if (x_dtype == MOE_FP16) launch_router_bwd<DT_F16, DT_F32>(pl, stream, grad_out, x, probs, grad_x, grad_probs, t, h);
    else launch_router_bwd<DT_F32, DT_F32>(pl, stream, grad_out, x, probs, grad_x, grad_probs, t, h);
    return launched();
}

moe_status_t moe_squared_relu_probs_fwd(const uint16_t *x, const float *probs, uint16_t *y,
                                        int64_t rows, int64_t hidden, int clamp,
                                        float clamp_scale, const int32_t *n_used,
                                        const int32_t *permutation_map, int zero_padding,
                                        hipStream_t stream, int num_workgroups)
{
    if (rows < 0 || hidden <= 0 || rows > kMaxRows || hidden > kMaxHidden || bad_grid(num_workgroups))
        return MOE_ERR_INVALID_ARG;
    if (clamp && !(clamp_scale > 0.0f && std::isfinite(clamp_scale)))
        return MOE_ERR_INVALID_ARG;
    if (hidden % 8 != 0)
        return MOE_ERR_ALIGNMENT;
    if (rows == 0)
        return MOE_OK;
    if (!x || !probs || !y)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(probs, 4) || !aligned(n_used, 4) ||
        !aligned(permutation_map, 4))
        return MOE_ERR_ALIGNMENT;
    const uint64_t R = (uint64_t)rows, H = (uint64_t)hidden;
    const Range o = span(y, R * H * 2);
    const Range ins[] = {span(x, R * H * 2), span(probs, R * 4), span(n_used, 4), span(permutation_map, R * 4)};
    for (const Range &i : ins)
        if (overlap(o, i))
            return MOE_ERR_INVALID_ARG;
    int cus = 0;
    hipError_t he = device_cus(&cus);
    if (he != hipSuccess)
        return fail_hip(he);
    const int U = squared_relu_u(hidden / 8, clamp);
    const float s = clamp ? clamp_scale : 1.0f;
    const int flags = row_flags(zero_padding ? 1 : 0, n_used, permutation_map);
    if (num_workgroups == 0 &&
        (clamp ? launch_sqrelu_row<true>(false, U, stream, rows, hidden, s, 1.0f / s, flags, x, nullptr, y, probs,
                                         nullptr, n_used, permutation_map)
               : launch_sqrelu_row<false>(false, U, stream, rows, hidden, s, 1.0f, flags, x, nullptr, y, probs,
                                          nullptr, n_used, permutation_map)))
        return launched();
    const int blocks = num_workgroups > 0 ? num_workgroups : squared_relu_workgroups(rows, hidden, cus, clamp);
    if (clamp)
        launch_sqrelu<true>(U, blocks, stream, x, probs, y, (int)rows, (int)hidden, s, 1.0f / s, n_used,
                            permutation_map, zero_padding ? 1 : 0);
    else
        launch_sqrelu<false>(U, blocks, stream, x, probs, y, (int)rows, (int)hidden, s, 1.0f, n_used,
                             permutation_map, zero_padding ? 1 : 0);
    return launched();
}

moe_status_t moe_squared_relu_probs_bwd(const uint16_t *x, const float *probs, const uint16_t *grad_y,
                                        uint16_t *grad_x, float *grad_probs, int64_t rows,
                                        int64_t hidden, int clamp, float clamp_scale,
                                        const int32_t *n_used, const int32_t *permutation_map,
                                        int zero_padding, hipStream_t stream, int num_workgroups)
{
    if (rows < 0 || hidden <= 0 || rows > kMaxRows || hidden > kMaxHidden || bad_grid(num_workgroups))
        return MOE_ERR_INVALID_ARG;
    if (clamp && !(clamp_scale > 0.0f && std::isfinite(clamp_scale)))
        return MOE_ERR_INVALID_ARG;
    if (hidden % 8 != 0)
        return MOE_ERR_ALIGNMENT;
    if (rows == 0)
        return MOE_OK;
    if (!x || !probs || !grad_y || !grad_x)
        return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(grad_y, 16) || !aligned(grad_x, 16) || !aligned(probs, 4) ||
        !aligned(grad_probs, 4) || !aligned(n_used, 4) || !aligned(permutation_map, 4))
        return MOE_ERR_ALIGNMENT;
    const uint64_t R = (uint64_t)rows, H = (uint64_t)hidden;
    const Range outs[] = {span(grad_x, R * H * 2), span(grad_probs, R * 4)};
    const Range ins[] = {span(x, R * H * 2), span(grad_y, R * H * 2), span(probs, R * 4), span(n_used, 4),
                         span(permutation_map, R * 4)};
    for (const Range &o : outs)
        for (const Range &i : ins)
            if (overlap(o, i))
                return MOE_ERR_INVALID_ARG;
    if (overlap(outs[0], outs[1]))
        return MOE_ERR_INVALID_ARG;
    int cus = 0;
    hipError_t he = device_cus(&cus);
    if (he != hipSuccess)
        return fail_hip(he);
    const int U = squared_relu_u(hidden / 8, clamp);
    const float s = clamp ? clamp_scale : 1.0f;
    const int flags = row_flags(zero_padding ? 1 : 0, n_used, permutation_map);
    if (num_workgroups == 0 &&
        (clamp ? launch_sqrelu_row<true>(true, U, stream, rows, hidden, s, 1.0f / s, flags, x, grad_y, grad_x,
                                         probs, grad_probs, n_used, permutation_map)
               : launch_sqrelu_row<false>(true, U, stream, rows, hidden, s, 1.0f, flags, x, grad_y, grad_x,
                                          probs, grad_probs, n_used, permutation_map)))
        return launched();
    const int blocks = num_workgroups > 0 ? num_workgroups : squared_relu_workgroups(rows, hidden, cus, clamp);
    if (clamp)
        launch_sqrelu_bwd<true>(U, blocks, stream, x, probs, grad_y, grad_x, grad_probs, (int)rows,
                                (int)hidden, s, 1.0f / s, n_used, permutation_map, zero_padding ? 1 : 0);
    else
        launch_sqrelu_bwd<false>(U, blocks, stream, x, probs, grad_y, grad_x, grad_probs, (int)rows,
                                 (int)hidden, s, 1.0f, n_used, permutation_map, zero_padding ? 1 : 0);
    return launched();
}

moe_status_t moe_unpermute_expert_order(const uint16_t *expert_output, int64_t expert_rows,
                                        const int32_t *inverse_map, const int32_t *valid_tokens,
                                        void *out, moe_dtype_t out_dtype, int64_t tokens,
                                        int64_t hidden, int num_local_experts, hipStream_t stream,
                                        int num_workgroups)
{
    if (tokens < 0 || hidden <= 0 || expert_rows < 0 || tokens > kMaxRows || hidden > kMaxHidden ||
        expert_rows > kMaxRows || num_local_experts < 1 || num_local_experts > 1024 ||
        bad_grid(num_workgroups) || !(out_dtype == MOE_FP32 || out_dtype == MOE_BF16))
        return MOE_ERR_INVALID_ARG;
    if (hidden % 8 != 0)
        return MOE_ERR_ALIGNMENT;
    if (tokens == 0)
        return MOE_OK;
    if (!inverse_map || !out || (expert_rows > 0 && !expert_output))
        return MOE_ERR_INVALID_ARG;
    if (!aligned(expert_output, 16) || !aligned(out, 16) || !aligned(inverse_map, 4) ||
        !aligned(valid_tokens, 4))
        return MOE_ERR_ALIGNMENT;
    const uint64_t T = (uint64_t)tokens, H = (uint64_t)hidden;
    const Range o = span(out, T * H * elem_bytes(out_dtype));
    const Range ins[] = {span(expert_output, (uint64_t)expert_rows * H * 2),
                         span(inverse_map, T * (uint64_t)num_local_experts * 4), span(valid_tokens, 4)};
    for (const Range &i : ins)
        if (overlap(o, i))
            return MOE_ERR_INVALID_ARG;
    int cus = 0;
    hipError_t he = device_cus(&cus);
    if (he != hipSuccess)
        return fail_hip(he);
    const int unit_u = out_dtype == MOE_FP32 ? kUnpermuteUnitU<DT_F32> : kUnpermuteUnitU<DT_BF16>;
    const int64_t units = tokens * row_chunks(hidden / 8, unit_u);
    if (num_workgroups == 0 && num_local_experts <= 8 &&
        (units + kWavesPerBlock - 1) / kWavesPerBlock <= kMaxWorkgroups && units <= 0x7fffffffLL) {
        const int blocks = (int)((units + kWavesPerBlock - 1) / kWavesPerBlock);
        const int nch = (int)row_chunks(hidden / 8, unit_u);
        char *o = static_cast<char *>(out);
        if (out_dtype == MOE_FP32)
            hipLaunchKernelGGL((unpermute_unit_kernel<DT_F32, kUnpermuteUnitU<DT_F32>>), dim3(blocks), dim3(kBlock), 0,
                               stream, (int)tokens, (int)hidden, num_local_experts, nch, (int)expert_rows,
                               expert_output, inverse_map, o, valid_tokens);
        else
            hipLaunchKernelGGL((unpermute_unit_kernel<DT_BF16, kUnpermuteUnitU<DT_BF16>>), dim3(blocks), dim3(kBlock), 0,
                               stream, (int)tokens, (int)hidden, num_local_experts, nch, (int)expert_rows,
                               expert_output, inverse_map, o, valid_tokens);
        return launched();
    }
    const bool pipelined = num_local_experts <= kUnpermutePipelinedMaxExperts;
    const int blocks = num_workgroups > 0 ? num_workgroups
                       : pipelined ? walk_workgroups(tokens, row_chunks(hidden / 8, kUnpermutePipeU), cus,
                                                     kUnpermutePipeBlocksPerCU)
                                   : balanced_workgroups(tokens, cus * kUnpermuteBlocksPerCU, 1);
    if (pipelined) {
        char *o = static_cast<char *>(out);
        const int T32 = (int)tokens, H32 = (int)hidden, E = num_local_experts;
        if (out_dtype == MOE_FP32 && E <= 4)
            hipLaunchKernelGGL((unpermute_pipelined_kernel<DT_F32, kUnpermutePipeU, 4>), dim3(blocks), dim3(kBlock),
                               0, stream, expert_output, expert_rows, inverse_map, valid_tokens, o, T32, H32, E);
        else if (out_dtype == MOE_FP32)
            hipLaunchKernelGGL((unpermute_pipelined_kernel<DT_F32, kUnpermutePipeU, 8>), dim3(blocks), dim3(kBlock),
                               0, stream, expert_output, expert_rows, inverse_map, valid_tokens, o, T32, H32, E);
        else if (E <= 4)
            hipLaunchKernelGGL((unpermute_pipelined_kernel<DT_BF16, kUnpermutePipeU, 4>), dim3(blocks), dim3(kBlock),
                               0, stream, expert_output, expert_rows, inverse_map, valid_tokens, o, T32, H32, E);
        else
            hipLaunchKernelGGL((unpermute_pipelined_kernel<DT_BF16, kUnpermutePipeU, 8>), dim3(blocks), dim3(kBlock),
                               0, stream, expert_output, expert_rows, inverse_map, valid_tokens, o, T32, H32, E);
        return launched();
    }
    if (out_dtype == MOE_FP32)
        hipLaunchKernelGGL((unpermute_kernel<DT_F32, kUnpermuteU, kUnpermuteG>), dim3(blocks), dim3(kBlock), 0,
                           stream, expert_output, expert_rows, inverse_map, valid_tokens,
                           static_cast<char *>(out), (int)tokens, (int)hidden, num_local_experts);
    else
        hipLaunchKernelGGL((unpermute_kernel<DT_BF16, kUnpermuteU, kUnpermuteG>), dim3(blocks), dim3(kBlock), 0,
                           stream, expert_output, expert_rows, inverse_map, valid_tokens,
                           static_cast<char *>(out), (int)tokens, (int)hidden, num_local_experts);
    return launched();
}

const char *moe_elementwise_status_string(moe_status_t status)
{
    switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_ALIGNMENT: return "misaligned pointer or row width not a multiple of 8";
    case MOE_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int moe_elementwise_last_hip_error(void) { return t_last_hip_error; }

int moe_elementwise_abi_version(void) { return MOE_ELEMENTWISE_ABI_VERSION; }

}  // extern "C"
