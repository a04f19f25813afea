// Plain streaming kernels (copy, 2:1 and 3:2 read:write, and one-way read-only and
// write-only streams) for the practical HBM ceiling and for calibrating FETCH_SIZE /
// WRITE_SIZE. C ABI in hbm_probe.h.
//
// They move data the way the activation kernels do, minus the arithmetic: each
// wave streams 4 KiB blocks of every source (64 lanes x 4 x 16-byte buffer loads
// with the nontemporal hint), blocks interleaved across waves, through the same
// two-buffer pipeline (the next block's loads issued before the current block's
// stores), with the kernels' default grid (one wave per block). Destination vector i is the XOR of the source
// vectors i. With no destination (read-only), each lane keeps the XOR of everything it
// read and stores it to a 16-byte sink only if it equals a caller-chosen key, so the
// loads cannot be dropped but nothing is written in practice. With no source
// (write-only), every destination word becomes a caller-chosen value.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <mutex>

#include "cdna4_stream.h"
#include "hbm_probe.h"

namespace {

using namespace cdna4;

constexpr int kU = 4;  // 16-byte vectors per lane per stream per block
constexpr uint32_t kBlockBytes = kU * kWave * kVecBytes;  // 4 KiB per stream per block at kU = 4

struct Ptrs {
    const char *src[3];
    char *dst[2];
};

template <int NS, int ND>
struct StreamOp {
    struct Buf {
        u32x4 v[NS > 0 ? NS : 1][kU];
    };
    Ptrs p;
    int64_t bytes;
    uint32_t voff;
    uint32_t word;  // write-only: the value every word gets
    u32x4 acc;      // read-only: XOR of every vector this lane read

    __device__ __forceinline__ uint32_t valid(int64_t b) const
    {
        const int64_t left = bytes - b * kBlockBytes;
        return left <= 0 ? 0u : (left < kBlockBytes ? (uint32_t)left : kBlockBytes);
    }

    __device__ __forceinline__ void load(Buf &buf, int64_t b, bool live) const
    {
        const uint32_t n = live ? valid(b) : 0u;
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const rsrc_t r = make_rsrc(p.src[s] + b * kBlockBytes, n);
#pragma unroll
            for (int u = 0; u < kU; ++u)
                buf.v[s][u] = load_vec(r, voff + u * kWave * kVecBytes);
        }
    }

    __device__ __forceinline__ u32x4 combined(const Buf &buf, int u) const
    {
        if constexpr (NS == 0) {
            return u32x4{word, word, word, word};
        } else {
            u32x4 v = buf.v[0][u];
#pragma unroll
            for (int s = 1; s < NS; ++s)
                v ^= buf.v[s][u];
            return v;
        }
    }

    __device__ __forceinline__ void process(const Buf &buf, int64_t b)
    {
        if constexpr (ND == 0) {
#pragma unroll
            for (int u = 0; u < kU; ++u)
                acc ^= combined(buf, u);
        } else {
            const uint32_t n = valid(b);
#pragma unroll
            for (int d = 0; d < ND; ++d) {
                const rsrc_t r = make_rsrc(p.dst[d] + b * kBlockBytes, n);
#pragma unroll
                for (int u = 0; u < kU; ++u)
                    store_vec(r, combined(buf, u), voff + u * kWave * kVecBytes);
            }
        }
    }
};

template <int NS, int ND>
__global__ __launch_bounds__(kBlock) void stream_kernel(Ptrs p, int64_t n_vec, uint32_t word, u32x4 *sink)
{
    StreamOp<NS, ND> op{p, n_vec * kVecBytes, (uint32_t)lane_id() * kVecBytes, word, u32x4{0u, 0u, 0u, 0u}};
    walk_blocks(op, (n_vec * kVecBytes + kBlockBytes - 1) / kBlockBytes);
    if constexpr (ND == 0) {
        if (op.acc[0] == word && op.acc[1] == word && op.acc[2] == word && op.acc[3] == word)
            *sink = op.acc;
    }
}

template <int NS, int ND>
int launch(const Ptrs &p, int64_t n_vec, int blocks, hipStream_t stream, uint32_t word = 0,
           u32x4 *sink = nullptr)
{
    if (blocks <= 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return 3;
        blocks = walk_workgroups((n_vec * kVecBytes + kBlockBytes - 1) / kBlockBytes, 1,
                                 prop.multiProcessorCount, 1);
    }
    hipLaunchKernelGGL((stream_kernel<NS, ND>), dim3(blocks), dim3(kBlock), 0, stream, p, n_vec, word, sink);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

bool aligned16(const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

bool overlap(const void *a, uintptr_t na, const void *b, uintptr_t nb)
{
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

bool bad_count(int64_t n_vec, int num_workgroups)
{
    // n_vec at most 2^44 (2^48 bytes per array): byte counts and offsets stay in 64 bits
    return n_vec < 0 || n_vec > (int64_t(1) << 44) || num_workgroups < 0 || num_workgroups > kMaxWorkgroups;
}

}  // namespace

extern "C" int hbm_probe_stream(const void *const *src, int n_src, void *const *dst, int n_dst,
                                int64_t n_vec, int num_workgroups, hipStream_t stream)
{
    // n_vec at most 2^44 (2^48 bytes per array): byte counts and offsets stay in 64 bits
    if (!src || !dst || n_src < 1 || n_src > 3 || n_dst < 1 || n_dst > 2 || n_vec < 0 ||
        n_vec > (int64_t(1) << 44) || num_workgroups < 0 || num_workgroups > kMaxWorkgroups)
        return 1;
    if (n_vec == 0)
        return 0;
    Ptrs p = {};
    for (int s = 0; s < n_src; ++s) {
        if (!src[s] || !aligned16(src[s]))
            return 1;
        p.src[s] = static_cast<const char *>(src[s]);
    }
    for (int d = 0; d < n_dst; ++d) {
        if (!dst[d] || !aligned16(dst[d]))
            return 1;
        p.dst[d] = static_cast<char *>(dst[d]);
    }
    const uintptr_t bytes = (uintptr_t)n_vec * 16;
    for (int d = 0; d < n_dst; ++d)
        for (int s = 0; s < n_src; ++s) {
            uintptr_t a = reinterpret_cast<uintptr_t>(dst[d]), b = reinterpret_cast<uintptr_t>(src[s]);
            if (a < b + bytes && b < a + bytes)
                return 1;
        }
    if (n_src == 1 && n_dst == 1) return launch<1, 1>(p, n_vec, num_workgroups, stream);
    if (n_src == 2 && n_dst == 1) return launch<2, 1>(p, n_vec, num_workgroups, stream);
    if (n_src == 3 && n_dst == 2) return launch<3, 2>(p, n_vec, num_workgroups, stream);
    if (n_src == 1 && n_dst == 2) return launch<1, 2>(p, n_vec, num_workgroups, stream);
    if (n_src == 2 && n_dst == 2) return launch<2, 2>(p, n_vec, num_workgroups, stream);
    if (n_src == 3 && n_dst == 1) return launch<3, 1>(p, n_vec, num_workgroups, stream);
    return 1;
}

extern "C" int hbm_probe_read(const void *const *src, int n_src, int64_t n_vec, uint32_t key, void *sink,
                              int num_workgroups, hipStream_t stream)
{
    if (!src || !sink || !aligned16(sink) || n_src < 1 || n_src > 3 || bad_count(n_vec, num_workgroups))
        return 1;
    Ptrs p = {};
    for (int s = 0; s < n_src; ++s) {
        if (!src[s] || !aligned16(src[s]) || overlap(src[s], (uintptr_t)n_vec * 16, sink, 16))
            return 1;
        p.src[s] = static_cast<const char *>(src[s]);
    }
    if (n_vec == 0)
        return 0;
    u32x4 *out = static_cast<u32x4 *>(sink);
    if (n_src == 1) return launch<1, 0>(p, n_vec, num_workgroups, stream, key, out);
    if (n_src == 2) return launch<2, 0>(p, n_vec, num_workgroups, stream, key, out);
    return launch<3, 0>(p, n_vec, num_workgroups, stream, key, out);
}

extern "C" int hbm_probe_fill(void *const *dst, int n_dst, int64_t n_vec, uint32_t value, int num_workgroups,
                              hipStream_t stream)
{
    if (!dst || n_dst < 1 || n_dst > 2 || bad_count(n_vec, num_workgroups))
        return 1;
    Ptrs p = {};
    for (int d = 0; d < n_dst; ++d) {
        if (!dst[d] || !aligned16(dst[d]))
            return 1;
        p.dst[d] = static_cast<char *>(dst[d]);
    }
    if (n_dst == 2 && overlap(dst[0], (uintptr_t)n_vec * 16, dst[1], (uintptr_t)n_vec * 16))
        return 1;
    if (n_vec == 0)
        return 0;
    if (n_dst == 1) return launch<0, 1>(p, n_vec, num_workgroups, stream, value);
    return launch<0, 2>(p, n_vec, num_workgroups, stream, value);
}
