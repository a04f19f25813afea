// Plain streaming kernels (copy, 2:1 and 3:2 read:write) for the practical HBM
// ceiling and for calibrating FETCH_SIZE / WRITE_SIZE. C ABI in hbm_probe.h.
//
// They move data the way the activation kernels do, minus the arithmetic: each
// wave streams 4 KiB blocks of every source (64 lanes x 4 x 16-byte buffer loads
// with the nontemporal hint), blocks interleaved across waves, through the same
// two-buffer pipeline (the next block's loads issued before the current block's
// stores), with the kernels' default grid (one wave per block). Destination vector i is the XOR of the source
// vectors i.
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
        u32x4 v[NS][kU];
    };
    Ptrs p;
    int64_t bytes;
    uint32_t voff;

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

    __device__ __forceinline__ void process(const Buf &buf, int64_t b) const
    {
        const uint32_t n = valid(b);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
            const rsrc_t r = make_rsrc(p.dst[d] + b * kBlockBytes, n);
#pragma unroll
            for (int u = 0; u < kU; ++u) {
                u32x4 v = buf.v[0][u];
#pragma unroll
                for (int s = 1; s < NS; ++s)
                    v ^= buf.v[s][u];
                store_vec(r, v, voff + u * kWave * kVecBytes);
            }
        }
    }
};

template <int NS, int ND>
__global__ __launch_bounds__(kBlock) void stream_kernel(Ptrs p, int64_t n_vec)
{
    StreamOp<NS, ND> op{p, n_vec * kVecBytes, (uint32_t)lane_id() * kVecBytes};
    walk_blocks(op, (n_vec * kVecBytes + kBlockBytes - 1) / kBlockBytes);
}

template <int NS, int ND>
int launch(const Ptrs &p, int64_t n_vec, int blocks, hipStream_t stream)
{
    if (blocks <= 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return 3;
        blocks = walk_workgroups((n_vec * kVecBytes + kBlockBytes - 1) / kBlockBytes, 1,
                                 prop.multiProcessorCount, 1);
    }
    hipLaunchKernelGGL((stream_kernel<NS, ND>), dim3(blocks), dim3(kBlock), 0, stream, p, n_vec);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

bool aligned16(const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

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
