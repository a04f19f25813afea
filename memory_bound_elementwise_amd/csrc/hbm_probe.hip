// Plain streaming kernels (copy, 2:1 and 3:2 read:write) for the practical HBM
// ceiling and for calibrating FETCH_SIZE / WRITE_SIZE. C ABI in hbm_probe.h.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "hbm_probe.h"

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;
constexpr int kUnroll = 4;

struct Ptrs {
    const u32x4 *src[3];
    u32x4 *dst[2];
};

// Each thread moves kUnroll vectors per stream per step, all loads issued first.
template <int NS, int ND>
__global__ __launch_bounds__(kBlock) void stream_kernel(Ptrs p, int64_t n_vec)
{
    const int64_t stride = (int64_t)gridDim.x * kBlock;
    const int64_t step = stride * kUnroll;
    for (int64_t base = (int64_t)blockIdx.x * kBlock + threadIdx.x; base < n_vec; base += step) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * stride;
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (i < n_vec) {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    v[u] ^= p.src[s][i];
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = base + u * stride;
            if (i < n_vec) {
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    p.dst[d][i] = v[u];
            }
        }
    }
}

template <int NS, int ND>
int launch(const Ptrs &p, int64_t n_vec, int blocks, hipStream_t stream)
{
    if (blocks <= 0) {
        int dev = 0, per_cu = 1;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return 3;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void *>(stream_kernel<NS, ND>), kBlock, 0) != hipSuccess)
            return 3;
        blocks = prop.multiProcessorCount * (per_cu > 0 ? per_cu : 1);
    }
    hipLaunchKernelGGL((stream_kernel<NS, ND>), dim3(blocks), dim3(kBlock), 0, stream, p, n_vec);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

bool aligned16(const void *q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; }

}  // namespace

extern "C" int hbm_probe_stream(const void *const *src, int n_src, void *const *dst, int n_dst,
                                int64_t n_vec, int num_workgroups, hipStream_t stream)
{
    if (!src || !dst || n_src < 1 || n_src > 3 || n_dst < 1 || n_dst > 2 || n_vec < 0 ||
        num_workgroups < 0)
        return 1;
    if (n_vec == 0)
        return 0;
    Ptrs p = {};
    for (int s = 0; s < n_src; ++s) {
        if (!src[s] || !aligned16(src[s]))
            return 1;
        p.src[s] = static_cast<const u32x4 *>(src[s]);
    }
    for (int d = 0; d < n_dst; ++d) {
        if (!dst[d] || !aligned16(dst[d]))
            return 1;
        p.dst[d] = static_cast<u32x4 *>(dst[d]);
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
