// Plain streaming kernels (copy, 2:1 and 3:2 read:write) for the practical HBM
// ceiling and for calibrating FETCH_SIZE / WRITE_SIZE. C ABI in hbm_probe.h.
// Loads and stores carry the nontemporal hint and the default grid is one
// workgroup per CU: the configuration that streamed fastest on MI355X.
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

// Each wave moves blocks of kUnroll * 64 vectors (4 KiB) per stream, blocks
// interleaved across waves (block b + k * waves); all loads of a block are issued
// before its stores. This row-per-wave mapping with nontemporal loads and stores
// streamed fastest on MI355X in steady back-to-back runs.
template <int NS, int ND>
__global__ __launch_bounds__(kBlock) void stream_kernel(Ptrs p, int64_t n_vec)
{
    constexpr int kWave = 64;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t waves = (int64_t)gridDim.x * (kBlock / kWave);
    const int64_t w = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
    const int64_t per_block = (int64_t)kUnroll * kWave;
    const int64_t n_blocks = (n_vec + per_block - 1) / per_block;
    for (int64_t b = w; b < n_blocks; b += waves) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = b * per_block + u * kWave + lane;
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (i < n_vec) {
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    v[u] ^= __builtin_nontemporal_load(p.src[s] + i);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int64_t i = b * per_block + u * kWave + lane;
            if (i < n_vec) {
#pragma unroll
                for (int d = 0; d < ND; ++d)
                    __builtin_nontemporal_store(v[u], p.dst[d] + i);
            }
        }
    }
}

template <int NS, int ND>
int launch(const Ptrs &p, int64_t n_vec, int blocks, hipStream_t stream)
{
    if (blocks <= 0) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
            return 3;
        blocks = prop.multiProcessorCount;
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
