/*
 * hbm_probe.h - plain streaming kernels that measure what HBM delivers on the
 * device they run on, for comparison with the activation kernels.
 *
 * hbm_probe_stream reads n_src arrays and writes n_dst arrays of n_vec 16-byte
 * vectors each: every destination vector becomes the XOR of the source vectors at
 * the same index (a plain copy for n_src = n_dst = 1). Ratios 1:1, 2:1 and 3:2
 * mirror a copy, the activation forward (gate + up -> y) and its backward
 * (gate + up + grad_y -> two halves of grad_x). The kernel moves exactly
 * (n_src + n_dst) * n_vec * 16 bytes, so it also calibrates the hardware byte
 * counters (FETCH_SIZE / WRITE_SIZE) against a known size.
 *
 * Pointers: device memory on the current HIP device, 16-byte aligned, caller-owned,
 * destinations must not overlap sources. 1 <= n_src <= 3, 1 <= n_dst <= 2,
 * 0 <= n_vec <= 2^44.
 * num_workgroups = 0 launches one wave per 4 KiB block (at most 16,777,215
 * workgroups), the activation kernels' default grid for short rows; an explicit
 * count must not exceed 16,777,215. Accesses are 128-bit buffer loads/stores with the
 * nontemporal hint, pipelined like the activation kernels, without their arithmetic. Work is enqueued on
 * `stream`; no synchronisation, no allocation.
 * Returns 0 on success, 1 for invalid arguments, 3 when the launch failed.
 */
#ifndef HBM_PROBE_H
#define HBM_PROBE_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

int hbm_probe_stream(const void *const *src, int n_src, void *const *dst, int n_dst,
                     int64_t n_vec, int num_workgroups, hipStream_t stream);

/*
 * One-way streams, the two ends of the read:write range, with the same access pattern,
 * grid and limits as hbm_probe_stream.
 *
 * hbm_probe_read reads n_src (1..3) arrays of n_vec 16-byte vectors and writes nothing
 * in practice: each lane keeps the XOR of the vectors it read and stores it to `sink`
 * (one 16-byte device buffer, 16-byte aligned, not inside a source) only where all four
 * of its 32-bit words equal `key`. Pick a key the data cannot produce (with every source
 * holding one repeated word w, an odd count of sources gives w, an even count 0); the
 * conditional store only keeps the loads from being dropped. A lane's XOR covers the
 * vectors it read, so which lanes match depends on the grid.
 *
 * hbm_probe_fill writes `value` to every 32-bit word of n_dst (1..2) arrays of n_vec
 * 16-byte vectors (non-overlapping), reading nothing.
 *
 * Return codes as hbm_probe_stream.
 */
int hbm_probe_read(const void *const *src, int n_src, int64_t n_vec, uint32_t key, void *sink,
                   int num_workgroups, hipStream_t stream);

int hbm_probe_fill(void *const *dst, int n_dst, int64_t n_vec, uint32_t value, int num_workgroups,
                   hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HBM_PROBE_H */
