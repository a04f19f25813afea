// Streaming building blocks for HBM-bound elementwise kernels on MI355X (gfx950):
// per-row buffer resources whose hardware range check does all masking, 128-bit
// accesses with cache-policy hints, bf16 packing, a fixed-order wave reduction, and
// the fixed-grid row walk with device-side row bounds, permutation slots and a
// two-buffer software pipeline. Internal to this package's HIP libraries.
#ifndef MBE_CDNA4_STREAM_H
#define MBE_CDNA4_STREAM_H

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace cdna4 {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kWave = 64;
constexpr int kBlock = 256;                       // threads per workgroup
constexpr int kWavesPerBlock = kBlock / kWave;
constexpr int kVecBytes = 16;                     // one lane access

// ---------------------------------------------------------------------------
// Buffer resources and streaming accesses
// ---------------------------------------------------------------------------
// Word 3 of a gfx9-family buffer descriptor for raw (unformatted, stride 0) access.
constexpr int kRsrcWord3 = 0x00020000;

// Cache-policy bits of streaming accesses (1 = sc0, 2 = nt, 16 = sc1). Nontemporal
// loads and stores measured fastest in back-to-back runs on MI355X: plain stores
// leave lines dirty in the 256 MB Infinity Cache for the next kernel to drain.
constexpr int kLoadAux = 2;
constexpr int kStoreAux = 2;

// Every caller passes wave-uniform values (row addresses and lengths); readfirstlane
// states that to the compiler, so the descriptor lives in SGPRs and no access needs a
// per-lane descriptor loop.
__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
    void *p = reinterpret_cast<void *>(((uint64_t)hi << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(p, (short)0, (int)n, kRsrcWord3);
}

// Resource for the part of a row from byte `off` on: `bytes` is the row's valid
// length (0 for a row that is not live). Offsets are range-checked relative to the
// resource, so every access uses only the lane's VGPR offset: lanes past the end
// read zeros without touching memory and their stores are dropped.
// Row lengths and offsets stay below 2^31 (the hosts bound row widths), so the
// remaining length is taken as a signed max, which the scalar unit has. The unsigned
// form (a saturating subtract) has only a vector instruction: each descriptor then
// borrowed a VGPR, often one a pending load was about to fill, and the compiler
// drained the loads in flight before the write.
__device__ __forceinline__ rsrc_t chunk_rsrc(const void *row, uint32_t bytes, uint32_t off)
{
    const int rem = (int)bytes - (int)off;
    return make_rsrc(reinterpret_cast<const char *>(row) + off, (uint32_t)(rem > 0 ? rem : 0));
}

__device__ __forceinline__ u32x4 load_vec(rsrc_t r, uint32_t voff)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kLoadAux);
}

__device__ __forceinline__ void store_vec(rsrc_t r, u32x4 v, uint32_t voff)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, voff, 0, kStoreAux);
}

// ---------------------------------------------------------------------------
// bf16 / fp16 <-> fp32
// ---------------------------------------------------------------------------
// bf16 is the upper half of an fp32, so widening is a shift or a mask.
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values to two bf16 (v_cvt_pk_bf16_f32: round to nearest even, subnormals
// kept, NaN stays NaN).
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ f32x2 unpack_f16x2(unsigned w)
{
    return __builtin_convertvector(__builtin_bit_cast(f16x2, w), f32x2);
}

// Two fp32 values to two fp16, round to nearest even.
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi)
{
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(v, f16x2));
}

// ---------------------------------------------------------------------------
// Wave-wide sum with a fixed combination order, returned as a wave-uniform value.
// ---------------------------------------------------------------------------
// DPP move of v from the lane `kCtrl` selects; lanes of rows (16 lanes) outside
// `kRowMask` get +0.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask, 0xf, false));
}

// Pairs of lanes, then quads, halves of a row, rows: after the four in-row steps every
// lane of a 16-lane row holds that row's total R_k. The two broadcasts then form
// (R_3 + R_2) + (R_1 + R_0) in lane 63. fp32 addition is commutative, so every step
// adds the same two values however its operands are ordered, and the order depends on
// nothing but the lane.
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp<0xB1>(v);        // quad_perm [1,0,3,2]: lanes ^1
    v += dpp<0x4E>(v);        // quad_perm [2,3,0,1]: lanes ^2
    v += dpp<0x141>(v);       // row_half_mirror: the other quad of each 8
    v += dpp<0x140>(v);       // row_mirror: the other half of each 16
    v += dpp<0x142, 0xa>(v);  // row_bcast:15: rows 1 and 3 add the total of rows 0 and 2
    v += dpp<0x143, 0xc>(v);  // row_bcast:31: rows 2 and 3 add lane 31 (rows 0 + 1)
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), kWave - 1));
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// The calling wave's index in its workgroup (0 .. 3); uniform, so kept in an SGPR.
__device__ __forceinline__ int wave_in_block() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// The calling wave's index in the grid; uniform, so kept in an SGPR.
__device__ __forceinline__ int wave_id() { return blockIdx.x * kWavesPerBlock + wave_in_block(); }

// ---------------------------------------------------------------------------
// Row schedule: a fixed grid of waves strides over rows (r, r + W, r + 2W, ...)
// ---------------------------------------------------------------------------
struct RowSchedule {
    int rows;     // rows of every row-indexed tensor (max_rows)
    int live;     // clamp(*n_used, 0, rows), or rows
    int row_end;  // rows a launch visits: rows with zero_padding, else live
};

__device__ __forceinline__ RowSchedule make_schedule(int rows, const int *__restrict__ n_used,
                                                     int zero_padding)
{
    RowSchedule s;
    s.rows = rows;
    s.live = rows;
    if (n_used) {
        int n = *n_used;
        s.live = n < 0 ? 0 : (n > rows ? rows : n);
    }
    s.row_end = zero_padding ? rows : s.live;
    return s;
}

// Gathers (slot, probability) of row `ri` for the calling lane; slot -1 = not live.
__device__ __forceinline__ void row_meta(int64_t ri, const RowSchedule &s, const int *__restrict__ perm,
                                         const float *__restrict__ probs, int &slot, float &p)
{
    slot = -1;
    p = 0.0f;
    if (ri < s.live) {
        int v = perm ? perm[ri] : (int)ri;
        if ((unsigned)v < (unsigned)s.rows) {
            slot = v;
            p = probs[v];
        }
    }
}

// Bits of the `flags` argument of kernels that handle one row per wave or workgroup. The
// flags say which optional row arguments exist, so a kernel reads those pointers (kernel
// arguments past the preloaded ones) only when they are there.
constexpr int kZeroPadding = 1;
constexpr int kHasNUsed = 2;
constexpr int kHasPerm = 4;

// Slot of row `r` for a kernel that handles one row per wave or workgroup (r uniform):
// -1 when the row is not live, i.e. at or past clamp(*n_used, 0, rows) or mapped outside
// [0, rows). The loads are scalar; without n_used and map there are none.
__device__ __forceinline__ int row_slot(int r, int rows, int flags, const int *__restrict__ n_used,
                                        const int *__restrict__ perm)
{
    int live = rows;
    if (flags & kHasNUsed) {
        const int n = *n_used;
        live = n < 0 ? 0 : (n > rows ? rows : n);
    }
    if (r >= live)
        return -1;
    const int v = (flags & kHasPerm) ? perm[r] : r;
    return (unsigned)v < (unsigned)rows ? v : -1;
}

// probs[slot] for every lane (0 for slot < 0), through the vector memory path: a buffer
// load of one dword at a wave-uniform address, issued like the row's streaming loads.
__device__ __forceinline__ float load_row_prob(const float *__restrict__ probs, int slot)
{
    const rsrc_t r = make_rsrc(probs + (slot >= 0 ? slot : 0), slot >= 0 ? 4u : 0u);
    return __int_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, 0, 0, 0));
}

// Row sums. An Op with `kRowSum` true keeps a lane partial `acc` of a per-row sum; it
// adds to it in process() and provides row_sum_wanted() (false when there is nowhere
// to write) and store_row_sum(slot, total). The walks reset acc before a row's first
// chunk and, after its last, combine the lanes with wave_sum (and, when waves share a
// row, the waves in wave order) and store the total for rows that have a slot. Each
// lane's columns are visited in increasing order, so the bits do not depend on the
// grid.
template <class Op>
__device__ __forceinline__ void row_sum_reset(Op &op)
{
    if constexpr (Op::kRowSum)
        op.acc = 0.0f;
}

// One wave's walk over its rows, in batches of up to 64 rows (one metadata lane
// each), as a sequence of items (row k of the batch, column chunk c). `Op` loads an
// item into a register buffer (`Op::Buf`) and processes an item from one; the walk
// issues the loads of item t + 1 before processing item t, alternating two buffers.
// Loads of items past the end use an empty buffer resource, so they move no data.
// `nch` = column chunks per row.
template <class Op>
__device__ __forceinline__ void walk_rows(Op &op, const RowSchedule &sched, const int *__restrict__ perm,
                                          const float *__restrict__ probs, int nch)
{
    const int lane = lane_id();
    const int W = gridDim.x * kWavesPerBlock;
    const int w = wave_id();

    for (int64_t base = w; base < sched.row_end; base += (int64_t)kWave * W) {
        int slot_l;
        float p_l;
        row_meta(base + (int64_t)lane * W, sched, perm, probs, slot_l, p_l);
        const int64_t left = (sched.row_end - base + W - 1) / W;
        const int nk = left < kWave ? (int)left : kWave;
        const int T = nk * nch;

        // Item t is (row k of the batch, chunk c), t = k * nch + c. The loads and the
        // processing each keep a cursor and step it, rather than dividing t. The rows of
        // a batch lie below 2^31 (the hosts bound the row count), so their indices are
        // 32-bit: 64-bit compares and divisions have no scalar form, and the vector
        // registers they borrow can be ones a pending load is about to fill, which the
        // compiler then waits on.
        auto step = [nch](int &k, int &c) {
            if (++c == nch) {
                c = 0;
                ++k;
            }
        };
        // Without a map a row is live iff it is below the live bound, so its loads do
        // not wait for the metadata gather; with a map the slot decides. Past the last
        // item the load names the batch's last row through an empty resource.
        auto prefetch = [&](int t, int k, int c, typename Op::Buf &buf) {
            if (k >= nk)
                k = nk - 1;
            const int r = (int)base + k * W;
            const bool live = perm ? __builtin_amdgcn_readlane(slot_l, k) >= 0 : r < sched.live;
            op.load(buf, r, c, live && t < T);
        };
        auto process = [&](int k, int c, const typename Op::Buf &buf) {
            const int slot = __builtin_amdgcn_readlane(slot_l, k);
            const float p = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p_l), k));
            if (c == 0)
                row_sum_reset(op);
            op.process(buf, (int)base + k * W, c, slot, p);
            if constexpr (Op::kRowSum) {
                if (c == nch - 1 && slot >= 0 && op.row_sum_wanted())
                    op.store_row_sum(slot, wave_sum(op.acc));
            }
        };

        // The scheduling barriers keep each item's loads ahead of the previous item's
        // arithmetic, which the scheduler would otherwise hoist above them.
        typename Op::Buf A, B;
        int pk = 0, pc = 0, qk = 0, qc = 0;  // next item to load, next item to process
        prefetch(0, pk, pc, A);
        step(pk, pc);
        for (int t = 0; t < T; t += 2) {
            prefetch(t + 1, pk, pc, B);
            step(pk, pc);
            __builtin_amdgcn_sched_barrier(0);
            process(qk, qc, A);
            step(qk, qc);
            if (t + 1 >= T)
                break;
            prefetch(t + 2, pk, pc, A);
            step(pk, pc);
            __builtin_amdgcn_sched_barrier(0);
            process(qk, qc, B);
            step(qk, qc);
        }
    }
}

// The row total of a row whose four quarters the four waves of a workgroup hold as lane
// partials `acc`: each wave writes its partials to part[w], and after one barrier wave 0
// adds, lane by lane, the partials of waves 0, 1, 2, 3 in that order, then reduces the
// 64 sums with wave_sum. The result is meaningful in wave 0 only. Every wave of the
// workgroup must call it (it holds a barrier). The barrier is fenced on LDS alone:
// only the partials cross it, and __syncthreads would also wait for every global
// access in flight, the next item's prefetched loads included.
__device__ __forceinline__ float row_sum_split(float (*part)[kWave], float acc, int w, int lane)
{
    part[w][lane] = acc;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    float t = 0.0f;
    if (w == 0) {
        t = part[0][lane];
#pragma unroll
        for (int i = 1; i < kWavesPerBlock; ++i)
            t += part[i][lane];
        t = wave_sum(t);
    }
    return t;
}

// The same row total for a workgroup that handles one row, without a barrier at the
// end: each wave writes its partials to part[w] and counts itself in `arrived`; the
// wave that arrives last (whichever it is) adds the partials of waves 0, 1, 2, 3 in that
// order and reduces them with wave_sum, exactly as row_sum_split does, and returns true
// with the total. The others return false at once instead of waiting for the slowest
// wave's loads. `arrived` must be zero and visible to every wave first:
// row_sum_last_init, called by every wave (it holds a barrier) before any wave can
// arrive; early in the kernel the four waves reach it together. The fences are on LDS
// alone, so global accesses in flight are not waited for.
__device__ __forceinline__ void row_sum_last_init(unsigned *arrived, int w, int lane)
{
    if (w == 0 && lane == 0)
        *arrived = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ bool row_sum_last(float (*part)[kWave], unsigned *arrived, float acc, int w, int lane,
                                             float &total)
{
    part[w][lane] = acc;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    unsigned before = 0u;
    if (lane == 0)
        before = __hip_atomic_fetch_add(arrived, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    before = __builtin_amdgcn_readfirstlane(before);
    if (before != kWavesPerBlock - 1)
        return false;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    float t = part[0][lane];
#pragma unroll
    for (int i = 1; i < kWavesPerBlock; ++i)
        t += part[i][lane];
    total = wave_sum(t);
    return true;
}

// One row per wave (row = the wave's index in the grid), all `NCH` column chunks of it
// loaded at once, for the default launch of rows of at most a couple of chunks: no walk,
// no per-row bookkeeping beyond the row's own slot (row_slot) and probability
// (load_row_prob). Op, the chunks' order and the row-sum order are walk_rows', so the
// bits are the same as a walk over the same rows.
template <int NCH, class Op>
__device__ __forceinline__ void row_per_wave(Op &op, int rows, int flags, const int *__restrict__ n_used,
                                             const int *__restrict__ perm, const float *__restrict__ probs)
{
    const int r = wave_id();
    if (r >= rows)
        return;
    const int slot = row_slot(r, rows, flags, n_used, perm);
    if (slot < 0 && !(flags & kZeroPadding))
        return;
    typename Op::Buf b[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        op.load(b[c], r, c, slot >= 0);
    const float p = load_row_prob(probs, slot);
    row_sum_reset(op);
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        op.process(b[c], r, c, slot, p);
    if constexpr (Op::kRowSum) {
        if (slot >= 0 && op.row_sum_wanted())
            op.store_row_sum(slot, wave_sum(op.acc));
    }
}

// A workgroup's walk over its rows (row r, r + G, r + 2G, ... for workgroup r of G), the
// four waves sharing each row: wave w takes the column chunks
// [floor(w nch / 4), floor((w + 1) nch / 4)), at least one each for nch >= 4. With
// `spans` (uniform), the op has already given each wave its own quarter of the row and
// nch counts the chunks of one quarter: every wave takes all nch of them. Per wave the
// items (row, chunk) run through the same two-buffer pipeline as walk_rows. Row sums
// (kRowSum ops) go through LDS first: every wave writes its 64 lane partials, and after
// one barrier per row wave 0 adds, lane by lane, the partials of waves 0, 1, 2, 3 in
// that order and reduces the 64 results with wave_sum (row_sum_split above). The LDS
// pair alternates by row so a fast wave cannot overwrite a partial that wave 0 has not
// read yet. When the grid gives each workgroup at most one row (the default grid), the
// sum goes through row_sum_last instead, in the same order and with the same bits, and
// no wave waits at the row's end: at 53,760 x 7,168 that took the router-weight
// backward from 370.3 to 362.9 us. Every wave of a workgroup visits the same rows, so
// every barrier is reached by all four.
template <class Op>
__device__ __forceinline__ void walk_row_split(Op &op, const RowSchedule &sched, const int *__restrict__ perm,
                                               const float *__restrict__ probs, int nch,
                                               bool spans = false)
{
    if (!spans && nch < kWavesPerBlock) {
        // a wave without chunks would miss the barriers: rows this short go one per wave
        // (the condition is the same for the whole grid)
        walk_rows(op, sched, perm, probs, nch);
        return;
    }
    __shared__ float partials[2][kWavesPerBlock][kWave];
    __shared__ unsigned arrived;
    const int lane = lane_id();
    const int G = gridDim.x;
    const bool one_row = sched.row_end <= G;
    const int w = wave_in_block();
    const int c_lo = spans ? 0 : (int)((int64_t)w * nch / kWavesPerBlock);
    const int nc = spans ? nch : (int)((int64_t)(w + 1) * nch / kWavesPerBlock) - c_lo;  // >= 1
    const int wg = __builtin_amdgcn_readfirstlane((int)blockIdx.x);
    int parity = 0;

    for (int64_t base = wg; base < sched.row_end; base += (int64_t)kWave * G) {
        int slot_l;
        float p_l;
        row_meta(base + (int64_t)lane * G, sched, perm, probs, slot_l, p_l);
        const int64_t left = (sched.row_end - base + G - 1) / G;
        const int nk = left < kWave ? (int)left : kWave;
        const int T = nk * nc;

        // items (row k, the wave's chunk j), stepped as in walk_rows
        auto step = [nc](int &k, int &jj) {
            if (++jj == nc) {
                jj = 0;
                ++k;
            }
        };
        auto prefetch = [&](int t, int k, int jj, typename Op::Buf &buf) {
            if (k >= nk)
                k = nk - 1;
            const int r = (int)base + k * G;
            const bool live = perm ? __builtin_amdgcn_readlane(slot_l, k) >= 0 : r < sched.live;
            op.load(buf, r, c_lo + jj, live && t < T);
        };
        auto process = [&](int k, int jj, const typename Op::Buf &buf) {
            const int slot = __builtin_amdgcn_readlane(slot_l, k);
            const float p = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(p_l), k));
            if (jj == 0)
                row_sum_reset(op);
            op.process(buf, (int)base + k * G, c_lo + jj, slot, p);
            if constexpr (Op::kRowSum) {
                // slot and the op's state are the same for all four waves: all or none sync
                if (jj == nc - 1 && slot >= 0 && op.row_sum_wanted()) {
                    if (one_row) {
                        float total;
                        if (row_sum_last(partials[0], &arrived, op.acc, w, lane, total))
                            op.store_row_sum(slot, total);
                    } else {
                        const float total = row_sum_split(partials[parity], op.acc, w, lane);
                        if (w == 0)
                            op.store_row_sum(slot, total);
                        parity ^= 1;
                    }
                }
            }
        };

        typename Op::Buf A, B;
        int pk = 0, pj = 0, qk = 0, qj = 0;  // next item to load, next item to process
        prefetch(0, pk, pj, A);
        if constexpr (Op::kRowSum) {
            // one row per workgroup: zero the arrival count behind one barrier, taken by
            // all four waves (the row's slot and the op are the same for all of them)
            if (one_row && __builtin_amdgcn_readlane(slot_l, 0) >= 0 && op.row_sum_wanted())
                row_sum_last_init(&arrived, w, lane);
        }
        step(pk, pj);
        for (int t = 0; t < T; t += 2) {
            prefetch(t + 1, pk, pj, B);
            step(pk, pj);
            __builtin_amdgcn_sched_barrier(0);
            process(qk, qj, A);
            step(qk, qj);
            if (t + 1 >= T)
                break;
            prefetch(t + 2, pk, pj, A);
            step(pk, pj);
            __builtin_amdgcn_sched_barrier(0);
            process(qk, qj, B);
            step(qk, qj);
        }
    }
}

// The same two-buffer pipeline over `n_blocks` equal blocks of a flat array, with no
// per-row metadata: block b goes to wave b mod W. Op::load(buf, b, live) and
// Op::process(buf, b).
template <class Op>
__device__ __forceinline__ void walk_blocks(Op &op, int64_t n_blocks)
{
    const int64_t W = (int64_t)gridDim.x * kWavesPerBlock;
    const int64_t w = wave_id();
    if (w >= n_blocks)
        return;
    const int64_t T = (n_blocks - w + W - 1) / W;  // blocks of this wave
    auto block = [&](int64_t t) { return w + (t < T ? t : T - 1) * W; };
    typename Op::Buf A, B;
    op.load(A, block(0), true);
    for (int64_t t = 0; t < T; t += 2) {
        op.load(B, block(t + 1), t + 1 < T);
        op.process(A, block(t));
        if (t + 1 >= T)
            break;
        op.load(A, block(t + 2), t + 2 < T);
        op.process(B, block(t + 1));
    }
}

// ---------------------------------------------------------------------------
// Host side: launch sizing
// ---------------------------------------------------------------------------
// Workgroups per CU of a default launch: one (four waves, one per SIMD). Each wave
// keeps its next chunk's loads in flight while it computes the current one, and on
// MI355X's HBM3E more resident waves only add concurrent request streams: measured
// throughput of the activation at the 1.1 GB shape falls from ~6.0 TB/s at one
// workgroup per CU to ~5.6 TB/s at two to four.
constexpr int kLaunchBlocksPerCU = 1;

// Workgroups so that `units` (rows, blocks) split evenly over the waves: with at most
// M waves, rounds = ceil(units / M) and waves = ceil(units / rounds). M is the CU count
// times min(resident workgroups per CU, kLaunchBlocksPerCU) times four.
inline int balanced_workgroups(int64_t units, int cus, int resident_blocks_per_cu)
{
    int blocks_per_cu = resident_blocks_per_cu < kLaunchBlocksPerCU ? resident_blocks_per_cu
                                                                     : kLaunchBlocksPerCU;
    if (blocks_per_cu < 1)
        blocks_per_cu = 1;
    if (cus < 1)
        cus = 1;
    const int64_t max_waves = (int64_t)cus * blocks_per_cu * kWavesPerBlock;
    if (units <= 0)
        return 1;
    const int64_t rounds = (units + max_waves - 1) / max_waves;
    const int64_t waves = (units + rounds - 1) / rounds;
    return (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
}

// A dispatch packet holds the grid size in work-items as a 32-bit count, so a launch of
// kBlock-thread workgroups has at most this many. The walks stride over whatever the
// grid does not cover, so a capped grid gives the same result bits.
constexpr int kMaxWorkgroups = (int)(0xffffffffu / kBlock);  // 16,777,215

inline int cap_workgroups(int64_t n) { return n > kMaxWorkgroups ? kMaxWorkgroups : (int)n; }

// Default grid of a walk over `units` rows (or blocks) of `chunks` chunks each.
//   * Units of one or two chunks: one wave per unit, ceil(units / 4) workgroups (at
//     most kMaxWorkgroups), which the dispatcher starts as slots free up. The rows in
//     flight then stay one contiguous window of the arrays. Measured on MI355X at
//     53760 x 2048: activation
//     forward 6.38 and backward 6.28 TB/s, against 6.10 / 5.76 TB/s with one persistent
//     workgroup per CU; the plain streaming probe gains alike (2:1 6.26 -> 6.50, 3:2
//     6.15 -> 6.31 TB/s). Grids of 4 to 16 persistent workgroups per CU were slower
//     than either.
//   * Longer units: one persistent workgroup per CU (at most `resident_blocks_per_cu`),
//     balanced over the units, so each wave's two-buffer pipeline overlaps its own
//     chunks. For 7168-column rows (7 chunks) this was 2-4% faster than one wave per row.
// The grid depends only on host sizes, never on device data.
constexpr int64_t kPerWaveMaxChunks = 2;

inline int walk_workgroups(int64_t units, int64_t chunks, int cus, int resident_blocks_per_cu)
{
    if (units <= 0)
        return 1;
    if (chunks <= kPerWaveMaxChunks)
        return cap_workgroups((units + kWavesPerBlock - 1) / kWavesPerBlock);
    return balanced_workgroups(units, cus, resident_blocks_per_cu);
}

// Default grid of walk_row_split: one workgroup per row (at most kMaxWorkgroups) when
// the four waves share it (at least 4 chunks), else the walk_rows grid above. For the
// 7168-column MoE router rows this measured 6.19 / 6.28 TB/s (forward / backward)
// against 5.79 / 5.87 with one persistent workgroup per CU walking whole rows per wave.
inline int split_walk_workgroups(int64_t units, int64_t chunks, int cus, int resident_blocks_per_cu)
{
    if (units <= 0)
        return 1;
    if (chunks >= kWavesPerBlock)
        return cap_workgroups(units);
    return walk_workgroups(units, chunks, cus, resident_blocks_per_cu);
}

}  // namespace cdna4

#endif  // MBE_CDNA4_STREAM_H
