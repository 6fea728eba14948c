// Single-launch DSpark block drafting (Markov head, bf16, matrix cores):
// the whole left-to-right loop of Eq 4/5 (DSpark paper as transcribed on the
// dormouse "DSpark - paper verification" page, section 1) in one persistent
// kernel, with W2 loaded from HBM once per call instead of once per step.
//
//   persistent kernel, grid = every workgroup that can be resident:
//     start: the workgroups clear the argmax keys and the barrier words and
//           raise a per-call flag; before step 0 publishes anything, every
//           workgroup waits for all flags (see start_barrier_*)
//     load: wave w keeps W2 tile w (64 columns) in registers as MFMA
//           A-fragments; tiles beyond 4 x grid live, pre-transposed, in the
//           LDS of workgroup (tile - 4 x grid)
//     for k = 0 .. gamma-1:
//       every (tile, 16-block group): bias by MFMA from E = W1[x_{k-1}],
//         + U_k, Gumbel-max statistics (see unit_stats)
//       workgroup merge -> one 64-bit atomicMax per block on the
//         (perturbed logit, lowest index) key; softmax partials stored
//       grid barrier (8 arrival counters polled by every workgroup, bounded
//         spin, no cache flushes)
//       read x_k of every block from the keys; stage W1[x_k] for step k+1
//   finish (grid B)          x_k, log p_k from the partials, the Eq 7
//                            confidences c_k and the survival products S_k
//
// The only cross-workgroup dependency per step is the argmax over V; the
// softmax normaliser and the confidence head are computed after the loop.
#include <math.h>
#include <stdio.h>

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <mutex>
#include <vector>

#include "device_common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace dspark {

constexpr int kPWaves = 8;        // waves per workgroup (one workgroup per compute unit)
constexpr int kPThreads = kPWaves * kWave;
constexpr int kKeyStride = 16;    // uint64 per argmax key copy: one 128-byte line each
constexpr int kBarGroups = 8;     // arrival counters at bar[32 g]
constexpr int kTimeoutWord = 320; // set when a barrier wait gave up
static_assert(kTimeoutWord < kDraftBarWords, "barrier words");
constexpr int kMaxGamma = 64;     // largest gamma the C ABI accepts
// noise buffer: [block group][q = 0..3][threads][4 columns] floats, so that a
// thread's 4 terms of one Philox block are one 16-byte slot and the 64 slots
// of a wave's access are consecutive (conflict-free)
constexpr int kNoiseQStride = 4 * kPThreads;  // floats between the q slots of a thread

struct PersistArgs {
    const uint16_t* U;
    const uint16_t* W2;
    const uint16_t* W1;
    const uint16_t* w_conf;
    const int32_t* anchor;
    const float* temperature;
    const uint16_t* h;   // [B, gamma, d]
    int V, r, d, gamma, B, Bpad, nWG;
    uint32_t key0, key1, ctr3;
    uint64_t* best;      // [gamma, B, copies, 16]  argmax keys, one 128-byte line each (cleared at the start)
    uint32_t* bar;       // barrier words (cleared at the kernel's start)
    uint64_t* flags;     // [nWG + 1] start-barrier flags, then the start barrier's time-out slot
    uint64_t epoch;      // this call's flag value (never repeats within a process)
    uint32_t spin_limit; // polling rounds before a barrier wait gives up
    int fail_waits;      // test hook: every barrier wait gives up at once
    float2* pms;         // [gamma, B, nWG] softmax (max, sum) partials of every step, base 2
    int32_t* dead;       // [B]
    int32_t* tokens;
    float* logp;
    float* conf;
    float* survival;
};

// ---------------------------------------------------------- start barrier

// The workspace arrives with arbitrary contents, so the argmax keys and the
// barrier words are cleared inside the kernel, and one more barrier makes
// the clearing visible before anything uses them.  That barrier cannot use
// counters (they would need clearing first): each workgroup stores the
// call's epoch -- a value no earlier call in the process used -- in its own
// flag word, and waits until every flag holds it.  Stale flags hold older
// epochs, so they never pass.  All of it is device-scope atomics, like the
// step barrier below.
__device__ __forceinline__ void start_barrier_arrive(const PersistArgs& a, int n_keys) {
    const int wg = blockIdx.x;
    for (int i = wg * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x); i < n_keys;
         i += a.nWG * static_cast<int>(blockDim.x))
        __hip_atomic_store(a.best + static_cast<size_t>(i) * kKeyStride, kKeyNone, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    if (wg == 0)
        for (int i = threadIdx.x; i < kDraftBarWords; i += blockDim.x)
            __hip_atomic_store(a.bar + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // every wave's clearing stores complete before the flag is raised (a
    // late clear would otherwise overwrite a step-0 maximum)
    wait_vmem_complete();
    __syncthreads();
    if (threadIdx.x == 0) __hip_atomic_store(a.flags + wg, a.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait (first wave, each lane a few flags) until every workgroup's flag
// holds this call's epoch; bounded like the step barrier, with the time-out
// recorded in slot nWG (the finish kernel then marks every block invalid).
__device__ __forceinline__ void start_barrier_wait(const PersistArgs& a) {
    if (threadIdx.x < kWave) {
        uint32_t spins = 0;
        // (read here: kept live from the kernel's start it would take registers)
        uint64_t epoch = a.epoch;
        asm volatile("" : "+s"(epoch));
        if (a.fail_waits && threadIdx.x == 0)
            __hip_atomic_store(a.flags + a.nWG, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (!a.fail_waits) {
            bool late = false;
            for (int i = threadIdx.x; i < a.nWG; i += kWave)
                late |= __hip_atomic_load(a.flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != epoch;
            if (__ballot(late) == 0) break;
            __builtin_amdgcn_s_sleep(2);
            if (++spins > a.spin_limit) {
                if (threadIdx.x == 0)
                    __hip_atomic_store(a.flags + a.nWG, epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// ------------------------------------------------------- grid barrier

// Grid barrier number `step` (1, 2, ...), in two halves (below).
// Everything one workgroup hands
// to another inside this kernel is a device-scope atomic (the argmax keys and
// the barrier words; the softmax partials are only read after the kernel):
// those are coherent at the device level (sc1), so the barrier needs no L2
// write-back or invalidate, which on this chip flush or drop a whole XCD's L2
// and cost several microseconds each.  Before the arrival every wave waits
// until its own memory operations, the key atomics included, have completed
// (an explicit vmcnt wait: a workgroup-scope fence emits none), then the
// workgroup barrier; so when a workgroup sees the last arrival, every key
// maximum of the step is already in place.  Arrivals
// are spread over 8 counters to limit the contention on any one of them:
// workgroup wg adds 1 to counter wg % 8.  Every workgroup then polls all
// 8 counters at once (one device-scope load per lane of its first wave, a
// short sleep between rounds) until each holds `step` times its group's
// size.  Measured on the Qwen3-4B-shaped drafting workload this single
// level is about 1.3 us per step faster than counting the arrivals in two
// levels and publishing a release word, which puts two more dependent
// device-scope round trips after the last arrival; 16 or 32 counters, or
// one flag per workgroup, were no better.  The wait is bounded: after
// ~2^20 polling rounds the timeout word is set and the workgroup proceeds,
// so a broken launch cannot hang the device.
// The barrier in two halves, so that independent work (the next step's
// Gumbel terms) can run while the arrival's atomic is in flight:
// barrier_arrive (after the completion wait and a workgroup barrier) issues
// thread 0's add to its group counter; barrier_finish waits for all
// counters.
__device__ __forceinline__ void barrier_arrive(uint32_t* bar, uint32_t wg) {
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(bar + 32 * (wg % kBarGroups), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void barrier_finish(uint32_t* bar, uint32_t step, uint32_t nwg, uint32_t spin_limit,
                                               int fail_waits) {
    if (threadIdx.x < kWave) {
        // (opaque: the per-lane group size would otherwise be kept in a
        // register across the whole step loop)
        uint32_t l = threadIdx.x;
        asm volatile("" : "+v"(l));
        const uint32_t ngroups = nwg < kBarGroups ? nwg : kBarGroups;
        // group l holds the workgroups wg = l, l + 8, ... < nwg
        const uint32_t target = l < ngroups ? step * ((nwg - l + kBarGroups - 1) / kBarGroups) : 0u;
        uint32_t spins = 0;
        if (fail_waits && l == 0) __hip_atomic_store(bar + kTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        while (!fail_waits) {
            const uint32_t v =
                l < ngroups ? __hip_atomic_load(bar + 32 * l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
            if (__ballot(v < target) == 0) break;
            __builtin_amdgcn_s_sleep(2);
            if (++spins > spin_limit) {
                if (l == 0) __hip_atomic_store(bar + kTimeoutWord, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

// Slot of workgroup wg in the per-step partial arrays.  Workgroups are
// dealt to the 8 XCDs in turn (wg % 8), so slots are grouped by wg % 8: the
// partials one XCD writes fill whole cache lines instead of every eighth
// word of many lines.
__host__ __device__ __forceinline__ int partial_slot(int wg, int nwg) {
    const int x = wg % kBarGroups, per = nwg / kBarGroups, extra = nwg % kBarGroups;
    return x * per + (x < extra ? x : extra) + wg / kBarGroups;
}

// Device-scope (coherent) load of data other workgroups wrote in this kernel.
template <typename T>
__device__ __forceinline__ T get_shared(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------- the kernel

// Columns are split over the waves of the grid as follows: wave wv = 4 wg +
// wave keeps the 64 columns 64 wv .. 64 wv + 63 in registers (W2Tile), and
// the 16 columns C0 + 16 wv .. C0 + 16 wv + 15 (C0 = 256 x grid) in its own
// LDS area as one extra MFMA A-operand (XFrag): every wave then does the
// same work per (16-block group), 80 columns of it at full size.

// The 16-column W2 fragments of a workgroup's waves as MFMA A-operands:
// wave w's fragment covers columns c0 + 16 w .. c0 + 16 w + 15, and for
// chunk kc lane (g, n) keeps W2[32 kc + 8 g + e][c0 + 16 w + n], e = 0..7,
// i.e. row n of A is column c0 + 16 w + n; the MFMA result in lane (g, n) is
// then columns c0 + 16 w + 4 g + q (q = 0..3) of block row n.  The whole
// workgroup loads the (16 kPWaves) x r block once per call with 16-byte row
// loads (two rows per thread and pass) and writes each pair of rows as packed
// words into the transposed layout.  Columns >= V read 0 (V % 8 == 0).
//
// Lane L of wave w finds its 16 bytes of chunk kc at 16-byte slot
// kc * 64 + (L ^ w): with the slot index swizzled by the wave, the 64
// threads of one staging store (8 waves' columns x 4 row pairs) write 32
// distinct banks instead of 4, while a wave's operand reads stay one
// contiguous, conflict-free kilobyte.
__device__ __forceinline__ int xfrag_slot(int kc, int lane, int wave) { return kc * kWave + (lane ^ wave); }

template <int KC>
__device__ __forceinline__ void load_xfrags(const uint16_t* __restrict__ W2, int V, int c0, uint32_t* xf_all) {
    constexpr int kPairs = KC * 16;             // row pairs
    constexpr int kSegs = 2 * kPWaves;          // 8-column segments of the workgroup's 16 kPWaves columns
    const int cseg = threadIdx.x % kSegs;
    const int col = c0 + 8 * cseg;
    const bool ok = col < V;
    for (int rp = threadIdx.x / kSegs; rp < kPairs; rp += kPThreads / kSegs) {
        const size_t j0 = static_cast<size_t>(2 * rp);
        u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
        if (ok) {
            a = *reinterpret_cast<const u32x4*>(W2 + j0 * V + col);
            b = *reinterpret_cast<const u32x4*>(W2 + (j0 + 1) * V + col);
        }
        const int kc = rp >> 4, g = (rp >> 2) & 3, p = rp & 3;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int cc = 8 * cseg + q;  // column within the workgroup's 16 kPWaves
            const int w = cc >> 4, n = cc & 15;
            const uint32_t lo = (q & 1) ? (a[q >> 1] >> 16) : (a[q >> 1] & 0xFFFFu);
            const uint32_t hi = (q & 1) ? (b[q >> 1] & 0xFFFF0000u) : (b[q >> 1] << 16);
            xf_all[w * (KC * kWave * 4) + xfrag_slot(kc, 16 * g + n, w) * 4 + p] = lo | hi;
        }
    }
}

// acc[c] += bias from the register tile (when REG), accx += bias from the
// LDS fragment (when XW), for the 16 block rows whose E rows start at erow
// (this lane's row, offset 8 g).  The choice is a template parameter so the
// chunk loop is straight-line code: the LDS reads of two chunks are issued
// ahead of their matrix-core instructions instead of each waiting behind a
// branch.
template <int KC, bool REG, bool XW>
__device__ __forceinline__ void unit_mul(const W2Tile<KC>& w2, const uint32_t* xf, const uint16_t* erow, int lane,
                                         int wave, f32x4 (&acc)[4], f32x4& accx) {
    u32x4 ev[2], xv[2];
    auto fetch = [&](int kc, int slot) {
        ev[slot] = *reinterpret_cast<const u32x4*>(erow + kc * 32);
        if (XW) xv[slot] = *reinterpret_cast<const u32x4*>(&xf[xfrag_slot(kc, lane, wave) * 4]);
    };
    fetch(0, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, XW ? 2 : 1, 0);
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const int cur = kc & 1;
        if (kc + 1 < KC) fetch(kc + 1, cur ^ 1);
        const bf16x8 bop = __builtin_bit_cast(bf16x8, ev[cur]);
        if (REG) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 av = {w2.f[kc][c][0], w2.f[kc][c][1], w2.f[kc][c][2], w2.f[kc][c][3]};
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bop,
                                                                 acc[c], 0, 0, 0);
            }
        }
        if (XW) accx = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, xv[cur]), bop, accx, 0, 0, 0);
        // keep the order: the next chunk's LDS reads, then this chunk's
        // products (the reads then have the products' duration to land)
        if (kc + 1 < KC) __builtin_amdgcn_sched_group_barrier(0x100, XW ? 2 : 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, (REG ? 4 : 0) + (XW ? 1 : 0), 0);
    }
}

// Per-lane statistics of one unit, in base-2 units: the running maximum m
// of z2 = z log2(e) / T, sum of 2^(z2 - m), and the argmax key of the
// perturbed values.  The logit at the argmax is not carried: the finish
// kernel recomputes it from U, W1 and W2.
struct PStats {
    float m;
    float s;
    uint64_t key;
};

__device__ __forceinline__ PStats pstats_empty() { return PStats{-INFINITY, 0.0f, kKeyNone}; }

__device__ __forceinline__ PStats pstats_merge(const PStats& a, const PStats& b) {
    PStats r;
    r.m = fmaxf(a.m, b.m);
    const float sa = (a.s > 0.0f) ? a.s * __builtin_amdgcn_exp2f(a.m - r.m) : 0.0f;
    const float sb = (b.s > 0.0f) ? b.s * __builtin_amdgcn_exp2f(b.m - r.m) : 0.0f;
    r.s = sa + sb;
    r.key = b.key > a.key ? b.key : a.key;
    return r;
}

// pstats_merge of the statistics of lanes l and l ^ 16, l ^ 32 or l ^ 8 (the
// merge is commutative bit for bit: max, max, and one float sum)
__device__ __forceinline__ PStats pstats_of(uint32_t m, uint32_t s, uint32_t lo, uint32_t hi) {
    return PStats{__uint_as_float(m), __uint_as_float(s), (static_cast<uint64_t>(hi) << 32) | lo};
}
template <int X>
__device__ __forceinline__ PStats pstats_merge_xor(const PStats& a) {
    const uint32_t w[4] = {__float_as_uint(a.m), __float_as_uint(a.s), static_cast<uint32_t>(a.key),
                           static_cast<uint32_t>(a.key >> 32)};
    if (X == 8) {
        return pstats_merge(a, pstats_of(dpp_ror8(w[0]), dpp_ror8(w[1]), dpp_ror8(w[2]), dpp_ror8(w[3])));
    } else {
        LanePair p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) p[i] = X == 16 ? swap16(w[i]) : swap32(w[i]);
        return pstats_merge(pstats_of(p[0].a, p[1].a, p[2].a, p[3].a), pstats_of(p[0].b, p[1].b, p[2].b, p[3].b));
    }
}

// Statistics of the 20 logits z[j] of one lane (columns v0 + j for j < 16,
// vx + j - 16 after, ascending; a column that does not exist holds -inf).  Sampling: y = z2 -
// g with g[j] = log2(-log2 u), the Gumbel-max value up to a positive factor
// and a constant (see log2_of_neg_log2_uniform); greedy: y = z2.  The key
// takes the maximum y and the lowest column attaining it.
// The softmax reference is the largest perturbed value ŷ, not the largest
// scaled logit: z2 - ŷ <= g <= log2(24) for every column (u >= 2^-24), so no
// term of the sum overflows, and the winner's term is 2^g >= 2^-24, so the
// sum keeps its mass; greedy (g = 0) it is the plain maximum.
template <bool SAMPLING>
__device__ __forceinline__ PStats unit_stats(const float (&z)[20], const float (&g)[20], int v0, int vx,
                                             float scale) {
    float y[20];
#pragma unroll
    for (int j = 0; j < 20; ++j) y[j] = SAMPLING ? fmaf(z[j], scale, -g[j]) : z[j] * scale;
    float ybest = y[0];
#pragma unroll
    for (int j = 1; j < 20; ++j) ybest = fmaxf(ybest, y[j]);
    int idx = 19;
#pragma unroll
    for (int j = 18; j >= 0; --j) idx = (y[j] == ybest) ? j : idx;
    if (ybest == -INFINITY) return pstats_empty();  // no column of this lane exists
    const float m = ybest;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 20; ++j) s += __builtin_amdgcn_exp2f(fmaf(z[j], scale, -m));
    const int c = idx < 16 ? v0 + idx : vx + (idx - 16);
    return PStats{m, s, argmax_key(ybest, static_cast<uint32_t>(c))};
}

// The same statistics when the Gumbel terms are precomputed (g = 0 for a
// greedy block, so that y = z2 - g covers both cases without a branch), for
// the 20 accumulator values of a lane (absent columns already -inf).  The
// softmax reference is the lane's largest perturbed value ybest instead of
// the largest z2: z2 - ybest <= g <= log2(24) for every column, so no term
// of the sum overflows, and the largest term is at least 2^-24, so none of
// the mass is lost.  This saves the second maximum and keeps the code
// branch-free.
__device__ __forceinline__ PStats unit_stats_pre(const f32x4 (&acc)[4], const f32x4& accx, const float* gnu,
                                                 const float (&nx)[4], float scale, int v0, int vx) {
    float z[20], y[20];
    f32x4 gq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) gq[q] = *reinterpret_cast<const f32x4*>(gnu + q * kNoiseQStride);
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            z[4 * q + c] = acc[c][q];
            y[4 * q + c] = fmaf(acc[c][q], scale, -gq[q][c]);
        }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        z[16 + c] = accx[c];
        y[16 + c] = fmaf(accx[c], scale, -nx[c]);
    }
    float ybest = y[0];
#pragma unroll
    for (int j = 1; j < 20; ++j) ybest = fmaxf(ybest, y[j]);
    int idx = 19;
#pragma unroll
    for (int j = 18; j >= 0; --j) idx = (y[j] == ybest) ? j : idx;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 20; ++j) s += __builtin_amdgcn_exp2f(fmaf(z[j], scale, -ybest));
    const int c = idx < 16 ? v0 + idx : vx + (idx - 16);
    if (ybest == -INFINITY) return pstats_empty();  // no column of this lane exists
    return PStats{ybest, s, argmax_key(ybest, static_cast<uint32_t>(c))};
}

// U values of one unit, loaded one unit ahead of use: 16 columns of the
// register tile (two 16-byte loads) and the 4 columns of the LDS fragment.
// They become the initial MFMA accumulators, so z = U + E W2 comes out of
// the matrix cores directly.
struct UAhead {
    u32x4 a, b;
    uint2 x;
};

// LDS of one workgroup: [kPWaves LDS fragments][E rows][prev tokens]
// [temperatures][per-wave statistics slots][noise].  The E rows
// W1[x_{k-1}] are staged either all at once after each barrier, or
// (GROUPED, when all rows would not fit) 16 at a time in two buffers, the
// next group's rows loaded while the current group is computed.  Either way
// the MFMA operand comes from LDS, so its wait never covers the U loads
// still in flight.  AHEAD (B <= 32, at most two block groups): the Gumbel
// terms of every block group are computed while memory or other workgroups
// are busy -- under the W2 loads before step 0; at each step end after the
// barrier arrival, spread over the wait for the other workgroups, the key
// read and the W1 row loads -- and kept in LDS (16-byte slots, see
// kNoiseQStride) for the register-tile columns and in registers for the 4
// LDS-fragment columns.
constexpr size_t kPersistLdsMax = 160 * 1024;  // one workgroup per CU

template <int KC>
__host__ __device__ constexpr size_t persist_xfrag_bytes() {
    return static_cast<size_t>(kPWaves) * KC * kWave * 16;
}
template <int KC>
__host__ __device__ constexpr size_t persist_e_bytes(int rows) {
    return static_cast<size_t>(rows) * (KC * 32 + 8) * 2;
}
constexpr size_t kNoiseBytesPerGroup = 4 * kNoiseQStride * 4;
template <int KC>
__host__ __device__ constexpr size_t persist_lds(int Bpad, int B, bool grouped, bool ahead) {
    return persist_xfrag_bytes<KC>() + persist_e_bytes<KC>(grouped ? 32 : Bpad) +
           2 * align_up(static_cast<size_t>(Bpad) * 4, 16) +
           align_up(sizeof(PStats) * kPWaves * static_cast<size_t>(B), 16) +
           (ahead ? (Bpad / 16) * kNoiseBytesPerGroup : 0);
}

template <int KC, bool GROUPED, bool AHEAD>
__global__ __launch_bounds__(kPThreads, 1) void k_draft_persistent(PersistArgs a) {
    static_assert(!(GROUPED && AHEAD), "noise ahead needs all E rows staged");
    constexpr int r = KC * 32;
    constexpr int ldE = r + 8;  // padded row stride of the staged E rows (bank spread)
    constexpr int kGroupChunks = 16 * (r / 8);                       // 16-byte pieces of 16 rows
    constexpr int kStage = (kGroupChunks + kPThreads - 1) / kPThreads;  // per thread
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const size_t e_bytes = persist_e_bytes<KC>(GROUPED ? 32 : a.Bpad);
    const size_t bp4 = align_up(static_cast<size_t>(a.Bpad) * 4, 16);
    uint16_t* Es = reinterpret_cast<uint16_t*>(smem + persist_xfrag_bytes<KC>());
    int32_t* prev = reinterpret_cast<int32_t*>(smem + persist_xfrag_bytes<KC>() + e_bytes);
    // per block: log2(e) / T when the block samples (T > 0), -log2(e) when greedy
    float* scale_s = reinterpret_cast<float*>(smem + persist_xfrag_bytes<KC>() + e_bytes + bp4);
    PStats* slot = reinterpret_cast<PStats*>(smem + persist_xfrag_bytes<KC>() + e_bytes + 2 * bp4);
    float* gn = reinterpret_cast<float*>(smem + persist_xfrag_bytes<KC>() + e_bytes + 2 * bp4 +
                                         align_up(sizeof(PStats) * kPWaves * static_cast<size_t>(a.B), 16)) +
                4 * threadIdx.x;  // this thread's noise slot

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // scalar: wave-uniform branches
    const int n = lane & 15, g = lane >> 4;
    const int wg = blockIdx.x, nWG = a.nWG;
    const int NB = a.Bpad / 16;
    const int wv = wg * kPWaves + wave;
    uint32_t* xf = reinterpret_cast<uint32_t*>(smem) + wave * (KC * kWave * 4);

    // this wave's columns: register tile (16 per lane) and LDS fragment (4 per lane)
    const int v0 = wv * 64 + 16 * g;
    const int c0 = kPWaves * nWG * 64 + 16 * wv;
    const int vx = c0 + 4 * g;
    const bool has_reg = wv * 64 < a.V, has_x = c0 < a.V;
    const bool reg_live = v0 < a.V, x_live = vx < a.V;

    const bool active = has_reg || has_x;
    // AHEAD: Gumbel terms of block group nb at step kk (zero when the
    // block is greedy, on = false): the 16 register-tile columns into LDS,
    // the 4 LDS-fragment columns into registers (nx0 / nx1)
    float nx0[4] = {0.0f, 0.0f, 0.0f, 0.0f}, nx1[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    auto noise_ahead = [&](int kk, int nb, bool on, int q0 = 0, int q1 = 4, bool with_x = true) {
        const int b = nb * 16 + n;
        if (!AHEAD || b >= a.B) return;
        // the counter words are opaque here, so that the compiler does not
        // keep products of the first Philox round (which do not depend on
        // the step) live across the whole loop
        uint32_t cb = static_cast<uint32_t>(b), cv = static_cast<uint32_t>(v0) >> 2;
        asm volatile("" : "+v"(cb), "+v"(cv));
        if (reg_live) {
            float* dst = gn + nb * 4 * kNoiseQStride;
#pragma unroll 2  // two independent Philox blocks at a time: their rounds interleave
            for (int q = q0; q < q1; ++q) {
                const u32x4 w = philox4x32_10(u32x4{cv + static_cast<uint32_t>(q), static_cast<uint32_t>(kk), cb, a.ctr3},
                                              a.key0, a.key1);
                f32x4 gv;
#pragma unroll
                for (int c = 0; c < 4; ++c) gv[c] = on ? log2_of_neg_log2_uniform(w[c]) : 0.0f;
                *reinterpret_cast<f32x4*>(dst + q * kNoiseQStride) = gv;
            }
        }
        if (with_x && x_live) {
            uint32_t cx = static_cast<uint32_t>(vx) >> 2;
            asm volatile("" : "+v"(cx));
            const u32x4 w = philox4x32_10(u32x4{cx, static_cast<uint32_t>(kk), cb, a.ctr3}, a.key0, a.key1);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float gx = on ? log2_of_neg_log2_uniform(w[c]) : 0.0f;
                if (nb == 0)
                    nx0[c] = gx;
                else
                    nx1[c] = gx;
            }
        }
    };

    start_barrier_arrive(a, a.gamma * a.B * kDraftKeyCopies);
    // Waves w and w + 4 share a SIMD: the second starts its tile loads a
    // little later and products are issued at raised priority (see
    // mul_any), so that one wave's matrix-core work tends to overlap the
    // other's statistics (about 1 us per call at the Qwen3-4B shape).
    if (wave >= 4) __builtin_amdgcn_s_sleep(8);
    W2Tile<KC> w2;
    if (has_reg) w2.load(a.W2, a.V, wv * 64, g, n);
    // while the tile loads are in flight
    noise_ahead(0, 0, AHEAD && n < a.B && a.temperature[n] > 0.0f);
    noise_ahead(0, 1, AHEAD && 16 + n < a.B && a.temperature[16 + n] > 0.0f);
    load_xfrags<KC>(a.W2, a.V, kPWaves * nWG * 64 + 16 * kPWaves * wg, reinterpret_cast<uint32_t*>(smem));
    // previous tokens of step 0: the anchors (an out-of-range anchor reads
    // row 0; the finish kernel marks its block invalid)
    for (int b = threadIdx.x; b < a.Bpad; b += blockDim.x) {
        const int x = b < a.B ? a.anchor[b] : 0;
        prev[b] = (x >= 0 && x < a.V) ? x : 0;
        const float t = b < a.B ? a.temperature[b] : 0.0f;
        scale_s[b] = t > 0.0f ? kLog2e / t : -kLog2e;
    }
    __syncthreads();
    // E rows W1[prev[b]] of the coming step: all rows (or, GROUPED, the
    // first group into buffer 0), then a workgroup barrier
    auto stage_rows = [&]() {
        const int chunks = (GROUPED ? 16 : a.Bpad) * (r / 8);
        for (int t = threadIdx.x; t < chunks; t += blockDim.x) {
            const int row = t / (r / 8), col = t % (r / 8);
            *reinterpret_cast<u32x4*>(&Es[row * ldE + col * 8]) =
                *reinterpret_cast<const u32x4*>(a.W1 + static_cast<size_t>(prev[row]) * r + col * 8);
        }
        __syncthreads();
    };
    // AHEAD (Bpad <= 32): the same in two halves, every load issued
    // first (rows_issue), the stores and the barrier later (rows_store), so
    // that other work can run while the loads are in flight
    constexpr int kMaxChunks = (32 * (r / 8) + kPThreads - 1) / kPThreads;
    u32x4 e[kMaxChunks];
    auto rows_issue = [&]() {
        const int chunks = a.Bpad * (r / 8);
#pragma unroll
        for (int i = 0; i < kMaxChunks; ++i) {
            const int t = (threadIdx.x + kPThreads * i) % chunks;  // unconditional: stays in flight
            const int row = t / (r / 8), col = t % (r / 8);
            e[i] = *reinterpret_cast<const u32x4*>(a.W1 + static_cast<size_t>(prev[row]) * r + col * 8);
        }
    };
    auto rows_store = [&]() {
        const int chunks = a.Bpad * (r / 8);
#pragma unroll
        for (int i = 0; i < kMaxChunks; ++i) {
            const int t = threadIdx.x + kPThreads * i;
            if (t < chunks) {
                const int row = t / (r / 8), col = t % (r / 8);
                *reinterpret_cast<u32x4*>(&Es[row * ldE + col * 8]) = e[i];
            }
        }
        __syncthreads();
    };
    // GROUPED: rows of block group nb, loaded into registers two units
    // before their unit (the gathered rows come from anywhere in W1, and a
    // greedy unit is shorter than that load) ...
    u32x4 staged0[kStage], staged1[kStage];  // groups of even / odd index
    auto load_group = [&](int nb, u32x4 (&dst)[kStage]) {
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int t = threadIdx.x + kPThreads * i;
            if (t < kGroupChunks) {
                const int row = t / (r / 8), col = t % (r / 8);
                dst[i] = *reinterpret_cast<const u32x4*>(a.W1 + static_cast<size_t>(prev[nb * 16 + row]) * r +
                                                         col * 8);
            }
        }
    };
    // ... and stored to buffer nb % 2 once the unit before it is done
    auto store_group = [&](int nb, const u32x4 (&src)[kStage]) {
        uint16_t* buf = Es + (nb & 1) * 16 * ldE;
#pragma unroll
        for (int i = 0; i < kStage; ++i) {
            const int t = threadIdx.x + kPThreads * i;
            if (t < kGroupChunks) {
                const int row = t / (r / 8), col = t % (r / 8);
                *reinterpret_cast<u32x4*>(&buf[row * ldE + col * 8]) = src[i];
            }
        }
    };
    // U of unit (step kk, block group nb), issued one unit ahead of its use.
    // The loads are unconditional, from addresses clamped into U (values of
    // padding blocks and of columns past V are never used), so the compiler
    // can leave them in flight across the unit instead of waiting at once.
    const int ua = reg_live ? v0 : 0, ub = (reg_live && v0 + 8 < a.V) ? v0 + 8 : ua;
    const int ux = x_live ? vx : 0;
    auto fetch_u = [&](int kk, int nb) {
        UAhead p;
        const int b = min(nb * 16 + n, a.B - 1);
        const uint16_t* row = a.U + (static_cast<size_t>(b) * a.gamma + kk) * a.V;
        p.a = *reinterpret_cast<const u32x4*>(row + ua);
        p.b = *reinterpret_cast<const u32x4*>(row + ub);
        p.x = *reinterpret_cast<const uint2*>(row + ux);
        return p;
    };
    stage_rows();
    UAhead ahead = fetch_u(0, 0);
    // GROUPED: U is loaded two units ahead, units of even index through
    // `ahead`, of odd index through `ahead1` (NB >= 3 there)
    UAhead ahead1 = GROUPED ? fetch_u(0, 1) : ahead;

    // accumulators start from U (bf16 -> f32 is exact)
    auto acc_from = [&](const UAhead& u, f32x4 (&acc)[4], f32x4& accx) {
        const uint32_t w[8] = {u.a[0], u.a[1], u.a[2], u.a[3], u.b[0], u.b[1], u.b[2], u.b[3]};
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * q + c;
                acc[c][q] = (j & 1) ? hi_bf16(w[j >> 1]) : lo_bf16(w[j >> 1]);
            }
        accx = f32x4{lo_bf16(u.x.x), hi_bf16(u.x.x), lo_bf16(u.x.y), hi_bf16(u.x.y)};
    };
    auto erow_of = [&](int nb) -> const uint16_t* {
        return GROUPED ? &Es[((nb & 1) * 16 + n) * ldE + 8 * g] : &Es[(nb * 16 + n) * ldE + 8 * g];
    };
    // bias of one unit on the matrix cores, for whichever column parts the
    // wave has (has_x implies has_reg: the fragment columns start past all
    // tiles), issued at raised wave priority
    auto mul_any = [&](int nb, f32x4 (&acc)[4], f32x4& accx) {
        __builtin_amdgcn_s_setprio(2);
        if (has_x)
            unit_mul<KC, true, true>(w2, xf, erow_of(nb), lane, wave, acc, accx);
        else if (has_reg)
            unit_mul<KC, true, false>(w2, xf, erow_of(nb), lane, wave, acc, accx);
    };
    // lane statistics of a unit for any wave: absent columns hold -inf
    auto any_stats = [&](int kk, int nb, const f32x4 (&acc)[4], const f32x4& accx) {
        const int b = nb * 16 + n;
        PStats st = pstats_empty();
        if (active && b < a.B) {
            const float sc = scale_s[b];
            const bool sampling = sc > 0.0f;
            const float scale = fabsf(sc);
            // the lane's 16 register-tile columns and 4 LDS-fragment
            // columns; columns past V (V % 8 == 0) and absent parts hold -inf
            const bool reg_hi = reg_live && v0 + 16 <= a.V;
            float z[20];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const bool ok = q < 2 ? reg_live : reg_hi;
                    z[4 * q + c] = ok ? acc[c][q] : -INFINITY;
                }
#pragma unroll
            for (int c = 0; c < 4; ++c) z[16 + c] = x_live ? accx[c] : -INFINITY;
            if (sampling) {
                float gs[20];
#pragma unroll
                for (int q = 0; q < 5; ++q) {
                    const int cq = q < 4 ? v0 + 4 * q : vx;
                    const u32x4 w = philox4x32_10(u32x4{static_cast<uint32_t>(cq) >> 2, static_cast<uint32_t>(kk),
                                                        static_cast<uint32_t>(b), a.ctr3},
                                                  a.key0, a.key1);
#pragma unroll
                    for (int c = 0; c < 4; ++c) gs[4 * q + c] = log2_of_neg_log2_uniform(w[c]);
                }
                st = unit_stats<true>(z, gs, v0, vx, scale);
            } else {
                float gs[20];
#pragma unroll
                for (int j = 0; j < 20; ++j) gs[j] = 0.0f;
                st = unit_stats<false>(z, gs, v0, vx, scale);
            }
        }
        return st;
    };
    // the unit's statistics over the 4 lanes of each block row, into this
    // wave's slot of each block (written once per step: every unit covers
    // other blocks)
    auto to_slot = [&](PStats st, int nb) {
        const int b = nb * 16 + n;
        st = pstats_merge_xor<16>(st);
        st = pstats_merge_xor<32>(st);
        if (g == 0 && b < a.B) slot[wave * a.B + b] = st;
    };

    // wave-uniform: every column of the wave's register tile and LDS
    // fragment exists
    const bool full = has_x && c0 + 16 <= a.V;

    // One unit: step kk, block group nb (16 blocks): accumulators from U
    // (held in u), bias on the matrix cores, lane statistics, merged into
    // this wave's slots.  u then receives the U of a later unit of the step:
    // the next one, or (GROUPED) the one after it.
    auto run_unit = [&](int kk, int nb, UAhead& u) {
        f32x4 acc[4], accx;
        acc_from(u, acc, accx);
        // (the next step's first units are fetched after the barrier
        // arrival: a load in flight at the arrival's completion wait would
        // be waited for)
        if (GROUPED) {
            if (nb + 2 < NB) u = fetch_u(kk, nb + 2);
        } else if (nb + 1 < NB) {
            u = fetch_u(kk, nb + 1);
        }
        mul_any(nb, acc, accx);
        __builtin_amdgcn_s_setprio(0);
        PStats st;
        if (AHEAD) {
            if (active) {
                // (the noise reads stay after the products: hoisted into
                // them they would hold registers the tile needs)
                __builtin_amdgcn_sched_barrier(0);
                if (!full) {
                    // columns past V (V % 8 == 0) and absent parts: -inf
                    const bool reg_hi = reg_live && v0 + 16 <= a.V;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            if (!(q < 2 ? reg_live : reg_hi)) acc[c][q] = -INFINITY;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (!x_live) accx[c] = -INFINITY;
                }
                st = unit_stats_pre(acc, accx, gn + nb * 4 * kNoiseQStride, nb == 0 ? nx0 : nx1,
                                    fabsf(scale_s[nb * 16 + n]), v0, vx);
            } else {
                st = pstats_empty();
            }
        } else {
            st = any_stats(kk, nb, acc, accx);
        }
        to_slot(st, nb);
    };
    // Workgroup merge of blocks [b0, b1), then publish: the argmax key
    // atomics and the softmax partials (read after the kernel).  Each wave
    // takes 8 blocks at a time: lane l reads wave l / 8's slot of block
    // l % 8 (consecutive lanes, consecutive slots), and three exchange
    // steps (lane distance 8, 16, 32) merge the 8 waves' slots in a fixed
    // tree order.
    auto publish = [&](int kk, int b0, int b1) {
        __syncthreads();
        const int groups = (b1 - b0 + 7) / 8;
        for (int q = wave; q < groups; q += kPWaves) {  // wave-uniform trip count
            const int b = b0 + 8 * q + (lane & 7), w = lane >> 3;
            PStats t = b < b1 ? slot[w * a.B + b] : pstats_empty();
            t = pstats_merge_xor<8>(t);
            t = pstats_merge_xor<16>(t);
            t = pstats_merge_xor<32>(t);
            if (w == 0 && b < b1) {
                if (t.key != kKeyNone)
                    __hip_atomic_fetch_max(&a.best[((static_cast<size_t>(kk) * a.B + b) * kDraftKeyCopies +
                                                    wg % kDraftKeyCopies) * kKeyStride],
                                           t.key, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                const size_t o = (static_cast<size_t>(kk) * a.B + b) * nWG + partial_slot(wg, nWG);
                a.pms[o] = make_float2(t.m, t.s);
            }
        }
    };
    // x_kk of blocks [b0, b1) from the keys: the copies of a block's key sit
    // in 8 consecutive lanes (b0 is a multiple of 16)
    auto read_keys = [&](int kk, int b0, int b1) {
        static_assert(kDraftKeyCopies == 8, "copies merged by max_key8");
        auto finish_key = [&](int t, uint64_t key) {
            key = max_key8(key);
            const uint32_t x = key_index(key);
            if (t < b1 * kDraftKeyCopies && t % kDraftKeyCopies == 0)
                prev[t / kDraftKeyCopies] = (key != kKeyNone && x < static_cast<uint32_t>(a.V)) ? static_cast<int>(x) : 0;
        };
        const size_t base = static_cast<size_t>(kk) * a.B * kDraftKeyCopies;
        for (int t = b0 * kDraftKeyCopies + static_cast<int>(threadIdx.x); t < b1 * kDraftKeyCopies; t += blockDim.x)
            finish_key(t, get_shared(&a.best[(base + t) * kKeyStride]));
        __syncthreads();
    };
    // AHEAD (B * copies <= 256 < threads): the same in two halves, the load
    // of one key copy per thread first (keys_issue), the merge, prev[] and
    // the barrier later (keys_finish)
    auto keys_issue = [&](int kk) -> uint64_t {
        const int t = threadIdx.x;
        const size_t base = static_cast<size_t>(kk) * a.B * kDraftKeyCopies;
        return t < a.B * kDraftKeyCopies ? get_shared(&a.best[(base + t) * kKeyStride]) : kKeyNone;
    };
    auto keys_finish = [&](uint64_t key) {
        const int t = threadIdx.x;
        key = max_key8(key);
        const uint32_t x = key_index(key);
        if (t < a.B * kDraftKeyCopies && t % kDraftKeyCopies == 0)
            prev[t / kDraftKeyCopies] = (key != kKeyNone && x < static_cast<uint32_t>(a.V)) ? static_cast<int>(x) : 0;
        __syncthreads();
    };

    for (int k = 0; k < a.gamma; ++k) {
        // every wave runs all NB units (GROUPED stages rows between
        // them); waves without columns skip the arithmetic
        if (GROUPED) {
            // unit nb loads group nb + 2 into the registers group nb came
            // through (its rows are in LDS by then) and stores group nb + 1;
            // the loop runs two units per trip so that both register sets
            // are named at compile time
            if (NB > 1) load_group(1, staged1);
            auto grouped_unit = [&](int nb, u32x4 (&nxt2)[kStage], const u32x4 (&nxt1)[kStage], UAhead& u) {
                if (nb + 2 < NB) load_group(nb + 2, nxt2);
                run_unit(k, nb, u);
                if (nb + 1 < NB) {
                    store_group(nb + 1, nxt1);
                    __syncthreads();
                }
            };
            for (int nb = 0; nb < NB; nb += 2) {
                grouped_unit(nb, staged0, staged1, ahead);
                if (nb + 1 < NB) grouped_unit(nb + 1, staged1, staged0, ahead1);
            }
        } else {
            for (int nb = 0; nb < NB; ++nb) run_unit(k, nb, ahead);
        }
        // the keys and barrier words are cleared everywhere before step 0
        // publishes or arrives (step 0's units do not touch them, so the
        // wait runs after them)
        if (k == 0) start_barrier_wait(a);
        publish(k, 0, a.B);
        if (k + 1 == a.gamma) break;  // the last keys are read after the kernel
        if (AHEAD) {
            // The next step's Gumbel terms fill the waits of the step's end,
            // all after the arrival: the completion wait for the key
            // atomics comes first (a workgroup that arrives earlier lets the
            // barrier complete earlier), then group 0's terms and half of
            // group 1's while the arrivals spread (about 2 us from a
            // workgroup's own arrival to the last one being seen), the rest
            // of group 1's register-tile terms while the keys are read, and
            // its fragment terms while the W1 rows load.
            const bool on0 = scale_s[n] > 0.0f, on1 = 16 + n < a.B && scale_s[16 + n] > 0.0f;
            wait_vmem_complete();
            __syncthreads();
            barrier_arrive(a.bar, static_cast<uint32_t>(wg));
            ahead = fetch_u(k + 1, 0);
            noise_ahead(k + 1, 0, on0);
            noise_ahead(k + 1, 1, on1, 0, 2, false);
            barrier_finish(a.bar, static_cast<uint32_t>(k + 1), static_cast<uint32_t>(nWG), a.spin_limit, a.fail_waits);
            const uint64_t key = keys_issue(k);
            noise_ahead(k + 1, 1, on1, 2, 4, false);
            keys_finish(key);
            rows_issue();
            noise_ahead(k + 1, 1, on1, 0, 0, true);
            rows_store();
        } else {
            wait_vmem_complete();
            __syncthreads();
            barrier_arrive(a.bar, static_cast<uint32_t>(wg));
            ahead = fetch_u(k + 1, 0);
            if (GROUPED) ahead1 = fetch_u(k + 1, 1);
            barrier_finish(a.bar, static_cast<uint32_t>(k + 1), static_cast<uint32_t>(nWG), a.spin_limit, a.fail_waits);
            read_keys(k, 0, a.B);
            stage_rows();
        }
    }
}

// --------------------------------------------------------------- finish

constexpr int kFinishWaves = 8;

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// sum over j < n of x[j] * y[j] (bf16), lane-strided, 8 elements per load
// when both rows are 16-byte aligned; partial sum of this lane.
__device__ __forceinline__ float lane_dot_bf16(const uint16_t* x, const uint16_t* y, int n, int lane) {
    float acc = 0.0f;
    if (n % 8 == 0 && (reinterpret_cast<uintptr_t>(x) & 15) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0) {
#pragma unroll 4
        for (int c = lane; c < n / 8; c += kWave) {
            const u32x4 a = *reinterpret_cast<const u32x4*>(x + 8 * c);
            const u32x4 b = *reinterpret_cast<const u32x4*>(y + 8 * c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fmaf(lo_bf16(a[q]), lo_bf16(b[q]), acc);
                acc = fmaf(hi_bf16(a[q]), hi_bf16(b[q]), acc);
            }
        }
    } else {
#pragma unroll 4
        for (int j = lane; j < n; j += kWave) acc = fmaf(bf16_to_f32(x[j]), bf16_to_f32(y[j]), acc);
    }
    return acc;
}

// Workgroup b, after the loop.  Wave w handles positions k = w, w + 8, ...:
// x_k from the argmax keys, log p_k = (z2 - m) ln 2 - ln s from the step's
// base-2 (max, sum) partials (merged lane-strided, then across the wave) and
// z2 = z log2(e) / T, the scaled logit of x_k, recovered as the key's
// perturbed value plus the Gumbel term of (x_k, k, b) (zero when greedy) --
// the very sum the drafting kernel formed, so no column of W2 is re-read --
// and c_k = sigma(w[0:d] . h_{b,k} + w[d:d+r] . W1[x_{k-1}]) (Eq 7, x_{-1} =
// the anchor); then S_k = c_0 ... c_k in position order.  A block is invalid from its first position whose
// previous token is out of range, or entirely when a grid barrier gave up.
// Loads of the finish kernel held in registers so that they are issued
// before the keys are known: the partials of up to 4 x 64 workgroups and the
// h / w_conf operands of up to 12 x 64 16-byte chunks (d <= 6144).
constexpr int kFinPms = 4;
constexpr int kFinDot = 12;

__global__ __launch_bounds__(kFinishWaves * kWave) void k_persist_finish(PersistArgs a) {
    __shared__ int xs[kMaxGamma + 1];  // xs[0] = anchor, xs[k + 1] = x_k
    __shared__ float ys[kMaxGamma];    // perturbed value at x_k (scaled units)
    __shared__ float cs[kMaxGamma];
    __shared__ int first_bad_s, timed_out_s;
    const int b = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;

    // The first position of each wave (k = wave): its softmax partials and
    // the h_{b,k} . w[0:d] operands do not depend on the keys, so they are
    // loaded before the keys are read; only the W1 row of x_{k-1} waits.
    const int k0 = wave;
    const uint16_t* hrow0 = a.h + (static_cast<size_t>(b) * a.gamma + (k0 < a.gamma ? k0 : 0)) * a.d;
    const bool pre = k0 < a.gamma && a.nWG <= kFinPms * kWave && a.d % 8 == 0 && a.d / 8 <= kFinDot * kWave &&
                     (reinterpret_cast<uintptr_t>(a.w_conf) & 15) == 0 && (reinterpret_cast<uintptr_t>(hrow0) & 15) == 0;
    float2 q[kFinPms];
    u32x4 hw[kFinDot], hh[kFinDot];
    if (pre) {
        const size_t base = (static_cast<size_t>(k0) * a.B + b) * a.nWG;
#pragma unroll
        for (int i = 0; i < kFinPms; ++i) {
            const int p = lane + kWave * i;
            q[i] = p < a.nWG ? a.pms[base + p] : make_float2(-INFINITY, 0.0f);
        }
#pragma unroll
        for (int i = 0; i < kFinDot; ++i) {
            const int c = lane + kWave * i;
            if (c < a.d / 8) {
                hw[i] = *reinterpret_cast<const u32x4*>(a.w_conf + 8 * c);
                hh[i] = *reinterpret_cast<const u32x4*>(hrow0 + 8 * c);
            }
        }
    }
    if (wave == 0) {
        bool inval = false;
        if (lane < a.gamma) {
            uint64_t key = kKeyNone;
            for (int c = 0; c < kDraftKeyCopies; ++c) {
                const uint64_t kc = a.best[((static_cast<size_t>(lane) * a.B + b) * kDraftKeyCopies + c) * kKeyStride];
                key = kc > key ? kc : key;
            }
            const uint32_t x = key_index(key);
            inval = key == kKeyNone || x >= static_cast<uint32_t>(a.V);
            xs[lane + 1] = static_cast<int>(x);
            // the float back from the order-preserving key bits
            const uint32_t kb = static_cast<uint32_t>(key >> 32);
            ys[lane] = __uint_as_float((kb & 0x80000000u) ? (kb ^ 0x80000000u) : ~kb);
        }
        const int x0 = a.anchor[b];
        const uint64_t m = __ballot(inval);
        const bool timed_out = a.bar[kTimeoutWord] != 0 || a.flags[a.nWG] == a.epoch;
        const bool head_bad = timed_out || x0 < 0 || x0 >= a.V;
        if (lane == 0) {
            xs[0] = x0;
            timed_out_s = timed_out ? 1 : 0;
            first_bad_s = head_bad ? 0 : (m ? __ffsll(static_cast<unsigned long long>(m)) - 1 : a.gamma);
        }
    }
    // (max, sum) over all workgroups, lane-strided then across the wave
    auto merge_pms = [&](float& m, float& sum, const float2 qq) {
        const float mm = fmaxf(m, qq.x);
        sum = (sum > 0.0f ? sum * __builtin_amdgcn_exp2f(m - mm) : 0.0f) +
              (qq.y > 0.0f ? qq.y * __builtin_amdgcn_exp2f(qq.x - mm) : 0.0f);
        m = mm;
    };
    auto wave_merge = [&](float& m, float& sum) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(sum, o);
            const float mm = fmaxf(m, m2);
            sum = (sum > 0.0f ? sum * __builtin_amdgcn_exp2f(m - mm) : 0.0f) +
                  (s2 > 0.0f ? s2 * __builtin_amdgcn_exp2f(m2 - mm) : 0.0f);
            m = mm;
        }
    };
    float m0 = -INFINITY, sum0 = 0.0f, part0 = 0.0f;
    if (pre) {
        // (a partial of a missing workgroup is (-inf, 0): merging it changes nothing)
#pragma unroll
        for (int i = 0; i < kFinPms; ++i) merge_pms(m0, sum0, q[i]);
        wave_merge(m0, sum0);
#pragma unroll
        for (int i = 0; i < kFinDot; ++i) {
            if (lane + kWave * i < a.d / 8) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    part0 = fmaf(lo_bf16(hw[i][j]), lo_bf16(hh[i][j]), part0);
                    part0 = fmaf(hi_bf16(hw[i][j]), hi_bf16(hh[i][j]), part0);
                }
            }
        }
    }
    __syncthreads();
    const int first_bad = first_bad_s;
    for (int k = wave; k < a.gamma; k += kFinishWaves) {
        const bool bad = k >= first_bad;
        float m = m0, sum = sum0, part = part0;
        if (!(pre && k == k0)) {
            const size_t base = (static_cast<size_t>(k) * a.B + b) * a.nWG;
            m = -INFINITY;
            sum = 0.0f;
            for (int p = lane; p < a.nWG; p += kWave) merge_pms(m, sum, a.pms[base + p]);
            wave_merge(m, sum);
            part = lane_dot_bf16(a.w_conf, a.h + (static_cast<size_t>(b) * a.gamma + k) * a.d, a.d, lane);
        }
        const uint32_t xk = bad ? 0u : static_cast<uint32_t>(xs[k + 1]);  // in range unless bad
        float g2 = 0.0f;
        if (a.temperature[b] > 0.0f) {
            const u32x4 w = philox4x32_10(u32x4{xk >> 2, static_cast<uint32_t>(k), static_cast<uint32_t>(b), a.ctr3},
                                          a.key0, a.key1);
            const uint32_t qi = xk & 3u;
            g2 = log2_of_neg_log2_uniform(qi == 0 ? w[0] : qi == 1 ? w[1] : qi == 2 ? w[2] : w[3]);
        }
        const float zx = ys[k] + g2;
        if (!bad) part += lane_dot_bf16(a.w_conf + a.d, a.W1 + static_cast<size_t>(xs[k]) * a.r, a.r, lane);
        const float logit = wave_sum(part);
        if (lane == 0) {
            const size_t out = static_cast<size_t>(b) * a.gamma + k;
            a.tokens[out] = bad ? -1 : xs[k + 1];
            if (a.logp) a.logp[out] = bad ? NAN : (zx - m) * kLn2 - logf(sum);
            cs[k] = bad ? NAN : sigmoidf_(logit);
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float S = 1.0f;
        for (int k = 0; k < a.gamma; ++k) {
            const size_t out = static_cast<size_t>(b) * a.gamma + k;
            S *= cs[k];
            a.conf[out] = cs[k];
            a.survival[out] = S;
        }
        // 2: a grid barrier gave up (every block of the call), 1: a token
        // id out of range in this block
        a.dead[b] = timed_out_s ? 2 : (first_bad < a.gamma ? 1 : 0);
    }
}

// ---------------------------------------------------------------- launch

struct PersistPlan {
    bool ok = false;
    bool grouped = false;
    bool ahead = false;
    int nWG = 0;
    size_t lds = 0;
};

template <int KC>
static void (*persist_kernel(bool grouped, bool ahead))(PersistArgs) {
    if (grouped) return k_draft_persistent<KC, true, false>;
    return ahead ? k_draft_persistent<KC, false, true> : k_draft_persistent<KC, false, false>;
}

// Device facts a plan needs, cached per (device, kernel, LDS bytes): the
// compute-unit count and the occupancy answer do not change while the
// process runs, and asking the runtime again on every call costs host time
// on a path that is otherwise a single launch.  The kernel's dynamic-LDS
// limit is raised to the most any plan uses once per (device, kernel), so a
// smaller plan met first cannot leave it too low for a larger one.
struct SlotCacheEntry {
    int dev;
    const void* fn;
    size_t lds;
    int cus;
    int per_cu;
};
static std::mutex g_slot_mu;
static std::vector<SlotCacheEntry> g_slot_cache;

static bool resident_slots(const void* fn, size_t lds, int* cus_out, int* per_cu_out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return false;
    std::lock_guard<std::mutex> lock(g_slot_mu);
    bool attr_set = false;
    for (const SlotCacheEntry& e : g_slot_cache) {
        if (e.dev != dev || e.fn != fn) continue;
        attr_set = true;
        if (e.lds == lds) {
            *cus_out = e.cus;
            *per_cu_out = e.per_cu;
            return true;
        }
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return false;
    if (!attr_set && hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                         static_cast<int>(kPersistLdsMax)) != hipSuccess)
        return false;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kPThreads, lds) != hipSuccess) return false;
    g_slot_cache.push_back(SlotCacheEntry{dev, fn, lds, cus, per_cu});
    *cus_out = cus;
    *per_cu_out = per_cu;
    return true;
}

template <int KC>
static PersistPlan plan_for(const dspark_dims& D) {
    PersistPlan p;
    const int Bpad = (D.B + 15) / 16 * 16;
    p.grouped = persist_lds<KC>(Bpad, D.B, false, false) > kPersistLdsMax;
    p.ahead = !p.grouped && Bpad <= 32 && persist_lds<KC>(Bpad, D.B, false, true) <= kPersistLdsMax;
    p.lds = persist_lds<KC>(Bpad, D.B, p.grouped, p.ahead);
    if (p.lds > kPersistLdsMax) return p;
    int cus = 0, per_cu = 0;
    void (*fn)(PersistArgs) = persist_kernel<KC>(p.grouped, p.ahead);
    if (!resident_slots(reinterpret_cast<const void*>(fn), p.lds, &cus, &per_cu)) {
        (void)hipGetLastError();
        return p;
    }
    if (per_cu < 1) return p;
    const int nWG = cus;  // one workgroup per compute unit
    // columns held on chip: 64 per wave in registers + 16 per wave in LDS
    if (static_cast<int64_t>(D.V) > static_cast<int64_t>(kPWaves) * nWG * 80) return p;
    if (nWG > draft_persist_max_wg()) return p;
    p.ok = true;
    p.nWG = nWG;
    return p;
}

bool persist_path_ok(const dspark_dims& D) {
    if (D.head != DSPARK_HEAD_MARKOV || !mfma_path_ok(D)) return false;
    switch (D.r / 32) {
        case 1: return plan_for<1>(D).ok;
        case 2: return plan_for<2>(D).ok;
        case 4: return plan_for<4>(D).ok;
        case 8: return plan_for<8>(D).ok;
        default: return false;
    }
}

template <int KC>
static const char* persist_name_kc(const dspark_dims& D) {
    static const char* names[3] = {"k_draft_persistent<%d, true, false>", "k_draft_persistent<%d, false, true>",
                                   "k_draft_persistent<%d, false, false>"};
    static char buf[3][64];
    const PersistPlan p = plan_for<KC>(D);
    if (!p.ok) return "";
    const int which = p.grouped ? 0 : (p.ahead ? 1 : 2);
    snprintf(buf[which], sizeof buf[which], names[which], KC);
    return buf[which];
}

const char* persist_kernel_name(const dspark_dims& D) {
    if (D.head != DSPARK_HEAD_MARKOV || !mfma_path_ok(D)) return "";
    switch (D.r / 32) {
        case 1: return persist_name_kc<1>(D);
        case 2: return persist_name_kc<2>(D);
        case 4: return persist_name_kc<4>(D);
        case 8: return persist_name_kc<8>(D);
        default: return "";
    }
}

// Epochs of the start barrier: a process-wide counter, started from the
// clock and the process id so that memory left by another process is
// unlikely to hold a value it will produce.
static uint64_t next_epoch() {
    static std::atomic<uint64_t> counter{(static_cast<uint64_t>(std::chrono::steady_clock::now().time_since_epoch().count()) *
                                          0x9E3779B97F4A7C15ull) ^
                                         (static_cast<uint64_t>(getpid()) << 40)};
    uint64_t e = counter.fetch_add(1, std::memory_order_relaxed) + 1;
    return e != 0 ? e : counter.fetch_add(1, std::memory_order_relaxed) + 1;
}

template <int KC>
static hipError_t launch_persist_kc(const DraftArgs& A) {
    const dspark_dims& D = A.dims;
    const PersistPlan plan = plan_for<KC>(D);
    if (!plan.ok) return hipErrorNotSupported;
    const DraftLayout L = draft_layout(D);
    char* ws = A.ws;
    PersistArgs p{};
    p.U = static_cast<const uint16_t*>(A.U);
    p.W2 = static_cast<const uint16_t*>(A.W2);
    p.W1 = static_cast<const uint16_t*>(A.W1);
    p.w_conf = static_cast<const uint16_t*>(A.w_conf);
    p.anchor = A.anchor;
    p.temperature = A.temperature;
    p.h = static_cast<const uint16_t*>(A.h);
    p.V = D.V; p.r = D.r; p.d = D.d; p.gamma = D.gamma; p.B = D.B; p.Bpad = L.Bpad;
    p.nWG = plan.nWG;
    p.key0 = static_cast<uint32_t>(A.seed);
    p.key1 = static_cast<uint32_t>(A.seed >> 32);
    p.ctr3 = static_cast<uint32_t>(A.offset);
    p.best = reinterpret_cast<uint64_t*>(ws + L.best);
    p.bar = reinterpret_cast<uint32_t*>(ws + L.bar);
    p.pms = reinterpret_cast<float2*>(ws + L.qms);
    p.dead = reinterpret_cast<int32_t*>(ws + L.dead);
    p.tokens = A.tokens; p.logp = A.logp; p.conf = A.conf; p.survival = A.survival;

    p.flags = reinterpret_cast<uint64_t*>(ws + L.flags);
    p.epoch = next_epoch();
    const int spin = barrier_spin_option();
    p.spin_limit = spin > 0 ? static_cast<uint32_t>(spin) : (1u << 20);
    p.fail_waits = spin < 0 ? 1 : 0;
    hipError_t e = profile_begin(A.stream);
    if (e != hipSuccess) return e;
    void* args[] = {&p};
    void (*fn)(PersistArgs) = persist_kernel<KC>(plan.grouped, plan.ahead);
    e = hipLaunchKernel(reinterpret_cast<const void*>(fn), dim3(plan.nWG), dim3(kPThreads), args, plan.lds,
                        A.stream);
    if (e != hipSuccess) return e;
    if ((e = profile_end(A.stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_persist_finish, dim3(D.B), dim3(kFinishWaves * kWave), 0, A.stream, p);
    return hipGetLastError();
}

hipError_t launch_draft_persistent(const DraftArgs& A) {
    switch (A.dims.r / 32) {
        case 1: return launch_persist_kc<1>(A);
        case 2: return launch_persist_kc<2>(A);
        case 4: return launch_persist_kc<4>(A);
        case 8: return launch_persist_kc<8>(A);
        default: return hipErrorNotSupported;
    }
}

}  // namespace dspark
