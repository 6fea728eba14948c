// Single-launch DSpark block drafting (Markov head, bf16, matrix cores):
// the whole left-to-right loop of Eq 4/5 (DSpark paper as transcribed on the
// dormouse "DSpark - paper verification" page, section 1) in one cooperative
// kernel, with W2 loaded from HBM once per call instead of once per step.
//
//   prepare (small kernel)   h part of every confidence logit, c_1, S_1,
//                            token checks; clears the argmax keys and the
//                            barrier counter
//   persistent kernel, grid = every workgroup that can be resident:
//     load: wave w keeps W2 tile w (64 columns) in registers as MFMA
//           A-fragments; tiles beyond 4 x grid live, pre-transposed, in the
//           LDS of workgroup (tile - 4 x grid)
//     for k = 0 .. gamma-1:
//       every (tile, 16-block group): bias by MFMA from E = W1[x_{k-1}],
//         + U_k, Gumbel-max statistics (see lane_stats16)
//       workgroup merge -> one 64-bit atomicMax per block on the
//         (perturbed logit, lowest index) key; softmax partials stored
//       grid barrier (one monotonic counter, bounded spin, no cache flushes)
//       read x_k of every block from the keys; stage W1[x_k] for step k+1
//   finish (small kernel, grid B x gamma)   x_k, log p_k from the partials,
//                            c_k and S_k
//
// The only cross-workgroup dependency per step is the argmax over V; the
// softmax normaliser and the confidence head are computed after the loop.
#include <math.h>

#include <algorithm>
#include <mutex>

#include "device_common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace dspark {

constexpr int kPWaves = 4;        // waves per workgroup
constexpr int kKeyStride = 16;    // uint64 per argmax key: one 128-byte line each
constexpr int kReleaseWord = 32;  // barrier release flag, on its own line

struct PersistArgs {
    const uint16_t* U;
    const uint16_t* W2;
    const uint16_t* W1;
    const uint16_t* w_conf;
    const int32_t* anchor;
    const float* temperature;
    const float* hdot;   // [B, gamma]
    int V, d, gamma, B, Bpad, T, nWG;
    uint32_t key0, key1, ctr3;
    uint64_t* best;      // [gamma, B, 16]  argmax keys, one 128-byte line each (cleared by prepare)
    uint32_t* bar;       // [0] arrivals, [1] timeout flag, [32] release flag (cleared by prepare)
    float* pm;           // [gamma, B, nWG] softmax partials of every step
    float* ps;
    uint64_t* pkey;
    float* pzx;
    int32_t* dead;       // [B]
    int32_t* tokens;
    float* logp;
    float* conf;
    float* survival;
};

// -------------------------------------------------------------- prepare

// Grid (B, gamma): w[0:d] . h_{b,k}; workgroups (b, 0) also check the
// anchor and emit c_1, S_1; workgroup (0, 0) clears keys and the barrier.
__global__ __launch_bounds__(256) void k_persist_prepare(
    const int32_t* __restrict__ anchor, const uint16_t* __restrict__ W1,
    const uint16_t* __restrict__ w_conf, const uint16_t* __restrict__ h, int V, int r, int d,
    int gamma, int B, float* __restrict__ hdot, int32_t* __restrict__ dead,
    uint64_t* __restrict__ best, uint32_t* __restrict__ bar, float* __restrict__ conf,
    float* __restrict__ survival) {
    __shared__ float red[16];
    const int b = blockIdx.x, k = blockIdx.y;
    if (b == 0 && k == 0) {
        for (int i = threadIdx.x; i < gamma * B; i += blockDim.x) best[static_cast<size_t>(i) * kKeyStride] = kKeyNone;
        if (threadIdx.x < 64) bar[threadIdx.x] = 0u;
    }
    const int64_t hrow = (static_cast<int64_t>(b) * gamma + k) * d;
    float hp = 0.0f;
    for (int i = threadIdx.x; i < d; i += blockDim.x) hp += bf16_to_f32(w_conf[i]) * bf16_to_f32(h[hrow + i]);
    const float hk = block_sum(hp, red);
    if (threadIdx.x == 0) hdot[static_cast<size_t>(b) * gamma + k] = hk;
    if (k != 0) return;
    const int prev = anchor[b];
    const bool bad = prev < 0 || prev >= V;
    float part = 0.0f;
    for (int j = threadIdx.x; j < r; j += blockDim.x)
        part += bad ? 0.0f : bf16_to_f32(w_conf[d + j]) * bf16_to_f32(W1[static_cast<size_t>(prev) * r + j]);
    const float ae = block_sum(part, red);
    if (threadIdx.x == 0) {
        dead[b] = bad ? 1 : 0;
        const float c = bad ? NAN : sigmoidf_(hk + ae);
        conf[static_cast<size_t>(b) * gamma] = c;
        survival[static_cast<size_t>(b) * gamma] = c;
    }
}

// ------------------------------------------------------- grid barrier

// Grid barrier number `step` (1, 2, ...).  Everything one workgroup hands
// to another inside this kernel is a device-scope atomic (the argmax keys and
// the barrier words; the softmax partials are only read after the kernel):
// those are coherent at the device level (sc1), so the barrier needs no L2
// write-back or invalidate, which on
// this chip flush or drop a whole XCD's L2 and cost several microseconds
// each.  A workgroup-scope release (each wave waits for its own memory
// operations to complete) and the workgroup barrier come before the arrival;
// the workgroup whose arrival completes the count publishes `step` on a
// separate release line, which the others poll about every 0.5 us (polling
// one line back-to-back from hundreds of workgroups slows the stragglers).
// The wait is bounded: after ~2^20 polls bar[1] is set and the workgroup
// proceeds, so a broken launch cannot hang the device.
__device__ __forceinline__ void grid_barrier(uint32_t* bar, uint32_t step, uint32_t nwg) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t before = __hip_atomic_fetch_add(bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before + 1 == step * nwg) {
            __hip_atomic_store(bar + kReleaseWord, step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            uint32_t spins = 0;
            while (__hip_atomic_load(bar + kReleaseWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < step) {
                __builtin_amdgcn_s_sleep(20);
                if (++spins > (1u << 20)) {
                    __hip_atomic_store(bar + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
        }
    }
    __syncthreads();
}

// Device-scope (coherent) load of data other workgroups wrote in this kernel.
template <typename T>
__device__ __forceinline__ T get_shared(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------- the kernel

template <int KC>
struct XTile {  // a W2 tile kept in LDS as ready MFMA A-fragments
    static constexpr int kWords = KC * 4 * 64 * 4;
};

template <int KC>
__device__ __forceinline__ void build_xtile(const uint16_t* __restrict__ W2, int V, int vt, int g,
                                            int n, int lane, uint32_t* xf) {
    const int va = vt + 4 * n;
    const bool ok = va < V;
    for (int kc = 0; kc < KC; ++kc) {
        uint2 raw[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = kc * 32 + 8 * g + e;
            raw[e] = ok ? *reinterpret_cast<const uint2*>(W2 + static_cast<size_t>(j) * V + va)
                        : make_uint2(0u, 0u);
        }
        u32x4 f[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            f[0][p] = __builtin_amdgcn_perm(raw[2 * p + 1].x, raw[2 * p].x, 0x05040100u);
            f[1][p] = __builtin_amdgcn_perm(raw[2 * p + 1].x, raw[2 * p].x, 0x07060302u);
            f[2][p] = __builtin_amdgcn_perm(raw[2 * p + 1].y, raw[2 * p].y, 0x05040100u);
            f[3][p] = __builtin_amdgcn_perm(raw[2 * p + 1].y, raw[2 * p].y, 0x07060302u);
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) *reinterpret_cast<u32x4*>(&xf[((kc * 4 + c) * 64 + lane) * 4]) = f[c];
    }
}

// Bias of 16 blocks x 64 columns from the LDS tile (same layout as W2Tile).
template <int KC>
__device__ __forceinline__ void xtile_mul(const uint32_t* xf, const uint16_t* erow, int lane,
                                          f32x4 (&acc)[4]) {
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
        const u32x4 ev = *reinterpret_cast<const u32x4*>(erow + kc * 32);
        const bf16x8 bop = __builtin_bit_cast(bf16x8, ev);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const u32x4 av = *reinterpret_cast<const u32x4*>(&xf[((kc * 4 + c) * 64 + lane) * 4]);
            acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bop, acc[c], 0, 0, 0);
        }
    }
}

// Statistics of one (tile, 16-block group): lane (g, n) -> block 16 nb + n,
// columns vt + 16g .. vt + 16g + 15.
template <bool FULL>
__device__ __forceinline__ Stats lane_stats16p(const float (&z)[16], int v0, int V, int b, int k,
                                               bool sampling, float invT, uint32_t key0,
                                               uint32_t key1, uint32_t ctr3) {
    float zs[16], y[16];
    const int nvalid = V - v0;
#pragma unroll
    for (int j = 0; j < 16; ++j) zs[j] = (FULL || j < nvalid) ? z[j] * invT : -INFINITY;
    if (sampling) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const u32x4 ctr = {static_cast<uint32_t>(v0 + 4 * q) >> 2, static_cast<uint32_t>(k),
                               static_cast<uint32_t>(b), ctr3};
            const u32x4 w = philox4x32_10(ctr, key0, key1);
#pragma unroll
            for (int c = 0; c < 4; ++c) y[4 * q + c] = zs[4 * q + c] + gumbel_from_word(w[c]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) y[j] = zs[j];
    }
    float m = zs[0], ybest = y[0];
#pragma unroll
    for (int j = 1; j < 16; ++j) {
        m = fmaxf(m, zs[j]);
        ybest = fmaxf(ybest, y[j]);
    }
    const float mb = m * kLog2e;
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += __builtin_amdgcn_exp2f(fmaf(zs[j], kLog2e, -mb));
    int idx = 15;
    float zx = zs[15];
#pragma unroll
    for (int j = 14; j >= 0; --j) {
        const bool hit = y[j] == ybest;
        idx = hit ? j : idx;
        zx = hit ? zs[j] : zx;
    }
    return Stats{m, s, argmax_key(ybest, static_cast<uint32_t>(v0 + idx)), zx};
}

// LDS of one workgroup: [LDS W2 tile][E rows (when staged)][prev tokens]
// [per-wave statistics slots].
template <int KC>
__host__ __device__ constexpr size_t persist_e_bytes(int Bpad) {
    return static_cast<size_t>(Bpad) * (KC * 32 + 8) * 2;
}
template <int KC>
__host__ __device__ constexpr bool persist_stage_e(int Bpad) {
    return persist_e_bytes<KC>(Bpad) <= 24 * 1024;
}

template <int KC>
__global__ __launch_bounds__(256, 2) void k_draft_persistent(PersistArgs a) {
    constexpr int r = KC * 32;
    constexpr int ldE = r + 8;  // padded row stride of the staged E rows (bank spread)
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    const bool stage_e = persist_stage_e<KC>(a.Bpad);
    const size_t e_bytes = stage_e ? persist_e_bytes<KC>(a.Bpad) : 0;
    uint32_t* xf = reinterpret_cast<uint32_t*>(smem);
    uint16_t* Es = reinterpret_cast<uint16_t*>(smem + XTile<KC>::kWords * 4);
    int32_t* prev = reinterpret_cast<int32_t*>(smem + XTile<KC>::kWords * 4 + e_bytes);
    Stats* slot = reinterpret_cast<Stats*>(smem + XTile<KC>::kWords * 4 + e_bytes +
                                           align_up(static_cast<size_t>(a.Bpad) * 4, 16));

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int wg = blockIdx.x, nWG = a.nWG;
    const int NB = a.Bpad / 16;
    const int t_reg = wg * kPWaves + wave;
    const int t_x = kPWaves * nWG + wg;
    const bool has_reg = t_reg < a.T, has_x = t_x < a.T;

    W2Tile<KC> w2;
    if (has_reg) w2.load(a.W2, a.V, t_reg * 64, g, n);
    if (has_x && wave == 0) build_xtile<KC>(a.W2, a.V, t_x * 64, g, n, lane, xf);
    // previous tokens of step 0: the anchors (an out-of-range anchor reads
    // row 0; the prepare kernel marked its block dead)
    for (int b = threadIdx.x; b < a.Bpad; b += blockDim.x) {
        const int x = b < a.B ? a.anchor[b] : 0;
        prev[b] = (x >= 0 && x < a.V) ? x : 0;
    }
    __syncthreads();
    // E rows of the coming step, W1[prev[b]], staged once per workgroup
    auto stage_rows = [&]() {
        if (!stage_e) return;
        for (int t = threadIdx.x; t < a.Bpad * (r / 8); t += blockDim.x) {
            const int row = t / (r / 8), col = t % (r / 8);
            *reinterpret_cast<u32x4*>(&Es[row * ldE + col * 8]) =
                *reinterpret_cast<const u32x4*>(a.W1 + static_cast<size_t>(prev[row]) * r + col * 8);
        }
        __syncthreads();
    };
    stage_rows();

    for (int k = 0; k < a.gamma; ++k) {
        for (int b = lane; b < a.B; b += 64) slot[wave * a.B + b] = stats_empty();
        // own tile: all block groups; LDS tile: groups nb = wave (mod 4)
        const int units = (has_reg ? NB : 0) + (has_x ? (NB - wave + kPWaves - 1) / kPWaves : 0);
        for (int u = 0; u < units; ++u) {
            const bool from_x = u >= (has_reg ? NB : 0);
            const int nb = from_x ? wave + kPWaves * (u - (has_reg ? NB : 0)) : u;
            const int tile = from_x ? t_x : t_reg;
            const int b = nb * 16 + n;
            const int v0 = tile * 64 + 16 * g;
            const bool live = b < a.B && v0 < a.V;
            // U of this unit first: its latency overlaps the MFMA below
            float z[16];
            float temp = 0.0f;
            if (live) {
                load16_bf16(a.U + (static_cast<size_t>(b) * a.gamma + k) * a.V + v0, v0 + 8 < a.V, z);
                temp = a.temperature[b];
            }
            const uint16_t* erow = stage_e ? &Es[b * ldE + 8 * g]
                                           : a.W1 + static_cast<size_t>(prev[b]) * r + 8 * g;
            f32x4 acc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (from_x)
                xtile_mul<KC>(xf, erow, lane, acc);
            else
                w2.mul(erow, acc);
            Stats st = stats_empty();
            if (live) {
                const bool sampling = temp > 0.0f;
                const float invT = sampling ? 1.0f / temp : 1.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int c = 0; c < 4; ++c) z[4 * q + c] += acc[c][q];
                if (v0 + 16 <= a.V)
                    st = lane_stats16p<true>(z, v0, a.V, b, k, sampling, invT, a.key0, a.key1, a.ctr3);
                else
                    st = lane_stats16p<false>(z, v0, a.V, b, k, sampling, invT, a.key0, a.key1, a.ctr3);
            }
            st = stats_merge(st, shfl_xor_stats(st, 16));
            st = stats_merge(st, shfl_xor_stats(st, 32));
            if (g == 0 && b < a.B) slot[wave * a.B + b] = stats_merge(slot[wave * a.B + b], st);
        }
        __syncthreads();
        // workgroup merge in wave order, then publish
        for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
            Stats t = slot[b];
#pragma unroll
            for (int w = 1; w < kPWaves; ++w) t = stats_merge(t, slot[w * a.B + b]);
            if (t.key != kKeyNone)
                __hip_atomic_fetch_max(&a.best[(static_cast<size_t>(k) * a.B + b) * kKeyStride], t.key,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            // softmax partials are read after the kernel (k_persist_finish)
            const size_t o = (static_cast<size_t>(k) * a.B + b) * nWG + wg;
            a.pm[o] = t.m;
            a.ps[o] = t.s;
            a.pkey[o] = t.key;
            a.pzx[o] = t.zx;
        }
        if (k + 1 == a.gamma) break;  // the last keys are read after the kernel
        grid_barrier(a.bar, static_cast<uint32_t>(k + 1), static_cast<uint32_t>(nWG));
        // x_k of every block from the keys -> the E rows of step k+1
        for (int b = threadIdx.x; b < a.B; b += blockDim.x) {
            const uint64_t key = get_shared(&a.best[(static_cast<size_t>(k) * a.B + b) * kKeyStride]);
            const uint32_t x = key_index(key);
            prev[b] = (key != kKeyNone && x < static_cast<uint32_t>(a.V)) ? static_cast<int>(x) : 0;
        }
        __syncthreads();
        stage_rows();
    }
}

// --------------------------------------------------------------- finish

// Workgroup (b, k), after the loop: x_k from the argmax keys, log p_k from
// the step's softmax partials (merged in workgroup order), c_k (Eq 7 on
// x_{k-1}) and S_k = c_1 ... c_k.  None of these feed the sampling loop, so
// they are kept out of it; each workgroup recomputes c_1 .. c_k itself
// (k <= 64 dot products of length r), which keeps every S_k a fixed-order
// product without a second pass.
__global__ __launch_bounds__(256) void k_persist_finish(PersistArgs a, int r) {
    __shared__ float red[16];
    __shared__ int xs[64];
    __shared__ int bad_s;
    const int b = blockIdx.x, k = blockIdx.y;
    if (threadIdx.x == 0) {
        bool bad = a.dead[b] != 0 || a.bar[1] != 0;
        for (int i = 0; i <= k; ++i) {
            const uint64_t key = a.best[(static_cast<size_t>(i) * a.B + b) * kKeyStride];
            const uint32_t x = key_index(key);
            bad = bad || key == kKeyNone || x >= static_cast<uint32_t>(a.V);
            xs[i] = static_cast<int>(x);
        }
        bad_s = bad;
    }
    __syncthreads();
    const bool bad = bad_s != 0;
    const size_t out = static_cast<size_t>(b) * a.gamma + k;
    // log p_k
    Stats t = stats_empty();
    const size_t base = (static_cast<size_t>(k) * a.B + b) * a.nWG;
    for (int p = threadIdx.x; p < a.nWG; p += blockDim.x)
        t = stats_merge(t, Stats{a.pm[base + p], a.ps[base + p], a.pkey[base + p], a.pzx[base + p]});
    for (int o = 32; o > 0; o >>= 1) t = stats_merge(t, shfl_xor_stats(t, o));
    __shared__ Stats wred[4];
    if ((threadIdx.x & 63) == 0) wred[threadIdx.x >> 6] = t;
    __syncthreads();
    if (threadIdx.x == 0) {
        Stats m = wred[0];
        for (int w = 1; w < static_cast<int>(blockDim.x / kWave); ++w) m = stats_merge(m, wred[w]);
        a.tokens[out] = bad ? -1 : xs[k];
        if (a.logp) a.logp[out] = bad ? NAN : m.zx - (m.m + logf(m.s));
        if (bad) a.dead[b] = 1;
    }
    // c_1 .. c_k and the survival product
    float S = a.survival[static_cast<size_t>(b) * a.gamma];  // S_0 = c_0 from prepare
    float c = S;
    for (int i = 1; i <= k; ++i) {
        float part = 0.0f;
        if (!bad)
            for (int j = threadIdx.x; j < r; j += blockDim.x)
                part += bf16_to_f32(a.w_conf[a.d + j]) * bf16_to_f32(a.W1[static_cast<size_t>(xs[i - 1]) * r + j]);
        const float ae = block_sum(part, red);
        c = bad ? NAN : sigmoidf_(a.hdot[static_cast<size_t>(b) * a.gamma + i] + ae);
        S *= c;
    }
    if (threadIdx.x == 0 && k > 0) {
        a.conf[out] = c;
        a.survival[out] = S;
    }
}

// ---------------------------------------------------------------- launch

template <int KC>
static size_t persist_lds(int Bpad, int B) {
    return XTile<KC>::kWords * 4 + (persist_stage_e<KC>(Bpad) ? persist_e_bytes<KC>(Bpad) : 0) +
           align_up(static_cast<size_t>(Bpad) * 4, 16) + sizeof(Stats) * kPWaves * static_cast<size_t>(B);
}

struct PersistPlan {
    bool ok = false;
    int nWG = 0;
};

template <int KC>
static PersistPlan plan_for(const dspark_dims& D) {
    PersistPlan p;
    const int Bpad = (D.B + 15) / 16 * 16;
    const size_t lds = persist_lds<KC>(Bpad, D.B);
    if (lds > 64 * 1024) return p;
    int dev = 0, cus = 0, coop = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return p;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return p;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop) return p;
    void (*fn)(PersistArgs) = k_draft_persistent<KC>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(fn), 256, lds) !=
        hipSuccess)
        return p;
    if (per_cu < 1) return p;
    const int nWG = std::min(per_cu, 2) * cus;
    const int T = (D.V + 63) / 64;
    if (T > kPWaves * nWG + nWG) return p;  // W2 does not fit on chip
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
    p.hdot = reinterpret_cast<const float*>(ws + L.hdot);
    p.V = D.V; p.d = D.d; p.gamma = D.gamma; p.B = D.B; p.Bpad = L.Bpad;
    p.T = (D.V + 63) / 64;
    p.nWG = plan.nWG;
    p.key0 = static_cast<uint32_t>(A.seed);
    p.key1 = static_cast<uint32_t>(A.seed >> 32);
    p.ctr3 = static_cast<uint32_t>(A.offset);
    p.best = reinterpret_cast<uint64_t*>(ws + L.best);
    p.bar = reinterpret_cast<uint32_t*>(ws + L.bar);
    p.pm = reinterpret_cast<float*>(ws + L.qm);
    p.ps = reinterpret_cast<float*>(ws + L.qs);
    p.pkey = reinterpret_cast<uint64_t*>(ws + L.qkey);
    p.pzx = reinterpret_cast<float*>(ws + L.qzx);
    p.dead = reinterpret_cast<int32_t*>(ws + L.dead);
    p.tokens = A.tokens; p.logp = A.logp; p.conf = A.conf; p.survival = A.survival;

    hipLaunchKernelGGL(k_persist_prepare, dim3(D.B, D.gamma), dim3(256), 0, A.stream, A.anchor,
                       p.W1, p.w_conf, static_cast<const uint16_t*>(A.h), D.V, D.r, D.d, D.gamma, D.B,
                       reinterpret_cast<float*>(ws + L.hdot), p.dead, p.best, p.bar, A.conf, A.survival);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if ((e = profile_begin(A.stream)) != hipSuccess) return e;
    void* args[] = {&p};
    void (*fn)(PersistArgs) = k_draft_persistent<KC>;
    e = hipLaunchCooperativeKernel(reinterpret_cast<const void*>(fn), dim3(plan.nWG),
                                   dim3(256), args, persist_lds<KC>(L.Bpad, D.B), A.stream);
    if (e != hipSuccess) return e;
    if ((e = profile_end(A.stream)) != hipSuccess) return e;
    hipLaunchKernelGGL(k_persist_finish, dim3(D.B, D.gamma), dim3(256), 0, A.stream, p, D.r);
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
