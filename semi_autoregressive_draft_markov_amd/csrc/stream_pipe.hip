// Per-step streaming of the transition bias for the per-step drafting
// driver: z = U_k + coef W2 over all V columns (Eq 5 / Eq 6 of the DSpark
// paper as transcribed on the dormouse "DSpark - paper verification" page,
// section 1), then per-block softmax and Gumbel-argmax partial statistics
// (Eq 4), as k_stream_mfma computes them, for B <= 128 and r = 256.
//
// k_stream_mfma gives every workgroup one 256-column W2 tile in registers:
// all resident workgroups load their tiles at the same time and then all
// compute, so HBM and the vector ALUs take turns.  Here one 8-wave workgroup
// per compute unit walks a list of 32-column tiles instead, and the next
// tile's loads are in flight while the current tile is computed:
//
//   stage all coef rows (bf16 planes) and 1/T in LDS, once per step
//   for each 32-column tile of this wave (half of a 64-column region):
//     for each 16-block unit:
//       issue U of the next unit and one 32-row chunk of the next tile
//       bias on the matrix cores (A = this tile's fragments, B = coef rows)
//       lane statistics of 8 columns, merged into the unit's running ones
//   running statistics merged over the lanes of a block, then over the
//   waves in wave order -> one partial per (block, workgroup)
//
// A 64-column region is one 128-byte line per W2 (and U) row; its two
// 32-column halves are taken by two waves of one workgroup at the same time,
// so each line is fetched from HBM once.
#include <math.h>

#include <atomic>

#include "device_common.h"
#include "internal.h"

namespace dspark {

constexpr int kSpWaves = 8;
constexpr int kSpThreads = kSpWaves * kWave;
constexpr int kSpMaxUnits = 8;  // Bpad <= 128: running statistics of 8 units per lane
constexpr int kSpKC = 8;        // r = 256
constexpr int kSpRows = 16 * kSpMaxUnits;  // block stride of the staged coef pieces

// One 32-column W2 tile as MFMA A operands.  Lane (g, n) loads, for chunk
// kc, the 4-byte pairs W2[32 kc + 8 g + e][c0 + 2n .. c0 + 2n + 1] (e =
// 0..7); transpose() then packs them by row pairs into fragment c = 0
// (column c0 + 2n) in w[kc][0..3] and fragment c = 1 (column c0 + 2n + 1)
// in w[kc][4..7].  With A row i = column c0 + 2i + c and B = 16 coef rows,
// v_mfma_f32_16x16x32_bf16 leaves the bias of block row n at column
// c0 + 8 g + 2 q + c in accumulator element q of fragment c: every lane
// ends up with the 8 consecutive columns c0 + 8 g .. c0 + 8 g + 7.
template <int KC>
struct Tile32 {
    uint32_t w[KC][8];

    // chunk kc of the tile at column c0 (columns past V: any in-bounds
    // address, their statistics are masked)
    __device__ __forceinline__ void issue(const uint16_t* __restrict__ W2, int V, int c0, int g, int n, int kc) {
        const int col = c0 + 2 * n < V ? c0 + 2 * n : 0;
        const uint16_t* base = W2 + static_cast<size_t>(32 * kc + 8 * g) * V + col;
#pragma unroll
        for (int e = 0; e < 8; ++e) w[kc][e] = *reinterpret_cast<const uint32_t*>(base + static_cast<size_t>(e) * V);
    }
    __device__ __forceinline__ void transpose() {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint32_t t[8];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                t[p] = __builtin_amdgcn_perm(w[kc][2 * p + 1], w[kc][2 * p], 0x05040100u);
                t[4 + p] = __builtin_amdgcn_perm(w[kc][2 * p + 1], w[kc][2 * p], 0x07060302u);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) w[kc][i] = t[i];
        }
    }
    __device__ __forceinline__ bf16x8 frag(int kc, int c) const {
        const u32x4 v = {w[kc][4 * c], w[kc][4 * c + 1], w[kc][4 * c + 2], w[kc][4 * c + 3]};
        return __builtin_bit_cast(bf16x8, v);
    }
};

// Running statistics of a lane in base-2 units: with z2 = z log2(e) / T
// (z log2(e) when greedy), s = sum of 2^(z2 - m) over the columns seen so
// far for a reference m no smaller than their largest perturbed value, and
// the argmax key of the perturbed values y = z2 - log2(-log2 u) (sampling;
// the Gumbel-max value up to a positive factor and a constant, as in
// log2_of_neg_log2_uniform) or y = z2 (greedy).  z at the argmax is not
// carried: it is recovered once per block from the winning key at the end.
struct RStats {
    float m;
    float s;
    uint64_t key;
};

__device__ __forceinline__ RStats rstats_merge(const RStats& a, const RStats& b) {
    RStats r;
    r.m = fmaxf(a.m, b.m);
    const float sa = (a.s > 0.0f) ? a.s * __builtin_amdgcn_exp2f(a.m - r.m) : 0.0f;
    const float sb = (b.s > 0.0f) ? b.s * __builtin_amdgcn_exp2f(b.m - r.m) : 0.0f;
    r.s = sa + sb;
    r.key = b.key > a.key ? b.key : a.key;
    return r;
}

// rstats_merge of lanes l and l ^ X (X = 16 or 32); commutative bit for bit
template <int X>
__device__ __forceinline__ RStats rstats_merge_xor(const RStats& a) {
    const uint32_t w[4] = {__float_as_uint(a.m), __float_as_uint(a.s), static_cast<uint32_t>(a.key),
                           static_cast<uint32_t>(a.key >> 32)};
    LanePair p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = X == 16 ? swap16(w[i]) : swap32(w[i]);
    const RStats x{__uint_as_float(p[0].a), __uint_as_float(p[1].a), (static_cast<uint64_t>(p[3].a) << 32) | p[2].a};
    const RStats y{__uint_as_float(p[0].b), __uint_as_float(p[1].b), (static_cast<uint64_t>(p[3].b) << 32) | p[2].b};
    return rstats_merge(x, y);
}

// Adds the 8 columns v0 .. v0 + 7 of block b (all present: V % 8 == 0) to
// the running statistics st; scale = log2(e) / T (sampling) or log2(e).  The
// new reference is the larger of the old one and the columns' largest
// perturbed value: z2 - y <= log2(24) for every column, so no term of the
// sum overflows, and the winner's term is at least 2^-24.
__device__ __forceinline__ void lane_update8(RStats& st, const float (&z)[8], int v0, int b, int k, bool sampling,
                                             float scale, uint32_t key0, uint32_t key1, uint32_t ctr3) {
    float y[8];
    if (sampling) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const u32x4 ctr = {(static_cast<uint32_t>(v0) >> 2) + static_cast<uint32_t>(q), static_cast<uint32_t>(k),
                               static_cast<uint32_t>(b), ctr3};
            const u32x4 w = philox4x32_10(ctr, key0, key1);
#pragma unroll
            for (int c = 0; c < 4; ++c) y[4 * q + c] = fmaf(z[4 * q + c], scale, -log2_of_neg_log2_uniform(w[c]));
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) y[j] = z[j] * scale;
    }
    float ybest = y[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) ybest = fmaxf(ybest, y[j]);
    int idx = 7;
#pragma unroll
    for (int j = 6; j >= 0; --j) idx = y[j] == ybest ? j : idx;
    const float m = fmaxf(st.m, ybest);
    float s = st.s > 0.0f ? st.s * __builtin_amdgcn_exp2f(st.m - m) : 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += __builtin_amdgcn_exp2f(fmaf(z[j], scale, -m));
    const uint64_t key = argmax_key(ybest, static_cast<uint32_t>(v0 + idx));
    st.m = m;
    st.s = s;
    st.key = key > st.key ? key : st.key;
}

template <int NPL>
__host__ __device__ constexpr size_t stream_pipe_lds() {
    return static_cast<size_t>(NPL) * (kSpKC * 32 / 8) * kSpRows * 16 + kSpRows * 4;
}

// NPL = coef planes (1: bf16 coef; 2: hi + lo bf16 planes of an fp32 coef).
// Partial of workgroup p for block b at pm/ps/pkey/pzx[b P + p], P = grid.
template <int NPL, int NU>
__global__ __launch_bounds__(kSpThreads, 1) void k_stream_pipe(
    const uint16_t* __restrict__ U, const uint16_t* __restrict__ W2, const uint16_t* __restrict__ ebf,
    const float* __restrict__ temperature, int V, int B, int Bpad, int gamma, int k, uint32_t key0,
    uint32_t key1, uint32_t ctr3, float* __restrict__ pm, float* __restrict__ ps, uint64_t* __restrict__ pkey,
    float* __restrict__ pzx) {
    constexpr int KC = kSpKC;
    constexpr int r = KC * 32;
    constexpr int kPieces = r / 8;  // 16-byte pieces of one coef row
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    // coef rows as [plane][piece][block] 16-byte pieces, block stride
    // kSpRows (a compile-time stride keeps every operand address an
    // immediate offset from one per-lane base): lane (g, n) of a unit reads
    // piece 4 kc + g of block 16 nb + n, so a read's bank group is n + const
    // (conflict-free) without padding
    u32x4* Es = reinterpret_cast<u32x4*>(smem);
    // per block: log2(e) / T when it samples, -log2(e) when greedy
    float* inv_s = reinterpret_cast<float*>(smem + static_cast<size_t>(NPL) * kPieces * kSpRows * 16);

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;

    {
        const int pieces = NPL * kPieces * Bpad;
        for (int t = threadIdx.x; t < pieces; t += kSpThreads) {
            const int b = t % Bpad, rest = t / Bpad;
            const int c = rest % kPieces, pl = rest / kPieces;
            Es[rest * kSpRows + b] = *reinterpret_cast<const u32x4*>(ebf + (static_cast<size_t>(pl) * Bpad + b) * r + c * 8);
        }
        for (int b = threadIdx.x; b < Bpad; b += kSpThreads) {
            const float t = b < B ? temperature[b] : 0.0f;
            inv_s[b] = t > 0.0f ? kLog2e / t : -kLog2e;
        }
    }
    __syncthreads();

    // Waves 2p and 2p + 1 take the two 32-column halves of the same 64-column
    // regions at the same time (one 128-byte line per W2 or U row, read by
    // both halves together): this wave's tiles s = 0 .. S-1 are region
    // pw + NP s, half wave % 2.
    const int NP = gridDim.x * (kSpWaves / 2), pw = blockIdx.x * (kSpWaves / 2) + (wave >> 1);
    const int nreg = (V + 63) / 64;
    const int S = pw < nreg ? (nreg - 1 - pw) / NP + 1 : 0;
    auto col0 = [&](int s) { return 64 * (pw + NP * s) + 32 * (wave & 1); };

    RStats st[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) st[u] = RStats{-INFINITY, 0.0f, kKeyNone};

    // U of unit nb at the lane's 8 columns from c0 (an in-bounds address for
    // padding blocks and columns past V, whose values are never used)
    auto fetch_u = [&](int c0, int nb) {
        // (the block index is opaque here and in the statistics, so that the
        // compiler does not keep per-unit row offsets or first Philox
        // rounds, which do not change from tile to tile, live across the
        // tile loop: at 8 units they would not fit in registers)
        int b = min(nb * 16 + n, B - 1);
        asm volatile("" : "+v"(b));
        const int col = c0 + 8 * g < V ? c0 + 8 * g : 0;
        return *reinterpret_cast<const u32x4*>(U + (static_cast<size_t>(b) * gamma + k) * V + col);
    };

    // One tile at a time, chunk-major: the products of chunk kc for every
    // unit, then chunk kc of the next tile is loaded into the same registers
    // (its last use is issued), and halfway through the statistics the next
    // tile's U values; the U values start the accumulators (z = U + bias
    // comes out of the matrix cores).  Every load is waited for only at the start of the
    // next tile, a whole statistics phase later (vector-memory counts
    // complete in issue order, so a load issued before a later wait would be
    // waited for too).  The loads are unconditional (after the last tile
    // they repeat it).
    // Waves w and w + 4 share a SIMD.  The second starts about a microsecond
    // later, and a wave's products run at raised priority, so that one
    // wave's matrix-core phase tends to overlap the other's statistics
    // (measured: 71.2 -> 69.0 us per step at the Gemma4 shape).
    if (wave >= 4) __builtin_amdgcn_s_sleep(40);
    Tile32<KC> t;
    u32x4 uall[NU];
    if (S > 0) {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) t.issue(W2, V, col0(0), g, n, kc);
#pragma unroll
        for (int u = 0; u < NU; ++u) uall[u] = fetch_u(col0(0), u);
    }
    for (int s = 0; s < S; ++s) {
        const int c0 = col0(s);
        const int c1 = s + 1 < S ? col0(s + 1) : c0;
        const int v0 = c0 + 8 * g;
        const bool live = v0 < V;
        t.transpose();
        f32x4 acc[NU][2];
#pragma unroll
        for (int u = 0; u < NU; ++u)
#pragma unroll
            for (int c = 0; c < 2; ++c)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int j = 2 * q + c;
                    acc[u][c][q] = (j & 1) ? hi_bf16(uall[u][j >> 1]) : lo_bf16(uall[u][j >> 1]);
                }
        // products in the order i = (kc, plane, unit), the coef piece of
        // product i + kAhead read while product i is issued (LDS latency off
        // the matrix-core path); chunk kc of the next tile is loaded after
        // the last product of chunk kc
        __builtin_amdgcn_s_setprio(2);
        const u32x4* erow = Es + g * kSpRows + n;
        constexpr int kN = KC * NPL * NU, kAhead = 2;
        auto piece = [&](int i) {
            const int kc = i / (NPL * NU), pl = (i / NU) % NPL, u = i % NU;
            return erow[(pl * kPieces + 4 * kc) * kSpRows + 16 * u];
        };
        u32x4 ev[kAhead + 1];
#pragma unroll
        for (int i = 0; i < kAhead; ++i) ev[i] = piece(i);
        __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
        for (int i = 0; i < kN; ++i) {
            const int kc = i / (NPL * NU), u = i % NU;
            if (i + kAhead < kN) ev[(i + kAhead) % (kAhead + 1)] = piece(i + kAhead);
            const bf16x8 bop = __builtin_bit_cast(bf16x8, ev[i % (kAhead + 1)]);
            acc[u][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.frag(kc, 0), bop, acc[u][0], 0, 0, 0);
            acc[u][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(t.frag(kc, 1), bop, acc[u][1], 0, 0, 0);
            if (i + kAhead < kN) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            if ((i + 1) % (NPL * NU) == 0) {
                t.issue(W2, V, c1, g, n, kc);
                __builtin_amdgcn_sched_group_barrier(0x020, 8, 0);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            int b = u * 16 + n;
            asm volatile("" : "+v"(b));
            if (live && b < B) {
                const float sc = inv_s[b];
                const bool sampling = sc > 0.0f;
                float z[8];
#pragma unroll
                for (int q = 0; q < 4; ++q)
#pragma unroll
                    for (int c = 0; c < 2; ++c) z[2 * q + c] = acc[u][c][q];
                lane_update8(st[u], z, v0, b, k, sampling, fabsf(sc), key0, key1, ctr3);
            }
            // one unit's statistics at a time (interleaving units would hold
            // all their temporaries at once)
            __builtin_amdgcn_sched_barrier(0);
            // the next tile's U values once half the accumulators are free
            if (u == (NU - 1) / 2) {
#pragma unroll
                for (int w = 0; w < NU; ++w) uall[w] = fetch_u(c1, w);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }

    // every wave is done with the coef rows: their LDS takes the per-wave
    // statistics [wave][block] (8 x 16 bytes per block, against 512 bytes
    // per block of one coef plane)
    __syncthreads();
    RStats* red = reinterpret_cast<RStats*>(smem);
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        RStats m = rstats_merge_xor<16>(st[u]);
        m = rstats_merge_xor<32>(m);
        if (g == 0) red[wave * kSpRows + u * 16 + n] = m;
    }
    __syncthreads();
    // back to the units of the partials (natural log): m ln 2, and z/T at
    // the argmax = (the winning perturbed value, from the key's high word
    // with the order-preserving bits inverted, plus the winner's
    // log2(-log2 u) recomputed from its counter; nothing when greedy) ln 2
    const int P = gridDim.x;
    for (int b = threadIdx.x; b < B; b += kSpThreads) {
        RStats t = red[b];
#pragma unroll
        for (int w = 1; w < kSpWaves; ++w) t = rstats_merge(t, red[w * kSpRows + b]);
        float zx = 0.0f;
        if (t.key != kKeyNone) {
            const uint32_t kb = static_cast<uint32_t>(t.key >> 32);
            const float y = __uint_as_float((kb & 0x80000000u) ? (kb ^ 0x80000000u) : ~kb);
            float z2 = y;
            if (inv_s[b] > 0.0f) {
                const uint32_t x = key_index(t.key);
                const u32x4 w = philox4x32_10(u32x4{x >> 2, static_cast<uint32_t>(k), static_cast<uint32_t>(b), ctr3},
                                              key0, key1);
                const uint32_t q = x & 3u;
                z2 = y + log2_of_neg_log2_uniform(q == 0 ? w[0] : q == 1 ? w[1] : q == 2 ? w[2] : w[3]);
            }
            zx = z2 * kLn2;
        }
        const size_t o = static_cast<size_t>(b) * P + blockIdx.x;
        pm[o] = t.m * kLn2;
        ps[o] = t.s;
        pkey[o] = t.key;
        pzx[o] = zx;
    }
}

// The pipelined kernel applies when r = 256, Bpad <= 128 and the coef rows
// fit in LDS; it needs no co-residency, so any grid works (one workgroup per
// compute unit, cached per device, capped by the partial slots).
bool stream_pipe_ok(const dspark_dims& d, int npl) {
    const int Bpad = (d.B + 15) / 16 * 16;
    const size_t lds = npl == 2 ? stream_pipe_lds<2>() : stream_pipe_lds<1>();
    return d.dtype == DSPARK_BF16 && d.r == kSpKC * 32 && d.V % 8 == 0 && Bpad <= kSpRows &&
           lds <= 160 * 1024 && npl >= 1 && npl <= 2;
}

static int stream_pipe_grid(const DraftLayout& L) {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        cus = 256;
    } else if ((cus = cached[dev].load(std::memory_order_relaxed)) <= 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
            (void)hipGetLastError();
            cus = 256;
        }
        cached[dev].store(cus, std::memory_order_relaxed);
    }
    return cus < L.P ? cus : L.P;
}

template <int NPL, int NU>
static hipError_t launch_pipe(const DraftArgs& a, const DraftLayout& L, int k, char* ws, int* P) {
    const dspark_dims& D = a.dims;
    constexpr int kMaxDevices = 64;
    static std::atomic<int> attr_done[kMaxDevices] = {};
    constexpr size_t lds = stream_pipe_lds<NPL>();
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return hipGetLastError();
    if (dev < 0 || dev >= kMaxDevices || !attr_done[dev].load(std::memory_order_relaxed)) {
        const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&k_stream_pipe<NPL, NU>),
                                                 hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
        if (e != hipSuccess) return e;
        if (dev >= 0 && dev < kMaxDevices) attr_done[dev].store(1, std::memory_order_relaxed);
    }
    const int grid = stream_pipe_grid(L);
    *P = grid;
    hipLaunchKernelGGL((k_stream_pipe<NPL, NU>), dim3(grid), dim3(kSpThreads), lds, a.stream,
                       static_cast<const uint16_t*>(a.U), static_cast<const uint16_t*>(a.W2),
                       reinterpret_cast<const uint16_t*>(ws + L.ebf), a.temperature, D.V, D.B, L.Bpad, D.gamma, k,
                       static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32),
                       static_cast<uint32_t>(a.offset), reinterpret_cast<float*>(ws + L.pm),
                       reinterpret_cast<float*>(ws + L.ps), reinterpret_cast<uint64_t*>(ws + L.pkey),
                       reinterpret_cast<float*>(ws + L.pzx));
    return hipGetLastError();
}

template <int NPL>
static hipError_t launch_pipe_nu(const DraftArgs& a, const DraftLayout& L, int k, char* ws, int* P) {
    switch (L.Bpad / 16) {
        case 1: return launch_pipe<NPL, 1>(a, L, k, ws, P);
        case 2: return launch_pipe<NPL, 2>(a, L, k, ws, P);
        case 3: return launch_pipe<NPL, 3>(a, L, k, ws, P);
        case 4: return launch_pipe<NPL, 4>(a, L, k, ws, P);
        case 5: return launch_pipe<NPL, 5>(a, L, k, ws, P);
        case 6: return launch_pipe<NPL, 6>(a, L, k, ws, P);
        case 7: return launch_pipe<NPL, 7>(a, L, k, ws, P);
        case 8: return launch_pipe<NPL, 8>(a, L, k, ws, P);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_stream_pipe(const DraftArgs& a, const DraftLayout& L, int k, char* ws, int npl, int* P) {
    return npl == 2 ? launch_pipe_nu<2>(a, L, k, ws, P) : launch_pipe_nu<1>(a, L, k, ws, P);
}

const char* stream_pipe_name(int npl, int Bpad) {
    static const char* const names[2][kSpMaxUnits] = {
        {"k_stream_pipe<1, 1>", "k_stream_pipe<1, 2>", "k_stream_pipe<1, 3>", "k_stream_pipe<1, 4>",
         "k_stream_pipe<1, 5>", "k_stream_pipe<1, 6>", "k_stream_pipe<1, 7>", "k_stream_pipe<1, 8>"},
        {"k_stream_pipe<2, 1>", "k_stream_pipe<2, 2>", "k_stream_pipe<2, 3>", "k_stream_pipe<2, 4>",
         "k_stream_pipe<2, 5>", "k_stream_pipe<2, 6>", "k_stream_pipe<2, 7>", "k_stream_pipe<2, 8>"}};
    const int nu = Bpad / 16;
    return (npl == 1 || npl == 2) && nu >= 1 && nu <= kSpMaxUnits ? names[npl - 1][nu - 1] : "";
}

}  // namespace dspark
