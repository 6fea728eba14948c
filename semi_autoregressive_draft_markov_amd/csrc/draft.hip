// DSpark block drafting on gfx950: Eq 4 sampling with the Eq 5 (Markov) or
// Eq 6 (RNN) transition bias, Eq 7 confidence and the prefix survival
// product (DSpark paper as transcribed on the dormouse "DSpark - paper
// verification" page, section 1; survival per the Meridian note, section 3).
//
// One call runs the whole left-to-right loop on the device:
//   init                      e = W1[x_0], c_1, S_1
//   for k = 0 .. gamma-1:
//     [RNN] gates + update    G = W_rnn [s; e; h_k] (h columns for all k
//                             before the loop); s, o = tanh(G_o)
//     stream                  z = U_k + coef W2 over V tiles -> per-tile
//                             softmax / Gumbel-argmax partial statistics
//     combine                 x_k, log p_k; e = W1[x_k]; c_{k+1}, S_{k+1}
// The only step-to-step dependency is the reduction over V inside combine.
#include <math.h>
#include <stdio.h>

#include <atomic>
#include <type_traits>

#include "device_common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace dspark {

constexpr int kTileV = 64;                       // columns per wave (MFMA path)
constexpr int kWavesPerWG = 4;
constexpr int kColsPerWG = kTileV * kWavesPerWG;  // 256 columns per workgroup
constexpr int kGenericCols = 4 * 256;             // generic path: 4 columns per thread

bool mfma_path_ok(const dspark_dims& d) {
    return d.dtype == DSPARK_BF16 && d.r % 32 == 0 && d.r <= 256 && d.V % 8 == 0;
}

int draft_partials(const dspark_dims& d) {
    return mfma_path_ok(d) ? (d.V + kColsPerWG - 1) / kColsPerWG
                           : (d.V + kGenericCols - 1) / kGenericCols;
}

// Upper bound on the single-launch grid: two workgroups per compute unit of
// the current device (256 units if no device can be queried).  The count is
// cached per device: it sizes the workspace of every call.
int draft_persist_max_wg() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cached[kMaxDevices] = {};
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 2 * 256;
    }
    if (dev >= 0 && dev < kMaxDevices && (cus = cached[dev].load(std::memory_order_relaxed)) > 0) return 2 * cus;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        return 2 * 256;
    }
    if (dev >= 0 && dev < kMaxDevices) cached[dev].store(cus, std::memory_order_relaxed);
    return 2 * cus;
}

DraftLayout draft_layout(const dspark_dims& d) {
    DraftLayout L{};
    L.Bpad = (d.B + 15) / 16 * 16;
    L.P = draft_partials(d);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t rows = static_cast<size_t>(L.Bpad);
    L.dead = take(sizeof(int32_t) * d.B);
    L.emb = take(sizeof(float) * rows * d.r);
    L.coef = take(sizeof(float) * rows * d.r);
    L.ebf = take(sizeof(uint16_t) * 2 * rows * d.r);
    L.state = take(sizeof(float) * rows * d.r);
    L.state2 = take(d.head == DSPARK_HEAD_RNN ? sizeof(float) * rows * d.r : 0);
    L.gates = take(sizeof(float) * rows * 3 * d.r);
    L.gh = take(d.head == DSPARK_HEAD_RNN ? sizeof(float) * static_cast<size_t>(d.B) * d.gamma * 3 * d.r : 0);
    L.hdot = take(sizeof(float) * static_cast<size_t>(d.B) * d.gamma);
    L.best = take(sizeof(uint64_t) * 16 * kDraftKeyCopies * static_cast<size_t>(d.B) * d.gamma);
    L.bar = take(sizeof(uint32_t) * kDraftBarWords);
    L.flags = take(sizeof(uint64_t) * (static_cast<size_t>(draft_persist_max_wg()) + 1));
    const size_t nq = static_cast<size_t>(d.gamma) * d.B * draft_persist_max_wg();
    L.qms = take(sizeof(float) * 2 * nq);
    const size_t np = static_cast<size_t>(d.B) * L.P;
    L.pm = take(sizeof(float) * np);
    L.ps = take(sizeof(float) * np);
    L.pkey = take(sizeof(uint64_t) * np);
    L.pzx = take(sizeof(float) * np);
    L.total = off;
    return L;
}

// ------------------------------------------------------------------ init

// Arguments of the per-block set-up before the sequential loop.
template <typename T>
struct InitArgs {
    const int32_t* anchor;
    const T* W1;
    const T* w_conf;
    const T* h;
    int V, r, d, gamma, B, Bpad, head;
    int32_t* dead;
    float* emb;
    float* coef;
    uint16_t* ebf;
    float* state;
    float* hdot;
    float* conf;
    float* survival;
};

constexpr int kInitPos = 8;  // positions whose h rows are read at the same time

// Block b, by one workgroup: the h part of every position's confidence
// logit, w[0:d] . h_{b,k}, which does not depend on the drafted tokens and
// so leaves the sequential loop (kInitPos positions at a time, partial sums
// added over the waves in wave order); then e = W1[anchor_b] (Eq 5 at the
// first position), c_1 and S_1 (Eq 7).  Rows b in [B, Bpad) only clear the
// padding rows of the MFMA operand.  red: 16 x kInitPos floats of LDS.
template <typename T>
__device__ void draft_init_block(const InitArgs<T>& a, int b, float* red) {
    const size_t row = static_cast<size_t>(b) * a.r;
    if (b >= a.B) {
        for (int j = threadIdx.x; j < a.r; j += blockDim.x) {
            a.emb[row + j] = 0.0f;
            a.coef[row + j] = 0.0f;
            a.state[row + j] = 0.0f;
            a.ebf[row + j] = 0;
            a.ebf[static_cast<size_t>(a.Bpad) * a.r + row + j] = 0;
        }
        return;
    }
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nw = blockDim.x / kWave;
    float hk0 = 0.0f;  // thread 0: the h part of position 0
    for (int k0 = 0; k0 < a.gamma; k0 += kInitPos) {
        float hp[kInitPos];
#pragma unroll
        for (int j = 0; j < kInitPos; ++j) hp[j] = 0.0f;
        const int64_t hrow = (static_cast<int64_t>(b) * a.gamma + k0) * a.d;
        bool vec = false;
        if constexpr (std::is_same<T, uint16_t>::value)
            vec = a.d % 8 == 0 && (reinterpret_cast<uintptr_t>(a.h) & 15) == 0 &&
                  (reinterpret_cast<uintptr_t>(a.w_conf) & 15) == 0;
        if (vec) {
            // 8 bf16 values per 16-byte load, the rows' loads issued together
            for (int c = threadIdx.x; c < a.d / 8; c += blockDim.x) {
                const u32x4 wv = *reinterpret_cast<const u32x4*>(a.w_conf + 8 * c);
                u32x4 hv[kInitPos];
#pragma unroll
                for (int j = 0; j < kInitPos; ++j)
                    if (k0 + j < a.gamma)
                        hv[j] = *reinterpret_cast<const u32x4*>(a.h + hrow + static_cast<int64_t>(j) * a.d + 8 * c);
#pragma unroll
                for (int j = 0; j < kInitPos; ++j)
                    if (k0 + j < a.gamma)
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            hp[j] = fmaf(lo_bf16(wv[q]), lo_bf16(hv[j][q]), hp[j]);
                            hp[j] = fmaf(hi_bf16(wv[q]), hi_bf16(hv[j][q]), hp[j]);
                        }
            }
        } else {
            for (int i = threadIdx.x; i < a.d; i += blockDim.x) {
                const float wi = load_f(a.w_conf, i);
#pragma unroll
                for (int j = 0; j < kInitPos; ++j)
                    if (k0 + j < a.gamma) hp[j] = fmaf(wi, load_f(a.h, hrow + static_cast<int64_t>(j) * a.d + i), hp[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < kInitPos; ++j)
            for (int o = 32; o > 0; o >>= 1) hp[j] += __shfl_xor(hp[j], o);
        __syncthreads();  // red is free
        if (lane == 0)
#pragma unroll
            for (int j = 0; j < kInitPos; ++j) red[wave * kInitPos + j] = hp[j];
        __syncthreads();
        if (threadIdx.x < kInitPos && k0 + static_cast<int>(threadIdx.x) < a.gamma) {
            float t = 0.0f;
            for (int w = 0; w < nw; ++w) t += red[w * kInitPos + threadIdx.x];
            a.hdot[static_cast<size_t>(b) * a.gamma + k0 + threadIdx.x] = t;
            if (k0 == 0) hk0 = t;
        }
    }

    const int prev = a.anchor[b];
    const bool bad = prev < 0 || prev >= a.V;
    if (threadIdx.x == 0) a.dead[b] = bad ? 1 : 0;
    float part = 0.0f;
    for (int j = threadIdx.x; j < a.r; j += blockDim.x) {
        const float ej = bad ? 0.0f : load_f(a.W1, static_cast<int64_t>(prev) * a.r + j);
        a.emb[row + j] = ej;
        a.state[row + j] = 0.0f;  // Eq 6: s_0 = 0
        if (a.head == DSPARK_HEAD_MARKOV) {
            a.coef[row + j] = ej;
            a.ebf[row + j] = static_cast<uint16_t>(f32_to_bf16(ej));  // exact: W1 is bf16 here
            a.ebf[static_cast<size_t>(a.Bpad) * a.r + row + j] = 0;
        }
        part += load_f(a.w_conf, a.d + j) * ej;
    }
    const float ae = block_sum(part, red);
    if (threadIdx.x == 0) {
        const float c = bad ? NAN : sigmoidf_(hk0 + ae);
        a.conf[static_cast<size_t>(b) * a.gamma] = c;
        a.survival[static_cast<size_t>(b) * a.gamma] = c;
    }
}

constexpr int kInitThreads = 512;

template <typename T>
__global__ __launch_bounds__(kInitThreads) void k_draft_init(InitArgs<T> a) {
    __shared__ float red[16 * kInitPos];
    draft_init_block(a, blockIdx.x, red);
}

// ------------------------------------------------------------ RNN step

// G[b, q] = sum_c W_rnn[q, c] zeta_b[c] with zeta_b = [s_b; e_b; h_{b,k}]
// (Eq 6).  A 16 (rows q) x 16 (blocks b) output tile per workgroup, K staged
// through LDS in slices of 64.
template <typename T>
__global__ __launch_bounds__(256) void k_rnn_gates(
    const T* __restrict__ W_rnn, const float* __restrict__ state, const float* __restrict__ emb,
    const T* __restrict__ h, int r, int d, int gamma, int k, int B, float* __restrict__ gates) {
    __shared__ float Ws[16][65];
    __shared__ float Zs[16][65];
    const int tq = threadIdx.x & 15, tb = threadIdx.x >> 4;
    const int q0 = blockIdx.x * 16, b0 = blockIdx.y * 16;
    const int width = 2 * r + d, Q = 3 * r;
    float acc = 0.0f;
    for (int c0 = 0; c0 < width; c0 += 64) {
        for (int t = threadIdx.x; t < 16 * 64; t += blockDim.x) {
            const int row = t >> 6, col = t & 63;
            const int q = q0 + row, c = c0 + col;
            Ws[row][col] = (q < Q && c < width) ? load_f(W_rnn, static_cast<int64_t>(q) * width + c) : 0.0f;
            const int b = b0 + row;
            float zv = 0.0f;
            if (b < B && c < width) {
                if (c < r)
                    zv = state[static_cast<size_t>(b) * r + c];
                else if (c < 2 * r)
                    zv = emb[static_cast<size_t>(b) * r + (c - r)];
                else
                    zv = load_f(h, (static_cast<int64_t>(b) * gamma + k) * d + (c - 2 * r));
            }
            Zs[row][col] = zv;
        }
        __syncthreads();
#pragma unroll 16
        for (int cc = 0; cc < 64; ++cc) acc = fmaf(Ws[tq][cc], Zs[tb][cc], acc);
        __syncthreads();
    }
    if (q0 + tq < Q && b0 + tb < B) gates[static_cast<size_t>(b0 + tb) * Q + q0 + tq] = acc;
}

// Matrix-core form of the same projection (bf16 weights, r % 32 == 0,
// d % 8 == 0).  The columns of W_rnn that multiply h_k do not depend on the
// drafted tokens, so their part of G is one GEMM over all B x gamma
// positions before the loop (gate_h_tile); each step then only adds the s and
// e columns (k_gate_update).  D[q][m] = sum_j W_rnn[q][col(j)] A[m][j] is
// built from v_mfma_f32_16x16x32_bf16 tiles with A = 16 rows of W_rnn and
// B = 16 operand rows: lane (g, n) supplies W_rnn row q0 + n and operand row
// m0 + n at k = 8 g .. 8 g + 7 of a 32-wide chunk and receives D[q0 + 4 g +
// i][m0 + n] in accumulator element i.  The waves of a workgroup take
// interleaved chunks of K and their partial tiles are added in a fixed
// order through LDS (deterministic).  Products of bf16 values are exact in
// fp32; the fp32 state s is fed as three bf16 pieces hi + mid + lo, which
// sum to s exactly, so the step GEMM keeps fp32 accuracy.
constexpr int kGateTile = 32;
constexpr int kGateHWaves = 8;  // h projection (K = d): K split over 8 waves

__device__ __forceinline__ u32x4 load8_bf16_or0(const uint16_t* p, bool ok) {
    return ok ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
}

// 8 consecutive floats -> 8 bf16 (round to nearest even) packed in pairs.
__device__ __forceinline__ u32x4 pack8_bf16(const float (&x)[8]) {
    u32x4 r;
#pragma unroll
    for (int p = 0; p < 4; ++p) r[p] = f32_to_bf16(x[2 * p]) | (f32_to_bf16(x[2 * p + 1]) << 16);
    return r;
}

// bf16 element q (0..7) of a packed 8-element operand, as float.
__device__ __forceinline__ float unpack8_at(const u32x4& v, int q) {
    return (q & 1) ? hi_bf16(v[q >> 1]) : lo_bf16(v[q >> 1]);
}

// Gh[m][q] = sum_{i<d} W_rnn[q][2r + i] h[m][i] for the M = B x gamma rows
// of h (row m = b gamma + k).  One workgroup per 64 (q) x 64 (m) tile, so
// that each operand row is read by fewer workgroups (K = d is long); each of
// its 8 waves accumulates the whole 4 x 4 grid of 16 x 16 tiles over every
// 8th 32-wide chunk of K with two chunks in flight, and the 8 partial tiles
// are added in a fixed order through LDS (waves w and w + 4 first).
constexpr int kGhTile = 64;

__device__ __forceinline__ void gate_h_tile(const uint16_t* __restrict__ W_rnn, const uint16_t* __restrict__ h,
                                            int r, int d, int M, float* __restrict__ Gh, int tile,
                                            f32x4 (*part)[16][kWave] /* [4][16][kWave] */) {
    const int Q = 3 * r, ldw = 2 * r + d;
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    const int wave = threadIdx.x >> 6;
    const int tq = (Q + kGhTile - 1) / kGhTile;
    const int q0 = (tile % tq) * kGhTile, m0 = (tile / tq) * kGhTile;
    // rows past Q or M read row 0 (their results are not stored)
    const uint16_t* wrow[4];
    const uint16_t* hrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = q0 + 16 * i + n, m = m0 + 16 * i + n;
        wrow[i] = W_rnn + static_cast<size_t>(q < Q ? q : 0) * ldw + 2 * r;
        hrow[i] = h + static_cast<size_t>(m < M ? m : 0) * d;
    }
    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int kStride = 32 * kGateHWaves;
    u32x4 wa[2][4], ob[2][4];
    auto fetch = [&](int slot, int k0) {
        const int kk = k0 + 8 * g;
        const bool kin = kk < d;  // d % 8 == 0: a lane's 8 values are all in or all out
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            wa[slot][i] = load8_bf16_or0(wrow[i] + kk, kin);
            ob[slot][i] = load8_bf16_or0(hrow[i] + kk, kin);
        }
    };
    auto mma = [&](int slot) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, wa[slot][i]),
                                                                    __builtin_bit_cast(bf16x8, ob[slot][j]), acc[i][j],
                                                                    0, 0, 0);
    };
    const int kfirst = 32 * wave;
    fetch(0, kfirst);
    fetch(1, kfirst + kStride);
    for (int k0 = kfirst; k0 < d; k0 += 2 * kStride) {
        mma(0);
        if (k0 + 2 * kStride < d) fetch(0, k0 + 2 * kStride);
        if (k0 + kStride >= d) break;
        mma(1);
        if (k0 + 3 * kStride < d) fetch(1, k0 + 3 * kStride);
    }
    // waves 4..7 hand their tiles to waves 0..3, which then publish the sums
    if (wave >= 4)
#pragma unroll
        for (int t = 0; t < 16; ++t) part[wave - 4][t][lane] = acc[t >> 2][t & 3];
    __syncthreads();
    if (wave < 4)
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const f32x4 u = part[wave][t][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[t >> 2][t & 3][e] += u[e];
        }
    __syncthreads();
    if (wave < 4)
#pragma unroll
        for (int t = 0; t < 16; ++t) part[wave][t][lane] = acc[t >> 2][t & 3];
    __syncthreads();
    // wave w stores tiles w and w + 8: the four pair sums added in order
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int t = wave + 8 * tt, i = t >> 2, j = t & 3;
        f32x4 v = part[0][t][lane];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            const f32x4 u = part[w][t][lane];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += u[e];
        }
        const int m = m0 + 16 * j + n;
        if (m < M)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int q = q0 + 16 * i + 4 * g + e;
                if (q < Q) Gh[static_cast<size_t>(m) * Q + q] = v[e];
            }
    }
}

// The RNN head's set-up in one launch: workgroups [0, tiles) compute the
// h-projection tiles, the rest the per-block set-up (block = index -
// tiles).  The two are independent and the tiles leave compute units idle,
// which the set-up then uses.
__global__ __launch_bounds__(kGateHWaves * kWave) void k_rnn_prologue(const uint16_t* __restrict__ W_rnn,
                                                                      int M, float* __restrict__ Gh, int tiles,
                                                                      InitArgs<uint16_t> ia) {
    __shared__ f32x4 part[4][16][kWave];
    __shared__ float red[16 * kInitPos];
    if (static_cast<int>(blockIdx.x) < tiles)
        gate_h_tile(W_rnn, ia.h, ia.r, ia.d, M, Gh, blockIdx.x, part);
    else
        draft_init_block(ia, static_cast<int>(blockIdx.x) - tiles, red);
}

// One step of Eq 6 after the h columns, in one launch: G[b][q] = Gh[b gamma
// + k][q] + sum_j W_rnn[q][j] s[b][j] + sum_j W_rnn[q][r + j] e[b][j], then
// the gated state update and the bias coefficients o = tanh(G_o), with the
// formulas of k_rnn_update.  A workgroup owns state columns j0 .. j0 + 15
// of blocks m0 .. m0 + 31 and computes the three gate rows that update them
// (q = j, r + j, 2r + j) as 16 x 16 matrix-core tiles (the fp32 state as
// three exact bf16 pieces, as in gate_h_tile's layout); its 8 waves take every
// 8th 32-wide chunk of K, the partial tiles are added in wave order through
// LDS, and each thread updates one (block, column).  The state is read from
// s_in and written to s_out (two buffers, alternating by step): the other
// workgroups still read s_in as the projection's operand.
constexpr int kGuWaves = 8;
constexpr int kGuCols = 16;

__global__ __launch_bounds__(kGuWaves * kWave) void k_gate_update(
    const uint16_t* __restrict__ W_rnn, const float* __restrict__ Gh, const float* __restrict__ s_in,
    const float* __restrict__ emb, int r, int d, int gamma, int k, int B, int Bpad, float* __restrict__ s_out,
    float* __restrict__ coef, uint16_t* __restrict__ ebf) {
    __shared__ f32x4 part[kGuWaves][6][kWave];
    const int Q = 3 * r, ldw = 2 * r + d;
    const int lane = threadIdx.x & 63, g = lane >> 4, n = lane & 15;
    const int wave = threadIdx.x >> 6;
    const int tj = r / kGuCols;
    const int j0 = (blockIdx.x % tj) * kGuCols, m0 = (blockIdx.x / tj) * kGateTile;
    const bool mok[2] = {m0 + n < B, m0 + 16 + n < B};
    const size_t brow[2] = {static_cast<size_t>(mok[0] ? m0 + n : 0) * r,
                            static_cast<size_t>(mok[1] ? m0 + 16 + n : 0) * r};
    f32x4 acc[3][2];
#pragma unroll
    for (int h = 0; h < 3; ++h) acc[h][0] = acc[h][1] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int k0 = 32 * wave; k0 < r; k0 += 32 * kGuWaves) {
        const int kk = k0 + 8 * g;
        u32x4 ws_[3], we[3];
#pragma unroll
        for (int h = 0; h < 3; ++h) {
            const uint16_t* wrow = W_rnn + static_cast<size_t>(h * r + j0 + n) * ldw;
            ws_[h] = *reinterpret_cast<const u32x4*>(wrow + kk);
            we[h] = *reinterpret_cast<const u32x4*>(wrow + r + kk);
        }
        f32x4 sv[2][2], ev[2][2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
                const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
                sv[j][h2] = mok[j] ? *reinterpret_cast<const f32x4*>(s_in + brow[j] + kk + 4 * h2) : z;
                ev[j][h2] = mok[j] ? *reinterpret_cast<const f32x4*>(emb + brow[j] + kk + 4 * h2) : z;
            }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            float s8[8], e8[8], t[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                s8[q] = sv[j][q >> 2][q & 3];
                e8[q] = ev[j][q >> 2][q & 3];
            }
            const u32x4 shi = pack8_bf16(s8);
#pragma unroll
            for (int q = 0; q < 8; ++q) t[q] = s8[q] - unpack8_at(shi, q);
            const u32x4 smid = pack8_bf16(t);
#pragma unroll
            for (int q = 0; q < 8; ++q) t[q] -= unpack8_at(smid, q);
            const u32x4 slo = pack8_bf16(t);
            const u32x4 eb = pack8_bf16(e8);  // exact: e is a bf16 row of W1
#pragma unroll
            for (int h = 0; h < 3; ++h) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, ws_[h]), ae = __builtin_bit_cast(bf16x8, we[h]);
                acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, shi), acc[h][j], 0, 0, 0);
                acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, smid), acc[h][j], 0, 0, 0);
                acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, slo), acc[h][j], 0, 0, 0);
                acc[h][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ae, __builtin_bit_cast(bf16x8, eb), acc[h][j], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int h = 0; h < 3; ++h)
#pragma unroll
        for (int j = 0; j < 2; ++j) part[wave][2 * h + j][lane] = acc[h][j];
    __syncthreads();
    // thread (wave, lane g n): block m0 + 16 (wave % 2) + n, column
    // j0 + 4 g + wave / 2 (accumulator element wave / 2 of lane g n)
    const int j = wave & 1, e = wave >> 1;
    const int m = m0 + 16 * j + n;
    if (m >= B) return;
    float G[3];
#pragma unroll
    for (int h = 0; h < 3; ++h) {
        float v = part[0][2 * h + j][lane][e];
#pragma unroll
        for (int w = 1; w < kGuWaves; ++w) v += part[w][2 * h + j][lane][e];
        G[h] = v;
    }
    const int jc = j0 + 4 * g + e;
    const float* gh = Gh + (static_cast<size_t>(m) * gamma + k) * Q;
    const size_t row = static_cast<size_t>(m) * r;
    const float gate = 1.0f / (1.0f + expf(-(gh[jc] + G[0])));
    const float cand = tanhf(gh[r + jc] + G[1]);
    const float o = tanhf(gh[2 * r + jc] + G[2]);
    s_out[row + jc] = gate * s_in[row + jc] + (1.0f - gate) * cand;
    coef[row + jc] = o;
    const uint32_t hi = f32_to_bf16(o);
    const uint32_t lo = f32_to_bf16(o - __uint_as_float(hi << 16));
    ebf[row + jc] = static_cast<uint16_t>(hi);
    ebf[static_cast<size_t>(Bpad) * r + row + jc] = static_cast<uint16_t>(lo);
}

bool rnn_gate_mfma_ok(const dspark_dims& d) {
    return d.dtype == DSPARK_BF16 && d.r % 32 == 0 && d.d % 8 == 0;
}

// Gated state update of Eq 6 and the bias coefficients o = tanh(W_o z).
// o is not exact in bf16, so the MFMA operand carries it as hi + lo planes.
__global__ __launch_bounds__(256) void k_rnn_update(const float* __restrict__ gates,
                                                    float* __restrict__ state,
                                                    float* __restrict__ coef,
                                                    uint16_t* __restrict__ ebf, int r, int Bpad) {
    const int b = blockIdx.x;
    const float* G = gates + static_cast<size_t>(b) * 3 * r;
    const size_t row = static_cast<size_t>(b) * r;
    for (int j = threadIdx.x; j < r; j += blockDim.x) {
        const float gate = 1.0f / (1.0f + expf(-G[j]));
        const float cand = tanhf(G[r + j]);
        const float o = tanhf(G[2 * r + j]);
        state[row + j] = gate * state[row + j] + (1.0f - gate) * cand;
        coef[row + j] = o;
        const uint32_t hi = f32_to_bf16(o);
        const uint32_t lo = f32_to_bf16(o - __uint_as_float(hi << 16));
        ebf[row + j] = static_cast<uint16_t>(hi);
        ebf[static_cast<size_t>(Bpad) * r + row + j] = static_cast<uint16_t>(lo);
    }
}

// -------------------------------------------------------- stream (MFMA)

// Per-lane statistics of the 16 consecutive columns v0 .. v0+15 of block b
// (z[j] = U + bias of column v0 + j).  Columns at or past V are masked to
// -inf, so they never win and add exp(-inf) = 0.  One argmax key per lane:
// the maximum perturbed logit, then the lowest column attaining it.
template <bool FULL>
__device__ __forceinline__ Stats lane_stats16(const float (&z)[16], int v0, int V, int b, int k,
                                              bool sampling, float invT, uint32_t key0,
                                              uint32_t key1, uint32_t ctr3) {
    float zs[16], y[16];
    const int nvalid = V - v0;  // >= 8 here (V % 8 == 0 and v0 < V)
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


// ------------------------------------------------------ stream (generic)

// Any dtype / rank: each thread owns 4 consecutive columns and walks the
// blocks; the bias is a plain float dot product with coef.
template <typename T>
__global__ __launch_bounds__(256) void k_stream_generic(
    const T* __restrict__ U, const T* __restrict__ W2, const float* __restrict__ coef,
    const float* __restrict__ temperature, int V, int r, int B, int gamma, int k, uint32_t key0,
    uint32_t key1, uint32_t ctr3, float* __restrict__ pm, float* __restrict__ ps,
    uint64_t* __restrict__ pkey, float* __restrict__ pzx) {
    __shared__ Stats red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int v0 = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
    const int P = gridDim.x;
    for (int b = 0; b < B; ++b) {
        Stats st = stats_empty();
        if (v0 < V) {
            const float temp = temperature[b];
            const bool sampling = temp > 0.0f;
            const float invT = sampling ? 1.0f / temp : 1.0f;
            const int64_t urow = (static_cast<int64_t>(b) * gamma + k) * V;
            float z[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) z[c] = (v0 + c < V) ? load_f(U, urow + v0 + c) : 0.0f;
            const float* cb = coef + static_cast<size_t>(b) * r;
            for (int j = 0; j < r; ++j) {
                const float cj = cb[j];
                const int64_t wrow = static_cast<int64_t>(j) * V + v0;
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (v0 + c < V) z[c] = fmaf(cj, load_f(W2, wrow + c), z[c]);
            }
            u32x4 w = {0u, 0u, 0u, 0u};
            if (sampling) {
                const u32x4 ctr = {static_cast<uint32_t>(v0) >> 2, static_cast<uint32_t>(k),
                                   static_cast<uint32_t>(b), ctr3};
                w = philox4x32_10(ctr, key0, key1);
            }
            float m = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if (v0 + c < V) m = fmaxf(m, z[c] * invT);
            float s = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                if (v0 + c < V) {
                    const float zs = z[c] * invT;
                    s += __expf(zs - m);
                    const float y = sampling ? zs + gumbel_from_word(w[c]) : zs;
                    const uint64_t key = argmax_key(y, static_cast<uint32_t>(v0 + c));
                    if (key > st.key) {
                        st.key = key;
                        st.zx = zs;
                    }
                }
            }
            st.m = m;
            st.s = s;
        }
        for (int o = 32; o > 0; o >>= 1) st = stats_merge(st, shfl_xor_stats(st, o));
        if (lane == 0) red[wave] = st;
        __syncthreads();
        if (threadIdx.x == 0) {
            Stats t = red[0];
            for (int w2 = 1; w2 < static_cast<int>(blockDim.x / kWave); ++w2) t = stats_merge(t, red[w2]);
            const size_t o = static_cast<size_t>(b) * P + blockIdx.x;
            pm[o] = t.m;
            ps[o] = t.s;
            pkey[o] = t.key;
            pzx[o] = t.zx;
        }
        __syncthreads();
    }
}

// One step over V (per-step driver): workgroup = 4 waves = 256 columns, wave
// = a 64-column W2 tile held in registers as MFMA A-fragments (see
// mfma_tile.h) for all blocks.  Per 16-block unit: z = U_k + E W2 on the
// matrix cores (NPL = 2: E as bf16 hi + lo planes); lane (g, n) ends up with
// the 16 consecutive columns vt + 16g .. vt + 16g + 15 of block row b =
// 16 nb + n, so all of a lane's softmax and argmax work is for one block
// row; the per-lane statistics are merged across the 4 lanes of a column
// group and the 4 waves.  The unit's E rows (all planes) are staged through
// a double-buffered LDS area, and its U values and temperatures are loaded a
// unit ahead, unconditionally from clamped addresses so that the loads stay
// in flight across the previous unit; one workgroup barrier per unit.
template <int KC, int NPL>
__global__ __launch_bounds__(256, 2) void k_stream_mfma(
    const uint16_t* __restrict__ U, const uint16_t* __restrict__ W2,
    const uint16_t* __restrict__ ebf, const float* __restrict__ temperature, int V, int B,
    int Bpad, int gamma, int k, uint32_t key0, uint32_t key1, uint32_t ctr3,
    float* __restrict__ pm, float* __restrict__ ps, uint64_t* __restrict__ pkey,
    float* __restrict__ pzx) {
    constexpr int r = KC * 32;
    constexpr int ldE = r + 8;                        // padded row stride (bank spread)
    constexpr int kChunks = NPL * 16 * (r / 8);       // 16-byte pieces of one unit's E rows
    constexpr int kPer = (kChunks + 255) / 256;       // per thread
    __shared__ __attribute__((aligned(16))) uint16_t Es[2][NPL * 16 * ldE];
    __shared__ Stats red[2][kWavesPerWG][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int vt = (blockIdx.x * kWavesPerWG + wave) * kTileV;
    const int P = gridDim.x;
    const int NB = Bpad / 16;

    const int v0 = vt + 16 * g;
    const bool live = v0 < V;
    const int ua = live ? v0 : 0, ub = (live && v0 + 8 < V) ? v0 + 8 : ua;
    u32x4 estage[kPer];
    auto fetch_e = [&](int nb) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = (threadIdx.x + 256 * i) % kChunks;
            const int pl = t / (16 * (r / 8)), rem = t % (16 * (r / 8));
            const int row = rem / (r / 8), col = rem % (r / 8);
            estage[i] = *reinterpret_cast<const u32x4*>(ebf + (static_cast<size_t>(pl) * Bpad + nb * 16 + row) * r +
                                                        col * 8);
        }
    };
    auto stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int t = threadIdx.x + 256 * i;
            if (t < kChunks) {
                const int pl = t / (16 * (r / 8)), rem = t % (16 * (r / 8));
                const int row = rem / (r / 8), col = rem % (r / 8);
                *reinterpret_cast<u32x4*>(&Es[buf][(pl * 16 + row) * ldE + col * 8]) = estage[i];
            }
        }
    };
    struct UnitIn {
        u32x4 u0, u1;
        float temp;
    };
    auto fetch = [&](int nb) {
        UnitIn in;
        const int b = min(nb * 16 + n, B - 1);
        const uint16_t* row = U + (static_cast<size_t>(b) * gamma + k) * V;
        in.u0 = *reinterpret_cast<const u32x4*>(row + ua);
        in.u1 = *reinterpret_cast<const u32x4*>(row + ub);
        in.temp = temperature[b];
        return in;
    };

    W2Tile<KC> w2;
    w2.load(W2, V, vt, g, n);
    fetch_e(0);
    UnitIn nxt = fetch(0);
    stage(0);
    __syncthreads();
    for (int nb = 0; nb < NB; ++nb) {
        const UnitIn cur = nxt;
        if (nb + 1 < NB) {
            fetch_e(nb + 1);
            nxt = fetch(nb + 1);
        }
        const int b = nb * 16 + n;
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int pl = 0; pl < NPL; ++pl) w2.mul(&Es[nb & 1][(pl * 16 + n) * ldE + 8 * g], acc);

        Stats st = stats_empty();
        if (b < B && live) {
            const float temp = cur.temp;
            const bool sampling = temp > 0.0f;
            const float invT = sampling ? 1.0f / temp : 1.0f;
            const uint32_t w[8] = {cur.u0[0], cur.u0[1], cur.u0[2], cur.u0[3],
                                   cur.u1[0], cur.u1[1], cur.u1[2], cur.u1[3]};
            float z[16];
#pragma unroll
            for (int q = 0; q < 4; ++q)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int j = 4 * q + c;
                    z[j] = ((j & 1) ? hi_bf16(w[j >> 1]) : lo_bf16(w[j >> 1])) + acc[c][q];
                }
            if (v0 + 16 <= V)
                st = lane_stats16<true>(z, v0, V, b, k, sampling, invT, key0, key1, ctr3);
            else
                st = lane_stats16<false>(z, v0, V, b, k, sampling, invT, key0, key1, ctr3);
        }
        st = stats_merge_xor<16>(st);
        st = stats_merge_xor<32>(st);
        if (g == 0) red[nb & 1][wave][n] = st;
        if (nb + 1 < NB) stage((nb + 1) & 1);
        __syncthreads();
        // the 4 waves' statistics of this unit's 16 blocks, merged by one
        // wave (a different one each unit, so that no wave falls behind):
        // lane (w, n) takes wave w's statistics of block n, two exchange
        // steps merge the 4 in a fixed tree order
        if (wave == (nb & (kWavesPerWG - 1))) {
            static_assert(kWavesPerWG == 4, "one lane per (wave, block)");
            Stats t = red[nb & 1][g][n];
            t = stats_merge_xor<16>(t);
            t = stats_merge_xor<32>(t);
            if (g == 0 && b < B) {
                const size_t o = static_cast<size_t>(b) * P + blockIdx.x;
                pm[o] = t.m;
                ps[o] = t.s;
                pkey[o] = t.key;
                pzx[o] = t.zx;
            }
        }
    }
}

// --------------------------------------------------------------- combine

// Block b: merge the P partial statistics of step k in a fixed order, emit
// x_k and log p_k, then prepare step k+1: e = W1[x_k], c_{k+1}, S_{k+1}.
template <typename T>
__global__ __launch_bounds__(256) void k_combine(
    const float* __restrict__ pm, const float* __restrict__ ps, const uint64_t* __restrict__ pkey,
    const float* __restrict__ pzx, int P, const T* __restrict__ W1, const T* __restrict__ w_conf,
    const float* __restrict__ hdot, int V, int r, int d, int gamma, int k, int head, int write_bf16,
    int32_t* __restrict__ dead, float* __restrict__ emb, float* __restrict__ coef,
    uint16_t* __restrict__ ebf, int32_t* __restrict__ tokens, float* __restrict__ logp,
    float* __restrict__ conf, float* __restrict__ survival) {
    __shared__ Stats red[4];
    __shared__ int sx;
    __shared__ float rs[16];
    const int b = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    Stats st = stats_empty();
    for (int p = threadIdx.x; p < P; p += blockDim.x) {
        const size_t o = static_cast<size_t>(b) * P + p;
        st = stats_merge(st, Stats{pm[o], ps[o], pkey[o], pzx[o]});
    }
    for (int o = 32; o > 0; o >>= 1) st = stats_merge(st, shfl_xor_stats(st, o));
    if (lane == 0) red[wave] = st;
    __syncthreads();
    const size_t out = static_cast<size_t>(b) * gamma + k;
    if (threadIdx.x == 0) {
        Stats t = red[0];
        for (int w = 1; w < static_cast<int>(blockDim.x / kWave); ++w) t = stats_merge(t, red[w]);
        int x = static_cast<int>(key_index(t.key));
        const bool bad = dead[b] != 0 || t.key == kKeyNone || x < 0 || x >= V;
        if (bad) {
            dead[b] = 1;
            x = -1;
        }
        tokens[out] = x;
        if (logp) logp[out] = bad ? NAN : t.zx - (t.m + logf(t.s));
        sx = x;
    }
    __syncthreads();
    if (k + 1 >= gamma) return;
    const int x = sx;
    const size_t row = static_cast<size_t>(b) * r;
    float part = 0.0f;
    for (int j = threadIdx.x; j < r; j += blockDim.x) {
        const float ej = x >= 0 ? load_f(W1, static_cast<int64_t>(x) * r + j) : 0.0f;
        emb[row + j] = ej;
        if (head == DSPARK_HEAD_MARKOV) {
            coef[row + j] = ej;
            if (write_bf16) ebf[row + j] = static_cast<uint16_t>(f32_to_bf16(ej));
        }
        part += load_f(w_conf, d + j) * ej;
    }
    const float a = block_sum(part, rs) + hdot[out + 1];
    if (threadIdx.x == 0) {
        const float c = x >= 0 ? sigmoidf_(a) : NAN;
        conf[out + 1] = c;
        survival[out + 1] = survival[out] * c;
    }
}

// ---------------------------------------------------------------- launch

template <int KC, int NPL>
static void launch_mfma(const DraftArgs& a, const DraftLayout& L, int k, char* ws) {
    const dspark_dims& D = a.dims;
    hipLaunchKernelGGL((k_stream_mfma<KC, NPL>), dim3(L.P), dim3(256), 0, a.stream,
                       static_cast<const uint16_t*>(a.U), static_cast<const uint16_t*>(a.W2),
                       reinterpret_cast<const uint16_t*>(ws + L.ebf), a.temperature, D.V, D.B, L.Bpad,
                       D.gamma, k, static_cast<uint32_t>(a.seed), static_cast<uint32_t>(a.seed >> 32),
                       static_cast<uint32_t>(a.offset), reinterpret_cast<float*>(ws + L.pm),
                       reinterpret_cast<float*>(ws + L.ps), reinterpret_cast<uint64_t*>(ws + L.pkey),
                       reinterpret_cast<float*>(ws + L.pzx));
}

template <int NPL>
static void launch_mfma_kc(const DraftArgs& a, const DraftLayout& L, int k, char* ws) {
    switch (a.dims.r / 32) {
        case 1: launch_mfma<1, NPL>(a, L, k, ws); break;
        case 2: launch_mfma<2, NPL>(a, L, k, ws); break;
        case 3: launch_mfma<3, NPL>(a, L, k, ws); break;
        case 4: launch_mfma<4, NPL>(a, L, k, ws); break;
        case 5: launch_mfma<5, NPL>(a, L, k, ws); break;
        case 6: launch_mfma<6, NPL>(a, L, k, ws); break;
        case 7: launch_mfma<7, NPL>(a, L, k, ws); break;
        default: launch_mfma<8, NPL>(a, L, k, ws); break;
    }
}

template <typename T>
static hipError_t launch_draft_t(const DraftArgs& a) {
    const dspark_dims& D = a.dims;
    const DraftLayout L = draft_layout(D);
    char* ws = a.ws;
    const bool mfma = mfma_path_ok(D);
    int32_t* dead = reinterpret_cast<int32_t*>(ws + L.dead);
    float* emb = reinterpret_cast<float*>(ws + L.emb);
    float* coef = reinterpret_cast<float*>(ws + L.coef);
    uint16_t* ebf = reinterpret_cast<uint16_t*>(ws + L.ebf);
    float* state = reinterpret_cast<float*>(ws + L.state);
    float* state2 = reinterpret_cast<float*>(ws + L.state2);
    float* gates = reinterpret_cast<float*>(ws + L.gates);
    const T* U = static_cast<const T*>(a.U);
    const T* h = static_cast<const T*>(a.h);
    const T* W1 = static_cast<const T*>(a.W1);
    const T* W2 = static_cast<const T*>(a.W2);
    const T* wc = static_cast<const T*>(a.w_conf);
    const T* Wr = static_cast<const T*>(a.W_rnn);

    const InitArgs<T> ia{a.anchor, W1,     wc,   h,     D.V,   D.r,   D.d,
                         D.gamma,  D.B,    L.Bpad, D.head, dead, emb,  coef,
                         ebf,      state,  reinterpret_cast<float*>(ws + L.hdot), a.conf, a.survival};
    // RNN on matrix cores: the h columns of the joint projection for every
    // position at once, before the loop, in the same launch as the set-up
    const bool gate_mfma = D.head == DSPARK_HEAD_RNN && rnn_gate_mfma_ok(D) &&
                           (reinterpret_cast<uintptr_t>(a.W_rnn) & 15) == 0 &&
                           (reinterpret_cast<uintptr_t>(a.h) & 15) == 0;
    float* gh = reinterpret_cast<float*>(ws + L.gh);
    bool set_up = false;
    if constexpr (std::is_same<T, uint16_t>::value) {  // gate_mfma implies bf16
        if (gate_mfma) {
            const int M = D.B * D.gamma;
            const int tiles = ((3 * D.r + kGhTile - 1) / kGhTile) * ((M + kGhTile - 1) / kGhTile);
            hipLaunchKernelGGL(k_rnn_prologue, dim3(tiles + L.Bpad), dim3(kGateHWaves * kWave), 0, a.stream,
                               reinterpret_cast<const uint16_t*>(Wr), M, gh, tiles, ia);
            set_up = true;
        }
    }
    if (!set_up) hipLaunchKernelGGL((k_draft_init<T>), dim3(L.Bpad), dim3(kInitThreads), 0, a.stream, ia);
    for (int k = 0; k < D.gamma; ++k) {
        if (D.head == DSPARK_HEAD_RNN) {
            if (gate_mfma) {
                // s_k in buffer k % 2, s_{k+1} into the other
                float* s_in = (k & 1) ? state2 : state;
                float* s_out = (k & 1) ? state : state2;
                const int tiles = (D.r / kGuCols) * ((D.B + kGateTile - 1) / kGateTile);
                hipLaunchKernelGGL(k_gate_update, dim3(tiles), dim3(kGuWaves * kWave), 0, a.stream,
                                   reinterpret_cast<const uint16_t*>(Wr), gh, s_in, emb, D.r, D.d, D.gamma, k, D.B,
                                   L.Bpad, s_out, coef, ebf);
            } else {
                hipLaunchKernelGGL((k_rnn_gates<T>), dim3((3 * D.r + 15) / 16, (D.B + 15) / 16), dim3(256), 0,
                                   a.stream, Wr, state, emb, h, D.r, D.d, D.gamma, k, D.B, gates);
                hipLaunchKernelGGL(k_rnn_update, dim3(D.B), dim3(256), 0, a.stream, gates, state, coef, ebf,
                                   D.r, L.Bpad);
            }
        }
        hipError_t pe = profile_begin(a.stream);
        if (pe != hipSuccess) return pe;
        int P = L.P;
        const int npl = D.head == DSPARK_HEAD_RNN ? 2 : 1;
        if (mfma && stream_pipe_ok(D, npl)) {
            pe = launch_stream_pipe(a, L, k, ws, npl, &P);
            if (pe != hipSuccess) return pe;
        } else if (mfma) {
            if (npl == 2)
                launch_mfma_kc<2>(a, L, k, ws);
            else
                launch_mfma_kc<1>(a, L, k, ws);
        } else {
            hipLaunchKernelGGL((k_stream_generic<T>), dim3(L.P), dim3(256), 0, a.stream, U, W2, coef,
                               a.temperature, D.V, D.r, D.B, D.gamma, k, static_cast<uint32_t>(a.seed),
                               static_cast<uint32_t>(a.seed >> 32), static_cast<uint32_t>(a.offset),
                               reinterpret_cast<float*>(ws + L.pm), reinterpret_cast<float*>(ws + L.ps),
                               reinterpret_cast<uint64_t*>(ws + L.pkey),
                               reinterpret_cast<float*>(ws + L.pzx));
        }
        pe = profile_end(a.stream);
        if (pe != hipSuccess) return pe;
        hipLaunchKernelGGL((k_combine<T>), dim3(D.B), dim3(256), 0, a.stream,
                           reinterpret_cast<const float*>(ws + L.pm),
                           reinterpret_cast<const float*>(ws + L.ps),
                           reinterpret_cast<const uint64_t*>(ws + L.pkey),
                           reinterpret_cast<const float*>(ws + L.pzx), P, W1, wc,
                           reinterpret_cast<const float*>(ws + L.hdot), D.V, D.r, D.d,
                           D.gamma, k, D.head, mfma ? 1 : 0, dead, emb, coef, ebf, a.tokens, a.logp,
                           a.conf, a.survival);
    }
    return hipGetLastError();
}

const char* draft_kernel_name(const dspark_dims& d) {
    if (draft_path_option() != 1 && persist_path_ok(d)) return persist_kernel_name(d);
    if (draft_path_option() == 2) return "";
    if (!mfma_path_ok(d)) return d.dtype == DSPARK_BF16 ? "k_stream_generic<unsigned short>" : "k_stream_generic<float>";
    const int npl = d.head == DSPARK_HEAD_RNN ? 2 : 1;
    if (stream_pipe_ok(d, npl)) return stream_pipe_name(npl, (d.B + 15) / 16 * 16);
    static char buf[64];
    snprintf(buf, sizeof buf, "k_stream_mfma<%d, %d>", d.r / 32, d.head == DSPARK_HEAD_RNN ? 2 : 1);
    return buf;
}

hipError_t launch_draft(const DraftArgs& a) {
    const int opt = draft_path_option();  // 0 auto, 1 multi-kernel, 2 single launch
    if (opt != 1 && persist_path_ok(a.dims)) {
        const hipError_t e = launch_draft_persistent(a);
        if (e == hipSuccess || opt == 2) return e;
        (void)hipGetLastError();  // fall back to the multi-kernel path
    } else if (opt == 2) {
        return hipErrorNotSupported;
    }
    if (a.dims.dtype == DSPARK_BF16) return launch_draft_t<uint16_t>(a);
    return launch_draft_t<float>(a);
}

}  // namespace dspark
