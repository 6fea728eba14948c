// Backward of the teacher-forced DSpark objective past the logits: from
// dZ = dL/dz_d and dA = dL/d(confidence logit) to the gradients of the Markov
// table W1, the confidence weights w and the hidden states h.
//
// Row i = n gamma + k is fed prev_i (anchor at k = 0, the previous label
// after; the alignment the dormouse "DSpark - paper verification" page calls
// correct in its off-by-one discussion, section 2).  e_i = W1[prev_i] enters
// the bias z_d = U + e W2 (Eq 5) and the confidence logit a = w . [h; e]
// (Eq 7), and the same page's delta table (section 2, row D16) has training
// update the sequential block and the confidence head, so the chain rule
// gives
//   dE_i  = dZ_i W2^T + dA_i w[d : d + r]
//   dW1[x] = sum of dE_i over the rows fed x
//   dw    = sum_i dA_i [h_i; e_i],   dh_i = dA_i w[0 : d].
//
// Kernels, in stream order:
//   k_bwd_prev   prev_i, -1 where the token is out of range or dA_i is not
//                finite; per-block error flags
//   k_bwd_rank   stable counting sort of the rows by prev (O(R^2) compares,
//                rows in LDS tiles): sorted position, token and segment bounds
//   k_de_mfma    dE = dZ W2^T on the matrix cores, split over the vocabulary
//                into S slices of fp32 partial tiles (bf16 W2; bf16 dZ, or
//                fp32 dZ as an exact-product hi + lo bf16 pair)
//   k_de_reduce  sum of the S partials in slice order, plus dA_i w[d:]
//   k_de_vec     the same two steps on the vector units for other shapes
//   k_fill_zero, k_seg_chunk, k_seg_final
//                dW1: zero rows, then each token's rows summed in row order
//                (chunks of 64 sorted rows, then the chunks in order)
//   k_dw_part, k_dw_final, k_dh
// Every sum has a fixed order, so results are bitwise reproducible.
#include <algorithm>

#include "device_common.h"
#include "internal.h"

namespace dspark {

constexpr int kBwdTileRows = 256;   // rows of one dE tile (matrix-core path)
constexpr int kBwdChunk = 64;       // sorted rows per dW1 chunk sum
constexpr int kBwdCus = 256;        // workgroups the split-K grid aims at
constexpr int kBwdDwSplits = 64;    // row splits of the dw_conf sums
constexpr int kRankRows = 64;       // rows per k_bwd_rank workgroup
constexpr int kRankTile = 2048;     // prev entries per LDS tile

bool bwd_mfma_ok(const dspark_dims& d) { return loss_mfma_ok(d); }

BwdLayout bwd_layout(const dspark_dims& d) {
    BwdLayout L{};
    const int64_t R = static_cast<int64_t>(d.B) * d.gamma;
    L.R = static_cast<int>(R);
    L.mfma = bwd_mfma_ok(d);
    L.T = static_cast<int>((R + kBwdTileRows - 1) / kBwdTileRows);
    const int ks = 64;  // vocabulary entries per stage (bf16 dZ; fp32 dZ uses 32)
    const int stages = (d.V + ks - 1) / ks;
    L.S = L.mfma ? std::max(1, std::min(kBwdCus / L.T, stages)) : 0;
    L.RS = static_cast<int>(std::min<int64_t>(R, kBwdDwSplits));
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t rr = static_cast<size_t>(R);
    L.bad = take(sizeof(int32_t) * d.B);
    L.prev = take(sizeof(int32_t) * rr);
    L.srow = take(sizeof(int32_t) * rr);
    L.sprev = take(sizeof(int32_t) * rr);
    L.slo = take(sizeof(int32_t) * rr);
    L.shi = take(sizeof(int32_t) * rr);
    L.de = take(sizeof(float) * rr * d.r);
    L.seg = take(sizeof(float) * rr * d.r);
    // the fp32-dZ variant uses 32-entry stages and up to twice the slices,
    // so size the partials for the larger count
    const int s_max = L.mfma ? std::max(1, std::min(kBwdCus / L.T, 2 * stages)) : 0;
    L.part = take(sizeof(float) * static_cast<size_t>(L.T) * s_max * kBwdTileRows * d.r);
    L.dwp = take(sizeof(float) * static_cast<size_t>(L.RS) * (d.d + d.r));
    L.total = off;
    return L;
}

// ------------------------------------------------------------ prev tokens

// Thread per block n: prev of its gamma rows and its error flag (one writer
// per flag, so no clearing pass is needed).
__global__ __launch_bounds__(256) void k_bwd_prev(const int32_t* __restrict__ anchor,
                                                  const int32_t* __restrict__ labels,
                                                  const float* __restrict__ dA, int N, int gamma,
                                                  int V, int32_t* __restrict__ bad,
                                                  int32_t* __restrict__ prev) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= N) return;
    int flag = 0;
    for (int k = 0; k < gamma; ++k) {
        const int64_t i = static_cast<int64_t>(n) * gamma + k;
        const int x = k == 0 ? anchor[n] : labels[i - 1];
        const bool in_range = x >= 0 && x < V;
        flag |= !in_range;
        const bool finite = dA == nullptr || isfinite(dA[i]);
        prev[i] = (in_range && finite) ? x : -1;
    }
    bad[n] = flag;
}

// Stable counting sort by prev: position = #(prev_j < prev_i) + #(j < i,
// prev_j == prev_i).  Workgroup = 64 rows x 4 quarters of every LDS tile.
__global__ __launch_bounds__(256) void k_bwd_rank(const int32_t* __restrict__ prev, int R,
                                                  int32_t* __restrict__ srow,
                                                  int32_t* __restrict__ sprev,
                                                  int32_t* __restrict__ slo,
                                                  int32_t* __restrict__ shi) {
    __shared__ int32_t tile[kRankTile];
    __shared__ int32_t red[3][4][kRankRows];
    const int t = threadIdx.x;
    const int rl = t % kRankRows, qt = t / kRankRows;
    const int i = blockIdx.x * kRankRows + rl;
    const int p = i < R ? prev[i] : INT32_MAX;
    int lt = 0, eqb = 0, eq = 0;
    for (int j0 = 0; j0 < R; j0 += kRankTile) {
        const int m = min(kRankTile, R - j0);
        __syncthreads();
        for (int q = t; q < m; q += 256) tile[q] = prev[j0 + q];
        __syncthreads();
        const int per = (m + 3) / 4;
        const int qa = qt * per, qb = min(m, qa + per);
        for (int q = qa; q < qb; ++q) {
            const int x = tile[q];
            lt += x < p;
            const int e = x == p;
            eq += e;
            eqb += e & (j0 + q < i);
        }
    }
    red[0][qt][rl] = lt;
    red[1][qt][rl] = eqb;
    red[2][qt][rl] = eq;
    __syncthreads();
    if (qt == 0 && i < R) {
        lt = red[0][0][rl] + red[0][1][rl] + red[0][2][rl] + red[0][3][rl];
        eqb = red[1][0][rl] + red[1][1][rl] + red[1][2][rl] + red[1][3][rl];
        eq = red[2][0][rl] + red[2][1][rl] + red[2][2][rl] + red[2][3][rl];
        const int pos = lt + eqb;
        srow[pos] = i;
        sprev[pos] = p;
        slo[pos] = lt;
        shi[pos] = lt + eq;
    }
}

// ------------------------------------------------- dE on the matrix cores
//
// v_mfma_f32_16x16x32_bf16 with A = 16 dZ rows x 32 vocabulary entries and
// B = 32 entries x 16 columns j of W2^T: both operands are contiguous along
// the vocabulary in memory (dZ rows, W2 rows), so lane (g = lane / 16,
// n = lane % 16) reads 16 bytes of row n at entry 8 g for either operand and
// receives dE[4 g + q][n].
//
// Workgroup: 256 rows x all r columns, 4 WN waves, wave (wm, wn) owns rows
// 64 wm .. 64 wm + 63 and columns wn r / WN .. (JF = r / (16 WN) column
// fragments).  Stages of KS vocabulary entries go through two LDS buffers:
//   A tile [256][64] bf16, 128-byte rows.  bf16 dZ: entries 0..63 of the
//     stage.  fp32 dZ (KS = 32): hi(dZ) in 0..31, lo(dZ) = bf16(dZ - hi) in
//     32..63, so hi x W2 + lo x W2 carries dZ to 2^-16 of itself with exact
//     products.
//   B tile [r][KS] bf16 (W2 rows), 128-byte rows (KS = 64) or 64-byte rows.
// 16-byte segments are XOR-swizzled by row so that the 8 lanes of one LDS
// cycle hit 8 distinct bank groups.  Stage s + 2 is fetched into registers
// while stage s is multiplied; the vocabulary range of each slice is split
// in stages, entries at or past V load as zero.
struct DeArgs {
    const void* dz;
    const uint16_t* W2;
    float* part;
    int R, V, T, S, stages;
};

__device__ __forceinline__ int sw128(int row, int seg) { return (seg ^ (row & 7)) << 4; }
__device__ __forceinline__ int sw64(int row, int seg) { return (seg ^ ((row >> 1) & 3)) << 4; }

template <int JF, int WN, bool F32Z>
__global__ __launch_bounds__(256 * WN, 1) void k_de_mfma(DeArgs a) {
    constexpr int NT = 256 * WN;
    constexpr int RJ = JF * 16 * WN;           // r
    constexpr int KS = F32Z ? 32 : 64;          // vocabulary entries per stage
    constexpr int BRB = KS * 2;                 // B row bytes
    constexpr int BSEG = BRB / 16;              // 16-byte segments per B row
    constexpr int ABYTES = kBwdTileRows * 128;  // A tile bytes
    constexpr int BBYTES = RJ * BRB;
    constexpr int LA = kBwdTileRows * 8 / NT;           // A segments per thread
    constexpr int LB = (RJ * BSEG + NT - 1) / NT;      // B segments per thread
    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * (ABYTES + BBYTES)];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 3, wn = w >> 2;
    const int g = lane >> 4, n = lane & 15;
    const int tile = blockIdx.x % a.T, slice = blockIdx.x / a.T;
    const int s_begin = static_cast<int>(static_cast<int64_t>(slice) * a.stages / a.S);
    const int s_end = static_cast<int>(static_cast<int64_t>(slice + 1) * a.stages / a.S);
    const int ns = s_end - s_begin;
    const int64_t V = a.V;

    // per-thread global sources: A rows (clamped into [0, R)), B rows
    const int seg8 = tid & 7;
    int arow[LA];
#pragma unroll
    for (int q = 0; q < LA; ++q) arow[q] = q * (NT / 8) + (tid >> 3);
    const int bseg = tid % BSEG;
    int brow[LB];
#pragma unroll
    for (int q = 0; q < LB; ++q) brow[q] = q * (NT / BSEG) + tid / BSEG;

    u32x4 ra[LA];
    u32x4 rb[LB];

    auto gload = [&](int stage) {
        const int64_t v0 = static_cast<int64_t>(stage) * KS;
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int64_t gr = min(static_cast<int64_t>(tile) * kBwdTileRows + arow[q],
                                   static_cast<int64_t>(a.R - 1));
            const int64_t v = v0 + (F32Z ? 4 : 8) * seg8;
            const bool ok = v < V;
            const int64_t vc = ok ? v : V - 8;
            u32x4 x;
            if (F32Z)
                x = *reinterpret_cast<const u32x4*>(static_cast<const float*>(a.dz) + gr * V + vc);
            else
                x = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(a.dz) + gr * V + vc);
            const u32x4 zero = {0u, 0u, 0u, 0u};
            ra[q] = ok ? x : zero;
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int j = min(brow[q], RJ - 1);
            const int64_t v = v0 + 8 * bseg;
            const bool ok = v < V;
            const int64_t vc = ok ? v : V - 8;
            const u32x4 x = *reinterpret_cast<const u32x4*>(a.W2 + static_cast<int64_t>(j) * V + vc);
            const u32x4 zero = {0u, 0u, 0u, 0u};
            rb[q] = ok ? x : zero;
        }
    };

    auto lstore = [&](int buf) {
        unsigned char* As = smem + buf * (ABYTES + BBYTES);
        unsigned char* Bs = As + ABYTES;
#pragma unroll
        for (int q = 0; q < LA; ++q) {
            const int row = arow[q];
            if (F32Z) {
                // 4 fp32 entries 4 seg8 .. 4 seg8 + 3 -> hi at k, lo at 32 + k
                float f[4], hf[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(ra[q][e]);
                typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
                uint32_t hw[2], lw[2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const bf16x2 hb = {static_cast<__bf16>(f[2 * e]), static_cast<__bf16>(f[2 * e + 1])};
                    hw[e] = __builtin_bit_cast(uint32_t, hb);
                    hf[2 * e] = static_cast<float>(hb[0]);
                    hf[2 * e + 1] = static_cast<float>(hb[1]);
                    const bf16x2 lb = {static_cast<__bf16>(f[2 * e] - hf[2 * e]),
                                       static_cast<__bf16>(f[2 * e + 1] - hf[2 * e + 1])};
                    lw[e] = __builtin_bit_cast(uint32_t, lb);
                }
                const int half = (seg8 & 1) * 8;
                *reinterpret_cast<uint2*>(As + row * 128 + sw128(row, seg8 >> 1) + half) =
                    make_uint2(hw[0], hw[1]);
                *reinterpret_cast<uint2*>(As + row * 128 + sw128(row, 4 + (seg8 >> 1)) + half) =
                    make_uint2(lw[0], lw[1]);
            } else {
                *reinterpret_cast<u32x4*>(As + row * 128 + sw128(row, seg8)) = ra[q];
            }
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int j = brow[q];
            if (j < RJ) {
                const int off = BRB == 128 ? j * 128 + sw128(j, bseg) : j * 64 + sw64(j, bseg);
                *reinterpret_cast<u32x4*>(Bs + off) = rb[q];
            }
        }
    };

    f32x4 acc[4][JF];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int f = 0; f < JF; ++f) acc[m][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    if (ns > 0) {
        gload(s_begin);
        lstore(0);
        gload(s_begin + min(1, ns - 1));
        __syncthreads();
        for (int s = 0; s < ns; ++s) {
            const unsigned char* As = smem + (s & 1) * (ABYTES + BBYTES);
            const unsigned char* Bs = As + ABYTES;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                bf16x8 af[4];
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int row = wm * 64 + m * 16 + n;
                    af[m] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4*>(As + row * 128 + sw128(row, kk * 4 + g)));
                }
#pragma unroll
                for (int f = 0; f < JF; ++f) {
                    const int j = wn * (JF * 16) + f * 16 + n;
                    const int off = BRB == 128 ? j * 128 + sw128(j, kk * 4 + g) : j * 64 + sw64(j, g);
                    const bf16x8 bf = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs + off));
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[m], bf, acc[m][f], 0, 0, 0);
                }
            }
            // stage s + 1 (already in registers) to the other buffer, then
            // fetch stage s + 2; past the end both repeat the last stage
            lstore((s + 1) & 1);
            gload(s_begin + min(s + 2, ns - 1));
            __syncthreads();
        }
    }

    // raw accumulator dump: [slot][wave][m][f][lane] f32x4, coalesced
    float* out = a.part + static_cast<int64_t>(blockIdx.x) * (kBwdTileRows * RJ);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int f = 0; f < JF; ++f)
            *reinterpret_cast<f32x4*>(out + ((static_cast<int64_t>(w * 4 + m) * JF + f) * 64 + lane) * 4) =
                acc[m][f];
}

// Thread per f32x4 of a tile: the S slice partials in slice order, plus
// dA_i w[d + j] (rows with prev_i < 0 get 0 there; the dW1 sums skip them).
template <typename T>
__global__ __launch_bounds__(256) void k_de_reduce(const float* __restrict__ part,
                                                   const int32_t* __restrict__ prev,
                                                   const float* __restrict__ dA,
                                                   const T* __restrict__ w_conf, int R, int r,
                                                   int d, int T_, int S, int JF,
                                                   float* __restrict__ dE) {
    const int per_tile = kBwdTileRows * r / 4;
    const int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (e >= static_cast<int64_t>(T_) * per_tile) return;
    const int tile = static_cast<int>(e / per_tile), u = static_cast<int>(e % per_tile);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s = 0; s < S; ++s)
        acc += *reinterpret_cast<const f32x4*>(part + (static_cast<int64_t>(s) * T_ + tile) *
                                                          (kBwdTileRows * r) + 4 * static_cast<int64_t>(u));
    const int lane = u & 63, f = (u >> 6) % JF, wm_m = (u >> 6) / JF;  // wave * 4 + m
    const int wv = wm_m >> 2, m = wm_m & 3;
    const int WN = r / (16 * JF);
    const int wm = wv % 4, wn = wv / 4;
    (void)WN;
    const int j = wn * (JF * 16) + f * 16 + (lane & 15);
    const float wj = load_f(w_conf, d + j);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = tile * kBwdTileRows + wm * 64 + m * 16 + 4 * (lane >> 4) + q;
        if (row < R) {
            const float c = (dA != nullptr && prev[row] >= 0) ? dA[row] * wj : 0.0f;
            dE[static_cast<int64_t>(row) * r + j] = acc[q] + c;
        }
    }
}

// Vector path: workgroup per (row, 8 columns); fixed-order tree reduction.
template <typename T, typename DZ>
__global__ __launch_bounds__(256) void k_de_vec(const DZ* __restrict__ dz, const T* __restrict__ W2,
                                                const int32_t* __restrict__ prev,
                                                const float* __restrict__ dA,
                                                const T* __restrict__ w_conf, int V, int r, int d,
                                                float* __restrict__ dE) {
    __shared__ float red[8][256];
    const int64_t i = blockIdx.x;
    const int j0 = blockIdx.y * 8, t = threadIdx.x;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    for (int v = t; v < V; v += 256) {
        const float z = load_f(dz, i * V + v);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            if (j0 + jj < r) acc[jj] = fmaf(z, load_f(W2, static_cast<int64_t>(j0 + jj) * V + v), acc[jj]);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) red[jj][t] = acc[jj];
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (t < h)
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) red[jj][t] += red[jj][t + h];
        __syncthreads();
    }
    if (t < 8 && j0 + t < r) {
        const int j = j0 + t;
        const float c = (dA != nullptr && prev[i] >= 0) ? dA[i] * load_f(w_conf, d + j) : 0.0f;
        dE[i * r + j] = red[t][0] + c;
    }
}

// ------------------------------------------------------------------- dW1

__global__ __launch_bounds__(256) void k_fill_zero(float* __restrict__ p, int64_t n) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * 4;
    for (int64_t e = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4; e < n; e += stride) {
        if (e + 4 <= n && (reinterpret_cast<uintptr_t>(p + e) & 15) == 0) {
            *reinterpret_cast<f32x4*>(p + e) = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        } else {
            for (int64_t q = e; q < min(e + 4, n); ++q) p[q] = 0.0f;
        }
    }
}

// Wave per sorted position p that starts a chunk (its segment's first
// position, or 64, 128, ... after it): the dE rows at positions p .. up to
// 63 after it, summed in position (= row) order.
__global__ __launch_bounds__(256) void k_seg_chunk(const float* __restrict__ dE,
                                                   const int32_t* __restrict__ srow,
                                                   const int32_t* __restrict__ sprev,
                                                   const int32_t* __restrict__ slo,
                                                   const int32_t* __restrict__ shi, int R, int r,
                                                   float* __restrict__ seg) {
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= R) return;
    const int lo = slo[p];
    if (sprev[p] < 0 || (p - lo) % kBwdChunk != 0) return;
    const int cnt = min(kBwdChunk, shi[p] - p);
    const int myrow = lane < cnt ? srow[p + lane] : 0;
    for (int j = lane; j < r; j += 64) {
        float acc = 0.0f;
        for (int q = 0; q < cnt; ++q) {
            const int row = __builtin_amdgcn_readlane(myrow, q);
            acc += dE[static_cast<int64_t>(row) * r + j];
        }
        seg[static_cast<int64_t>(p) * r + j] = acc;
    }
}

// Wave per segment start p: dW1[token] = its chunk sums in order.
__global__ __launch_bounds__(256) void k_seg_final(const float* __restrict__ seg,
                                                   const int32_t* __restrict__ sprev,
                                                   const int32_t* __restrict__ slo,
                                                   const int32_t* __restrict__ shi, int R, int r,
                                                   float* __restrict__ dW1) {
    const int lane = threadIdx.x & 63;
    const int p = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= R) return;
    const int x = sprev[p];
    if (x < 0 || slo[p] != p) return;
    const int end = shi[p];
    for (int j = lane; j < r; j += 64) {
        float acc = 0.0f;
        for (int c = p; c < end; c += kBwdChunk) acc += seg[static_cast<int64_t>(c) * r + j];
        dW1[static_cast<int64_t>(x) * r + j] = acc;
    }
}

// ------------------------------------------------------------ dw_conf, dh

// Thread per column q of [h; e], rows of split blockIdx.y in row order.
template <typename T>
__global__ __launch_bounds__(256) void k_dw_part(const T* __restrict__ h, const T* __restrict__ W1,
                                                 const int32_t* __restrict__ prev,
                                                 const float* __restrict__ dA, int R, int r, int d,
                                                 int RS, float* __restrict__ dwp) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    const int cols = d + r;
    if (q >= cols) return;
    const int rs = blockIdx.y;
    const int i0 = static_cast<int>(static_cast<int64_t>(rs) * R / RS);
    const int i1 = static_cast<int>(static_cast<int64_t>(rs + 1) * R / RS);
    float acc = 0.0f;
    for (int i = i0; i < i1; ++i) {
        const int p = prev[i];
        if (p < 0) continue;
        const float x = q < d ? load_f(h, static_cast<int64_t>(i) * d + q)
                              : load_f(W1, static_cast<int64_t>(p) * r + (q - d));
        acc = fmaf(dA[i], x, acc);
    }
    dwp[static_cast<int64_t>(rs) * cols + q] = acc;
}

__global__ __launch_bounds__(256) void k_dw_final(const float* __restrict__ dwp, int cols, int RS,
                                                  float* __restrict__ dw) {
    const int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q >= cols) return;
    float acc = 0.0f;
    for (int rs = 0; rs < RS; ++rs) acc += dwp[static_cast<int64_t>(rs) * cols + q];
    dw[q] = acc;
}

// dh[i, q] = dA_i w[q] for every row (a row with a non-finite dA gets it).
template <typename T>
__global__ __launch_bounds__(256) void k_dh(const float* __restrict__ dA, const T* __restrict__ w_conf,
                                            int64_t R, int d, float* __restrict__ dh) {
    const int64_t n = R * d;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n; e += stride) {
        const int64_t i = e / d;
        const int q = static_cast<int>(e - i * d);
        dh[e] = dA[i] * load_f(w_conf, q);
    }
}

// ------------------------------------------------------------------ launch

template <int JF, int WN, bool F32Z>
static void launch_de_t(const DeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_de_mfma<JF, WN, F32Z>), dim3(a.T * a.S), dim3(256 * WN), 0, st, a);
}

template <bool F32Z>
static bool launch_de(int r, const DeArgs& a, hipStream_t st) {
    switch (r) {
        case 32: launch_de_t<2, 1, F32Z>(a, st); return true;
        case 64: launch_de_t<4, 1, F32Z>(a, st); return true;
        case 96: launch_de_t<6, 1, F32Z>(a, st); return true;
        case 128: launch_de_t<8, 1, F32Z>(a, st); return true;
        case 160: launch_de_t<5, 2, F32Z>(a, st); return true;
        case 192: launch_de_t<6, 2, F32Z>(a, st); return true;
        case 224: launch_de_t<7, 2, F32Z>(a, st); return true;
        case 256: launch_de_t<8, 2, F32Z>(a, st); return true;
        default: return false;
    }
}

static int grid_for(int64_t n, int per_block) {
    return static_cast<int>(std::max<int64_t>(1, std::min<int64_t>((n + per_block - 1) / per_block, 1 << 20)));
}

template <typename T>
static hipError_t launch_bwd_t(const BwdArgs& ba) {
    const dspark_dims& D = ba.dims;
    const BwdLayout L = bwd_layout(D);
    hipStream_t st = ba.stream;
    char* ws = ba.ws;
    int32_t* bad = reinterpret_cast<int32_t*>(ws + L.bad);
    int32_t* prev = reinterpret_cast<int32_t*>(ws + L.prev);
    int32_t* srow = reinterpret_cast<int32_t*>(ws + L.srow);
    int32_t* sprev = reinterpret_cast<int32_t*>(ws + L.sprev);
    int32_t* slo = reinterpret_cast<int32_t*>(ws + L.slo);
    int32_t* shi = reinterpret_cast<int32_t*>(ws + L.shi);
    float* dE = reinterpret_cast<float*>(ws + L.de);
    float* seg = reinterpret_cast<float*>(ws + L.seg);
    float* part = reinterpret_cast<float*>(ws + L.part);
    float* dwp = reinterpret_cast<float*>(ws + L.dwp);
    const T* h = static_cast<const T*>(ba.h);
    const T* W1 = static_cast<const T*>(ba.W1);
    const T* W2 = static_cast<const T*>(ba.W2);
    const T* w = static_cast<const T*>(ba.w_conf);
    const int R = L.R, r = D.r, d = D.d, V = D.V;

    hipLaunchKernelGGL(k_bwd_prev, dim3(grid_for(D.B, 256)), dim3(256), 0, st, ba.anchor, ba.labels,
                       ba.dA, D.B, D.gamma, V, bad, prev);
    if (ba.dW1) {
        hipLaunchKernelGGL(k_bwd_rank, dim3((R + kRankRows - 1) / kRankRows), dim3(256), 0, st, prev, R,
                           srow, sprev, slo, shi);
        if (L.mfma) {
            const bool f32z = ba.dz_dtype == DSPARK_F32;
            DeArgs a{};
            a.dz = ba.dz;
            a.W2 = static_cast<const uint16_t*>(ba.W2);
            a.part = part;
            a.R = R;
            a.V = V;
            a.T = L.T;
            const int ks = f32z ? 32 : 64;
            a.stages = (V + ks - 1) / ks;
            a.S = std::max(1, std::min(kBwdCus / L.T, a.stages));
            hipError_t pe = profile_begin(st);
            if (pe != hipSuccess) return pe;
            const bool ok = f32z ? launch_de<true>(r, a, st) : launch_de<false>(r, a, st);
            if (!ok) return hipErrorInvalidValue;
            if ((pe = profile_end(st)) != hipSuccess) return pe;
            const int JF = r > 128 ? r / 32 : r / 16;
            const int64_t n4 = static_cast<int64_t>(L.T) * kBwdTileRows * r / 4;
            hipLaunchKernelGGL((k_de_reduce<T>), dim3(grid_for(n4, 256)), dim3(256), 0, st, part, prev, ba.dA,
                               w, R, r, d, L.T, a.S, JF, dE);
        } else {
            if (ba.dz_dtype == DSPARK_F32)
                hipLaunchKernelGGL((k_de_vec<T, float>), dim3(R, (r + 7) / 8), dim3(256), 0, st,
                                   static_cast<const float*>(ba.dz), W2, prev, ba.dA, w, V, r, d, dE);
            else
                hipLaunchKernelGGL((k_de_vec<T, uint16_t>), dim3(R, (r + 7) / 8), dim3(256), 0, st,
                                   static_cast<const uint16_t*>(ba.dz), W2, prev, ba.dA, w, V, r, d, dE);
        }
        const int64_t nW1 = static_cast<int64_t>(V) * r;
        hipLaunchKernelGGL(k_fill_zero, dim3(grid_for(nW1 / 4 + 1, 256 * 8)), dim3(256), 0, st, ba.dW1, nW1);
        hipLaunchKernelGGL(k_seg_chunk, dim3((R + 3) / 4), dim3(256), 0, st, dE, srow, sprev, slo, shi, R, r,
                           seg);
        hipLaunchKernelGGL(k_seg_final, dim3((R + 3) / 4), dim3(256), 0, st, seg, sprev, slo, shi, R, r,
                           ba.dW1);
    }
    if (ba.dw_conf) {
        const int cols = d + r;
        hipLaunchKernelGGL((k_dw_part<T>), dim3((cols + 255) / 256, L.RS), dim3(256), 0, st, h, W1, prev,
                           ba.dA, R, r, d, L.RS, dwp);
        hipLaunchKernelGGL(k_dw_final, dim3((cols + 255) / 256), dim3(256), 0, st, dwp, cols, L.RS,
                           ba.dw_conf);
    }
    if (ba.dh) {
        const int64_t n = static_cast<int64_t>(R) * d;
        hipLaunchKernelGGL((k_dh<T>), dim3(grid_for(n, 256 * 8)), dim3(256), 0, st, ba.dA, w,
                           static_cast<int64_t>(R), d, ba.dh);
    }
    return hipGetLastError();
}

hipError_t launch_loss_backward(const BwdArgs& a) {
    return a.dims.dtype == DSPARK_BF16 ? launch_bwd_t<uint16_t>(a) : launch_bwd_t<float>(a);
}

}  // namespace dspark
