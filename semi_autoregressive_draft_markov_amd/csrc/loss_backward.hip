// Backward of the teacher-forced DSpark objective past the logits: from
// dZ = dL/dz_d and dA = dL/d(confidence logit) to the gradients of the Markov
// table W1, the confidence weights w and the hidden states h.
//
// Row i = n gamma + k is fed prev_i (anchor at k = 0, the previous label
// after; the alignment the dormouse "DSpark - paper verification" page calls
// correct in its off-by-one discussion, section 2).  e_i = W1[prev_i] enters
// the bias z_d = U + e W2 (Eq 5) and the confidence logit a = w . [h; e]
// (Eq 7), and the same page's delta table (section 4, row D16) has training
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
constexpr int kBwdDwSplits = 128;   // row splits of the dw_conf sums
constexpr int kRankRows = 16;       // rows per k_bwd_rank workgroup
constexpr int kRankSplits = 16;     // splits of each prev tile per row
constexpr int kRankTile = 4096;     // prev entries per LDS tile

bool bwd_mfma_ok(const dspark_dims& d) { return loss_mfma_ok(d); }

BwdLayout bwd_layout(const dspark_dims& d) {
    BwdLayout L{};
    const int64_t R = static_cast<int64_t>(d.B) * d.gamma;
    L.R = static_cast<int>(R);
    L.mfma = bwd_mfma_ok(d);
    L.T = static_cast<int>((R + kBwdTileRows - 1) / kBwdTileRows);
    const int stages = (d.V + 31) / 32;  // fp32 dZ: 32 entries per stage (bf16: 64)
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
    L.zpage = take(16);
    L.prev = take(sizeof(int32_t) * rr);
    L.srow = take(sizeof(int32_t) * rr);
    L.sprev = take(sizeof(int32_t) * rr);
    L.slo = take(sizeof(int32_t) * rr);
    L.shi = take(sizeof(int32_t) * rr);
    L.de = take(sizeof(float) * rr * d.r);
    L.seg = take(sizeof(float) * rr * d.r);
    L.part = take(sizeof(float) * static_cast<size_t>(L.T) * L.S * kBwdTileRows * d.r);
    L.dwp = take(sizeof(float) * static_cast<size_t>(L.RS) * (d.d + d.r));
    L.total = off;
    return L;
}

// ------------------------------------------------------------ prev tokens

// Thread per block n: prev of its gamma rows and its error flag (one writer
// per flag, so no clearing pass is needed).  Also zeroes the 16-byte page
// that the dE kernel loads for vocabulary entries past V.
__global__ __launch_bounds__(256) void k_bwd_prev(const int32_t* __restrict__ anchor,
                                                  const int32_t* __restrict__ labels,
                                                  const float* __restrict__ dA, int N, int gamma,
                                                  int V, int32_t* __restrict__ bad,
                                                  int32_t* __restrict__ prev,
                                                  uint32_t* __restrict__ zpage) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n < 4) zpage[n] = 0u;
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
// prev_j == prev_i).  Workgroup = 16 rows x 16 splits of each LDS tile of
// prev (read 4 entries at a time); the 16 partial counts of a row are added
// through LDS.
__global__ __launch_bounds__(256) void k_bwd_rank(const int32_t* __restrict__ prev, int R,
                                                  int32_t* __restrict__ srow,
                                                  int32_t* __restrict__ sprev,
                                                  int32_t* __restrict__ slo,
                                                  int32_t* __restrict__ shi) {
    __shared__ __attribute__((aligned(16))) int32_t tile[kRankTile];
    __shared__ int32_t red[3][kRankSplits][kRankRows];
    const int t = threadIdx.x;
    const int rl = t % kRankRows, qt = t / kRankRows;
    const int i = blockIdx.x * kRankRows + rl;
    const int p = i < R ? prev[i] : INT32_MAX;
    int lt = 0, eqb = 0, eq = 0;
    for (int j0 = 0; j0 < R; j0 += kRankTile) {
        const int m = min(kRankTile, R - j0);
        __syncthreads();
        // entries past R hold INT32_MAX: never below or equal to a real prev
        for (int q = t; q < kRankTile; q += 256) tile[q] = q < m ? prev[j0 + q] : INT32_MAX;
        __syncthreads();
        constexpr int per = kRankTile / kRankSplits;  // multiple of 4
        const int qa = qt * per;
#pragma unroll 4
        for (int q = qa; q < qa + per; q += 4) {
            const int4 x = *reinterpret_cast<const int4*>(tile + q);
            const int jj = j0 + q;
            lt += (x.x < p) + (x.y < p) + (x.z < p) + (x.w < p);
            const int e0 = x.x == p, e1 = x.y == p, e2 = x.z == p, e3 = x.w == p;
            eq += e0 + e1 + e2 + e3;
            eqb += (e0 & (jj < i)) + (e1 & (jj + 1 < i)) + (e2 & (jj + 2 < i)) + (e3 & (jj + 3 < i));
        }
    }
    red[0][qt][rl] = lt;
    red[1][qt][rl] = eqb;
    red[2][qt][rl] = eq;
    __syncthreads();
    if (qt == 0 && i < R) {
        lt = eqb = eq = 0;
        for (int u = 0; u < kRankSplits; ++u) {
            lt += red[0][u][rl];
            eqb += red[1][u][rl];
            eq += red[2][u][rl];
        }
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
// fragments).  The vocabulary range of a slice goes through LDS in stages of
// KS entries: A tile [256][KS] of dZ as stored (bf16, KS = 64; fp32,
// KS = 32: 128-byte rows either way) and B tile [r][KS] of bf16 W2 rows.
// Both stream straight from memory into LDS with global_load_lds_dwordx4
// (each wave instruction fills 1 KB, lane l the 16 bytes at 16 l), without
// staging registers: A through a ring of NA buffers (3 for bf16, 4 for
// fp32), B through 2, which fills the 160 KB of LDS at r = 256.  16-byte
// segments are XOR-swizzled by row (the lane that fills physical segment p
// of a row loads logical segment p ^ swizzle(row)), so the 8 lanes of one
// LDS read cycle hit 8 distinct bank groups.  Entries at or past V load from
// a zeroed 16-byte page.  fp32 dZ is split on the LDS read into
// hi = bf16(dZ) and lo = bf16(dZ - hi), both multiplied by the exact bf16
// W2: dZ is carried to 2^-18 of itself with exact products.
//
// The compiler does not order LDS reads after these loads, so the rings are
// synchronised by hand: every wave issues the same numbers DA and DB of
// loads per stage (chunk indices past the last are clamped, which rewrites
// the same bytes with the same data), loads complete in issue order, stage s
// issues B(s + 1) then A(s + NA - 1), and before stage s is read each wave
// waits until at most DA of its loads are outstanding (then A(s) and B(s)
// are in), then the workgroup meets at a barrier.
struct DeArgs {
    const void* dz;
    const uint16_t* W2;
    const uint32_t* zpage;  // 16 zero bytes (device)
    float* part;
    int R, V, T, S, stages;
    int per_xcd;  // work items (tile, slice) per XCD, ceil(T S / 8)
};

// 16 bytes per lane from global memory into LDS at lds + 16 lane (lds is
// wave-uniform).  The builtin exists for the device pass only; the host pass
// just needs the kernel's launch stub.
__device__ __forceinline__ void dma16(const void* src, void* lds) {
#if __HIP_DEVICE_COMPILE__
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#endif
}

__device__ __forceinline__ int sw128(int row, int seg) { return (seg ^ (row & 7)) << 4; }
__device__ __forceinline__ int sw64(int row, int seg) { return (seg ^ ((row >> 1) & 3)) << 4; }

template <int JF, int WN, bool F32Z>
__global__ __launch_bounds__(256 * WN, 1) void k_de_mfma(DeArgs a) {
    constexpr int NW = 4 * WN;
    constexpr int RJ = JF * 16 * WN;           // r
    constexpr int KS = F32Z ? 32 : 64;         // vocabulary entries per stage
    constexpr int BRB = KS * 2;                // B row bytes (A rows are 128 bytes)
    constexpr int ABYTES = kBwdTileRows * 128;
    constexpr int BBYTES = RJ * BRB;
    constexpr int NA = F32Z ? 4 : 3, NB = 2;   // ring depths of the A and B tiles
    constexpr int ACH = ABYTES / 1024, BCH = BBYTES / 1024;
    constexpr int DA = (ACH + NW - 1) / NW;   // A loads per wave per stage
    constexpr int DB = (BCH + NW - 1) / NW;   // B loads per wave per stage
    static_assert(BBYTES % 1024 == 0 && DA < 64, "ring accounting");
    static_assert(NA * ABYTES + NB * BBYTES <= 160 * 1024, "LDS");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NA * ABYTES + NB * BBYTES];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wm = w & 3, wn = w >> 2;
    const int g = lane >> 4, n = lane & 15;
    // Workgroups go round-robin to the 8 XCDs (blockIdx % 8); XCD x takes
    // work items [x per_xcd, (x + 1) per_xcd) in slice-major order, so that
    // the tiles sharing a W2 slice share an L2 (a slice spans at most two
    // XCDs when per_xcd >= T).
    const int item = (blockIdx.x & 7) * a.per_xcd + (blockIdx.x >> 3);
    if (item >= a.T * a.S) return;
    const int tile = item % a.T, slice = item / a.T;
    const int s_begin = static_cast<int>(static_cast<int64_t>(slice) * a.stages / a.S);
    const int s_end = static_cast<int>(static_cast<int64_t>(slice + 1) * a.stages / a.S);
    const int ns = s_end - s_begin;
    const int64_t V = a.V;

    // per load q: this lane's source row start and vocabulary offset in the stage
    const unsigned char* srcA[DA];
    int voffA[DA];
#pragma unroll
    for (int q = 0; q < DA; ++q) {
        const int byte = min(w + q * NW, ACH - 1) * 1024 + lane * 16;
        const int row = byte >> 7, lseg = ((byte & 127) >> 4) ^ (row & 7);
        const int64_t gr = min(static_cast<int64_t>(tile) * kBwdTileRows + row,
                               static_cast<int64_t>(a.R - 1));
        srcA[q] = static_cast<const unsigned char*>(a.dz) + gr * V * (F32Z ? 4 : 2);
        voffA[q] = lseg * (F32Z ? 4 : 8);
    }
    const unsigned char* srcB[DB];
    int voffB[DB];
#pragma unroll
    for (int q = 0; q < DB; ++q) {
        const int byte = min(w + q * NW, BCH - 1) * 1024 + lane * 16;
        const int j = byte / BRB, pseg = (byte % BRB) >> 4;
        srcB[q] = reinterpret_cast<const unsigned char*>(a.W2 + static_cast<int64_t>(j) * V);
        voffB[q] = (BRB == 128 ? (pseg ^ (j & 7)) : (pseg ^ ((j >> 1) & 3))) * 8;
    }
    unsigned char* const Aring = smem;
    unsigned char* const Bring = smem + NA * ABYTES;

    auto issueA = [&](int stage, int buf) {
        const int64_t v0 = static_cast<int64_t>(stage) * KS;
#pragma unroll
        for (int q = 0; q < DA; ++q) {
            const int64_t v = v0 + voffA[q];
            const void* p = v < V ? static_cast<const void*>(srcA[q] + v * (F32Z ? 4 : 2))
                                  : static_cast<const void*>(a.zpage);
            dma16(p, Aring + buf * ABYTES + min(w + q * NW, ACH - 1) * 1024);
        }
    };
    auto issueB = [&](int stage, int buf) {
        const int64_t v0 = static_cast<int64_t>(stage) * KS;
#pragma unroll
        for (int q = 0; q < DB; ++q) {
            const int64_t v = v0 + voffB[q];
            const void* p = v < V ? static_cast<const void*>(srcB[q] + v * 2)
                                  : static_cast<const void*>(a.zpage);
            dma16(p, Bring + buf * BBYTES + min(w + q * NW, BCH - 1) * 1024);
        }
    };

    f32x4 acc[4][JF];
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int f = 0; f < JF; ++f) acc[m][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // Issue order B(s + 1), A(s + NA - 1) per stage: loads complete in
    // order, so once at most DA loads are outstanding, A(s) and B(s) are in.
    issueB(s_begin, 0);
#pragma unroll
    for (int q = 0; q < NA - 1; ++q) issueA(s_begin + min(q, ns - 1), q);
    for (int s = 0; s < ns; ++s) {
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(DA) : "memory");
        issueB(s_begin + min(s + 1, ns - 1), (s + 1) & 1);
        issueA(s_begin + min(s + NA - 1, ns - 1), (s + NA - 1) % NA);
        const unsigned char* As = Aring + (s % NA) * ABYTES;
        const unsigned char* Bs = Bring + (s & 1) * BBYTES;
        // operand fragments: A for sub-step kk (32 entries), B for (kk, f);
        // B is fetched one step ahead and A of kk = 1 early, so that LDS
        // latency hides behind the matrix-core work of the step before
        auto ldA = [&](int kk, bf16x8 (&ah)[4], bf16x8 (&al)[4]) {
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int row = wm * 64 + m * 16 + n;
                if (F32Z) {
                    const f32x4 x0 = *reinterpret_cast<const f32x4*>(As + row * 128 + sw128(row, 2 * g));
                    const f32x4 x1 = *reinterpret_cast<const f32x4*>(As + row * 128 + sw128(row, 2 * g + 1));
                    const float x[8] = {x0[0], x0[1], x0[2], x0[3], x1[0], x1[1], x1[2], x1[3]};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        ah[m][e] = static_cast<__bf16>(x[e]);
                        al[m][e] = static_cast<__bf16>(x[e] - static_cast<float>(ah[m][e]));
                    }
                } else {
                    ah[m] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4*>(As + row * 128 + sw128(row, kk * 4 + g)));
                }
            }
        };
        auto ldB = [&](int kk, int f) {
            const int j = wn * (JF * 16) + f * 16 + n;
            const int boff = BRB == 128 ? j * 128 + sw128(j, kk * 4 + g) : j * 64 + sw64(j, g);
            return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(Bs + boff));
        };
        constexpr int KK = F32Z ? 1 : 2;
        bf16x8 ah0[4], al0[4], ah1[4], al1[4];
        ldA(0, ah0, al0);
        bf16x8 bcur = ldB(0, 0);
#pragma unroll
        for (int step = 0; step < KK * JF; ++step) {
            const int kk = step / JF, f = step % JF;
            bf16x8 bnext = bcur;
            if (step + 1 < KK * JF) bnext = ldB((step + 1) / JF, (step + 1) % JF);
            if (KK == 2 && step == 1) ldA(1, ah1, al1);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const bf16x8 ah = kk == 0 ? ah0[m] : ah1[m];
                acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bcur, acc[m][f], 0, 0, 0);
                if (F32Z) acc[m][f] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al0[m], bcur, acc[m][f], 0, 0, 0);
            }
            bcur = bnext;
            // keep the fetch-ahead order: the scheduler would otherwise sink
            // each LDS read next to its first use
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // raw accumulator dump: [item][wave][m][f][lane] f32x4, coalesced
    float* out = a.part + static_cast<int64_t>(item) * (kBwdTileRows * RJ);
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
// 63 after it, summed in position (= row) order.  Lane l holds columns
// 4 l + 256 t (r % 4 == 0) or l + 64 t; rows are fetched 8 at a time.
template <bool VEC4>
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
    constexpr int W = VEC4 ? 4 : 1;
    for (int j = lane * W; j < r; j += 64 * W) {
        float acc[W];
#pragma unroll
        for (int e = 0; e < W; ++e) acc[e] = 0.0f;
        for (int q0 = 0; q0 < cnt; q0 += 8) {
            float x[8][W];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int row = __builtin_amdgcn_readlane(myrow, min(q0 + u, cnt - 1));
                const float* src = dE + static_cast<int64_t>(row) * r + j;
                if (VEC4) {
                    const f32x4 v = *reinterpret_cast<const f32x4*>(src);
#pragma unroll
                    for (int e = 0; e < W; ++e) x[u][e] = v[e];
                } else {
                    x[u][0] = *src;
                }
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
                if (q0 + u < cnt)
#pragma unroll
                    for (int e = 0; e < W; ++e) acc[e] += x[u][e];
        }
        float* dst = seg + static_cast<int64_t>(p) * r + j;
        if (VEC4) {
            *reinterpret_cast<f32x4*>(dst) = f32x4{acc[0], acc[W > 1 ? 1 : 0], acc[W > 2 ? 2 : 0], acc[W > 3 ? 3 : 0]};
        } else {
            dst[0] = acc[0];
        }
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

// Thread per column q of [h; e] (h part first), rows of split blockIdx.y in
// row order.  Rows are fetched 8 at a time; a row left out contributes
// fma(0, 0, acc) = acc exactly.
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
    for (int b = i0; b < i1; b += 8) {
        float x[8], c[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = min(b + u, i1 - 1);
            const int p = prev[i];
            const bool use = p >= 0 && b + u < i1;
            const float v = q < d ? load_f(h, static_cast<int64_t>(i) * d + q)
                                  : load_f(W1, static_cast<int64_t>(max(p, 0)) * r + (q - d));
            x[u] = use ? v : 0.0f;
            c[u] = use ? dA[i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) acc = fmaf(c[u], x[u], acc);
    }
    dwp[static_cast<int64_t>(rs) * cols + q] = acc;
}

// Workgroup per 64 columns: 4 threads per column add every 4th split, then
// the 4 sums are added in order.
__global__ __launch_bounds__(256) void k_dw_final(const float* __restrict__ dwp, int cols, int RS,
                                                  float* __restrict__ dw) {
    __shared__ float red[4][64];
    const int c = threadIdx.x & 63, u = threadIdx.x >> 6;
    const int q = blockIdx.x * 64 + c;
    float acc = 0.0f;
    if (q < cols)
        for (int rs = u; rs < RS; rs += 4) acc += dwp[static_cast<int64_t>(rs) * cols + q];
    red[u][c] = acc;
    __syncthreads();
    if (u == 0 && q < cols) dw[q] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
}

// dh[i, q] = dA_i w[q] for every row (a row with a non-finite dA gets it).
// Workgroup per row; 4 columns per thread when the rows are 16-byte aligned.
template <typename T, bool VEC4>
__global__ __launch_bounds__(256) void k_dh(const float* __restrict__ dA, const T* __restrict__ w_conf,
                                            int R, int d, float* __restrict__ dh) {
    const int i = blockIdx.x;
    const float c = dA[i];
    float* out = dh + static_cast<int64_t>(i) * d;
    if (VEC4) {
        for (int q = threadIdx.x * 4; q < d; q += 1024)
            *reinterpret_cast<f32x4*>(out + q) = f32x4{c * load_f(w_conf, q), c * load_f(w_conf, q + 1),
                                                       c * load_f(w_conf, q + 2), c * load_f(w_conf, q + 3)};
    } else {
        for (int q = threadIdx.x; q < d; q += 256) out[q] = c * load_f(w_conf, q);
    }
}

// ------------------------------------------------------------------ launch

template <int JF, int WN, bool F32Z>
static void launch_de_t(const DeArgs& a, hipStream_t st) {
    hipLaunchKernelGGL((k_de_mfma<JF, WN, F32Z>), dim3(8 * a.per_xcd), dim3(256 * WN), 0, st, a);
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

    hipLaunchKernelGGL(k_bwd_prev, dim3(grid_for(std::max(D.B, 4), 256)), dim3(256), 0, st, ba.anchor, ba.labels,
                       ba.dA, D.B, D.gamma, V, bad, prev, reinterpret_cast<uint32_t*>(ws + L.zpage));
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
            a.zpage = reinterpret_cast<const uint32_t*>(ws + L.zpage);
            a.stages = f32z ? (V + 31) / 32 : (V + 63) / 64;
            a.S = std::min(L.S, a.stages);
            a.per_xcd = (L.T * a.S + 7) / 8;
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
        if (r % 4 == 0)
            hipLaunchKernelGGL(k_seg_chunk<true>, dim3((R + 3) / 4), dim3(256), 0, st, dE, srow, sprev, slo, shi,
                               R, r, seg);
        else
            hipLaunchKernelGGL(k_seg_chunk<false>, dim3((R + 3) / 4), dim3(256), 0, st, dE, srow, sprev, slo, shi,
                               R, r, seg);
        hipLaunchKernelGGL(k_seg_final, dim3((R + 3) / 4), dim3(256), 0, st, seg, sprev, slo, shi, R, r,
                           ba.dW1);
    }
    if (ba.dw_conf) {
        const int cols = d + r;
        hipLaunchKernelGGL((k_dw_part<T>), dim3((cols + 255) / 256, L.RS), dim3(256), 0, st, h, W1, prev,
                           ba.dA, R, r, d, L.RS, dwp);
        hipLaunchKernelGGL(k_dw_final, dim3((cols + 63) / 64), dim3(256), 0, st, dwp, cols, L.RS, ba.dw_conf);
    }
    if (ba.dh) {
        if (d % 4 == 0 && (reinterpret_cast<uintptr_t>(ba.dh) & 15) == 0)
            hipLaunchKernelGGL((k_dh<T, true>), dim3(R), dim3(256), 0, st, ba.dA, w, R, d, ba.dh);
        else
            hipLaunchKernelGGL((k_dh<T, false>), dim3(R), dim3(256), 0, st, ba.dA, w, R, d, ba.dh);
    }
    return hipGetLastError();
}

hipError_t launch_loss_backward(const BwdArgs& a) {
    return a.dims.dtype == DSPARK_BF16 ? launch_bwd_t<uint16_t>(a) : launch_bwd_t<float>(a);
}

}  // namespace dspark
