// Verification of drafted blocks against the target, Markov head: prefix
// trimming by confidence, the standard speculative accept/reject rule and
// the final draw.
//
// The target checks the drafted block and keeps the leading tokens up to the
// first rejection, leaving the output distribution the target's (bowenzhou
// "DSpark：既要猜得连贯，也要把验证算力花在刀刃上", "Why DSpark?");
// c* = 1 - TV(p_d, p_t) is that rule's single-step acceptance probability
// (Meridian "Phase-Conditioned Speculative Decoding", section 3); pruning by
// confidence only cuts a suffix of the proposal, the kept tokens are verified
// as usual (bowenzhou, "设计" and the static-threshold diagnostic of
// "Results").  Per block, with T its temperature:
//   m = number of leading positions with survival >= threshold;
//   for k < m: accept x_k iff u_k p_d(x_k) < p_t(x_k) (greedy: iff x_k is
//   the target's argmax); n = positions accepted before the first rejection;
//   next token: after a rejection at j = n, argmax of ln max(0, p_t - p_d)
//   + Gumbel over the vocabulary (the residual draw; p_d recomputed at j from
//   U and the Eq 5 bias of x_{j-1}); after m acceptances, argmax of
//   z_t / T + Gumbel at position m; greedy: the target's argmax at j.
// Random numbers: the accept uniform of (b, k) is word 0 of Philox4x32-10 at
// counter (0xFFFFFFFF, k, b, offset), the Gumbel variate of element v of the
// final draw at position j is word v mod 4 at counter
// (v / 4, 0x80000000 | j, b, offset); the key and the word -> u map are the
// drafting ones, and no counter coincides with a drafting counter.
//
// Kernels: k_vt_stats (chunk statistics of the target rows: max, sum of
// exp((z_t - max) / T), argmax), k_v_decide (wave per block: row
// normalisers, the accept tests of all positions at once, trim and first
// rejection by ballot, the mode of the final draw, E row of the residual
// position),
// k_v_bias_mfma / k_v_bias_vec (z_d / T at the residual position for every
// block, and per-column-group softmax partials), k_v_sample (the draft
// row's normaliser from those partials, partial argmax keys of the
// residual and the target draw, and in the block's last workgroup the
// next token).
#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace dspark {

constexpr int kVCols = 256;      // columns per bias workgroup (4 waves x 64)
constexpr int kVChunk = 4096;    // columns per sampling workgroup (256 threads x 16)
constexpr int kVTChunk = 8192;   // columns per target-statistics workgroup (256 threads x 32)
constexpr uint32_t kVerifyAcceptCtr0 = 0xFFFFFFFFu;
constexpr uint32_t kVerifyDrawCtr1 = 0x80000000u;

enum VerifyMode : int32_t { kModeGreedy = 0, kModeResidual = 1, kModeTarget = 2 };

bool verify_mfma_ok(const dspark_dims& d) {
    return d.dtype == DSPARK_BF16 && d.r % 32 == 0 && d.r <= 256 && d.V % 8 == 0;
}

VerifyLayout verify_layout(const dspark_dims& d) {
    VerifyLayout L{};
    L.mfma = verify_mfma_ok(d);
    L.Bpad = (d.B + 15) / 16 * 16;
    L.P = (d.V + kVCols - 1) / kVCols;
    L.C = (d.V + kVChunk - 1) / kVChunk;
    L.CT = (d.V + kVTChunk - 1) / kVTChunk;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t B = static_cast<size_t>(d.B), rows = B * (d.gamma + 1);
    L.bad = take(sizeof(int32_t) * B);
    L.lse_t = take(sizeof(float) * rows);
    L.amax = take(sizeof(int32_t) * rows);
    L.tmx = take(sizeof(float) * rows * L.CT);
    L.tsm = take(sizeof(float) * rows * L.CT);
    L.tkey = take(sizeof(uint64_t) * rows * L.CT);
    L.mode = take(sizeof(int32_t) * B);
    L.jpos = take(sizeof(int32_t) * B);
    L.invT = take(sizeof(float) * B);
    L.ebf = take(sizeof(uint16_t) * L.Bpad * d.r);
    L.ef = take(sizeof(float) * B * d.r);
    L.zd = take(sizeof(float) * B * d.V);
    L.pmx = take(sizeof(float) * B * L.P);
    L.psm = take(sizeof(float) * B * L.P);
    L.keys = take(sizeof(uint64_t) * B * 2);
    L.done = take(sizeof(uint32_t) * B);
    L.total = off;
    return L;
}

__device__ __forceinline__ uint32_t philox_word(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                uint32_t k0, uint32_t k1, int word) {
    const u32x4 out = philox4x32_10(u32x4{c0, c1, c2, c3}, k0, k1);
    return out[word];
}

// (max, sum of exp(x - max)) merge with empty partials (s = 0) allowed.
__device__ __forceinline__ void ms_merge(float& m, float& s, float m2, float s2) {
    const float mm = fmaxf(m, m2);
    const float a = s > 0.0f ? s * __expf(m - mm) : 0.0f;
    const float b = s2 > 0.0f ? s2 * __expf(m2 - mm) : 0.0f;
    m = mm;
    s = a + b;
}

// ------------------------------------------------------------ target rows

// Workgroup per (target row, 8192-column chunk), row = (b, position k in
// 0..gamma), thread per 32 columns: the chunk's max of z_t (and its argmax
// key, lowest index on a tie) and sum of exp((z_t - max) / T).  A thread
// takes its maximum first and the lowest of its columns attaining it after
// (one key per thread), then the workgroup merges across lanes (exchange
// steps) and across its 4 waves (in wave order).
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_vt_stats(const T* __restrict__ Tl,
                                                  const float* __restrict__ temperature, int V,
                                                  int gamma, int CT, float* __restrict__ tmx,
                                                  float* __restrict__ tsm, uint64_t* __restrict__ tkey) {
    constexpr int NX = kVTChunk / 256;
    __shared__ float sm[4], ss[4];
    __shared__ uint64_t sk[4];
    const int64_t row = blockIdx.x;
    const int chunk = blockIdx.y;
    const int b = static_cast<int>(row / (gamma + 1));
    const float Tb = temperature[b];
    const float invT = Tb > 0.0f ? 1.0f / Tb : 1.0f;
    const T* z = Tl + row * V;
    float x[NX];
    // column of element j of this thread (increasing in j)
    auto col = [&](int j) {
        return VEC ? chunk * kVTChunk + 2048 * (j / 8) + 8 * static_cast<int>(threadIdx.x) + (j % 8)
                   : chunk * kVTChunk + static_cast<int>(threadIdx.x) + 256 * j;
    };
    if (VEC) {
        // 4 runs of 8 consecutive columns per thread, 16-byte loads
#pragma unroll
        for (int i = 0; i < NX / 8; ++i) {
            const int v = col(8 * i);
            const u32x4 w = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(z) + min(v, V - 8));
#pragma unroll
            for (int e = 0; e < 8; ++e) x[8 * i + e] = v < V ? ((e & 1) ? hi_bf16(w[e >> 1]) : lo_bf16(w[e >> 1])) : -INFINITY;
        }
    } else {
#pragma unroll
        for (int i = 0; i < NX; ++i) {
            const int v = col(i);
            x[i] = v < V ? load_f(z, min(v, V - 1)) : -INFINITY;
        }
    }
    float m = x[0];
#pragma unroll
    for (int i = 1; i < NX; ++i) m = fmaxf(m, x[i]);
    int jb = NX - 1;
#pragma unroll
    for (int i = NX - 2; i >= 0; --i) jb = x[i] == m ? i : jb;
    uint64_t key = m > -INFINITY ? argmax_key(m, static_cast<uint32_t>(col(jb))) : kKeyNone;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NX; ++i) s += x[i] > -INFINITY ? __expf((x[i] - m) * invT) : 0.0f;
    float ms = m * invT;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const float m2 = __shfl_xor(ms, o), s2 = __shfl_xor(s, o);
        ms_merge(ms, s, m2, s2);
        const uint32_t lo = __shfl_xor(static_cast<uint32_t>(key), o);
        const uint32_t hi = __shfl_xor(static_cast<uint32_t>(key >> 32), o);
        const uint64_t k2 = (static_cast<uint64_t>(hi) << 32) | lo;
        key = k2 > key ? k2 : key;
    }
    const int wave = threadIdx.x / kWave;
    if ((threadIdx.x & (kWave - 1)) == 0) {
        sm[wave] = ms;
        ss[wave] = s;
        sk[wave] = key;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        float m1 = sm[0], s1 = ss[0];
        uint64_t k1 = sk[0];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            ms_merge(m1, s1, sm[w], ss[w]);
            k1 = sk[w] > k1 ? sk[w] : k1;
        }
        tmx[row * CT + chunk] = m1;
        tsm[row * CT + chunk] = s1;
        tkey[row * CT + chunk] = k1;
    }
}

// ----------------------------------------------------------------- decide

// Wave per block.  Lane k <= gamma merges the chunk statistics of target row
// k (lse of z_t / T, argmax); lane k < gamma runs the accept test of
// position k (independent of the others; the first failure ends the run);
// lane 0 then takes m, n, the mode and position of the final draw, and the
// wave copies the E row (W1[token before the residual position]) in bf16
// and fp32.
template <typename T>
__global__ __launch_bounds__(64) void k_v_decide(
    const T* __restrict__ Tl, const T* __restrict__ W1, const int32_t* __restrict__ anchor,
    const int32_t* __restrict__ tokens, const float* __restrict__ logp,
    const float* __restrict__ survival, const float* __restrict__ temperature,
    const float* __restrict__ tmx, const float* __restrict__ tsm, const uint64_t* __restrict__ tkey,
    int CT, int V, int r, int gamma, float tau, uint32_t key0, uint32_t key1, uint32_t ctr3,
    float* __restrict__ lse_t, int32_t* __restrict__ amax, uint64_t* __restrict__ keys,
    uint32_t* __restrict__ done, int32_t* __restrict__ bad,
    int32_t* __restrict__ mode, int32_t* __restrict__ jpos, float* __restrict__ invTo,
    uint16_t* __restrict__ ebf, float* __restrict__ ef, int32_t* __restrict__ n_keep,
    int32_t* __restrict__ n_accept, int32_t* __restrict__ next_token,
    float* __restrict__ accept_prob) {
    __shared__ int s_prev;
    __shared__ float s_lt[65];
    __shared__ int s_am[65];
    const int b = blockIdx.x, lane = threadIdx.x;
    const float Tb = temperature[b];
    const bool greedy = !(Tb > 0.0f);
    const float invT = greedy ? 1.0f : 1.0f / Tb;
    const int64_t i0 = static_cast<int64_t>(b) * gamma;
    // target row statistics (rows 0..gamma, gamma <= 64)
    for (int k = lane; k <= gamma; k += 64) {
        const int64_t row = static_cast<int64_t>(b) * (gamma + 1) + k;
        float m = -INFINITY, s = 0.0f;
        uint64_t key = kKeyNone;
        for (int c = 0; c < CT; ++c) {
            ms_merge(m, s, tmx[row * CT + c], tsm[row * CT + c]);
            const uint64_t k2 = tkey[row * CT + c];
            key = k2 > key ? k2 : key;
        }
        s_lt[k] = m + __logf(s);
        s_am[k] = static_cast<int32_t>(key_index(key));
        lse_t[row] = s_lt[k];
        amax[row] = s_am[k];
    }
    __syncthreads();
    const float lt = lane <= gamma ? s_lt[lane] : 0.0f;
    const int am = lane <= gamma ? s_am[lane] : 0;
    // per-position accept tests
    const int x = lane < gamma ? tokens[i0 + lane] : 0;
    const bool xbad = lane < gamma && (x < 0 || x >= V);
    const bool in_keep = lane < gamma && survival[i0 + lane] >= tau;
    bool ok = false;
    float ap = 0.0f;
    if (lane < gamma && !xbad) {
        if (greedy) {
            ok = x == am;
            ap = ok ? 1.0f : 0.0f;
        } else {
            const int64_t row = static_cast<int64_t>(b) * (gamma + 1) + lane;
            const float pt = __expf(load_f(Tl, row * V + x) * invT - lt);
            const float pd = __expf(logp[i0 + lane]);
            const uint32_t w = philox_word(kVerifyAcceptCtr0, static_cast<uint32_t>(lane),
                                           static_cast<uint32_t>(b), ctr3, key0, key1, 0);
            const float u = static_cast<float>((w >> 8) | 1u) * 5.9604644775390625e-8f;
            ok = u * pd < pt;
            ap = pt >= pd ? 1.0f : pt / pd;
        }
    }
    const uint64_t badmask = __ballot(xbad);
    const int flag = badmask != 0 || anchor[b] < 0 || anchor[b] >= V;
    // m = leading kept positions, n = leading accepted positions among them
    const uint64_t past = gamma < 64 ? (~0ull << gamma) : 0ull;
    const uint64_t notkeep = __ballot(lane < gamma && !in_keep) | past;
    const int m = notkeep ? __builtin_ctzll(notkeep) : 64;
    const uint64_t notok = __ballot(lane < gamma && !ok) | past;
    const int n = flag ? 0 : min(m, notok ? static_cast<int>(__builtin_ctzll(notok)) : 64);
    // tested positions: 0..n (the rejected one included) within the kept ones
    if (accept_prob && lane < gamma)
        accept_prob[i0 + lane] = (!flag && lane < m && lane <= n) ? ap : NAN;
    const int j = n;
    const int md = greedy ? kModeGreedy : (n < m ? kModeResidual : kModeTarget);
    if (lane < 2) keys[2 * b + lane] = kKeyNone;
    if (lane == 2) done[b] = 0u;
    if (lane == 0) {
        bad[b] = flag;
        mode[b] = flag ? -1 : md;
        jpos[b] = j;
        invTo[b] = invT;
        n_keep[b] = flag ? 0 : m;
        n_accept[b] = n;
        s_prev = (md == kModeResidual && !flag) ? (j == 0 ? anchor[b] : tokens[i0 + j - 1]) : -1;
    }
    // the greedy emission is the target's argmax at j
    if (lane == 0) next_token[b] = flag ? -1 : (greedy ? s_am[j] : -1);
    __syncthreads();
    const int prev = s_prev;
    for (int q = lane; q < r; q += 64) {
        const float e = prev >= 0 ? load_f(W1, static_cast<int64_t>(prev) * r + q) : 0.0f;
        ef[static_cast<int64_t>(b) * r + q] = e;
        ebf[static_cast<int64_t>(b) * r + q] = static_cast<uint16_t>(__float_as_uint(e) >> 16);  // exact: bf16 data
    }
}

// ------------------------------------------------------------ draft row

__global__ __launch_bounds__(256) void k_v_zero_u16(uint16_t* __restrict__ p, int n) {
    for (int i = threadIdx.x; i < n; i += 256) p[i] = 0;
}

// z_d / T at each block's residual position on the matrix cores: a wave owns
// 64 columns with the W2 tile in registers (W2Tile), 16 blocks per MFMA
// unit with their E rows staged in LDS; lane (g, n) ends up with 16
// consecutive columns of block n.  Writes zd and the (max, sum) partial of
// every 256-column group.
template <int KC>
__global__ __launch_bounds__(256) void k_v_bias_mfma(const uint16_t* __restrict__ U,
                                                     const uint16_t* __restrict__ W2,
                                                     const uint16_t* __restrict__ ebf,
                                                     const int32_t* __restrict__ jpos,
                                                     const float* __restrict__ invT, int V, int B,
                                                     int Bpad, int gamma, float* __restrict__ zd,
                                                     float* __restrict__ pmx, float* __restrict__ psm) {
    constexpr int r = KC * 32;
    constexpr int ldE = r + 8;
    __shared__ __attribute__((aligned(16))) uint16_t Es[16 * ldE];
    __shared__ float red_m[4][16], red_s[4][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int vt = (blockIdx.x * 4 + wave) * 64;
    const int P = gridDim.x;
    const int v0 = vt + 16 * g;
    const bool live = v0 < V;
    const int ua = live ? v0 : 0, ub = (live && v0 + 8 < V) ? v0 + 8 : ua;

    W2Tile<KC> w2;
    w2.load(W2, V, vt, g, n);
    for (int nb = 0; nb < Bpad / 16; ++nb) {
        __syncthreads();
        for (int t = threadIdx.x; t < 16 * (r / 8); t += 256) {
            const int row = t / (r / 8), col = t % (r / 8);
            *reinterpret_cast<u32x4*>(&Es[row * ldE + col * 8]) =
                *reinterpret_cast<const u32x4*>(ebf + (static_cast<size_t>(nb) * 16 + row) * r + col * 8);
        }
        __syncthreads();
        const int b = nb * 16 + n;
        const int bc = min(b, B - 1);
        // position of the residual draw (other modes: any valid row, unused)
        const uint16_t* urow = U + (static_cast<size_t>(bc) * gamma + min(jpos[bc], gamma - 1)) * V;
        const u32x4 u0 = *reinterpret_cast<const u32x4*>(urow + ua);
        const u32x4 u1 = *reinterpret_cast<const u32x4*>(urow + ub);
        const float it = invT[bc];
        f32x4 acc[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        w2.mul(&Es[n * ldE + 8 * g], acc);
        const uint32_t w[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
        float z[16];
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int jj = 4 * q + c;
                z[jj] = (((jj & 1) ? hi_bf16(w[jj >> 1]) : lo_bf16(w[jj >> 1])) + acc[c][q]) * it;
            }
        float m = -INFINITY, s = 0.0f;
        if (b < B && live) {
            float* out = zd + static_cast<size_t>(b) * V + v0;
            const int cnt = min(16, V - v0);  // 8 or 16 (V % 8 == 0)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (4 * q < cnt) *reinterpret_cast<f32x4*>(out + 4 * q) = f32x4{z[4 * q], z[4 * q + 1], z[4 * q + 2], z[4 * q + 3]};
#pragma unroll
            for (int jj = 0; jj < 16; ++jj)
                if (jj < cnt) ms_merge(m, s, z[jj], 1.0f);
        }
        // merge the 4 lanes of block n, then the 4 waves
        for (int o = 16; o < 64; o <<= 1) {
            const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
            ms_merge(m, s, m2, s2);
        }
        if (g == 0) {
            red_m[wave][n] = m;
            red_s[wave][n] = s;
        }
        __syncthreads();
        if (wave == 0 && g == 0 && b < B) {
            float mm = red_m[0][n], ss = red_s[0][n];
            for (int wv = 1; wv < 4; ++wv) ms_merge(mm, ss, red_m[wv][n], red_s[wv][n]);
            pmx[static_cast<size_t>(b) * P + blockIdx.x] = mm;
            psm[static_cast<size_t>(b) * P + blockIdx.x] = ss;
        }
    }
}

// Vector path: thread per column, blocks in turn; same outputs.
template <typename T>
__global__ __launch_bounds__(256) void k_v_bias_vec(const T* __restrict__ U, const T* __restrict__ W2,
                                                    const float* __restrict__ ef,
                                                    const int32_t* __restrict__ jpos,
                                                    const float* __restrict__ invT, int V, int r,
                                                    int B, int gamma, float* __restrict__ zd,
                                                    float* __restrict__ pmx, float* __restrict__ psm) {
    __shared__ float sm[256], ss[256];
    const int v = blockIdx.x * 256 + threadIdx.x;
    const int P = gridDim.x;
    for (int b = 0; b < B; ++b) {
        float m = -INFINITY, s = 0.0f;
        if (v < V) {
            float acc = load_f(U, (static_cast<int64_t>(b) * gamma + min(jpos[b], gamma - 1)) * V + v);
            for (int q = 0; q < r; ++q)
                acc = fmaf(ef[static_cast<int64_t>(b) * r + q], load_f(W2, static_cast<int64_t>(q) * V + v), acc);
            const float z = acc * invT[b];
            zd[static_cast<int64_t>(b) * V + v] = z;
            m = z;
            s = 1.0f;
        }
        sm[threadIdx.x] = m;
        ss[threadIdx.x] = s;
        __syncthreads();
        for (int h = 128; h > 0; h >>= 1) {
            if (threadIdx.x < h) {
                float m1 = sm[threadIdx.x], s1 = ss[threadIdx.x];
                ms_merge(m1, s1, sm[threadIdx.x + h], ss[threadIdx.x + h]);
                sm[threadIdx.x] = m1;
                ss[threadIdx.x] = s1;
            }
            __syncthreads();
        }
        if (threadIdx.x == 0) {
            pmx[static_cast<int64_t>(b) * P + blockIdx.x] = sm[0];
            psm[static_cast<int64_t>(b) * P + blockIdx.x] = ss[0];
        }
        __syncthreads();
    }
}

// Wave per block: lse of z_d / T from the P partials, in order.
// ------------------------------------------------------------ final draw

// Workgroup per (block, 4096-column chunk), thread per 16 columns: partial
// argmax keys of the residual draw (entries with p_t > p_d only) and of the
// target draw.  Greedy blocks are skipped.
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void k_v_sample(const T* __restrict__ Tl, const float* __restrict__ zd,
                                                  const float* __restrict__ lse_t,
                                                  const float* __restrict__ pmx, const float* __restrict__ psm,
                                                  int P, const int32_t* __restrict__ mode,
                                                  const int32_t* __restrict__ jpos,
                                                  const float* __restrict__ invT, int V, int gamma,
                                                  uint32_t key0, uint32_t key1, uint32_t ctr3,
                                                  uint64_t* __restrict__ keys, uint32_t* __restrict__ done,
                                                  int32_t* __restrict__ next_token) {
    __shared__ uint64_t kr[256], kt[256];
    __shared__ float sm[256 / kWave], ss[256 / kWave];
    __shared__ bool last;
    const int b = blockIdx.y, chunk = blockIdx.x;
    const int md = mode[b];
    if (md != kModeResidual && md != kModeTarget) return;
    const int j = jpos[b];
    const float it = invT[b];
    const int64_t row = static_cast<int64_t>(b) * (gamma + 1) + j;
    const float lt = lse_t[row];
    // log-normaliser of the draft row from the bias kernel's P partials,
    // merged in the same fixed order by every workgroup of the block
    float ld = 0.0f;
    if (md == kModeResidual) {
        float m = -INFINITY, s = 0.0f;
        for (int p = threadIdx.x; p < P; p += blockDim.x)
            ms_merge(m, s, pmx[static_cast<int64_t>(b) * P + p], psm[static_cast<int64_t>(b) * P + p]);
        for (int o = 1; o < kWave; o <<= 1) {
            const float m2 = __shfl_xor(m, o), s2 = __shfl_xor(s, o);
            ms_merge(m, s, m2, s2);
        }
        if ((threadIdx.x & (kWave - 1)) == 0) {
            sm[threadIdx.x / kWave] = m;
            ss[threadIdx.x / kWave] = s;
        }
        __syncthreads();
        m = sm[0];
        s = ss[0];
        for (int w = 1; w < static_cast<int>(blockDim.x) / kWave; ++w) ms_merge(m, s, sm[w], ss[w]);
        ld = m + __logf(s);
    }
    const T* zt = Tl + row * V;
    const float* zr = zd + static_cast<int64_t>(b) * V;
    uint64_t bres = kKeyNone, btgt = kKeyNone;
    const int v0 = chunk * kVChunk + threadIdx.x * 16;
    float xt[16], xd[16];
    if (VEC) {
        // 16 consecutive columns: two 16-byte loads of the target row, four
        // of the draft row (residual mode only); clamped past V
        const int va = min(v0, V - 8), vb = min(v0 + 8, V - 8);
        const u32x4 w0 = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(zt) + va);
        const u32x4 w1 = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(zt) + vb);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            xt[e] = (e & 1) ? hi_bf16(w0[e >> 1]) : lo_bf16(w0[e >> 1]);
            xt[8 + e] = (e & 1) ? hi_bf16(w1[e >> 1]) : lo_bf16(w1[e >> 1]);
        }
        if (md == kModeResidual) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const f32x4 d4 = *reinterpret_cast<const f32x4*>(zr + min(v0 + 4 * q, V - 4));
#pragma unroll
                for (int e = 0; e < 4; ++e) xd[4 * q + e] = d4[e];
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int v = min(v0 + e, V - 1);
            xt[e] = load_f(zt, v);
            xd[e] = md == kModeResidual ? zr[v] : 0.0f;
        }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int vb = v0 + 4 * q;
        const u32x4 wd = philox4x32_10(u32x4{static_cast<uint32_t>(vb >> 2), kVerifyDrawCtr1 | static_cast<uint32_t>(j),
                                             static_cast<uint32_t>(b), ctr3},
                                       key0, key1);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int v = vb + e;
            if (v < V) {
                const float g = gumbel_from_word(wd[e]);
                const float zl = xt[4 * q + e] * it;
                const uint64_t k2 = argmax_key(zl + g, static_cast<uint32_t>(v));
                btgt = k2 > btgt ? k2 : btgt;
                if (md == kModeResidual) {
                    const float res = __expf(zl - lt) - __expf(xd[4 * q + e] - ld);
                    if (res > 0.0f) {
                        const uint64_t k1 = argmax_key(__logf(res) + g, static_cast<uint32_t>(v));
                        bres = k1 > bres ? k1 : bres;
                    }
                }
            }
        }
    }
    kr[threadIdx.x] = bres;
    kt[threadIdx.x] = btgt;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (threadIdx.x < h) {
            kr[threadIdx.x] = kr[threadIdx.x + h] > kr[threadIdx.x] ? kr[threadIdx.x + h] : kr[threadIdx.x];
            kt[threadIdx.x] = kt[threadIdx.x + h] > kt[threadIdx.x] ? kt[threadIdx.x + h] : kt[threadIdx.x];
        }
        __syncthreads();
    }
    // a maximum does not depend on the order of the updates; the block's
    // last workgroup to finish (counted after its own keys are complete)
    // picks the token: the residual draw, or the target draw when no entry
    // of the residual is positive
    if (threadIdx.x == 0) {
        if (kr[0] != kKeyNone) atomicMax(reinterpret_cast<unsigned long long*>(keys + 2 * b), kr[0]);
        atomicMax(reinterpret_cast<unsigned long long*>(keys + 2 * b + 1), kt[0]);
        // the key atomics are device-coherent: waiting here until both have
        // completed (no cache write-back) orders them before the count, so
        // the workgroup that counts last reads both maxima complete
        wait_vmem_complete();
        last = __hip_atomic_fetch_add(done + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1;
    }
    __syncthreads();
    if (last && threadIdx.x == 0) {
        const uint64_t fr = __hip_atomic_load(keys + 2 * b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t ft = __hip_atomic_load(keys + 2 * b + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t k = (md == kModeResidual && fr != kKeyNone) ? fr : ft;
        next_token[b] = static_cast<int32_t>(key_index(k));
    }
}

// ------------------------------------------------------------------ launch

template <typename T>
static hipError_t launch_verify_t(const VerifyArgs& va) {
    const dspark_dims& D = va.dims;
    const VerifyLayout L = verify_layout(D);
    hipStream_t st = va.stream;
    char* ws = va.ws;
    int32_t* bad = reinterpret_cast<int32_t*>(ws + L.bad);
    float* lse_t = reinterpret_cast<float*>(ws + L.lse_t);
    int32_t* amax = reinterpret_cast<int32_t*>(ws + L.amax);
    int32_t* mode = reinterpret_cast<int32_t*>(ws + L.mode);
    int32_t* jpos = reinterpret_cast<int32_t*>(ws + L.jpos);
    float* invT = reinterpret_cast<float*>(ws + L.invT);
    uint16_t* ebf = reinterpret_cast<uint16_t*>(ws + L.ebf);
    float* ef = reinterpret_cast<float*>(ws + L.ef);
    float* zd = reinterpret_cast<float*>(ws + L.zd);
    float* pmx = reinterpret_cast<float*>(ws + L.pmx);
    float* psm = reinterpret_cast<float*>(ws + L.psm);
    uint64_t* keys = reinterpret_cast<uint64_t*>(ws + L.keys);
    uint32_t* done = reinterpret_cast<uint32_t*>(ws + L.done);
    const T* Tl = static_cast<const T*>(va.T_logits);
    const uint32_t key0 = static_cast<uint32_t>(va.seed), key1 = static_cast<uint32_t>(va.seed >> 32);
    const uint32_t ctr3 = static_cast<uint32_t>(va.offset);
    const int B = D.B, V = D.V, r = D.r, g = D.gamma;

    float* tmx = reinterpret_cast<float*>(ws + L.tmx);
    float* tsm = reinterpret_cast<float*>(ws + L.tsm);
    uint64_t* tkey = reinterpret_cast<uint64_t*>(ws + L.tkey);
    // 16-byte loads for bf16 rows (V % 8 == 0 keeps every row 16-byte aligned)
    const bool vec = sizeof(T) == 2 && V % 8 == 0 && (reinterpret_cast<uintptr_t>(Tl) & 15) == 0;
    if (vec)
        hipLaunchKernelGGL((k_vt_stats<T, true>), dim3(B * (g + 1), L.CT), dim3(256), 0, st, Tl, va.temperature,
                           V, g, L.CT, tmx, tsm, tkey);
    else
        hipLaunchKernelGGL((k_vt_stats<T, false>), dim3(B * (g + 1), L.CT), dim3(256), 0, st, Tl, va.temperature,
                           V, g, L.CT, tmx, tsm, tkey);
    hipLaunchKernelGGL((k_v_decide<T>), dim3(B), dim3(64), 0, st, Tl, static_cast<const T*>(va.W1),
                       va.anchor, va.tokens, va.logp, va.survival, va.temperature, tmx, tsm, tkey, L.CT,
                       V, r, g, va.threshold, key0, key1, ctr3, lse_t, amax, keys, done, bad, mode, jpos, invT, ebf,
                       ef, va.n_keep, va.n_accept, va.next_token, va.accept_prob);
    if (L.Bpad > B) {
        // padding E rows of the last 16-block unit (read by the MFMA, never used)
        hipLaunchKernelGGL(k_v_zero_u16, dim3(1), dim3(256), 0, st, ebf + static_cast<size_t>(B) * r,
                           (L.Bpad - B) * r);
    }
    hipError_t pe = profile_begin(st);
    if (pe != hipSuccess) return pe;
    if (L.mfma) {
        const uint16_t* U = static_cast<const uint16_t*>(va.U);
        const uint16_t* W2 = static_cast<const uint16_t*>(va.W2);
        switch (r / 32) {
#define DSPARK_VB(KC)                                                                                    \
    case KC:                                                                                             \
        hipLaunchKernelGGL((k_v_bias_mfma<KC>), dim3(L.P), dim3(256), 0, st, U, W2, ebf, jpos, invT, V, B, \
                           L.Bpad, g, zd, pmx, psm);                                                     \
        break;
            DSPARK_VB(1) DSPARK_VB(2) DSPARK_VB(3) DSPARK_VB(4) DSPARK_VB(5) DSPARK_VB(6) DSPARK_VB(7) DSPARK_VB(8)
#undef DSPARK_VB
            default: return hipErrorInvalidValue;
        }
    } else {
        hipLaunchKernelGGL((k_v_bias_vec<T>), dim3(L.P), dim3(256), 0, st, static_cast<const T*>(va.U),
                           static_cast<const T*>(va.W2), ef, jpos, invT, V, r, B, g, zd, pmx, psm);
    }
    if ((pe = profile_end(st)) != hipSuccess) return pe;
    if (vec)
        hipLaunchKernelGGL((k_v_sample<T, true>), dim3(L.C, B), dim3(256), 0, st, Tl, zd, lse_t, pmx, psm, L.P, mode,
                           jpos, invT, V, g, key0, key1, ctr3, keys, done, va.next_token);
    else
        hipLaunchKernelGGL((k_v_sample<T, false>), dim3(L.C, B), dim3(256), 0, st, Tl, zd, lse_t, pmx, psm, L.P, mode,
                           jpos, invT, V, g, key0, key1, ctr3, keys, done, va.next_token);
    return hipGetLastError();
}

hipError_t launch_verify(const VerifyArgs& a) {
    return a.dims.dtype == DSPARK_BF16 ? launch_verify_t<uint16_t>(a) : launch_verify_t<float>(a);
}

}  // namespace dspark
