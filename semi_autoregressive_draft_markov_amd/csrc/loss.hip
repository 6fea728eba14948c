// DSpark teacher-forced objective on gfx950: Eq 8-12 of the DSpark paper as
// transcribed on the dormouse "DSpark - paper verification" page, section 1,
// with teacher forcing as in mainlymatmul's "Training DSpark" (position k is
// fed the ground-truth x_{k-1}), plus dL/dz_d and dW2 = E^T dZ.
//
// Rows i = n * gamma + k.  z_d = U + E W2 (E = W1[prev]) is recomputed in
// each of three sweeps over V rather than stored (storing it in bf16 would
// break the tolerance, in fp32 it costs more bytes than re-reading U):
//   prep     prev tokens, E (row-major and transposed), confidence logits,
//            z_d at the label
//   pass 1   per row: log-sum-exp of z_d and z_t
//   pass 2   per row: sum |p_d - p_t|, sum min(p_d, p_t), sum p_d sign(p_d - p_t)
//   finalize c*, CE, BCE, dL/da per row; the four losses (fixed-order sums)
//   pass 3   dZ = (w_k/N)[a_ce (p_d - onehot) + a_tv p_d (s - S)]  -> dlogits
//            (matrix-core path: s from 2-bit signs pass 2 stored, T not read)
//   dW2      E^T dZ, MFMA over rows (split-bf16 when dZ is float32)
#include <math.h>

#include <algorithm>

#include "device_common.h"
#include "internal.h"
#include "mfma_tile.h"

namespace dspark {

constexpr int kLossWaves = 4;                  // waves per workgroup (MFMA passes)
constexpr int kLossColsPerWG = 64 * kLossWaves;
constexpr int kLossGenericCols = 4 * 256;
constexpr int kLossTargetItems = 2048;         // work items per pass (row chunks x column groups)

bool loss_mfma_ok(const dspark_dims& d) {
    return d.dtype == DSPARK_BF16 && d.r % 32 == 0 && d.r <= 256 && d.V % 8 == 0;
}

LossLayout loss_layout(const dspark_dims& d) {
    LossLayout L{};
    const int64_t R = static_cast<int64_t>(d.B) * d.gamma;
    L.R = static_cast<int>(R);
    L.Rpad = static_cast<int>((R + 31) / 32 * 32);
    L.mfma = loss_mfma_ok(d);
    L.P = L.mfma ? (d.V + kLossColsPerWG - 1) / kLossColsPerWG
                 : (d.V + kLossGenericCols - 1) / kLossGenericCols;
    const int rb = L.Rpad / 16;
    L.nrc = std::max(1, std::min(rb, (kLossTargetItems + L.P - 1) / L.P));
    L.rb_per_chunk = (rb + L.nrc - 1) / L.nrc;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off = align_up(off + bytes, 256);
        return at;
    };
    const size_t rp = static_cast<size_t>(L.Rpad);
    L.bad = take(sizeof(int32_t) * d.B);
    L.ebf = take(sizeof(uint16_t) * rp * d.r);
    L.ef = take(sizeof(float) * rp * d.r);
    L.et = take(sizeof(uint16_t) * rp * d.r);
    L.label = take(sizeof(int32_t) * rp);
    L.rowc = take(sizeof(float) * rp);
    L.alog = take(sizeof(float) * rp);
    L.lse_d = take(sizeof(float) * rp);
    L.lse_t = take(sizeof(float) * rp);
    L.zlab = take(sizeof(float) * rp);
    L.tv = take(sizeof(float) * rp);
    L.cmin = take(sizeof(float) * rp);
    L.S = take(sizeof(float) * rp);
    for (int q = 0; q < 5; ++q) L.part[q] = take(sizeof(float) * rp * L.P);
    // one extra column group: the store target of lanes past V
    L.smask = take(L.mfma ? sizeof(uint32_t) * rp * ((d.V + 15) / 16 + 1) : 0);
    L.tce = take(sizeof(float) * rp);
    L.ttv = take(sizeof(float) * rp);
    L.tbce = take(sizeof(float) * rp);
    L.total = off;
    return L;
}

// ------------------------------------------------------------------ prep

struct LossConsts {
    float alpha[3];
    float pos_weight[64];  // w_k / N for k < gamma
};

// Position of E[i][j] in the transposed copy the dW2 contraction reads:
// chunk-major, the 32-row chunk i / 32 of all r columns contiguous, column j
// of it 32 consecutive values.  An MFMA operand (16 columns j, 8 rows i of
// one chunk) is then 1 KB of whole cache lines, and a chunk is read once: in
// a plain [r, Rpad] layout each operand piece is half a line whose other
// half belongs to the next chunk, and the streaming dZ evicts it between
// the two.
__host__ __device__ __forceinline__ size_t et_index(int i, int j, int r) {
    return (static_cast<size_t>(i >> 5) * r + j) * 32 + (i & 31);
}

// Workgroup = one row i (rows in [R, Rpad) only zero their operand rows).
// Teacher forcing: prev = anchor[n] at k = 0, labels[n, k-1] after.  The row
// k = 0 workgroup of block n also checks every token id of the block.  Also
// the draft logit at the label, z_d[x*] = U[i, x*] + E_i . W2[:, x*] (Eq 9).
template <typename T>
__global__ __launch_bounds__(256) void k_loss_prep(
    const int32_t* __restrict__ anchor, const int32_t* __restrict__ labels,
    const T* __restrict__ W1, const T* __restrict__ w_conf, const T* __restrict__ h,
    const T* __restrict__ U, const T* __restrict__ W2, int V, int r,
    int d, int gamma, int R, int Rpad, LossConsts cst, int32_t* __restrict__ bad,
    uint16_t* __restrict__ ebf, float* __restrict__ ef, uint16_t* __restrict__ et,
    int32_t* __restrict__ label_out, float* __restrict__ rowc, float* __restrict__ alog,
    float* __restrict__ zlab) {
    __shared__ float red[16];
    const int i = blockIdx.x;
    if (i >= R) {
        for (int j = threadIdx.x; j < r; j += blockDim.x) {
            ebf[static_cast<size_t>(i) * r + j] = 0;
            ef[static_cast<size_t>(i) * r + j] = 0.0f;
            et[et_index(i, j, r)] = 0;
        }
        if (threadIdx.x == 0) {
            label_out[i] = 0;
            rowc[i] = 0.0f;
            alog[i] = 0.0f;
            zlab[i] = 0.0f;
        }
        return;
    }
    const int n = i / gamma, k = i % gamma;
    const int prev_raw = k == 0 ? anchor[n] : labels[i - 1];
    const int lab_raw = labels[i];
    const bool ok = prev_raw >= 0 && prev_raw < V && lab_raw >= 0 && lab_raw < V;
    const int prev = ok ? prev_raw : 0;
    if (k == 0 && threadIdx.x == 0) {
        bool all = anchor[n] >= 0 && anchor[n] < V;
        for (int q = 0; q < gamma; ++q) {
            const int t = labels[static_cast<size_t>(n) * gamma + q];
            all = all && t >= 0 && t < V;
        }
        bad[n] = all ? 0 : 1;
    }
    const int lab = ok ? lab_raw : 0;
    float part = 0.0f, zl = 0.0f;
    for (int j = threadIdx.x; j < r; j += blockDim.x) {
        const float e = load_f(W1, static_cast<int64_t>(prev) * r + j);
        const uint16_t eb = static_cast<uint16_t>(f32_to_bf16(e));
        ebf[static_cast<size_t>(i) * r + j] = eb;
        ef[static_cast<size_t>(i) * r + j] = e;
        et[et_index(i, j, r)] = eb;
        part += load_f(w_conf, d + j) * e;
        zl = fmaf(e, load_f(W2, static_cast<int64_t>(j) * V + lab), zl);
    }
    const int64_t hrow = static_cast<int64_t>(i) * d;
    for (int q = threadIdx.x; q < d; q += blockDim.x) part += load_f(w_conf, q) * load_f(h, hrow + q);
    const float a = block_sum(part, red);
    zl = block_sum(zl, red);
    if (threadIdx.x == 0) {
        label_out[i] = lab;
        rowc[i] = ok ? cst.pos_weight[k] : 0.0f;  // zero gradient rows for invalid ids
        alog[i] = ok ? a : NAN;
        zlab[i] = load_f(U, static_cast<int64_t>(i) * V + lab) + zl;
    }
}

// ------------------------------------------------------- pass epilogues

struct PassArgs {
    const uint16_t* U;     // bf16 (MFMA path)
    const uint16_t* T;
    const void* Ug;        // any dtype (vector path)
    const void* Tg;
    const void* W2g;
    const uint16_t* W2;
    const uint16_t* ebf;
    const float* ef;
    int V, r, R, Rpad, P, nrc, rb_per_chunk;
    const int32_t* label;
    const float *lse_d, *lse_t, *S, *rowc;
    float* part[5];        // partials [P][Rpad]
    uint32_t* smask;       // sign(p_d - p_t) as 2 bits per element, [V / 16 + 1][Rpad] (matrix-core path)
    int mask_groups;       // ceil(V / 16): index of the extra (discard) column group
    void* dz;
    int dz_bf16;
    float a_ce, a_tv;
};

constexpr int kPass1 = 1, kPass2 = 2, kPass3 = 3;
// partial values per row and column slice: pass 1 (max, sum) of z_d and of
// z_t; pass 2 sum |p_d - p_t|, sum min(p_d, p_t), sum p_d sign(p_d - p_t)
constexpr int kPartVals[4] = {0, 4, 3, 0};

// Partial values one pass contributes for one row and one column slice.
struct RowPart {
    float v[5];
};

__device__ __forceinline__ RowPart rowpart_empty(int pass) {
    RowPart p;
    if (pass == kPass1) {
        p.v[0] = -INFINITY; p.v[1] = 0.0f; p.v[2] = -INFINITY; p.v[3] = 0.0f; p.v[4] = 0.0f;
    } else {
        p.v[0] = 0.0f; p.v[1] = 0.0f; p.v[2] = 0.0f; p.v[3] = 0.0f; p.v[4] = 0.0f;
    }
    return p;
}

// (max, sum exp(x - max)) pairs merge with a rescale; pass-2 values are
// plain sums.
__device__ __forceinline__ RowPart rowpart_merge(int pass, const RowPart& a, const RowPart& b) {
    RowPart r;
    if (pass == kPass1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float m = fmaxf(a.v[2 * h], b.v[2 * h]);
            const float sa = a.v[2 * h + 1] > 0.0f ? a.v[2 * h + 1] * __builtin_amdgcn_exp2f((a.v[2 * h] - m) * kLog2e) : 0.0f;
            const float sb = b.v[2 * h + 1] > 0.0f ? b.v[2 * h + 1] * __builtin_amdgcn_exp2f((b.v[2 * h] - m) * kLog2e) : 0.0f;
            r.v[2 * h] = m;
            r.v[2 * h + 1] = sa + sb;
        }
        r.v[4] = 0.0f;
    } else {
#pragma unroll
        for (int q = 0; q < 5; ++q) r.v[q] = a.v[q] + b.v[q];
    }
    return r;
}

// rowpart_merge of the partials of lanes l and l ^ X (X = 16 or 32) through
// swap16 / swap32 (the merge is commutative bit for bit)
template <int PASS, int X>
__device__ __forceinline__ RowPart rowpart_merge_xor(const RowPart& a) {
    static_assert(X == 16 || X == 32, "lane distance");
    RowPart x = rowpart_empty(PASS), y = rowpart_empty(PASS);
#pragma unroll
    for (int q = 0; q < kPartVals[PASS]; ++q) {
        const LanePair p = X == 16 ? swap16(__float_as_uint(a.v[q])) : swap32(__float_as_uint(a.v[q]));
        x.v[q] = __uint_as_float(p.a);
        y.v[q] = __uint_as_float(p.b);
    }
    return rowpart_merge(PASS, x, y);
}

__device__ __forceinline__ RowPart rowpart_shfl(const RowPart& a, int mask) {
    RowPart r;
#pragma unroll
    for (int q = 0; q < 5; ++q) r.v[q] = __shfl_xor(a.v[q], mask);
    return r;
}

// Per-row values a pass reads (lse of z_d and z_t in base-2 units, w_k / N,
// the row's S and label), loaded ahead with the row's logits.
struct RowIn {
    float ld, lt, rowc, S;
    int label;
};

__device__ __forceinline__ RowIn row_in(const PassArgs& a, int pass, int row) {
    RowIn in{0.0f, 0.0f, 0.0f, 0.0f, -1};
    if (pass != kPass1) {
        in.ld = a.lse_d[row] * kLog2e;
        in.lt = a.lse_t[row] * kLog2e;
    }
    if (pass == kPass3) {
        in.rowc = a.rowc[row];
        in.S = a.S[row];
        in.label = a.label[row];
    }
    return in;
}

// float pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
    typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
    const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, v);
}

// Per-row work on NC consecutive columns v0 .. v0+NC-1 (zd = U + bias,
// zt = target logits; columns at or past V hold -inf).
// (DZB: pass 3 stores bf16 dZ, else float32.  MASK: pass 2 also returns
// sign(p_d - p_t) of its columns in `bits`, 2 bits per column (bit 2j: p_d >
// p_t, bit 2j + 1: p_d < p_t), and pass 3 takes the signs from `bits`
// instead of recomputing p_t, so it never reads the target logits.)
template <int PASS, int NC, int DZB, bool MASK>
__device__ __forceinline__ RowPart row_epilogue(const PassArgs& a, int row, int v0, const RowIn& ri,
                                                const float (&zd)[NC], const float (&zt)[NC], uint32_t& bits) {
    RowPart p = rowpart_empty(PASS);
    if (PASS == kPass1) {
        float md = zd[0], mt = zt[0];
#pragma unroll
        for (int j = 1; j < NC; ++j) {
            md = fmaxf(md, zd[j]);
            mt = fmaxf(mt, zt[j]);
        }
        float sd = 0.0f, st = 0.0f;
        const float mdl = md * kLog2e, mtl = mt * kLog2e;
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            sd += __builtin_amdgcn_exp2f(fmaf(zd[j], kLog2e, -mdl));
            st += __builtin_amdgcn_exp2f(fmaf(zt[j], kLog2e, -mtl));
        }
        p.v[0] = md; p.v[1] = sd; p.v[2] = mt; p.v[3] = st;
    } else {
        const float ld = ri.ld, lt = ri.lt;
        if (PASS == kPass2) {
            float tv = 0.0f, cm = 0.0f, S = 0.0f;
            uint32_t sb = 0u;
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                const float pd = __builtin_amdgcn_exp2f(fmaf(zd[j], kLog2e, -ld));
                const float pt = __builtin_amdgcn_exp2f(fmaf(zt[j], kLog2e, -lt));
                tv += fabsf(pd - pt);
                cm += fminf(pd, pt);
                S += pd > pt ? pd : (pd < pt ? -pd : 0.0f);
                if (MASK) sb |= (pd > pt ? 1u : 0u) << (2 * j) | (pd < pt ? 2u : 0u) << (2 * j);
            }
            p.v[0] = tv; p.v[1] = cm; p.v[2] = S;
            if (MASK) bits = sb;
        } else {
            const float coef = ri.rowc, S = ri.S;
            const int lab = ri.label;
            const size_t o = static_cast<size_t>(row) * a.V + v0;
            const int nvalid = a.V - v0;
            const bool vec = NC % 8 == 0 && nvalid >= NC && (o % 8) == 0;
            // 8 columns at a time: dZ, then one 16-byte (bf16) or two (f32) stores
#pragma unroll
            for (int h = 0; h < NC; h += 8) {
                float dz[8];
#pragma unroll
                for (int q = 0; q < 8 && h + q < NC; ++q) {
                    const int j = h + q;
                    const float pd = __builtin_amdgcn_exp2f(fmaf(zd[j], kLog2e, -ld));
                    float sg;
                    if (MASK) {
                        sg = static_cast<float>(static_cast<int>((bits >> (2 * j)) & 1u) -
                                                static_cast<int>((bits >> (2 * j + 1)) & 1u));
                    } else {
                        const float pt = __builtin_amdgcn_exp2f(fmaf(zt[j], kLog2e, -lt));
                        sg = pd > pt ? 1.0f : (pd < pt ? -1.0f : 0.0f);
                    }
                    const float onehot = (lab == v0 + j) ? 1.0f : 0.0f;
                    dz[q] = coef * (a.a_ce * (pd - onehot) + a.a_tv * pd * (sg - S));
                }
                if (DZB) {
                    uint16_t* dst = static_cast<uint16_t*>(a.dz) + o + h;
                    if (vec) {
                        u32x4 w;
#pragma unroll
                        for (int q = 0; q < 4; ++q) w[q] = pack2_bf16(dz[2 * q], dz[2 * q + 1]);
                        *reinterpret_cast<u32x4*>(dst) = w;
                    } else {
                        for (int q = 0; q < 8 && h + q < NC && h + q < nvalid; ++q)
                            dst[q] = static_cast<uint16_t>(f32_to_bf16(dz[q]));
                    }
                } else {
                    float* dst = static_cast<float*>(a.dz) + o + h;
                    if (vec) {
                        *reinterpret_cast<f32x4*>(dst) = f32x4{dz[0], dz[1], dz[2], dz[3]};
                        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{dz[4], dz[5], dz[6], dz[7]};
                    } else {
                        for (int q = 0; q < 8 && h + q < NC && h + q < nvalid; ++q) dst[q] = dz[q];
                    }
                }
            }
        }
    }
    return p;
}

// ----------------------------------------------------- pass kernels (MFMA)

// Inputs of one 16-row block for one lane, loaded a block ahead of use so
// that their latency overlaps the previous block's MFMA and epilogue: 16
// columns of U and T, the per-row values the pass needs, and this thread's
// share of the block's 16 E rows (staged into LDS for the whole workgroup).
struct BlockIn {
    u32x4 u0, u1, t0, t1;  // t: target logits (passes 1, 2)
    uint32_t sbits;        // pass 3: the sign bits pass 2 stored
    RowIn ri;
};

// Work item = (column group cg of 256 columns, row chunk rc).  The
// workgroup's 4 waves hold the 4 W2 tiles of cg in registers and walk the
// chunk 16 rows at a time; the 16 E rows of a block are shared through a
// double-buffered LDS area (row stride padded by 16 bytes against bank
// conflicts).  One workgroup barrier per block publishes the next block's E
// rows and, in passes 1 and 2, this block's per-wave row partials, which
// one wave merges (wave rb mod 4 for block rb).  Two workgroups fit per compute unit (at most 256 VGPRs),
// so the waves of one can run while the other's wait on memory.
template <int KC, int PASS, int DZB>
__global__ __launch_bounds__(256, 2) void k_loss_mfma(PassArgs a) {
    constexpr int r = KC * 32;
    constexpr int ldE = r + 8;
    constexpr int kEChunks = 16 * r / 8;  // 16-byte pieces of one block's E rows
    static_assert(kEChunks <= 2 * 256, "E rows of a block: two 16-byte pieces per thread");
    __shared__ __attribute__((aligned(16))) uint16_t Es[2][16 * ldE];
    __shared__ RowPart red[2][kLossWaves][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int items = a.P * a.nrc;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int cg = item % a.P, rc = item / a.P;
        const int vt = cg * kLossColsPerWG + wave * 64;
        const int v0 = vt + 16 * g;
        const bool cols = v0 < a.V, second = v0 + 8 < a.V;
        const bool full = vt + 64 <= a.V;  // wave-uniform: no masked columns
        const int rb0 = rc * a.rb_per_chunk;
        const int rb1 = min(a.Rpad / 16, rb0 + a.rb_per_chunk);
        // All loads below are unconditional, from addresses clamped into
        // the buffers (values of rows past R or columns past V are never
        // used), so the compiler can count them and wait only for the ones
        // a step needs instead of for every load in flight.
        u32x4 estage[2];  // this thread's pieces of the next block's E rows
        auto fetch_e = [&](int rb) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = (threadIdx.x + 256 * h) % kEChunks;  // E rows are padded to Rpad
                estage[h] = *reinterpret_cast<const u32x4*>(a.ebf + static_cast<size_t>(rb * 16) * r + 8 * t);
            }
        };
        const int vc0 = cols ? v0 : 0, vc1 = second ? v0 + 8 : vc0;
        auto fetch = [&](int rb) {
            BlockIn in;
            const int row = rb * 16 + n;  // < Rpad: the per-row arrays are padded
            const size_t ro = static_cast<size_t>(min(row, a.R - 1)) * a.V;
            in.u0 = *reinterpret_cast<const u32x4*>(a.U + ro + vc0);
            in.u1 = *reinterpret_cast<const u32x4*>(a.U + ro + vc1);
            if (PASS != kPass3) {
                in.t0 = *reinterpret_cast<const u32x4*>(a.T + ro + vc0);
                in.t1 = *reinterpret_cast<const u32x4*>(a.T + ro + vc1);
                in.sbits = 0u;
            } else {
                in.t0 = in.t1 = u32x4{0u, 0u, 0u, 0u};
                in.sbits = a.smask[static_cast<size_t>(vc0 >> 4) * a.Rpad + row];
            }
            in.ri = row_in(a, PASS, row);
            return in;
        };
        auto stage = [&](int buf) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int t = threadIdx.x + 256 * h;
                if (t < kEChunks) {
                    const int er = t / (r / 8), ec = t % (r / 8);
                    *reinterpret_cast<u32x4*>(&Es[buf][er * ldE + ec * 8]) = estage[h];
                }
            }
        };
        W2Tile<KC> w2;
        w2.load(a.W2, a.V, vt, g, n);
        fetch_e(rb0);
        BlockIn nxt = fetch(rb0);
        stage(rb0 & 1);
        __syncthreads();
        for (int rb = rb0; rb < rb1; ++rb) {
            const BlockIn cur = nxt;
            if (rb + 1 < rb1) {
                fetch_e(rb + 1);
                nxt = fetch(rb + 1);
            }
            f32x4 acc[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            w2.mul(&Es[rb & 1][n * ldE + 8 * g], acc);
            const int row = rb * 16 + n;
            RowPart p = rowpart_empty(PASS);
            uint32_t bits = cur.sbits;
            if (row < a.R && cols) {
                const uint32_t uw[8] = {cur.u0[0], cur.u0[1], cur.u0[2], cur.u0[3],
                                        cur.u1[0], cur.u1[1], cur.u1[2], cur.u1[3]};
                const uint32_t tw[8] = {cur.t0[0], cur.t0[1], cur.t0[2], cur.t0[3],
                                        cur.t1[0], cur.t1[1], cur.t1[2], cur.t1[3]};
                float zd[16], zt[16];
                if (full) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int j = 4 * q + c;
                            zd[j] = ((j & 1) ? hi_bf16(uw[j >> 1]) : lo_bf16(uw[j >> 1])) + acc[c][q];
                            zt[j] = (j & 1) ? hi_bf16(tw[j >> 1]) : lo_bf16(tw[j >> 1]);
                        }
                } else {
                    const int nvalid = a.V - v0;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
#pragma unroll
                        for (int c = 0; c < 4; ++c) {
                            const int j = 4 * q + c;
                            const bool in = j < nvalid;
                            zd[j] = in ? ((j & 1) ? hi_bf16(uw[j >> 1]) : lo_bf16(uw[j >> 1])) + acc[c][q] : -INFINITY;
                            zt[j] = in ? ((j & 1) ? hi_bf16(tw[j >> 1]) : lo_bf16(tw[j >> 1])) : -INFINITY;
                        }
                }
                p = row_epilogue<PASS, 16, DZB, true>(a, row, v0, cur.ri, zd, zt, bits);
            }
            // unconditional (padding rows and the extra column group
            // absorb the lanes without a row or columns)
            if (PASS == kPass2) a.smask[static_cast<size_t>(cols ? v0 >> 4 : a.mask_groups) * a.Rpad + row] = bits;
            if (PASS != kPass3) {
                p = rowpart_merge_xor<PASS, 16>(p);
                p = rowpart_merge_xor<PASS, 32>(p);
                if (g == 0) red[rb & 1][wave][n] = p;
            }
            if (rb + 1 < rb1) stage((rb + 1) & 1);
            __syncthreads();
            // the 4 waves' partials of this block's 16 rows, merged by one
            // wave (a different one each block, so that no wave falls
            // behind): lane (w, n) takes wave w's partial of row n, two
            // exchange steps merge the 4 in a fixed tree order
            if (PASS != kPass3 && wave == (rb & (kLossWaves - 1))) {
                static_assert(kLossWaves == 4, "one lane per (wave, row)");
                RowPart t = red[rb & 1][g][n];
                t = rowpart_merge_xor<PASS, 16>(t);
                t = rowpart_merge_xor<PASS, 32>(t);
                if (g == 0 && row < a.R) {
                    const size_t o = static_cast<size_t>(cg) * a.Rpad + row;
#pragma unroll
                    for (int q = 0; q < kPartVals[PASS]; ++q) a.part[q][o] = t.v[q];
                }
            }
        }
        __syncthreads();  // Es and red are reused by the next item
    }
}

// --------------------------------------------------- pass kernels (vector)

// Any dtype / rank: thread = 4 consecutive columns, rows of the item's chunk
// one at a time, bias as a float dot product with E.
template <typename T, int PASS, int DZB>
__global__ __launch_bounds__(256) void k_loss_generic(PassArgs a) {
    __shared__ RowPart red[4];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const T* U = static_cast<const T*>(a.Ug);
    const T* Tl = static_cast<const T*>(a.Tg);
    const T* W2 = static_cast<const T*>(a.W2g);
    const int items = a.P * a.nrc;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int cg = item % a.P, rc = item / a.P;
        const int v0 = (cg * static_cast<int>(blockDim.x) + static_cast<int>(threadIdx.x)) * 4;
        const int r0 = rc * a.rb_per_chunk * 16;
        const int r1 = min(a.R, r0 + a.rb_per_chunk * 16);
        for (int row = r0; row < r1; ++row) {
            RowPart p = rowpart_empty(PASS);
            if (v0 < a.V) {
                float zd[4], zt[4];
                const int64_t o = static_cast<int64_t>(row) * a.V + v0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    zd[c] = v0 + c < a.V ? load_f(U, o + c) : -INFINITY;
                    zt[c] = v0 + c < a.V ? load_f(Tl, o + c) : -INFINITY;
                }
                const float* e = a.ef + static_cast<size_t>(row) * a.r;
                for (int j = 0; j < a.r; ++j) {
                    const int64_t wrow = static_cast<int64_t>(j) * a.V + v0;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (v0 + c < a.V) zd[c] = fmaf(e[j], load_f(W2, wrow + c), zd[c]);
                }
                uint32_t bits = 0u;
                p = row_epilogue<PASS, 4, DZB, false>(a, row, v0, row_in(a, PASS, row), zd, zt, bits);
            }
            if (PASS == kPass3) continue;
            for (int o = 32; o > 0; o >>= 1) p = rowpart_merge(PASS, p, rowpart_shfl(p, o));
            if (lane == 0) red[wave] = p;
            __syncthreads();
            if (threadIdx.x == 0) {
                RowPart t = red[0];
                for (int w = 1; w < static_cast<int>(blockDim.x / kWave); ++w) t = rowpart_merge(PASS, t, red[w]);
                const size_t o = static_cast<size_t>(cg) * a.Rpad + row;
                for (int q = 0; q < kPartVals[PASS]; ++q) a.part[q][o] = t.v[q];
            }
            __syncthreads();
        }
    }
}

// ------------------------------------------------------- row reductions

// Merge the P column-group partials of a pass per row.  Workgroup = 16
// rows x 16 slices: thread (slice sl, row) merges groups sl, sl + 16, ...
// (16 consecutive rows per quarter wave: 64-byte reads), then slice 0 merges
// the 16 slice results in slice order through LDS (deterministic).
constexpr int kRowsPerWG = 16, kRowSlices = 16;

template <int PASS>
__global__ __launch_bounds__(256) void k_loss_rows(const PassArgs a, float* __restrict__ out0,
                                                   float* __restrict__ out1, float* __restrict__ out2) {
    __shared__ RowPart sl_part[kRowSlices][kRowsPerWG];
    const int rr = threadIdx.x % kRowsPerWG, sl = threadIdx.x / kRowsPerWG;
    const int row = blockIdx.x * kRowsPerWG + rr;
    RowPart t = rowpart_empty(PASS);
    if (row < a.R) {
        for (int p = sl; p < a.P; p += kRowSlices) {
            RowPart q = rowpart_empty(PASS);
            const size_t o = static_cast<size_t>(p) * a.Rpad + row;
#pragma unroll
            for (int k = 0; k < kPartVals[PASS]; ++k) q.v[k] = a.part[k][o];
            t = rowpart_merge(PASS, t, q);
        }
    }
    sl_part[sl][rr] = t;
    __syncthreads();
    if (sl != 0 || row >= a.R) return;
#pragma unroll 1
    for (int s2 = 1; s2 < kRowSlices; ++s2) t = rowpart_merge(PASS, t, sl_part[s2][rr]);
    if (PASS == kPass1) {
        out0[row] = t.v[0] + logf(t.v[1]);  // lse_d
        out1[row] = t.v[2] + logf(t.v[3]);  // lse_t
    } else {
        out0[row] = t.v[0];  // sum |p_d - p_t|
        out1[row] = t.v[1];  // sum min(p_d, p_t)
        out2[row] = t.v[2];  // sum p_d sign(p_d - p_t)
    }
}

// Thread = row: Eq 8 (c* as sum min(p_d, p_t), equal to 1 - tv/2 for
// normalised p, with the delta-table D7 clamp), Eq 9 and Eq 11 terms, the
// confidence gradient (c* held constant), and w_k/N-weighted loss terms.
__global__ __launch_bounds__(256) void k_loss_finalize(
    const float* __restrict__ lse_d, const float* __restrict__ zlab, const float* __restrict__ tv,
    const float* __restrict__ cmin, const float* __restrict__ alog, const float* __restrict__ rowc,
    int R, float a_conf, float* __restrict__ c_star, float* __restrict__ conf,
    float* __restrict__ dconf, float* __restrict__ tce, float* __restrict__ ttv,
    float* __restrict__ tbce) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= R) return;
    const float a = alog[i];
    const float cs = fminf(1.0f, fmaxf(0.0f, cmin[i]));
    const float c = 1.0f / (1.0f + expf(-a));
    // -(c* log c + (1 - c*) log(1 - c)) = softplus(a) - c* a
    const float softplus = fmaxf(a, 0.0f) + log1pf(expf(-fabsf(a)));
    const float bce = softplus - cs * a;
    const float ce = lse_d[i] - zlab[i];
    const float w = rowc[i];
    const bool ok = !isnan(a);  // invalid token ids make every loss NaN
    c_star[i] = ok ? cs : NAN;
    if (conf) conf[i] = c;
    if (dconf) dconf[i] = ok ? w * a_conf * (c - cs) : NAN;
    tce[i] = ok ? w * ce : NAN;
    ttv[i] = ok ? w * tv[i] : NAN;
    tbce[i] = ok ? w * bce : NAN;
}

// One workgroup: L_ce, L_tv, L_conf (each already carries w_k / N) in a
// fixed order, then L = alpha . (L_ce, L_tv, L_conf).
__global__ __launch_bounds__(256) void k_loss_sum(const float* __restrict__ tce,
                                                  const float* __restrict__ ttv,
                                                  const float* __restrict__ tbce, int R,
                                                  float a_ce, float a_tv, float a_conf,
                                                  float* __restrict__ loss4) {
    __shared__ float red[16];
    float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f;
    for (int i = threadIdx.x; i < R; i += blockDim.x) {
        s0 += tce[i];
        s1 += ttv[i];
        s2 += tbce[i];
    }
    s0 = block_sum(s0, red);
    s1 = block_sum(s1, red);
    s2 = block_sum(s2, red);
    if (threadIdx.x == 0) {
        loss4[0] = a_ce * s0 + a_tv * s1 + a_conf * s2;
        loss4[1] = s0;
        loss4[2] = s1;
        loss4[3] = s2;
    }
}

// ------------------------------------------------------------------ dW2

// dW2[j, v] = sum_i E[i, j] dZ[i, v], a GEMM with M = r, N = V, K = R on
// v_mfma_f32_16x16x32_bf16 (lane (g, n) supplies A[n][8g .. 8g+7] and
// B[8g .. 8g+7][n] and receives D[4g + q][n] in accumulator element q).
// Workgroup = 128 columns of V; wave w owns dW2 rows 64 w .. 64 w + 63 of
// them (4 x 8 tiles, accumulated over all rows of dZ).  K runs in 32-row
// chunks:
//   B (dZ) -- K runs along dZ's strided axis, so each chunk is staged
//     through LDS transposed: thread (row pair p, 8 columns) holds two
//     16-byte row pieces, pairs the rows of each column with v_perm and
//     stores column-major words, which lanes read back as 16-byte operand
//     fragments.  The global loads run kAhead chunks ahead of the LDS
//     stores (a register ring); the LDS tile is double-buffered with one
//     workgroup barrier per chunk.  A float32 dZ is split into bf16 hi + lo
//     planes (two MFMAs per tile), so the product keeps about 16 bits of its
//     mantissa.
//   A (E^T) -- from the chunk-major transposed copy of E (et_index), 16
//     contiguous bytes per lane and tile, loaded two chunks ahead.
constexpr int kDw2Cols = 128;
constexpr int kDw2Threads = 256;
// Word offset of row pair p (of 16) of staged column col (of 128): the
// 4-pair piece q = p / 4 of column tile t = col / 16 occupies a 64-word
// (one bank each) row of its own, in which column col % 16 sits at quad
// (col % 16 + t) % 16.  A ds_read_b128 serves, each cycle, one lane of each
// residue mod 16 (measured on gfx950: lanes 16 apart never share a cycle,
// and the cycle's 16 lanes are not always 16 consecutive ones), so the
// operand reads -- lane (g, n) takes piece g of column 16 t + n -- are
// conflict-free when a lane's bank depends on n alone: here quad (n + t) %
// 16 for every g.  The rotation by t also spreads the staging stores (16
// threads on columns 8 s + c, s = 0..15, times 4 row pairs) over all 64
// banks.
__device__ __forceinline__ int dw2_word(int col, int p) {
    const int t = col >> 4;
    return 64 * (4 * t + (p >> 2)) + 4 * (((col & 15) + t) & 15) + (p & 3);
}
constexpr int kDw2Words = kDw2Cols * 16;

// (float32 dZ: the hi/lo planes need more registers, one workgroup per CU)
template <int DZF32>
__global__ __launch_bounds__(kDw2Threads, DZF32 ? 1 : 2) void k_dw2_mfma(const void* __restrict__ dz,
                                                                         const uint16_t* __restrict__ et, int V,
                                                                         int r, int R, int Rpad,
                                                                         float* __restrict__ dW2) {
    constexpr int kPlanes = DZF32 ? 2 : 1;
    constexpr int kAhead = DZF32 ? 2 : 4;      // register ring depth of the dZ loads (chunks, even)
    constexpr int kLdPerRow = DZF32 ? 2 : 1;   // 16-byte pieces per row and thread
    static_assert(kAhead % 2 == 0, "chunk parity is the unrolled step's parity");
    __shared__ __attribute__((aligned(16))) uint32_t Bs[2][kPlanes][kDw2Words];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 15, g = lane >> 4;
    const int vt = blockIdx.x * kDw2Cols;
    const int j0 = 64 * wave;
    const bool rows_live = j0 < r;
    const int nchunks = Rpad / 32;
    // staging role: row pair p (rows 2p, 2p + 1 of the chunk), columns 8 cg .. 8 cg + 7
    const int sp = threadIdx.x >> 4, scg = threadIdx.x & 15;
    const int scol = vt + 8 * scg;
    const bool scol_ok = scol < V;  // V % 8 == 0: a thread's 8 columns are all in or all out
    u32x4 ring[kAhead][2][kLdPerRow];
    // Loads are unconditional, from addresses clamped into the buffers
    // (zeros are substituted when a chunk is staged), so the compiler can
    // count them and wait only for the chunk being staged.
    auto load_b = [&](int c, u32x4 (&dst)[2][kLdPerRow]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = min(32 * c + 2 * sp + h, R - 1);
            const size_t o = static_cast<size_t>(row) * V + (scol_ok ? scol : 0);
#pragma unroll
            for (int q = 0; q < kLdPerRow; ++q)
                dst[h][q] = DZF32 ? *reinterpret_cast<const u32x4*>(static_cast<const float*>(dz) + o + 4 * q)
                                  : *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(dz) + o);
        }
    };
    auto store_b = [&](const u32x4 (&src)[2][kLdPerRow], int buf, int chunk) {
        // rows past R and columns past V contribute zeros
        const bool ok0 = scol_ok && 32 * chunk + 2 * sp < R, ok1 = scol_ok && 32 * chunk + 2 * sp + 1 < R;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            uint32_t hi, lo = 0u;
            if (DZF32) {
                const float x0 = ok0 ? __uint_as_float(src[0][c >> 2][c & 3]) : 0.0f;
                const float x1 = ok1 ? __uint_as_float(src[1][c >> 2][c & 3]) : 0.0f;
                hi = pack2_bf16(x0, x1);
                lo = pack2_bf16(x0 - lo_bf16(hi), x1 - hi_bf16(hi));
            } else {
                const uint32_t w0 = ok0 ? src[0][0][c >> 1] : 0u, w1 = ok1 ? src[1][0][c >> 1] : 0u;
                hi = __builtin_amdgcn_perm(w1, w0, (c & 1) ? 0x07060302u : 0x05040100u);
            }
            const int at = dw2_word(8 * scg + c, sp);
            Bs[buf][0][at] = hi;
            if (DZF32) Bs[buf][kPlanes - 1][at] = lo;
        }
    };
    // E^T rows past r are never multiplied into a stored row of dW2, and
    // chunks past the end are never used: clamp, load unconditionally
    u32x4 afr[2][4];
    auto load_a = [&](int c, u32x4 (&dst)[4]) {
        const int cc = min(c, nchunks - 1);
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int j = min(j0 + 16 * it + n, r - 1);
            dst[it] = *reinterpret_cast<const u32x4*>(et + et_index(32 * cc + 8 * g, j, r));
        }
    };
    f32x4 acc[4][8];
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) acc[it][jt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // prologue: chunk 0 staged, chunks 1 .. kAhead in the ring, A of chunks 0 and 1
#pragma unroll
    for (int q = 0; q < kAhead; ++q) load_b(q, ring[q]);
    load_a(0, afr[0]);
    load_a(1, afr[1]);
    store_b(ring[0], 0, 0);
    load_b(kAhead, ring[0]);
    __syncthreads();
    // chunk c: B in Bs[c & 1], A in afr[c & 1]; ring slot (c + 1) % kAhead
    // holds chunk c + 1, staged at the end of the step, then refilled with
    // chunk c + 1 + kAhead.  The chunk count is padded to a multiple of
    // kAhead (chunks past the end stage zeros: their rows are past R, and
    // their A operands are clamped), so the unrolled body has no exit: with
    // one, the compiler's count of loads in flight became conservative at the
    // loop head and its waits drained the ring every step.
    const int nchunks_pad = (nchunks + kAhead - 1) / kAhead * kAhead;
    for (int c0 = 0; c0 < nchunks_pad; c0 += kAhead) {
#pragma unroll
        for (int u = 0; u < kAhead; ++u) {
            const int c = c0 + u;
            if (rows_live) {
#pragma unroll
                for (int pl = 0; pl < kPlanes; ++pl)
#pragma unroll
                    for (int jt = 0; jt < 8; ++jt) {
                        const u32x4 bv =
                            *reinterpret_cast<const u32x4*>(&Bs[u & 1][pl][dw2_word(16 * jt + n, 4 * g)]);
                        const bf16x8 bop = __builtin_bit_cast(bf16x8, bv);
#pragma unroll
                        for (int it = 0; it < 4; ++it)
                            acc[it][jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8, afr[u & 1][it]), bop, acc[it][jt], 0, 0, 0);
                    }
            }
            load_a(c + 2, afr[u & 1]);
            const int slot = (u + 1) % kAhead;
            store_b(ring[slot], (u + 1) & 1, c + 1);
            load_b(c + 1 + kAhead, ring[slot]);
            __syncthreads();
        }
    }
    if (!rows_live) return;
    // lane (g, n) of tile (it, jt): dW2 rows j0 + 16 it + 4 g + q, column vt + 16 jt + n
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int jt = 0; jt < 8; ++jt) {
            const int v = vt + 16 * jt + n;
            if (v >= V) continue;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int j = j0 + 16 * it + 4 * g + q;
                if (j < r) dW2[static_cast<size_t>(j) * V + v] = acc[it][jt][q];
            }
        }
}

// Vector dW2: thread = (row j of dW2, column v), plain sum over rows.
template <typename DZ>
__global__ __launch_bounds__(256) void k_dw2_generic(const DZ* __restrict__ dz,
                                                     const float* __restrict__ ef, int V, int r,
                                                     int R, float* __restrict__ dW2) {
    const int v = blockIdx.x * blockDim.x + threadIdx.x;
    const int j = blockIdx.y;
    if (v >= V) return;
    float acc = 0.0f;
    for (int i = 0; i < R; ++i) acc = fmaf(ef[static_cast<size_t>(i) * r + j], load_f(dz, static_cast<int64_t>(i) * V + v), acc);
    dW2[static_cast<size_t>(j) * V + v] = acc;
}

// ---------------------------------------------------------------- launch

template <int PASS, int DZB>
static void launch_pass_t(const LossArgs& la, const LossLayout& L, PassArgs& a, int grid) {
    const int r = la.dims.r;
    if (L.mfma) {
        switch (r / 32) {
            case 1: hipLaunchKernelGGL((k_loss_mfma<1, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            case 2: hipLaunchKernelGGL((k_loss_mfma<2, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            case 3: hipLaunchKernelGGL((k_loss_mfma<3, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            case 4: hipLaunchKernelGGL((k_loss_mfma<4, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            case 5: hipLaunchKernelGGL((k_loss_mfma<5, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            case 6: hipLaunchKernelGGL((k_loss_mfma<6, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            case 7: hipLaunchKernelGGL((k_loss_mfma<7, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
            default: hipLaunchKernelGGL((k_loss_mfma<8, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a); break;
        }
    } else if (la.dims.dtype == DSPARK_BF16) {
        hipLaunchKernelGGL((k_loss_generic<uint16_t, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a);
    } else {
        hipLaunchKernelGGL((k_loss_generic<float, PASS, DZB>), dim3(grid), dim3(256), 0, la.stream, a);
    }
}

// Passes 1 and 2 write no dZ; pass 3 is built for both dZ dtypes.
template <int PASS>
static void launch_pass(const LossArgs& la, const LossLayout& L, PassArgs& a, int grid) {
    if (PASS == kPass3 && a.dz_bf16)
        launch_pass_t<PASS, 1>(la, L, a, grid);
    else
        launch_pass_t<PASS, 0>(la, L, a, grid);
}

template <typename T>
static hipError_t launch_loss_t(const LossArgs& la) {
    const dspark_dims& D = la.dims;
    const LossLayout L = loss_layout(D);
    char* ws = la.ws;
    const int R = L.R;
    auto F = [&](size_t off) { return reinterpret_cast<float*>(ws + off); };

    LossConsts cst{};
    for (int q = 0; q < 3; ++q) cst.alpha[q] = la.alpha[q];
    for (int k = 0; k < D.gamma; ++k) cst.pos_weight[k] = la.pos_weight[k] / static_cast<float>(D.B);

    hipLaunchKernelGGL((k_loss_prep<T>), dim3(L.Rpad), dim3(256), 0, la.stream, la.anchor, la.labels,
                       static_cast<const T*>(la.W1), static_cast<const T*>(la.w_conf),
                       static_cast<const T*>(la.h), static_cast<const T*>(la.U), static_cast<const T*>(la.W2),
                       D.V, D.r, D.d, D.gamma, R, L.Rpad, cst,
                       reinterpret_cast<int32_t*>(ws + L.bad), reinterpret_cast<uint16_t*>(ws + L.ebf),
                       F(L.ef), reinterpret_cast<uint16_t*>(ws + L.et),
                       reinterpret_cast<int32_t*>(ws + L.label), F(L.rowc), F(L.alog), F(L.zlab));

    PassArgs a{};
    a.U = static_cast<const uint16_t*>(la.U);
    a.T = static_cast<const uint16_t*>(la.T_logits);
    a.Ug = la.U;
    a.Tg = la.T_logits;
    a.W2g = la.W2;
    a.W2 = static_cast<const uint16_t*>(la.W2);
    a.ebf = reinterpret_cast<const uint16_t*>(ws + L.ebf);
    a.ef = F(L.ef);
    a.V = D.V; a.r = D.r; a.R = R; a.Rpad = L.Rpad; a.P = L.P; a.nrc = L.nrc; a.rb_per_chunk = L.rb_per_chunk;
    a.label = reinterpret_cast<const int32_t*>(ws + L.label);
    a.lse_d = F(L.lse_d); a.lse_t = F(L.lse_t); a.S = F(L.S); a.rowc = F(L.rowc);
    for (int q = 0; q < 5; ++q) a.part[q] = F(L.part[q]);
    a.smask = reinterpret_cast<uint32_t*>(ws + L.smask);
    a.mask_groups = (D.V + 15) / 16;
    a.dz = la.dlogits;
    a.dz_bf16 = la.dlogits_dtype == DSPARK_BF16;
    a.a_ce = la.alpha[0];
    a.a_tv = la.alpha[1];
    const int grid = std::min(L.P * L.nrc, 2048);
    const int rgrid = (R + 255) / 256;

    hipError_t pe = profile_begin(la.stream);
    if (pe != hipSuccess) return pe;
    launch_pass<kPass1>(la, L, a, grid);
    if ((pe = profile_end(la.stream)) != hipSuccess) return pe;
    const int mgrid = (R + kRowsPerWG - 1) / kRowsPerWG;
    hipLaunchKernelGGL((k_loss_rows<kPass1>), dim3(mgrid), dim3(256), 0, la.stream, a, F(L.lse_d),
                       F(L.lse_t), nullptr);
    if ((pe = profile_begin(la.stream)) != hipSuccess) return pe;
    launch_pass<kPass2>(la, L, a, grid);
    if ((pe = profile_end(la.stream)) != hipSuccess) return pe;
    hipLaunchKernelGGL((k_loss_rows<kPass2>), dim3(mgrid), dim3(256), 0, la.stream, a, F(L.tv),
                       F(L.cmin), F(L.S));
    hipLaunchKernelGGL(k_loss_finalize, dim3(rgrid), dim3(256), 0, la.stream, F(L.lse_d), F(L.zlab),
                       F(L.tv), F(L.cmin), F(L.alog), F(L.rowc), R, la.alpha[2], la.c_star, la.conf,
                       la.dconf_logit, F(L.tce), F(L.ttv), F(L.tbce));
    hipLaunchKernelGGL(k_loss_sum, dim3(1), dim3(256), 0, la.stream, F(L.tce), F(L.ttv), F(L.tbce), R,
                       la.alpha[0], la.alpha[1], la.alpha[2], la.loss4);
    if (la.dlogits) {
        if ((pe = profile_begin(la.stream)) != hipSuccess) return pe;
        launch_pass<kPass3>(la, L, a, grid);
        if ((pe = profile_end(la.stream)) != hipSuccess) return pe;
    }
    if (la.dW2) {
        if ((pe = profile_begin(la.stream)) != hipSuccess) return pe;
        if (L.mfma) {
            const dim3 grid((D.V + kDw2Cols - 1) / kDw2Cols);
            if (a.dz_bf16)
                hipLaunchKernelGGL((k_dw2_mfma<0>), grid, dim3(kDw2Threads), 0, la.stream, la.dlogits,
                                   reinterpret_cast<const uint16_t*>(ws + L.et), D.V, D.r, R, L.Rpad, la.dW2);
            else
                hipLaunchKernelGGL((k_dw2_mfma<1>), grid, dim3(kDw2Threads), 0, la.stream, la.dlogits,
                                   reinterpret_cast<const uint16_t*>(ws + L.et), D.V, D.r, R, L.Rpad, la.dW2);
        } else if (a.dz_bf16) {
            hipLaunchKernelGGL((k_dw2_generic<uint16_t>), dim3((D.V + 255) / 256, D.r), dim3(256), 0,
                               la.stream, static_cast<const uint16_t*>(la.dlogits), F(L.ef), D.V, D.r, R,
                               la.dW2);
        } else {
            hipLaunchKernelGGL((k_dw2_generic<float>), dim3((D.V + 255) / 256, D.r), dim3(256), 0,
                               la.stream, static_cast<const float*>(la.dlogits), F(L.ef), D.V, D.r, R,
                               la.dW2);
        }
        if ((pe = profile_end(la.stream)) != hipSuccess) return pe;
    }
    return hipGetLastError();
}

hipError_t launch_loss(const LossArgs& a) {
    if (a.dims.dtype == DSPARK_BF16) return launch_loss_t<uint16_t>(a);
    return launch_loss_t<float>(a);
}

}  // namespace dspark
