// W2 tiles as MFMA operands for the DSpark bias contraction z = U + E W2
// (Eq 5 of the DSpark paper as transcribed on the dormouse verification
// page, section 1), shared by the drafting and the training kernels.
//
// W2 is read in its natural [r, V] row-major layout.  A wave owns a 64-column
// tile: lane (g = lane / 16, n = lane % 16) loads rows 32 kc + 8 g + e (e =
// 0..7) at the 4 columns vt + 4n .. vt + 4n + 3 with coalesced 8-byte loads,
// and v_perm_b32 transposes the 8 x 4 block into four operand fragments, one
// per column offset c, each holding the 8 consecutive rows of one column.
// v_mfma_f32_16x16x32_bf16 with A = that fragment (row i of A is column
// vt + 4i + c) and B = 16 rows of E gives, in lane (g, n), the bias of row n
// at columns vt + 16g + 4q + c (q = 0..3 in the accumulator): each lane ends
// up with 16 consecutive columns of one row.
#pragma once

#include "device_common.h"

namespace dspark {

template <int KC>
struct W2Tile {
    uint32_t f[KC][4][4];  // [k chunk][column offset c][packed bf16 pair]

    // vt: first column of the tile; columns at or past V load as zero
    // (V % 8 == 0, so a lane's 4 columns are all in or all out).
    __device__ __forceinline__ void load(const uint16_t* __restrict__ W2, int V, int vt, int g,
                                         int n) {
        const int va = vt + 4 * n;
        const bool ok = va < V;
        // lane base (row 8 g, column va) plus wave-uniform row offsets, so
        // that no per-row address stays live across calls
        const uint16_t* base = W2 + static_cast<size_t>(8 * g) * V + va;
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            uint2 raw[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const size_t j = static_cast<size_t>(kc * 32 + e);
                raw[e] = ok ? *reinterpret_cast<const uint2*>(base + j * V) : make_uint2(0u, 0u);
            }
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                f[kc][0][p] = __builtin_amdgcn_perm(raw[2 * p + 1].x, raw[2 * p].x, 0x05040100u);
                f[kc][1][p] = __builtin_amdgcn_perm(raw[2 * p + 1].x, raw[2 * p].x, 0x07060302u);
                f[kc][2][p] = __builtin_amdgcn_perm(raw[2 * p + 1].y, raw[2 * p].y, 0x05040100u);
                f[kc][3][p] = __builtin_amdgcn_perm(raw[2 * p + 1].y, raw[2 * p].y, 0x07060302u);
            }
        }
    }

    // acc[c][q] += bias of row n at column vt + 16 g + 4 q + c, with erow
    // pointing at this lane's operand row (row n of the 16-row block) plus
    // 8 g elements.
    __device__ __forceinline__ void mul(const uint16_t* erow, f32x4 (&acc)[4]) const {
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
            const u32x4 ev = *reinterpret_cast<const u32x4*>(erow + kc * 32);
            const bf16x8 bop = __builtin_bit_cast(bf16x8, ev);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const u32x4 av = {f[kc][c][0], f[kc][c][1], f[kc][c][2], f[kc][c][3]};
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av), bop,
                                                                 acc[c], 0, 0, 0);
            }
        }
    }
};

// The 16 bf16 values at p (16-byte aligned), widened to float.
__device__ __forceinline__ void load16_bf16(const uint16_t* p, bool second_half, float (&x)[16]) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(p);
    u32x4 b = {0u, 0u, 0u, 0u};
    if (second_half) b = *reinterpret_cast<const u32x4*>(p + 8);
    const uint32_t w[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = (j & 1) ? hi_bf16(w[j >> 1]) : lo_bf16(w[j >> 1]);
}

}  // namespace dspark
