// Device helpers shared by the gfx950 kernels of the DSpark sequential head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dspark {

constexpr int kWave = 64;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <typename T> __device__ __forceinline__ float load_f(const T* p, int64_t i);
template <> __device__ __forceinline__ float load_f<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float load_f<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11): ten rounds, each two 32x32 -> 64-bit products,
// with the key bumped by the Weyl constants between rounds.  The two
// three-way xors of a round are single v_bitop3_b32 instructions (truth
// table 0x96), which gfx950 has and earlier CDNA parts do not.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox4x32_10(u32x4 x, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
        const uint64_t pa = static_cast<uint64_t>(0xD2511F53u) * x[0];
        const uint64_t pc = static_cast<uint64_t>(0xCD9E8D57u) * x[2];
        const uint32_t b = x[1], d = x[3];
        x[0] = xor3(static_cast<uint32_t>(pc >> 32), b, k0);
        x[1] = static_cast<uint32_t>(pc);
        x[2] = xor3(static_cast<uint32_t>(pa >> 32), d, k1);
        x[3] = static_cast<uint32_t>(pa);
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return x;
}

// Standard Gumbel draw from one 32-bit word: u = (2 m + 1) 2^-24 with m the
// top 23 bits (exact in float, never 0 or 1), then g = -ln(-ln u).
// With L = -log2(u):  g = -ln(ln 2) - ln 2 * log2(L).  Both logarithms use
// the hardware log2 (v_log_f32); over all 2^23 possible u it is within 2 ulp
// of log2(u) relative to the result, including u -> 1, so -ln u keeps its
// relative accuracy without a log1p branch.
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegLnLn2 = 0.36651292058166432701f;  // -ln(ln 2)
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ float gumbel_from_word(uint32_t w) {
    const float u = static_cast<float>((w >> 8) | 1u) * 5.9604644775390625e-8f;  // (2m+1) 2^-24
    const float L = -__builtin_amdgcn_logf(u);
    return fmaf(-kLn2, __builtin_amdgcn_logf(L), kNegLnLn2);
}

// The same draw in base-2 units for a Gumbel-max argmax: with z2 = z log2(e)
// the perturbed value (z + g) log2(e) - log2(e) (-ln(ln 2)) equals
// z2 - log2(L), L = -log2(u), a positive multiple of z + g minus a constant,
// so it has the same argmax.  u is built without a conversion: v_alignbit
// puts the top 23 bits of w under the exponent of 1.0, giving
// f = 1 + m 2^-23 in [1, 2), and f - (1 - 2^-24) = (2 m + 1) 2^-24 is exact.
__device__ __forceinline__ float log2_of_neg_log2_uniform(uint32_t w) {
    const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9u));
    const float u = f + -0.99999994039535522461f;  // -(1 - 2^-24)
    return __builtin_amdgcn_logf(-__builtin_amdgcn_logf(u));
}

// ------------------------------------------------------- ordered argmax key
// 64-bit key whose unsigned maximum is the largest value, lowest index on a
// tie: order-preserving bits of the float (with -0 folded onto +0) in the
// high word, the complemented index in the low word.
__device__ __forceinline__ uint64_t argmax_key(float y, uint32_t idx) {
    uint32_t u = __float_as_uint(y + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(0xFFFFFFFFu - idx);
}
__device__ __forceinline__ uint32_t key_index(uint64_t key) {
    return 0xFFFFFFFFu - static_cast<uint32_t>(key);
}
constexpr uint64_t kKeyNone = 0;  // below every real key

// ------------------------------------------------- cross-lane exchanges
// Partner values for butterfly merges without an LDS round trip (the
// generic shuffle compiles to ds_bpermute).  swap16 / swap32 return, in
// every lane, its own 32-bit value and that of lane l ^ 16 / l ^ 32, in an
// order that depends on the lane (v_permlane16_swap / v_permlane32_swap,
// gfx950: each lane pair exchanges the halves); a merge that is
// commutative bit for bit then gives both lanes of a pair the same result
// as merge(own, partner).  dpp_ror8 is the value of lane l ^ 8 (a rotation
// by 8 within each row of 16 lanes), dpp_xor1 / dpp_xor2 that of l ^ 1 /
// l ^ 2, and dpp_half_mirror that of lane 8 r + 7 - (l - 8 r) (each half
// row reversed, so lanes 0..3 and 4..7 of every group of 8 face each
// other).
struct LanePair {
    uint32_t a, b;
};
__device__ __forceinline__ LanePair swap16(uint32_t x) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    return LanePair{static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])};
}
__device__ __forceinline__ LanePair swap32(uint32_t x) {
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return LanePair{static_cast<uint32_t>(r[0]), static_cast<uint32_t>(r[1])};
}
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t x) { return dpp<0xB1>(x); }        // quad_perm [1,0,3,2]
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t x) { return dpp<0x4E>(x); }        // quad_perm [2,3,0,1]
__device__ __forceinline__ uint32_t dpp_ror8(uint32_t x) { return dpp<0x128>(x); }       // row_ror:8
__device__ __forceinline__ uint32_t dpp_half_mirror(uint32_t x) { return dpp<0x141>(x); }  // row_half_mirror

// The larger 64-bit key over each group of 8 consecutive lanes, in every
// lane of the group.
__device__ __forceinline__ uint64_t max_key8(uint64_t key) {
    auto step = [](uint64_t k, uint32_t lo, uint32_t hi) {
        const uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        return o > k ? o : k;
    };
    key = step(key, dpp_xor1(static_cast<uint32_t>(key)), dpp_xor1(static_cast<uint32_t>(key >> 32)));
    key = step(key, dpp_xor2(static_cast<uint32_t>(key)), dpp_xor2(static_cast<uint32_t>(key >> 32)));
    key = step(key, dpp_half_mirror(static_cast<uint32_t>(key)), dpp_half_mirror(static_cast<uint32_t>(key >> 32)));
    return key;
}

// Softmax statistics of a slice: running max m, sum of exp(z - m), plus the
// argmax key of the (perturbed) logits and the tempered logit at that index.
struct Stats {
    float m;
    float s;
    uint64_t key;
    float zx;
};

__device__ __forceinline__ Stats stats_empty() { return Stats{-INFINITY, 0.0f, kKeyNone, 0.0f}; }

__device__ __forceinline__ Stats stats_merge(const Stats& a, const Stats& b) {
    Stats r;
    r.m = fmaxf(a.m, b.m);
    const float sa = (a.s > 0.0f) ? a.s * __expf(a.m - r.m) : 0.0f;
    const float sb = (b.s > 0.0f) ? b.s * __expf(b.m - r.m) : 0.0f;
    r.s = sa + sb;
    const bool take_b = b.key > a.key;
    r.key = take_b ? b.key : a.key;
    r.zx = take_b ? b.zx : a.zx;
    return r;
}

// stats_merge for statistics kept in base-2 units (m and zx multiplied by
// log2(e), s = sum of 2^(z2 - m2)).
__device__ __forceinline__ Stats stats_merge2(const Stats& a, const Stats& b) {
    Stats r;
    r.m = fmaxf(a.m, b.m);
    const float sa = (a.s > 0.0f) ? a.s * __builtin_amdgcn_exp2f(a.m - r.m) : 0.0f;
    const float sb = (b.s > 0.0f) ? b.s * __builtin_amdgcn_exp2f(b.m - r.m) : 0.0f;
    r.s = sa + sb;
    const bool take_b = b.key > a.key;
    r.key = take_b ? b.key : a.key;
    r.zx = take_b ? b.zx : a.zx;
    return r;
}

// stats_merge of the statistics of lanes l and l ^ X (X = 16 or 32) through
// swap16 / swap32; the merge is commutative bit for bit (keys of different
// lanes differ unless both are empty, when zx is 0 on both sides).
template <int X>
__device__ __forceinline__ Stats stats_merge_xor(const Stats& a) {
    static_assert(X == 16 || X == 32, "lane distance");
    const uint32_t w[5] = {__float_as_uint(a.m), __float_as_uint(a.s), static_cast<uint32_t>(a.key),
                           static_cast<uint32_t>(a.key >> 32), __float_as_uint(a.zx)};
    LanePair p[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) p[i] = X == 16 ? swap16(w[i]) : swap32(w[i]);
    const Stats x{__uint_as_float(p[0].a), __uint_as_float(p[1].a), (static_cast<uint64_t>(p[3].a) << 32) | p[2].a,
                  __uint_as_float(p[4].a)};
    const Stats y{__uint_as_float(p[0].b), __uint_as_float(p[1].b), (static_cast<uint64_t>(p[3].b) << 32) | p[2].b,
                  __uint_as_float(p[4].b)};
    return stats_merge(x, y);
}

__device__ __forceinline__ Stats shfl_xor_stats(const Stats& a, int mask) {
    Stats r;
    r.m = __shfl_xor(a.m, mask);
    r.s = __shfl_xor(a.s, mask);
    const uint32_t lo = __shfl_xor(static_cast<uint32_t>(a.key), mask);
    const uint32_t hi = __shfl_xor(static_cast<uint32_t>(a.key >> 32), mask);
    r.key = (static_cast<uint64_t>(hi) << 32) | lo;
    r.zx = __shfl_xor(a.zx, mask);
    return r;
}

__device__ __forceinline__ float sigmoidf_(float a) { return 1.0f / (1.0f + __expf(-a)); }

// Wait until every vector-memory operation this wave has issued -- loads,
// stores and atomics, with or without return -- has completed.  A
// workgroup-scope release fence does not do this on gfx950: the waves of a
// workgroup share one vector L1, so the memory model emits no wait for it
// and the operations may still be in flight.  A hand-off to other
// workgroups through device-scope atomics (an arrival count, a done count)
// must therefore be preceded by this wait in every wave whose earlier
// atomics the other side will read.
__device__ __forceinline__ void wait_vmem_complete() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Block-wide float sum over blockDim.x threads (multiple of 64), fixed order.
__device__ __forceinline__ float block_sum(float v, float* lds /* >= 16 */) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int nw = blockDim.x / kWave;
    __syncthreads();
    if (lane == 0) lds[wave] = v;
    __syncthreads();
    float t = 0.0f;
    for (int i = 0; i < nw; ++i) t += lds[i];
    __syncthreads();
    return t;
}

}  // namespace dspark
