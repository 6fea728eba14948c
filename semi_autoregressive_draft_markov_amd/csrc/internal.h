// Host-side plumbing shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Draft-call workspace carve-up.  Every region starts 256-byte aligned.
struct DraftLayout {
    int Bpad;          // B rounded up to 16 (MFMA column block)
    int P;             // partial-statistics slots per block row and step
    size_t dead;       // int32 [B]   1 if the block saw a token id out of range
    size_t emb;        // f32 [Bpad, r]  W1[x_{k-1}] of the current step
    size_t coef;       // f32 [Bpad, r]  bias coefficients (emb, or tanh(W_o z))
    size_t ebf;        // u16 [2, Bpad, r] bf16 planes of coef (hi, lo)
    size_t state;      // f32 [Bpad, r]  RNN state s
    size_t gates;      // f32 [Bpad, 3r] RNN joint projection output
    size_t hdot;       // f32 [B, gamma]  h part of the Eq 7 logit, w[0:d] . h_k
    size_t pm, ps, pkey, pzx;  // partials [B, P]: max, sum, key (u64), z at key
    size_t total;
};

bool mfma_path_ok(const dspark_dims& d);
int draft_partials(const dspark_dims& d);
DraftLayout draft_layout(const dspark_dims& d);

struct LossLayout {
    size_t bad;        // int32 [N]   1 if the block saw a token id out of range
    size_t total;
};
LossLayout loss_layout(const dspark_dims& d);

struct DraftArgs {
    dspark_dims dims;
    const void *U, *h, *W1, *W2, *w_conf, *W_rnn;
    const int32_t* anchor;
    const float* temperature;
    uint64_t seed, offset;
    int32_t* tokens;
    float *logp, *conf, *survival;
    char* ws;
    hipStream_t stream;
};

// Enqueue the whole draft call.  Returns hipSuccess or the first launch error.
hipError_t launch_draft(const DraftArgs& a);

// Per-thread event timing of the dominant kernel (see dspark_profile_*).
bool profiling_enabled();
hipError_t profile_begin(hipStream_t s);  // records a start event when enabled
hipError_t profile_end(hipStream_t s);    // records the matching end event

}  // namespace dspark
