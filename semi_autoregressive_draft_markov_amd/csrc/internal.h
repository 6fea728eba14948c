// Host-side plumbing shared by the C-ABI front end and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/dspark.h"

namespace dspark {

__host__ __device__ inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Single-launch drafting: each argmax key has this many copies (workgroup
// wg updates copy wg % kDraftKeyCopies), so that no more than 1/8 of the
// grid contends for one address; the grid barrier uses as many arrival
// counters for the same reason.
constexpr int kDraftKeyCopies = 8;
constexpr int kDraftBarWords = 512;

// Draft-call workspace carve-up.  Every region starts 256-byte aligned.
struct DraftLayout {
    int Bpad;          // B rounded up to 16 (MFMA column block)
    int P;             // partial-statistics slots per block row and step
    size_t dead;       // int32 [B]   1 if the block saw a token id out of range
    size_t emb;        // f32 [Bpad, r]  W1[x_{k-1}] of the current step
    size_t coef;       // f32 [Bpad, r]  bias coefficients (emb, or tanh(W_o z))
    size_t ebf;        // u16 [2, Bpad, r] bf16 planes of coef (hi, lo)
    size_t state;      // f32 [Bpad, r]  RNN state s
    size_t state2;     // f32 [Bpad, r]  second RNN state buffer (steps alternate)
    size_t gates;      // f32 [Bpad, 3r] RNN joint projection output
    size_t gh;         // f32 [B, gamma, 3r] h columns of the RNN projection (RNN head only)
    size_t hdot;       // f32 [B, gamma]  h part of the Eq 7 logit, w[0:d] . h_k
    size_t best;       // u64 [gamma, B, copies, 16]  argmax keys, one line each (single-launch path)
    size_t bar;        // u32 [512]  grid barrier: arrival counters and the time-out flag
    size_t flags;      // u64 [max workgroups + 1]  start-barrier flags of the single-launch kernel, then its time-out slot
    size_t qms;        // f32x2 [gamma, B, max workgroups] (max, sum) step partials (single-launch path)
    size_t pm, ps, pkey, pzx;  // partials [B, P]: max, sum, key (u64), z at key
    size_t total;
};

bool mfma_path_ok(const dspark_dims& d);
bool rnn_gate_mfma_ok(const dspark_dims& d);
bool persist_path_ok(const dspark_dims& d);
const char* persist_kernel_name(const dspark_dims& d);  // "" when the path does not fit
const char* draft_kernel_name(const dspark_dims& d);
int draft_persist_max_wg();
hipError_t launch_draft_persistent(const struct DraftArgs& a);
int draft_partials(const dspark_dims& d);
DraftLayout draft_layout(const dspark_dims& d);
// Pipelined per-step streaming kernel (r = 256, B <= 128); npl = coef
// planes.  launch_stream_pipe stores the number of partials per block in *P.
bool stream_pipe_ok(const dspark_dims& d, int npl);
hipError_t launch_stream_pipe(const struct DraftArgs& a, const DraftLayout& L, int k, char* ws, int npl, int* P);
const char* stream_pipe_name(int npl, int Bpad);

// Loss-call workspace carve-up.  Rows i = n * gamma + k, padded to Rpad.
struct LossLayout {
    int R, Rpad;       // rows, rows rounded up to 32
    bool mfma;         // matrix-core path (bf16, r % 32 == 0, r <= 256, V % 8 == 0)
    int P;             // column groups (partial slots per row)
    int nrc;           // row chunks per pass
    int rb_per_chunk;  // 16-row blocks per chunk
    size_t bad;        // int32 [N]  1 if the block saw a token id out of range
    size_t ebf;        // u16 [Rpad, r]  E = W1[prev] rows (MFMA operand)
    size_t ef;         // f32 [Rpad, r]  E rows (vector path, dW2 vector path)
    size_t et;         // u16 [r, Rpad]  E transposed (dW2 operand)
    size_t label;      // i32 [Rpad]  label per row (0 for invalid rows)
    size_t rowc;       // f32 [Rpad]  w_k / N (0 for invalid rows)
    size_t alog;       // f32 [Rpad]  confidence logit (NaN for invalid rows)
    size_t lse_d, lse_t, zlab, tv, cmin, S;  // f32 [Rpad] per-row statistics
    size_t part[5];    // f32 [P, Rpad] per-pass partials
    size_t smask;      // u32 [ceil(V/16), Rpad] sign(p_d - p_t), 2 bits per element (matrix-core path)
    size_t tce, ttv, tbce;  // f32 [Rpad] weighted loss terms
    size_t total;
};
LossLayout loss_layout(const dspark_dims& d);
bool loss_mfma_ok(const dspark_dims& d);

struct LossArgs {
    dspark_dims dims;
    const void *U, *T_logits, *h, *W1, *W2, *w_conf;
    const int32_t *anchor, *labels;
    float alpha[3];
    float pos_weight[64];
    float *loss4, *c_star, *conf, *dconf_logit, *dW2;
    void* dlogits;
    int32_t dlogits_dtype;
    char* ws;
    hipStream_t stream;
};

hipError_t launch_loss(const LossArgs& a);

// Workspace of the backward call past the logits.  Rows i = n * gamma + k.
struct BwdLayout {
    int R;             // rows
    bool mfma;         // matrix-core dE (the loss call's matrix-core shapes)
    int T;             // 256-row tiles of dE
    int S;             // vocabulary slices of dE
    int RS;            // row splits of the dw_conf sums
    size_t bad;        // int32 [N]  1 if a token fed to the block is out of range
    size_t zpage;      // 16 zero bytes, the source of vocabulary entries past V
    size_t prev;       // i32 [R]  token fed to row i, -1 when left out
    size_t srow, sprev, slo, shi;  // i32 [R]  rows sorted by prev: row, prev, segment bounds
    size_t de;         // f32 [R, r]  dL/dE
    size_t seg;        // f32 [R, r]  chunk sums of dE over sorted rows
    size_t part;       // f32 [T * S, 256 * r]  split-vocabulary partial tiles
    size_t dwp;        // f32 [RS, d + r]  dw_conf partial sums
    size_t total;
};
BwdLayout bwd_layout(const dspark_dims& d);
bool bwd_mfma_ok(const dspark_dims& d);

struct BwdArgs {
    dspark_dims dims;
    const void* dz;
    int32_t dz_dtype;
    const float* dA;
    const void *h, *W1, *W2, *w_conf;
    const int32_t *anchor, *labels;
    float *dW1, *dw_conf, *dh;
    char* ws;
    hipStream_t stream;
};

hipError_t launch_loss_backward(const BwdArgs& a);

// Workspace of the verification call.
struct VerifyLayout {
    bool mfma;         // matrix-core draft row (bf16, r % 32 == 0, r <= 256, V % 8 == 0)
    int Bpad;          // B rounded up to 16
    int P;             // 256-column groups of the draft row
    int C;             // 4096-column chunks of the final draw
    int CT;            // 8192-column chunks of the target-row statistics
    size_t bad;        // int32 [B]  1 if the block holds a token id out of range
    size_t lse_t;      // f32 [B, gamma+1]  lse of z_t / T
    size_t amax;       // i32 [B, gamma+1]  argmax of z_t
    size_t tmx, tsm, tkey;  // [B, gamma+1, CT] chunk max / sum / argmax key of the target rows
    size_t mode, jpos; // i32 [B]  final-draw mode and position
    size_t invT;       // f32 [B]  1 / T (1 when greedy)
    size_t ebf;        // u16 [Bpad, r]  E row of the residual position (bf16)
    size_t ef;         // f32 [B, r]     same, fp32
    size_t zd;         // f32 [B, V]  z_d / T at the residual position
    size_t pmx, psm;   // f32 [B, P]  (max, sum) partials of z_d / T
    size_t keys;       // u64 [B, 2]  residual and target argmax keys (atomic maxima)
    size_t done;       // u32 [B]  finished sampling workgroups of each block (the last one picks the token)
    size_t total;
};
VerifyLayout verify_layout(const dspark_dims& d);

struct VerifyArgs {
    dspark_dims dims;
    const void *U, *W1, *W2, *T_logits;
    const int32_t *anchor, *tokens;
    const float *logp, *survival, *temperature;
    float threshold;
    uint64_t seed, offset;
    int32_t *n_keep, *n_accept, *next_token;
    float* accept_prob;
    char* ws;
    hipStream_t stream;
};

hipError_t launch_verify(const VerifyArgs& a);

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

// Built-in device scratch of the allocation-free drafting entry point
// (noalloc.hip): its size, and its device address on the current device
// (looked up on the first call there, then cached).
constexpr size_t kDraftScratchBytes = size_t(32) << 20;
hipError_t draft_scratch(void** ptr);

// Device random numbers of the kernels, one element per thread (noise.hip).
hipError_t launch_noise(uint64_t seed, uint64_t offset, uint32_t ctr1, uint32_t ctr2, uint32_t v0, int n,
                        const uint32_t* words_in, uint32_t* words, float* gumbel, float* gumbel2,
                        hipStream_t stream);

// Host-side post-draft stages (schedule.cpp).
std::vector<double> sts_default_grid();
void sts_calibrate(int N, int gamma, const float* logit, const int32_t* accepted,
                   const std::vector<double>& grid, int bins, float* temperature, float* ece_before,
                   float* ece_after);
double schedule_prefixes(int R, int gamma, const float* survival, const float* sps, int32_t* length);

// Per-thread choice of drafting path (see dspark_set_option).
int draft_path_option();
// DSPARK_OPT_BARRIER_SPIN of the calling thread (0: the default limit)
int barrier_spin_option();

// Per-thread event timing of the dominant kernel (see dspark_profile_*).
bool profiling_enabled();
hipError_t profile_begin(hipStream_t s);  // records a start event when enabled
hipError_t profile_end(hipStream_t s);    // records the matching end event

}  // namespace dspark
