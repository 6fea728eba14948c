/*
 * dspark.h - C ABI of the MI355X (gfx950) DSpark sequential-head library.
 *
 * DSpark drafts a block of gamma tokens after an anchor token x_0.  A parallel
 * backbone gives base logits U_k and hidden states h_k for every position; a
 * light sequential head then samples left to right (DSpark paper, arXiv
 * 2607.05147, as transcribed on the dormouse "DSpark - paper verification"
 * page, section 1):
 *   Eq 4  p_k = softmax(U_k + B_k)
 *   Eq 5  Markov head  B_k = W1[x_{k-1}] W2,  W1 [V x r], W2 [r x V]
 *   Eq 6  RNN head     z_k = [s_{k-1}; W1[x_{k-1}]; h_k], joint projection
 *                      split into gate/candidate/output, s_0 = 0,
 *                      B_k = W2^T tanh(W_o z_k)
 *   Eq 7  confidence   c_k = sigmoid(w^T [h_k; W1[x_{k-1}]])
 * and the prefix survival is the running product of the c_k (Meridian
 * "Phase-Conditioned Speculative Decoding", section 3).  Training is teacher
 * forced (mainlymatmul "DSpark: Wait It's All Autoregressive?", section
 * "Training DSpark") with the Eq 8-12 objective.
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers unless stated, C-contiguous,
 *    row-major, owned by the caller, and must stay alive until the work
 *    enqueued on `hip_stream` has finished.  The library allocates nothing
 *    and keeps no pointer after a call returns.  Weights are never written.
 *  - `hip_stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous: a status of DSPARK_OK means the work was enqueued.
 *  - Floating tensors are float32 or bfloat16 as `dims->dtype` says (the
 *    temperature and all outputs are float32).  Accumulation is float32.
 *  - Results are deterministic: the same inputs, seed and offset give
 *    bitwise-identical outputs (no floating-point atomics).
 *  - A workspace serves one call at a time: calls that may run at the same
 *    time (on different streams) need workspaces of their own.  Entry
 *    points are otherwise reentrant.
 *  - No exceptions cross the ABI.  On failure the status says why and
 *    dspark_last_error() (thread-local) holds a message.  Token ids out of
 *    [0, V) are found on the device: the block's outputs become token -1 and
 *    NaN, and that block's flag in the workspace is raised; read the flags
 *    with dspark_read_device_error().
 */
#ifndef DSPARK_H
#define DSPARK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSPARK_VERSION 1

typedef enum dspark_status {
    DSPARK_OK = 0,
    DSPARK_EINVAL = 1,       /* null required pointer or meaningless size */
    DSPARK_EUNSUPPORTED = 2, /* a shape / dtype / head combination not built */
    DSPARK_EWORKSPACE = 3,   /* workspace smaller than dspark_workspace_size() */
    DSPARK_EDEVICE = 4       /* a HIP runtime call or kernel launch failed */
} dspark_status;

typedef enum dspark_dtype { DSPARK_F32 = 0, DSPARK_BF16 = 1 } dspark_dtype;
typedef enum dspark_head { DSPARK_HEAD_MARKOV = 0, DSPARK_HEAD_RNN = 1 } dspark_head;

/* Problem sizes.  V vocabulary, r Markov rank, d hidden width, gamma block
 * length (also the position-weight decay length, one gamma for both as the
 * dormouse delta table, row D2, requires), B blocks (anchors).
 * Limits: V >= 2, 1 <= r <= 1024, d >= 1, 1 <= gamma <= 64, B >= 1.
 * bf16 data with r a multiple of 32 (r <= 256) and V a multiple of 8 runs
 * on the matrix cores; other shapes take a plain vector path. */
typedef struct dspark_dims {
    int32_t V, r, d, gamma, B;
    int32_t dtype; /* dspark_dtype of U, h, W1, W2, w_conf, W_rnn, T_logits */
    int32_t head;  /* dspark_head */
} dspark_dims;

#define DSPARK_CALL_DRAFT 0
#define DSPARK_CALL_LOSS 1
#define DSPARK_CALL_LOSS_BACKWARD 2
#define DSPARK_CALL_VERIFY 3

/* Bytes of device workspace `which` (DSPARK_CALL_DRAFT, DSPARK_CALL_LOSS,
 * DSPARK_CALL_LOSS_BACKWARD or DSPARK_CALL_VERIFY) needs for `dims`; 0 if
 * dims are invalid or `which` is unknown.  Host function, no device work. */
size_t dspark_workspace_size(const dspark_dims* dims, int which);

/* Semi-autoregressive block drafting: Eq 4 with the Eq 5 (Markov) or Eq 6
 * (RNN) bias, Gumbel-max sampling, Eq 7 confidence and prefix survival.
 *
 * Inputs (device):
 *   U        [B, gamma, V]  base logits U_k of the parallel backbone
 *   h        [B, gamma, d]  hidden states h_k
 *   anchor   [B] int32      x_0, the anchor token of each block
 *   W1       [V, r]         Markov embedding table
 *   W2       [r, V]         logit projection
 *   w_conf   [d + r]        confidence weights, h part first (Eq 7)
 *   W_rnn    [3r, 2r + d]   RNN joint projection, rows (gate, candidate,
 *                           output), columns (s, W1[x], h); NULL for Markov
 *   temperature [B] float   per-block temperature; T_b > 0 samples
 *                           x_k = argmax_v (z_v / T_b + g_v) with standard
 *                           Gumbel noise g; T_b <= 0 is greedy argmax z.
 *                           Ties go to the lowest token id.
 *   seed, offset            Gumbel noise for element v of block b at 0-based
 *                           step k is -ln(-ln u), u = (2 m + 1) / 2^24 with m
 *                           the top 23 bits of word (v mod 4) of
 *                           Philox4x32-10(counter = (v/4, k, b, offset mod
 *                           2^32), key = (seed mod 2^32, seed >> 32)).
 * Outputs (device, [B, gamma]):
 *   tokens   int32  sampled x_k (-1 for a block with a bad token id)
 *   logp     float  log p_k(x_k) under softmax(z / T_b) (softmax(z) when
 *                   greedy); nullable
 *   conf     float  c_k (Eq 7) on the previous token actually drafted
 *   survival float  prod_{i <= k} c_i
 * workspace: device scratch of at least dspark_workspace_size(dims,
 *   DSPARK_CALL_DRAFT) bytes, 256-byte aligned; contents need not be
 *   initialised; afterwards only the per-block error flags at its start
 *   are defined (see dspark_read_device_error).
 * The whole block is always drafted (all gamma positions). */
dspark_status dspark_draft_block(const dspark_dims* dims, const void* U, const void* h,
                                 const int32_t* anchor, const void* W1, const void* W2,
                                 const void* w_conf, const void* W_rnn,
                                 const float* temperature, uint64_t seed, uint64_t offset,
                                 int32_t* tokens, float* logp, float* conf, float* survival,
                                 void* workspace, size_t workspace_bytes, void* hip_stream);

/* dspark_draft_block without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, serving loops or
 * harnesses that forbid allocation).  Same arguments, semantics and results
 * as dspark_draft_block; the workspace is a fixed 32 MiB array in the
 * library's device memory, one per GPU, held until the process ends (its
 * address is looked up on the first call on each device).  The call itself
 * allocates nothing.
 * Limit: DSPARK_EWORKSPACE when dspark_workspace_size(dims,
 * DSPARK_CALL_DRAFT) exceeds 32 MiB (the Qwen3-4B, Qwen3-14B and Gemma4
 * shaped workloads need 1.7, 13.4 and 10.4 MiB).
 * Every call on one GPU shares that GPU's array: calls that may overlap on
 * one GPU (different streams, or different host threads) race and must be
 * serialised by the caller.  The per-block error flags stay in the library's
 * array; a block with a bad token id is still reported as token -1 / NaN. */
dspark_status dspark_draft_block_noalloc(const dspark_dims* dims, const void* U, const void* h,
                                         const int32_t* anchor, const void* W1, const void* W2,
                                         const void* w_conf, const void* W_rnn,
                                         const float* temperature, uint64_t seed, uint64_t offset,
                                         int32_t* tokens, float* logp, float* conf, float* survival,
                                         void* hip_stream);

/* Teacher-forced DSpark objective (Eq 8-12) with dL/dlogits and dW2, Markov
 * head.  dims->B is the number of blocks N; rows i = n * gamma + k.
 * Position k is fed the previous ground-truth token (anchor[n] at k = 0,
 * labels[n, k-1] after) and predicts labels[n, k] (the alignment the dormouse
 * page's off-by-one discussion, section 2, calls correct).
 *
 * Inputs (device):
 *   U        [N, gamma, V]  draft base logits;  z_d = U + W1[prev] W2
 *   T_logits [N, gamma, V]  frozen target logits z_t (read only)
 *   h        [N, gamma, d]; anchor [N] int32; labels [N, gamma] int32
 *   W1, W2, w_conf          as for dspark_draft_block
 *   alpha    HOST float[3]  (alpha_ce, alpha_tv, alpha_conf); NULL means
 *                           (0.1, 0.9, 1.0), the Eq 12 defaults
 *   pos_weight HOST float[gamma]; NULL means w_k = exp(-(k-1)/gamma)
 * Per row: p_d = softmax(z_d), p_t = softmax(z_t), tv = sum |p_d - p_t|,
 *   c* = clamp(1 - tv/2, 0, 1) (Eq 8, clamp per delta-table row D7),
 *   ce = -log p_d(label), c = sigmoid(w^T [h; W1[prev]]),
 *   bce = -(c* log c + (1 - c*) log(1 - c)).
 * Outputs (device):
 *   loss4    float[4]  (L, L_ce, L_tv, L_conf), L_* = (1/N) sum_i w_k term_i,
 *                      L = alpha . (L_ce, L_tv, L_conf)
 *   c_star   [N, gamma] float; conf [N, gamma] float (nullable)
 *   dlogits  [N, gamma, V] dL/dz_d (= dL/dU), float32 or bfloat16 per
 *            dlogits_dtype; nullable.  c* is held constant (it is a label):
 *            dZ = (w_k/N)[alpha_ce (p_d - onehot) + alpha_tv p_d (s - sum p_d s)]
 *            with s = sign(p_d - p_t).
 *   dW2      [r, V] float32, overwritten with W1[prev]^T dZ; nullable
 *   dconf_logit [N, gamma] float dL/d(confidence logit) =
 *            (w_k/N) alpha_conf (c - c*); nullable
 * workspace: at least dspark_workspace_size(dims, DSPARK_CALL_LOSS) bytes. */
dspark_status dspark_block_loss(const dspark_dims* dims, const void* U, const void* T_logits,
                                const void* h, const int32_t* anchor, const int32_t* labels,
                                const void* W1, const void* W2, const void* w_conf,
                                const float* alpha, const float* pos_weight,
                                float* loss4, float* c_star, float* conf,
                                void* dlogits, int32_t dlogits_dtype, float* dW2,
                                float* dconf_logit,
                                void* workspace, size_t workspace_bytes, void* hip_stream);

/* The rest of the backward pass of the teacher-forced objective, Markov
 * head: from dZ = dL/dz_d and dA = dL/d(confidence logit), as
 * dspark_block_loss returns them, to the gradients of the Markov table, the
 * confidence weights and the hidden states.  Training updates the
 * sequential block and the confidence head (dormouse page, section 4, delta
 * table row D16); row i = n * gamma + k is fed prev_i (anchor[n] at k = 0,
 * labels[n, k-1] after), and e_i = W1[prev_i] enters both the bias (Eq 5)
 * and the confidence logit a_i = w . [h_i; e_i] (Eq 7), so
 *   dE_i     = dZ_i W2^T + dA_i w[d : d+r]
 *   dW1[x]   = sum of dE_i over the rows i with prev_i = x (0 for tokens
 *              never fed)
 *   dw_conf  = sum_i dA_i [h_i; e_i]
 *   dh_i     = dA_i w[0 : d]
 * Rows whose prev is outside [0, V) or whose dA is not finite (the loss
 * call returns NaN for a block with a bad token id) are left out of dW1
 * and dw_conf; such a block's flag is raised as for the other calls.
 *
 * Inputs (device): dlogits [N, gamma, V] float32 or bfloat16 per
 *   dlogits_dtype (required when dW1 is wanted, else nullable);
 *   dconf_logit [N, gamma] float (nullable only when dw_conf and dh are
 *   NULL: dW1 then has no confidence term); h, anchor, labels, W1, W2,
 *   w_conf as for dspark_block_loss (h is only read for dw_conf).
 * Outputs (device, float32, each nullable, overwritten):
 *   dW1 [V, r], dw_conf [d + r] (h part first), dh [N, gamma, d].
 * The dW1 sums run in row order per token, the others in fixed row order:
 * results are bitwise reproducible.  bf16 data on the matrix-core shapes
 * (r a multiple of 32 up to 256, V a multiple of 8) multiply dZ by W2^T
 * on the matrix cores (float32 dZ as a hi + lo pair of bf16 values, so dZ
 * is carried to 2^-16 relative); other shapes use the vector units.
 * workspace: at least dspark_workspace_size(dims, DSPARK_CALL_LOSS_BACKWARD)
 *   bytes, 256-byte aligned. */
dspark_status dspark_block_loss_backward(const dspark_dims* dims, const void* dlogits,
                                         int32_t dlogits_dtype, const float* dconf_logit,
                                         const void* h, const int32_t* anchor,
                                         const int32_t* labels, const void* W1, const void* W2,
                                         const void* w_conf, float* dW1, float* dw_conf, float* dh,
                                         void* workspace, size_t workspace_bytes,
                                         void* hip_stream);

/* Verification of drafted blocks against the target, Markov head: prefix
 * trimming by confidence, the standard speculative accept/reject rule and
 * the token emitted after the accepted prefix.  The target checks the block
 * and keeps the leading tokens up to the first rejection, so the output
 * follows the target's distribution (bowenzhou page, "Why DSpark?");
 * c* = 1 - TV(p_d, p_t) is the single-step acceptance probability of that
 * rule (Meridian page, section 3); confidence pruning only cuts a suffix of
 * the proposal (bowenzhou page, "设计" and "Results").  Per block b, with
 * T = temperature[b]:
 *   m = number of leading positions k with survival[b,k] >= threshold;
 *   for k < m, left to right: accept x_k iff u p_d(x_k) < p_t(x_k), where
 *     p_d(x_k) = exp(logp[b,k]), p_t = softmax(T_logits[b,k] / T) and u is
 *     word 0 of Philox4x32-10 at counter (0xFFFFFFFF, k, b, offset mod 2^32)
 *     mapped as for drafting; greedy (T <= 0): accept iff x_k is the argmax
 *     of T_logits[b,k] (lowest id on a tie); stop at the first rejection;
 *   n = number accepted;
 *   next token: after a rejection at position j = n, a draw from the residual
 *     max(0, p_t - p_d) at j, with p_d = softmax((U[b,j] + W1[x_{j-1}] W2) / T)
 *     (x_{-1} = anchor) recomputed here, as argmax_v ln(residual) + g_v;
 *     after m acceptances, argmax_v T_logits[b,m,v] / T + g_v (a residual
 *     with no positive entry also takes this draw); greedy: the argmax of
 *     T_logits[b,j].  g_v is the standard Gumbel draw from word v mod 4 of
 *     Philox4x32-10 at counter (v / 4, 0x80000000 | j, b, offset mod 2^32),
 *     key (seed mod 2^32, seed >> 32).
 * Inputs (device): U [B,gamma,V], anchor [B], W1, W2 as for drafting;
 *   T_logits [B, gamma+1, V] target logits for positions 1..gamma+1 (same
 *   dtype as U); tokens [B,gamma] int32, logp [B,gamma] float, survival
 *   [B,gamma] float as dspark_draft_block returns them (logp required, it
 *   is p_d at the drafted tokens); temperature [B] float.  threshold, seed,
 *   offset are values (a threshold <= 0 keeps every position).
 * Outputs (device): n_keep [B], n_accept [B], next_token [B] int32;
 *   accept_prob [B,gamma] float (nullable): min(1, p_t/p_d) (greedy 0 or 1)
 *   at the tested positions, NaN elsewhere.  A block whose anchor or drafted
 *   tokens hold an id outside [0, V) gets n_keep = n_accept = 0,
 *   next_token = -1 and its flag raised (dspark_read_device_error).
 * workspace: at least dspark_workspace_size(dims, DSPARK_CALL_VERIFY) bytes,
 *   256-byte aligned.  dims->d is not used; dims->head must be Markov. */
dspark_status dspark_verify_block(const dspark_dims* dims, const void* U, const int32_t* anchor,
                                  const void* W1, const void* W2, const void* T_logits,
                                  const int32_t* tokens, const float* logp, const float* survival,
                                  const float* temperature, float threshold, uint64_t seed,
                                  uint64_t offset, int32_t* n_keep, int32_t* n_accept,
                                  int32_t* next_token, float* accept_prob, void* workspace,
                                  size_t workspace_bytes, void* hip_stream);

/* ---- Host-side post-draft stages.  HOST pointers, no device work, no
 * stream; results are deterministic. ---- */

/* Sequential Temperature Scaling of the confidence head (dormouse page,
 * section 1, the post-hoc calibration paragraph; bowenzhou page, "设计"):
 * the survival of a (k+1)-token prefix is prod_{i<=k} c_i, and STS fits one
 * temperature per position, left to right, by a 1-D grid search minimising
 * the expected calibration error of that product with the earlier positions
 * held at their fitted temperatures.  Position k's calibrated confidence is
 * sigmoid(conf_logit / temperature[k]).
 *   conf_logit [N, gamma] raw confidence logits a = w . [h; e] (Eq 7);
 *   accepted [N] int32: accepted prefix length of each block (0..gamma), so
 *     the outcome at position k is accepted > k;
 *   grid [G] candidate temperatures (> 0); NULL uses 201 geometric points
 *     from 0.05 to 20 (the middle one exactly 1); bins: equal-width ECE
 *     bins over [0, 1] (<= 0 means 15);
 *   temperature [gamma] out; ece_before / ece_after [gamma] (nullable): ECE
 *     of the uncalibrated and the calibrated product at each position.
 * The first grid point wins a tie.  EINVAL for a bad size or pointer or a
 * non-positive grid entry. */
dspark_status dspark_sts_calibrate(int32_t N, int32_t gamma, const float* conf_logit,
                                   const int32_t* accepted, const float* grid, int32_t G,
                                   int32_t bins, float* temperature, float* ece_before,
                                   float* ece_after);

/* Hardware-aware prefix scheduler (bowenzhou page, "设计"; Meridian page,
 * section 3): choose each request's verified prefix length l_r in 0..gamma
 * to maximise Theta = (R + sum_r sum_{k<l_r} survival[r,k]) * sps[B] with
 * B = R + sum_r l_r tokens in the verification batch (each request also
 * verifies its bonus position, which always yields one token).  Tokens are
 * added in order of survival (ties: lower request first), each only as the
 * next position of its request, and the best count is kept (the first on a
 * tie); for survivals that do not increase along each request this is the
 * exact optimum.  survival [R, gamma]; sps [T + 1] steps per second at a
 * batch of t tokens, T >= R (gamma + 1); length [R] out; theta (nullable)
 * out.  The engine's measured capacity (the production system estimates it
 * two steps late) is the caller's sps table. */
dspark_status dspark_schedule_prefixes(int32_t R, int32_t gamma, const float* survival,
                                       const float* sps, int32_t T, int32_t* length,
                                       float* theta);

/* The random numbers the kernels draw, for checking them against an
 * independent Philox4x32-10 (Salmon et al., SC'11; the pages name no
 * generator).  For i < n and v = v0 + i (v0 >= 0, n >= 0, v0 + n <= 2^31):
 *   words[i]  = word (v mod 4) of Philox4x32-10 at counter (v / 4, c1, c2,
 *               offset mod 2^32), key (seed mod 2^32, seed >> 32) -- the word
 *               dspark_draft_block uses for element v of block b at 0-based
 *               step k when c1 = k, c2 = b (the verification's final draw at
 *               position j uses c1 = 0x80000000 | j) -- or words_in[i] when
 *               words_in is not NULL;
 *   gumbel[i]      = -ln(-ln u) and
 *   gumbel_log2[i] = log2(-log2 u), both as the kernels evaluate them in
 *               float32, u = (2 m + 1) / 2^24 with m the top 23 bits of the
 *               word (gumbel_log2 is the form the single-launch drafting
 *               kernel subtracts from z log2(e) / T: same argmax).
 * DEVICE pointers; every output is nullable; asynchronous on hip_stream.
 * EINVAL for n < 0, v0 < 0 or a range past 2^31. */
dspark_status dspark_noise(uint64_t seed, uint64_t offset, uint32_t c1, uint32_t c2, int32_t v0, int32_t n,
                           const uint32_t* words_in, uint32_t* words, float* gumbel, float* gumbel_log2,
                           void* hip_stream);

/* Synchronises `hip_stream`, then reads the per-block error flags the last
 * call with these dims left at the start of `workspace`: *code (HOST
 * pointer) = the number of blocks whose outputs are invalid (0 when all
 * are valid): a block that met a token id outside [0, V), or every block
 * when a grid barrier of the single-launch kernel gave up waiting (for
 * ~2^20 polling rounds, ~0.5 s: it assumes one workgroup per compute unit
 * can run at once, which other work on the device can prevent).  Returns
 * DSPARK_EDEVICE, with *code set, when a barrier gave up, or when the
 * synchronisation or the copy fails. */
dspark_status dspark_read_device_error(const dspark_dims* dims, const void* workspace,
                                       int32_t* code, void* hip_stream);

/* Per-thread options.  DSPARK_OPT_DRAFT_PATH selects how dspark_draft_block
 * runs the gamma steps: 0 (default) = the single-launch kernel when the
 * problem fits it (Markov head, bf16, r in {32, 64, 128, 256}, V % 8 == 0,
 * W2 fits in the registers and LDS of the device), else one launch per
 * step; 1 = always one launch per step; 2 = always the single-launch kernel
 * (DSPARK_EUNSUPPORTED when the problem does not fit it).  Both paths give
 * the same results.  Returns DSPARK_EINVAL for an unknown option or value. */
#define DSPARK_OPT_DRAFT_PATH 1
/* DSPARK_OPT_BARRIER_SPIN: polling rounds before a grid barrier of the
 * single-launch kernel gives up (0, the default: 2^20); -1 makes every wait
 * give up at once, which lets a caller test its handling of that failure
 * (the kernel then completes normally with every block invalid). */
#define DSPARK_OPT_BARRIER_SPIN 3
dspark_status dspark_set_option(int option, int value);

/* Kernel timing for measurement.  While enabled on the calling thread, each
 * call records a pair of HIP events on `hip_stream` around every launch of
 * its timed kernels, in this order per call:
 *   dspark_draft_block          the single-launch drafting kernel (one pair),
 *                               or the V-streaming step kernel (one per step);
 *   dspark_block_loss           pass 1, pass 2, pass 3 (when dlogits is
 *                               given) of the V-streaming passes, then the
 *                               dW2 contraction (when dW2 is given);
 *   dspark_block_loss_backward  the matrix-core dZ W2^T kernel;
 *   dspark_verify_block         the draft-row kernel.
 * dspark_profile_read() waits for those events and returns (HOST
 * out-pointers) the summed milliseconds and the number of timed launches
 * since the previous read, then forgets them; dspark_profile_read_each()
 * returns each launch's milliseconds in recording order instead (EINVAL,
 * with *launches set to the count, if `capacity` is too small; nothing is
 * forgotten then).  Events are created on first use and reused; enable = 0
 * stops recording.  Returns DSPARK_EDEVICE if a HIP event call fails. */
dspark_status dspark_profile_enable(int enable);
dspark_status dspark_profile_read(float* kernel_ms, int32_t* launches);
dspark_status dspark_profile_read_each(float* kernel_ms, int32_t capacity, int32_t* launches);

/* Name of the dominant kernel dspark_draft_block runs for `dims` on the
 * current device with this thread's options, as a kernel trace lists it
 * without the namespace (the single-launch variant, or the per-step
 * V-streaming kernel): for measurement reports.  Host function, no device
 * work; "" if dims are invalid.  The string is static. */
const char* dspark_draft_kernel_name(const dspark_dims* dims);

/* Message describing the last failure on this thread ("" if none). */
const char* dspark_last_error(void);

/* DSPARK_VERSION of the built library. */
int dspark_version(void);

#ifdef __cplusplus
}
#endif
#endif /* DSPARK_H */
