/*
 * CPU reference ("oracle") for the DSpark sequential head.  TEST
 * INFRASTRUCTURE ONLY: the tests, the package's smoke check and the
 * benchmark's CPU-baseline leg may call it; the product path never does.
 * It shares no code with the HIP library.
 *
 * Plain, slow, double precision.  Inputs are the exact bytes the GPU sees
 * (float32, or bfloat16 bit patterns), widened exactly to double.
 *
 * Sources (DSpark, arXiv 2607.05147, as transcribed on the pages):
 *  - dormouse "DSpark - paper verification", section 1: Eq 4 (block
 *    factorisation), Eq 5 (Markov head), Eq 6 (RNN head), Eq 7 (confidence
 *    head), Eq 8 (soft acceptance label), Eq 9-12 (losses), position weights.
 *  - same page, section 4 (delta table): D7 clamp of c*, D8 RNN split order
 *    gate/candidate/output, D5 CE by gather, D6 TV on probabilities.
 *  - mainlymatmul "DSpark: Wait It's All Autoregressive?", "Training DSpark":
 *    teacher forcing (ground-truth previous token feeds the Markov head).
 *  - Meridian "Phase-Conditioned Speculative Decoding", section 3: the prefix
 *    survival is the cumulative product of the c_k.
 * Readings where the pages are silent (RNG, tie-break, temperature, batch
 * reduction, stop-gradient through c*) are each stated at their point of
 * use in dspark_oracle.c.
 *
 * Parity status: every function here is pinned by tests/test_oracle_*.py
 * except the points the pages leave open (overall loss scale, the logp
 * convention at T != 1, the concrete Gumbel values), which are "parity
 * unpinned" by the pages and fixed by reading.
 */
#ifndef DSPARK_ORACLE_H
#define DSPARK_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dtype: 0 = float32, 1 = bfloat16 bits (uint16).  head: 0 = Markov, 1 = RNN. */

/* Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11). */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);

/* The uniform and Gumbel draw used for element v of block b at step k
 * (0-based), as defined in dspark_oracle.c. */
double oracle_uniform(uint64_t seed, uint64_t offset, int b, int k, int v);
double oracle_gumbel(uint64_t seed, uint64_t offset, int b, int k, int v);

/* Semi-autoregressive block sampling (Eq 4-7 + prefix survival).
 *   U [B,gamma,V], h [B,gamma,d], anchor [B], W1 [V,r], W2 [r,V],
 *   w_conf [d+r], W_rnn [3r, 2r+d] (head 1 only), temperature [B] (0 = greedy).
 *   forced_prev [B,gamma] nullable: when set, the previous token fed to step
 *   k+1 is forced_prev[b,k] instead of the oracle's own sample (so a parity
 *   test can condition on another implementation's prefix).
 *   block_ids [B] nullable: the block index b that selects the Gumbel noise
 *   of each block (default: its position), so a subset of a larger batch
 *   can be recomputed with its original noise.
 * Outputs (all [B,gamma]): tokens, logp, conf, surv, and for tie analysis gap
 * (largest minus second-largest perturbed logit) and second (its index).
 * Returns 0, or -1 on an out-of-range token id / bad argument. */
int oracle_draft_block(int V, int r, int d, int gamma, int B, int dtype, int head,
                       const void* U, const void* h, const int32_t* anchor,
                       const void* W1, const void* W2, const void* w_conf,
                       const void* W_rnn, const float* temperature,
                       uint64_t seed, uint64_t offset, const int32_t* forced_prev,
                       const int32_t* block_ids,
                       int32_t* tokens, double* logp, double* conf, double* surv,
                       double* gap, int32_t* second, int nthreads);

/* Eq 4 log-probability of given blocks: out[b] = sum_k log p_k(x_k | x_0,
 * x_<k) with p_k = softmax(z_k / T_b) (softmax(z_k) when T_b = 0), where the
 * previous tokens are the anchor then blk[b, 0..k-1].  blk is [B, gamma].
 * Returns 0, or -1 on an out-of-range token id / bad argument. */
int oracle_block_logprob(int V, int r, int d, int gamma, int B, int dtype, int head,
                         const void* U, const void* h, const int32_t* anchor,
                         const void* W1, const void* W2, const void* W_rnn,
                         const float* temperature, const int32_t* blk,
                         double* out, int nthreads);

/* Teacher-forced DSpark loss (Eq 8-12) with dL/dlogits and dW2.
 *   U, T_logits [N,gamma,V]; h [N,gamma,d]; anchor [N]; labels [N,gamma].
 *   alpha [3] = (ce, tv, conf); pos_weight [gamma].
 *   rows: nullable list of n_rows row indices i = n*gamma + k to evaluate;
 *   NULL means all rows.  loss4 and dW2 are only meaningful for all rows.
 * Outputs: loss4 [4] = (L, L_ce, L_tv, L_conf) over the evaluated rows;
 * per evaluated row t (t = position in `rows`, t = i when rows is NULL):
 * c_star, conf, dA (dL/d confidence logit), ce, tv, bce, and dZ [t, V]
 * (nullable); dW2 [r, V] (nullable, all rows only).  With `cols` (n_cols
 * ids in [0, V)), dZ is [t, n_cols] and dW2 [r, n_cols]: the same values at
 * those columns only.  Returns 0 or -1. */
int oracle_block_loss(int V, int r, int d, int gamma, int N, int dtype,
                      const void* U, const void* T_logits, const void* h,
                      const int32_t* anchor, const int32_t* labels,
                      const void* W1, const void* W2, const void* w_conf,
                      const double* alpha, const double* pos_weight,
                      const int64_t* rows, int64_t n_rows,
                      const int32_t* cols, int32_t n_cols,
                      double* loss4, double* c_star, double* conf, double* dA,
                      double* ce, double* tv, double* bce,
                      double* dZ, double* dW2, int nthreads);

/* Rest of the backward of the teacher-forced objective, from the loss's own
 * gradients dZ = dL/dz_d [R, V] and dA = dL/d(confidence logit) [R] (float64,
 * e.g. another implementation's stored outputs widened):
 *   dW1 [V, r]  sum over the rows fed token x of dZ_i W2^T + dA_i w[d:d+r]
 *   dw  [d + r] sum_i dA_i [h_i; W1[prev_i]]
 *   dh  [R, d]  dA_i w[0:d]
 * (each nullable; dZ may be NULL when dW1 is).  Rows with an out-of-range
 * previous token or a non-finite dA are left out of the sums.  Returns 0 or
 * -1. */
int oracle_block_loss_backward(int V, int r, int d, int gamma, int N, int dtype,
                               const void* h, const int32_t* anchor, const int32_t* labels,
                               const void* W1, const void* W2, const void* w_conf,
                               const double* dZ, const double* dA,
                               double* dW1, double* dw, double* dh, int nthreads);

/* Verification of drafted blocks, Markov head: confidence-driven prefix
 * trimming, the standard speculative accept/reject rule, and the final draw
 * (residual after a rejection, the target's next token after full
 * acceptance).  Inputs: U [B,gamma,V], anchor [B], W1, W2 as for sampling;
 * tokens [B,gamma] drafted; logp [B,gamma] their draft log-probabilities
 * (under softmax(z/T)); surv [B,gamma] prefix survival; temperature [B]
 * (<= 0: greedy); T_logits [B,gamma+1,V] target logits for positions
 * 1..gamma+1; tau the survival threshold.  Outputs [B]: keep (m, positions
 * kept), accept (n <= m, positions accepted), next (the token emitted after
 * them); margin (smallest relative distance |u p_d - p_t| / max of the two
 * over the accept tests, inf if none), gap (top-two gap of the final draw);
 * accept_prob [B,gamma] min(1, p_t/p_d) at the tested positions, NaN
 * elsewhere.  Returns 0, or -1 on a bad argument / token id. */
double oracle_verify_uniform(uint64_t seed, uint64_t offset, int b, int k);
double oracle_verify_gumbel(uint64_t seed, uint64_t offset, int b, int j, int v);
int oracle_verify_block(int V, int r, int gamma, int B, int dtype, const void* U,
                        const int32_t* anchor, const void* W1, const void* W2,
                        const int32_t* tokens, const double* logp, const double* surv,
                        const float* temperature, const void* T_logits, double tau,
                        uint64_t seed, uint64_t offset, int32_t* keep, int32_t* accept,
                        int32_t* next, double* margin, double* gap, double* accept_prob,
                        int nthreads);

#ifdef __cplusplus
}
#endif
#endif
