/*
 * CPU reference ("oracle") for the DSpark sequential head.  TEST
 * INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline); the
 * product path never calls it and it shares no code with the HIP library.
 *
 * Everything is computed from the definitions in double precision, one block
 * (sampling) or one row (training) at a time, with plain loops.  Threads only
 * split independent blocks/rows; every sum runs in a fixed order, so results
 * do not depend on the thread count.
 *
 * Equation numbers are those of the DSpark paper (arXiv 2607.05147) as
 * transcribed on the dormouse "DSpark - paper verification" page, section 1.
 */
#include "dspark_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- inputs */

/* Exact widening of one stored element (float32 or bfloat16 bits). */
static double load_elem(const void* p, int dtype, int64_t i)
{
    if (dtype == 0)
        return (double)((const float*)p)[i];
    uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int thread_count(int nthreads)
{
#ifdef _OPENMP
    return nthreads > 0 ? nthreads : omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* ---------------------------------------------------------------- Philox */

/* Philox4x32-10 as published by Salmon et al. (SC'11): ten rounds of two
 * 32x32->64 multiplications; the Weyl key schedule adds the golden-ratio and
 * sqrt(3)-1 constants between rounds. */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t x0 = ctr[0], x1 = ctr[1], x2 = ctr[2], x3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * x0;
        uint64_t p1 = (uint64_t)M1 * x2;
        uint32_t y0 = (uint32_t)(p1 >> 32) ^ x1 ^ k0;
        uint32_t y1 = (uint32_t)p1;
        uint32_t y2 = (uint32_t)(p0 >> 32) ^ x3 ^ k1;
        uint32_t y3 = (uint32_t)p0;
        x0 = y0; x1 = y1; x2 = y2; x3 = y3;
    }
    out[0] = x0; out[1] = x1; out[2] = x2; out[3] = x3;
}

/* Reading (the pages define no random number generator): element v of block
 * b at 0-based step k draws word v mod 4 of Philox4x32-10 with
 * key = (seed low 32 bits, seed high 32 bits) and
 * counter = (v / 4, k, b, offset low 32 bits).
 * The word's top 23 bits give u = (2m + 1) / 2^24, strictly inside (0, 1). */
double oracle_uniform(uint64_t seed, uint64_t offset, int b, int k, int v)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {(uint32_t)(v / 4), (uint32_t)k, (uint32_t)b, (uint32_t)offset};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    uint32_t m = out[v % 4] >> 9;
    return (2.0 * (double)m + 1.0) / 16777216.0;
}

/* Standard Gumbel variate by inversion: g = -ln(-ln u). */
double oracle_gumbel(uint64_t seed, uint64_t offset, int b, int k, int v)
{
    double u = oracle_uniform(seed, offset, b, k, v);
    return -log(-log(u));
}

static double sigmoid(double a) { return 1.0 / (1.0 + exp(-a)); }

/* ln sum_v exp(x_v), shifted by the maximum. */
static double log_sum_exp(const double* x, int V)
{
    double m = x[0];
    for (int v = 1; v < V; ++v)
        if (x[v] > m) m = x[v];
    double s = 0.0;
    for (int v = 0; v < V; ++v)
        s += exp(x[v] - m);
    return m + log(s);
}

/* ------------------------------------------------------------- sampling */

/* Logits of one step (Eq 4 with the Eq 5 or Eq 6 bias) for block b at
 * 0-based step k, given the previous token.  Fills e = W1[prev] and z; for
 * the RNN head also advances the state s from s_{k-1} to s_k. */
static void step_logits(int V, int r, int d, int gamma, int b, int k, int prev,
                        int dtype, int head, const void* U, const void* h,
                        const void* W1, const void* W2, const void* W_rnn,
                        double* z, double* e, double* s, double* coef,
                        double* zeta, double* G)
{
    const int width = 2 * r + d; /* Eq 6: z_k = [s_{k-1}; W1[x_{k-1}]; h_k] */
    const int64_t row = (int64_t)b * gamma + k;

    /* Eq 5: the Markov embedding of the previous token. */
    for (int j = 0; j < r; ++j)
        e[j] = load_elem(W1, dtype, (int64_t)prev * r + j);

    if (head == 1) {
        /* Eq 6: one joint projection of z_k, split by rows into the gate,
         * candidate and output parts (order per delta-table row D8). */
        for (int j = 0; j < r; ++j) zeta[j] = s[j];
        for (int j = 0; j < r; ++j) zeta[r + j] = e[j];
        for (int i = 0; i < d; ++i) zeta[2 * r + i] = load_elem(h, dtype, row * d + i);
        for (int q = 0; q < 3 * r; ++q) {
            double acc = 0.0;
            for (int c = 0; c < width; ++c)
                acc += load_elem(W_rnn, dtype, (int64_t)q * width + c) * zeta[c];
            G[q] = acc;
        }
        for (int j = 0; j < r; ++j) {
            double g = sigmoid(G[j]);
            double cand = tanh(G[r + j]);
            coef[j] = tanh(G[2 * r + j]); /* bias = W2^T tanh(W_o z_k) */
            s[j] = g * s[j] + (1.0 - g) * cand;
        }
    } else {
        for (int j = 0; j < r; ++j) coef[j] = e[j];
    }

    /* Eq 4: z = U_k + B_k, with B_k(v) = sum_j coef_j W2[j, v]. */
    for (int v = 0; v < V; ++v)
        z[v] = load_elem(U, dtype, row * V + v);
    for (int j = 0; j < r; ++j) {
        const double cj = coef[j];
        for (int v = 0; v < V; ++v)
            z[v] += cj * load_elem(W2, dtype, (int64_t)j * V + v);
    }
}

/* Eq 7: c_k = sigmoid(w^T [h_k; W1[x_{k-1}]]), h part first, no bias. */
static double confidence(int r, int d, int64_t row, int dtype, const void* h,
                         const void* w_conf, const double* e)
{
    double a = 0.0;
    for (int i = 0; i < d; ++i)
        a += load_elem(w_conf, dtype, i) * load_elem(h, dtype, row * d + i);
    for (int j = 0; j < r; ++j)
        a += load_elem(w_conf, dtype, d + j) * e[j];
    return sigmoid(a);
}

/* One block of Eq 4 sampling, left to right over the gamma positions. */
static int sample_one_block(int V, int r, int d, int gamma, int b, int dtype, int head,
                            const void* U, const void* h, const int32_t* anchor,
                            const void* W1, const void* W2, const void* w_conf,
                            const void* W_rnn, const float* temperature,
                            uint64_t seed, uint64_t offset, const int32_t* forced_prev,
                            int noise_id,
                            int32_t* tokens, double* logp, double* conf, double* surv,
                            double* gap, int32_t* second,
                            double* z, double* y, double* e, double* s, double* coef,
                            double* zeta, double* G)
{
    double survival = 1.0;       /* empty prefix survives with probability 1 */
    for (int j = 0; j < r; ++j)
        s[j] = 0.0;              /* Eq 6: s_0 = 0 */
    int prev = anchor[b];        /* Eq 4: x_0 is the anchor */
    for (int k = 0; k < gamma; ++k) {
        const int64_t row = (int64_t)b * gamma + k;
        if (k > 0)
            prev = forced_prev ? forced_prev[row - 1] : tokens[row - 1];
        if (prev < 0 || prev >= V)
            return -1;
        step_logits(V, r, d, gamma, b, k, prev, dtype, head, U, h, W1, W2, W_rnn,
                    z, e, s, coef, zeta, G);

        /* The prefix survival is the running product of the c_i. */
        const double c = confidence(r, d, row, dtype, h, w_conf, e);
        survival *= c;

        /* Reading: sample x_k = argmax_v (z_v / T + g_v) (Gumbel-max), greedy
         * argmax z at T = 0; ties go to the lowest index.  logp is taken under
         * softmax(z / T) (softmax(z) when greedy). */
        const double T = (double)temperature[b];
        for (int v = 0; v < V; ++v) {
            const double zs = T > 0.0 ? z[v] / T : z[v];
            z[v] = zs;
            y[v] = T > 0.0 ? zs + oracle_gumbel(seed, offset, noise_id, k, v) : zs;
        }
        int best = 0;
        for (int v = 1; v < V; ++v)
            if (y[v] > y[best]) best = v;
        int runner = -1;
        for (int v = 0; v < V; ++v)
            if (v != best && (runner < 0 || y[v] > y[runner])) runner = v;

        tokens[row] = best;
        logp[row] = z[best] - log_sum_exp(z, V);
        conf[row] = c;
        surv[row] = survival;
        if (gap) gap[row] = runner >= 0 ? y[best] - y[runner] : INFINITY;
        if (second) second[row] = runner;
    }
    return 0;
}

int oracle_block_logprob(int V, int r, int d, int gamma, int B, int dtype, int head,
                         const void* U, const void* h, const int32_t* anchor,
                         const void* W1, const void* W2, const void* W_rnn,
                         const float* temperature, const int32_t* blk,
                         double* out, int nthreads)
{
    if (V < 1 || r < 1 || d < 1 || gamma < 1 || B < 0 || (dtype != 0 && dtype != 1) ||
        (head != 0 && head != 1) || (head == 1 && !W_rnn))
        return -1;
    int failed = 0;
    const int width = 2 * r + d;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double* z = malloc(sizeof(double) * (size_t)V);
        double* e = malloc(sizeof(double) * (size_t)r);
        double* s = malloc(sizeof(double) * (size_t)r);
        double* coef = malloc(sizeof(double) * (size_t)r);
        double* zeta = malloc(sizeof(double) * (size_t)width);
        double* G = malloc(sizeof(double) * (size_t)(3 * r));
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b) {
            double total = 0.0;
            for (int j = 0; j < r; ++j) s[j] = 0.0;
            const double T = (double)temperature[b];
            for (int k = 0; k < gamma && !failed; ++k) {
                const int64_t row = (int64_t)b * gamma + k;
                const int prev = k == 0 ? anchor[b] : blk[row - 1];
                const int x = blk[row];
                if (prev < 0 || prev >= V || x < 0 || x >= V) { failed = 1; break; }
                step_logits(V, r, d, gamma, b, k, prev, dtype, head, U, h, W1, W2, W_rnn,
                            z, e, s, coef, zeta, G);
                if (T > 0.0)
                    for (int v = 0; v < V; ++v) z[v] /= T;
                total += z[x] - log_sum_exp(z, V);
            }
            out[b] = total;
        }
        free(z); free(e); free(s); free(coef); free(zeta); free(G);
    }
    return failed ? -1 : 0;
}

int oracle_draft_block(int V, int r, int d, int gamma, int B, int dtype, int head,
                       const void* U, const void* h, const int32_t* anchor,
                       const void* W1, const void* W2, const void* w_conf,
                       const void* W_rnn, const float* temperature,
                       uint64_t seed, uint64_t offset, const int32_t* forced_prev,
                       const int32_t* block_ids,
                       int32_t* tokens, double* logp, double* conf, double* surv,
                       double* gap, int32_t* second, int nthreads)
{
    if (V < 1 || r < 1 || d < 1 || gamma < 1 || B < 0 || (dtype != 0 && dtype != 1) ||
        (head != 0 && head != 1) || (head == 1 && !W_rnn))
        return -1;
    int failed = 0;
    const int width = 2 * r + d;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double* z = malloc(sizeof(double) * (size_t)V);
        double* y = malloc(sizeof(double) * (size_t)V);
        double* e = malloc(sizeof(double) * (size_t)r);
        double* s = malloc(sizeof(double) * (size_t)r);
        double* coef = malloc(sizeof(double) * (size_t)r);
        double* zeta = malloc(sizeof(double) * (size_t)width);
        double* G = malloc(sizeof(double) * (size_t)(3 * r));
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b)
            failed |= sample_one_block(V, r, d, gamma, b, dtype, head, U, h, anchor, W1, W2,
                                       w_conf, W_rnn, temperature, seed, offset, forced_prev,
                                       block_ids ? block_ids[b] : b, tokens, logp, conf, surv, gap, second,
                                       z, y, e, s, coef, zeta, G) != 0;
        free(z); free(y); free(e); free(s); free(coef); free(zeta); free(G);
    }
    return failed ? -1 : 0;
}

/* ------------------------------------------------------------- training */

/* One teacher-forced row i = n * gamma + k.  Writes the per-row terms and,
 * when dZrow is non-null, dL/dz_d for the row. */
static int loss_one_row(int V, int r, int d, int gamma, int N, int dtype, int64_t i,
                        const void* U, const void* T_logits, const void* h,
                        const int32_t* anchor, const int32_t* labels,
                        const void* W1, const void* W2, const void* w_conf,
                        const double* alpha, const double* pos_weight,
                        double* c_star, double* conf, double* dA,
                        double* ce, double* tv, double* bce, double* dZrow,
                        double* zd, double* zt, double* e)
{
    const int n = (int)(i / gamma), k = (int)(i % gamma);
    /* Teacher forcing: position k is fed the ground-truth previous token,
     * the anchor at the first position (alignment per the delta-table
     * discussion of the off-by-one, "with input_ids" row). */
    const int prev = k == 0 ? anchor[n] : labels[i - 1];
    const int label = labels[i];
    if (prev < 0 || prev >= V || label < 0 || label >= V)
        return -1;
    for (int j = 0; j < r; ++j)
        e[j] = load_elem(W1, dtype, (int64_t)prev * r + j);

    /* Eq 4/5: draft logits z_d = U + W1[prev] W2; target logits as given. */
    for (int v = 0; v < V; ++v) {
        zd[v] = load_elem(U, dtype, i * V + v);
        zt[v] = load_elem(T_logits, dtype, i * V + v);
    }
    for (int j = 0; j < r; ++j) {
        const double ej = e[j];
        for (int v = 0; v < V; ++v)
            zd[v] += ej * load_elem(W2, dtype, (int64_t)j * V + v);
    }
    const double lse_d = log_sum_exp(zd, V);
    const double lse_t = log_sum_exp(zt, V);

    /* Eq 10 term: L1 distance between the two probability vectors (D6). */
    double l1 = 0.0;
    for (int v = 0; v < V; ++v)
        l1 += fabs(exp(zd[v] - lse_d) - exp(zt[v] - lse_t));

    /* Eq 8 with the clamp of delta-table row D7. */
    double cs = 1.0 - 0.5 * l1;
    if (cs < 0.0) cs = 0.0;
    if (cs > 1.0) cs = 1.0;

    /* Eq 9 term: -log p_d(x*), by gather (D5). */
    const double ce_i = lse_d - zd[label];

    /* Eq 7 confidence on the teacher-forced previous token, Eq 11 term. */
    double a = 0.0;
    for (int q = 0; q < d; ++q)
        a += load_elem(w_conf, dtype, q) * load_elem(h, dtype, i * d + q);
    for (int j = 0; j < r; ++j)
        a += load_elem(w_conf, dtype, d + j) * e[j];
    const double c = sigmoid(a);
    const double bce_i = -(cs * log(c) + (1.0 - cs) * log(1.0 - c));

    const double wk = pos_weight[k];
    c_star[0] = cs;
    conf[0] = c;
    ce[0] = ce_i;
    tv[0] = l1;
    bce[0] = bce_i;
    /* Reading: c* is a label (Eq 8), so it is held constant (stop-gradient);
     * the batch reduction is a mean over blocks. */
    dA[0] = wk / N * alpha[2] * (c - cs);

    if (dZrow) {
        /* d/dz_u of sum_v |p_v - q_v| = p_u (s_u - sum_v p_v s_v) with
         * s_v = sign(p_v - q_v) (sign 0 at equality); d/dz_u of -log p_x =
         * p_u - [u = x]. */
        double S = 0.0;
        for (int v = 0; v < V; ++v) {
            const double p = exp(zd[v] - lse_d), q = exp(zt[v] - lse_t);
            const double sg = p > q ? 1.0 : (p < q ? -1.0 : 0.0);
            S += p * sg;
        }
        for (int v = 0; v < V; ++v) {
            const double p = exp(zd[v] - lse_d), q = exp(zt[v] - lse_t);
            const double sg = p > q ? 1.0 : (p < q ? -1.0 : 0.0);
            const double dce = p - (v == label ? 1.0 : 0.0);
            const double dtv = p * (sg - S);
            dZrow[v] = wk / N * (alpha[0] * dce + alpha[1] * dtv);
        }
    }
    return 0;
}

/* cols (optional, n_cols entries in [0, V)): dZ and dW2 are returned only
 * at these vocabulary columns -- dZ as [count, n_cols], dW2 as [r, n_cols]
 * -- so that every row can be checked without holding R x V values.  Each
 * row is still computed in full; only the stored columns change. */
int oracle_block_loss(int V, int r, int d, int gamma, int N, int dtype,
                      const void* U, const void* T_logits, const void* h,
                      const int32_t* anchor, const int32_t* labels,
                      const void* W1, const void* W2, const void* w_conf,
                      const double* alpha, const double* pos_weight,
                      const int64_t* rows, int64_t n_rows,
                      const int32_t* cols, int32_t n_cols,
                      double* loss4, double* c_star, double* conf, double* dA,
                      double* ce, double* tv, double* bce,
                      double* dZ, double* dW2, int nthreads)
{
    if (V < 1 || r < 1 || d < 1 || gamma < 1 || N < 1 || (dtype != 0 && dtype != 1))
        return -1;
    if (cols && n_cols < 1)
        return -1;
    for (int32_t c = 0; cols && c < n_cols; ++c)
        if (cols[c] < 0 || cols[c] >= V) return -1;
    const int64_t R = (int64_t)N * gamma;
    const int64_t count = rows ? n_rows : R;
    const int64_t W = cols ? n_cols : V; /* stored columns per dZ row */
    if (dW2 && rows)
        return -1; /* dW2 needs every row */
    double* dZbuf = dZ;
    if (dW2 && !dZ) {
        dZbuf = malloc(sizeof(double) * (size_t)R * (size_t)W);
        if (!dZbuf) return -1;
    }
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double* zd = malloc(sizeof(double) * (size_t)V);
        double* zt = malloc(sizeof(double) * (size_t)V);
        double* e = malloc(sizeof(double) * (size_t)r);
        double* full = (cols && dZbuf) ? malloc(sizeof(double) * (size_t)V) : NULL;
#pragma omp for schedule(static)
        for (int64_t t = 0; t < count; ++t) {
            const int64_t i = rows ? rows[t] : t;
            if (i < 0 || i >= R) { failed = 1; continue; }
            double* row_out = dZbuf ? (cols ? full : dZbuf + t * W) : NULL;
            failed |= loss_one_row(V, r, d, gamma, N, dtype, i, U, T_logits, h, anchor, labels,
                                   W1, W2, w_conf, alpha, pos_weight,
                                   c_star + t, conf + t, dA + t, ce + t, tv + t, bce + t,
                                   row_out, zd, zt, e) != 0;
            if (cols && dZbuf)
                for (int32_t c = 0; c < n_cols; ++c) dZbuf[t * W + c] = full[cols[c]];
        }
        free(zd); free(zt); free(e); free(full);
    }
    if (failed) {
        if (dZbuf != dZ) free(dZbuf);
        return -1;
    }

    /* Eq 9-12: position-weighted sums over k, mean over the N blocks, in a
     * fixed sequential order. */
    double Lce = 0.0, Ltv = 0.0, Lconf = 0.0;
    for (int64_t t = 0; t < count; ++t) {
        const int64_t i = rows ? rows[t] : t;
        const double wk = pos_weight[i % gamma];
        Lce += wk * ce[t];
        Ltv += wk * tv[t];
        Lconf += wk * bce[t];
    }
    Lce /= N; Ltv /= N; Lconf /= N;
    loss4[0] = alpha[0] * Lce + alpha[1] * Ltv + alpha[2] * Lconf;
    loss4[1] = Lce;
    loss4[2] = Ltv;
    loss4[3] = Lconf;

    if (dW2) {
        /* dW2[j, v] = sum_i W1[prev_i, j] dZ[i, v]: the chain rule through
         * z_d = U + e W2.  Rows of dW2 are split over threads; each sum runs
         * over i in order. */
#pragma omp parallel for schedule(static) num_threads(thread_count(nthreads))
        for (int j = 0; j < r; ++j) {
            double* out = dW2 + (int64_t)j * W;
            for (int64_t v = 0; v < W; ++v) out[v] = 0.0;
            for (int64_t i = 0; i < R; ++i) {
                const int k = (int)(i % gamma), n = (int)(i / gamma);
                const int prev = k == 0 ? anchor[n] : labels[i - 1];
                const double ej = load_elem(W1, dtype, (int64_t)prev * r + j);
                const double* dz = dZbuf + i * W;
                for (int64_t v = 0; v < W; ++v) out[v] += ej * dz[v];
            }
        }
    }
    if (dZbuf != dZ) free(dZbuf);
    return 0;
}

/* ------------------------------------------------------------ backward */

/* The rest of the teacher-forced backward (chain rule through z_d = U +
 * E W2 with E_i = W1[prev_i], Eq 5, and through the Eq 7 logit a_i =
 * w[0:d] . h_i + w[d:d+r] . E_i), given the loss's own gradients dZ =
 * dL/dz_d [R, V] and dA = dL/da [R]:
 *   dE_i[j] = sum_v dZ[i, v] W2[j, v] + dA_i w[d + j]
 *   dW1[x]  = sum over the rows i fed x (prev_i = x) of dE_i, in row order;
 *             rows of W1 no position was fed stay 0
 *   dw[q]   = sum_i dA_i h_i[q]  (q < d),  dw[d + j] = sum_i dA_i E_i[j]
 *   dh_i    = dA_i w[0:d]
 * c* is a label (held constant), so it contributes nothing.  Rows whose
 * previous token is out of range, or whose dA is not finite, are skipped by
 * the sums (their dh is dA_i w). */
int oracle_block_loss_backward(int V, int r, int d, int gamma, int N, int dtype,
                               const void* h, const int32_t* anchor, const int32_t* labels,
                               const void* W1, const void* W2, const void* w_conf,
                               const double* dZ, const double* dA,
                               double* dW1, double* dw, double* dh, int nthreads)
{
    if (V < 1 || r < 1 || d < 1 || gamma < 1 || N < 1 || (dtype != 0 && dtype != 1) || !dA)
        return -1;
    if (dW1 && !dZ)
        return -1; /* dZ is only read for dW1 */
    const int64_t R = (int64_t)N * gamma;
    int32_t* prev = malloc(sizeof(int32_t) * (size_t)R);
    double* dE = dW1 ? malloc(sizeof(double) * (size_t)R * (size_t)r) : NULL;
    if (!prev || (dW1 && !dE)) { free(prev); free(dE); return -1; }
    for (int64_t i = 0; i < R; ++i) {
        const int n = (int)(i / gamma), k = (int)(i % gamma);
        const int x = k == 0 ? anchor[n] : labels[i - 1];
        prev[i] = (x >= 0 && x < V && isfinite(dA[i])) ? x : -1;
    }
#pragma omp parallel for schedule(static) num_threads(thread_count(nthreads))
    for (int64_t i = 0; i < (dW1 ? R : 0); ++i) {
        for (int j = 0; j < r; ++j) {
            double acc = 0.0;
            for (int v = 0; v < V; ++v)
                acc += dZ[i * V + v] * load_elem(W2, dtype, (int64_t)j * V + v);
            dE[i * r + j] = acc + dA[i] * load_elem(w_conf, dtype, d + j);
        }
    }
    if (dW1) {
        for (int64_t t = 0; t < (int64_t)V * r; ++t) dW1[t] = 0.0;
        for (int64_t i = 0; i < R; ++i) {
            if (prev[i] < 0) continue;
            for (int j = 0; j < r; ++j) dW1[(int64_t)prev[i] * r + j] += dE[i * r + j];
        }
    }
    if (dw) {
        for (int q = 0; q < d + r; ++q) dw[q] = 0.0;
        for (int64_t i = 0; i < R; ++i) {
            if (prev[i] < 0) continue;
            for (int q = 0; q < d; ++q) dw[q] += dA[i] * load_elem(h, dtype, i * d + q);
            for (int j = 0; j < r; ++j) dw[d + j] += dA[i] * load_elem(W1, dtype, (int64_t)prev[i] * r + j);
        }
    }
    if (dh) {
        for (int64_t i = 0; i < R; ++i)
            for (int q = 0; q < d; ++q) dh[i * d + q] = dA[i] * load_elem(w_conf, dtype, q);
    }
    free(prev);
    free(dE);
    return 0;
}

/* ----------------------------------------------------------- verification */

/* Reading (the pages fix no random numbers for verification): the uniform
 * of the accept test at 0-based position k of block b is word 0 of
 * Philox4x32-10 at counter (0xFFFFFFFF, k, b, offset low 32 bits), and the
 * Gumbel variate of element v of the final draw (made at 0-based position j)
 * is word v mod 4 at counter (v / 4, 0x80000000 | j, b, offset low 32 bits),
 * both with the sampling key and the same word -> u map.  Neither counter can
 * equal one the drafting noise uses (its first word is v / 4 < 2^30 and its
 * second word a step index below 64). */
static double verify_u(uint64_t seed, uint64_t offset, uint32_t c0, uint32_t c1, int b, int word)
{
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t ctr[4] = {c0, c1, (uint32_t)b, (uint32_t)offset};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return (2.0 * (double)(out[word] >> 9) + 1.0) / 16777216.0;
}

double oracle_verify_uniform(uint64_t seed, uint64_t offset, int b, int k)
{
    return verify_u(seed, offset, 0xFFFFFFFFu, (uint32_t)k, b, 0);
}

double oracle_verify_gumbel(uint64_t seed, uint64_t offset, int b, int j, int v)
{
    double u = verify_u(seed, offset, (uint32_t)(v / 4), 0x80000000u | (uint32_t)j, b, v % 4);
    return -log(-log(u));
}

/* Index of the largest y (lowest index on a tie) and the gap to the runner-up. */
static int argmax_gap(const double* y, int V, double* gap)
{
    int best = -1;
    double b1 = -INFINITY, b2 = -INFINITY;
    for (int v = 0; v < V; ++v) {
        if (y[v] > b1) {
            b2 = b1;
            b1 = y[v];
            best = v;
        } else if (y[v] > b2) {
            b2 = y[v];
        }
    }
    *gap = b1 - b2;
    return best;
}

/* One block: trim, accept/reject left to right, then the final draw. */
static int verify_one_block(int V, int r, int gamma, int b, int dtype, const void* U,
                            const int32_t* anchor, const void* W1, const void* W2,
                            const int32_t* tokens, const double* logp, const double* surv,
                            const float* temperature, const void* T_logits, double tau,
                            uint64_t seed, uint64_t offset, int32_t* keep, int32_t* accept,
                            int32_t* next, double* margin, double* gap, double* accept_prob,
                            double* zt, double* zd, double* y, double* e)
{
    const double T = (double)temperature[b];
    const int greedy = !(T > 0.0);
    /* Static threshold pruning ([bowenzhou] "Results", static-threshold
     * diagnostic; [meridian] section 3: the survival is the product of the
     * c_k): keep the leading positions whose survival is at least tau. */
    int m = 0;
    while (m < gamma && surv[(int64_t)b * gamma + m] >= tau) ++m;
    for (int k = 0; k < gamma; ++k) accept_prob[(int64_t)b * gamma + k] = NAN;
    /* Standard speculative accept/reject ([bowenzhou] "Why DSpark?": the
     * target checks the block and keeps the leading tokens up to the first
     * rejection; [meridian] section 3: c* is the single-step acceptance
     * probability of that rule): accept x_k with probability
     * min(1, p_t(x_k) / p_d(x_k)); greedy accepts x_k iff it is the target's
     * argmax. */
    int n = 0;
    double mg = INFINITY;
    for (; n < m; ++n) {
        const int x = tokens[(int64_t)b * gamma + n];
        if (x < 0 || x >= V) return -1;
        for (int v = 0; v < V; ++v)
            zt[v] = load_elem(T_logits, dtype, ((int64_t)b * (gamma + 1) + n) * V + v);
        int ok;
        if (greedy) {
            double g_unused;
            ok = argmax_gap(zt, V, &g_unused) == x;
            accept_prob[(int64_t)b * gamma + n] = ok ? 1.0 : 0.0;
        } else {
            for (int v = 0; v < V; ++v) zt[v] /= T;
            const double pt = exp(zt[x] - log_sum_exp(zt, V));
            const double pd = exp(logp[(int64_t)b * gamma + n]);
            const double u = oracle_verify_uniform(seed, offset, b, n);
            accept_prob[(int64_t)b * gamma + n] = pt >= pd ? 1.0 : pt / pd;
            ok = u * pd < pt;
            const double rel = fabs(u * pd - pt) / fmax(pt, u * pd);
            if (rel < mg) mg = rel;
        }
        if (!ok) break;
    }
    /* The final draw at 0-based position j = n: after a rejection, from the
     * residual max(0, p_t - p_d) normalised (drawn as the argmax of
     * ln(residual) + Gumbel); after m acceptances, the target's own next
     * token.  Greedy takes the target's argmax either way. */
    const int j = n;
    for (int v = 0; v < V; ++v)
        zt[v] = load_elem(T_logits, dtype, ((int64_t)b * (gamma + 1) + j) * V + v);
    double gp;
    int out;
    if (greedy) {
        out = argmax_gap(zt, V, &gp);
    } else {
        for (int v = 0; v < V; ++v) zt[v] /= T;
        const double lse_t = log_sum_exp(zt, V);
        int residual = n < m;
        if (residual) {
            /* the draft distribution at position j (Eq 4 with the Eq 5 bias
             * of the token before it) */
            const int prev = j == 0 ? anchor[b] : tokens[(int64_t)b * gamma + j - 1];
            if (prev < 0 || prev >= V) return -1;
            for (int q = 0; q < r; ++q) e[q] = load_elem(W1, dtype, (int64_t)prev * r + q);
            for (int v = 0; v < V; ++v) {
                double acc = load_elem(U, dtype, ((int64_t)b * gamma + j) * V + v);
                for (int q = 0; q < r; ++q) acc += e[q] * load_elem(W2, dtype, (int64_t)q * V + v);
                zd[v] = acc / T;
            }
            const double lse_d = log_sum_exp(zd, V);
            int any = 0;
            for (int v = 0; v < V; ++v) {
                const double res = exp(zt[v] - lse_t) - exp(zd[v] - lse_d);
                y[v] = res > 0.0 ? log(res) + oracle_verify_gumbel(seed, offset, b, j, v) : -INFINITY;
                any |= res > 0.0;
            }
            /* Reading: a residual with no positive entry (p_t = p_d exactly)
             * falls back to the target distribution. */
            residual = any;
        }
        if (!residual)
            for (int v = 0; v < V; ++v) y[v] = zt[v] + oracle_verify_gumbel(seed, offset, b, j, v);
        out = argmax_gap(y, V, &gp);
    }
    keep[b] = m;
    accept[b] = n;
    next[b] = out;
    margin[b] = mg;
    gap[b] = gp;
    return 0;
}

int oracle_verify_block(int V, int r, int gamma, int B, int dtype, const void* U,
                        const int32_t* anchor, const void* W1, const void* W2,
                        const int32_t* tokens, const double* logp, const double* surv,
                        const float* temperature, const void* T_logits, double tau,
                        uint64_t seed, uint64_t offset, int32_t* keep, int32_t* accept,
                        int32_t* next, double* margin, double* gap, double* accept_prob,
                        int nthreads)
{
    if (V < 1 || r < 1 || gamma < 1 || B < 0 || (dtype != 0 && dtype != 1))
        return -1;
    int failed = 0;
#pragma omp parallel num_threads(thread_count(nthreads)) reduction(| : failed)
    {
        double* zt = malloc(sizeof(double) * (size_t)V);
        double* zd = malloc(sizeof(double) * (size_t)V);
        double* y = malloc(sizeof(double) * (size_t)V);
        double* e = malloc(sizeof(double) * (size_t)r);
#pragma omp for schedule(static)
        for (int b = 0; b < B; ++b)
            failed |= verify_one_block(V, r, gamma, b, dtype, U, anchor, W1, W2, tokens, logp, surv,
                                       temperature, T_logits, tau, seed, offset, keep, accept, next,
                                       margin, gap, accept_prob, zt, zd, y, e) != 0;
        free(zt); free(zd); free(y); free(e);
    }
    return failed ? -1 : 0;
}
