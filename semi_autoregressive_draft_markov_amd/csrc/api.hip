// C ABI of the DSpark sequential-head library: argument checks, workspace
// sizing and dispatch.  Declarations and the contract live in
// include/dspark.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

dspark_status fail(dspark_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
dspark_status fail(dspark_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

dspark_status ok() {
    g_last_error.clear();
    return DSPARK_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by both calls; returns DSPARK_OK or a failure with a message.
dspark_status check_dims(const dspark_dims* d) {
    if (!d) return fail(DSPARK_EINVAL, "dims is NULL");
    if (d->V < 2) return fail(DSPARK_EINVAL, "V = %d, need V >= 2", d->V);
    if (d->r < 1 || d->r > 1024) return fail(DSPARK_EINVAL, "r = %d, need 1 <= r <= 1024", d->r);
    if (d->d < 1) return fail(DSPARK_EINVAL, "d = %d, need d >= 1", d->d);
    if (d->gamma < 1 || d->gamma > 64)
        return fail(DSPARK_EINVAL, "gamma = %d, need 1 <= gamma <= 64", d->gamma);
    if (d->B < 1) return fail(DSPARK_EINVAL, "B = %d, need B >= 1", d->B);
    if (d->dtype != DSPARK_F32 && d->dtype != DSPARK_BF16)
        return fail(DSPARK_EINVAL, "dtype = %d is neither DSPARK_F32 nor DSPARK_BF16", d->dtype);
    if (d->head != DSPARK_HEAD_MARKOV && d->head != DSPARK_HEAD_RNN)
        return fail(DSPARK_EINVAL, "head = %d is neither MARKOV nor RNN", d->head);
    const int64_t rows = static_cast<int64_t>(d->B) * d->gamma;
    if (rows * d->V > (int64_t(1) << 40) || rows * d->d > (int64_t(1) << 40))
        return fail(DSPARK_EUNSUPPORTED, "tensor sizes beyond 2^40 elements are not supported");
    return DSPARK_OK;
}

}  // namespace

namespace dspark {

namespace {
struct Profile {
    bool on = false;
    std::vector<hipEvent_t> pool;  // even index = start, odd = end
    size_t used = 0;               // events recorded since the last read
};
thread_local Profile g_prof;

hipError_t record(hipStream_t s) {
    if (g_prof.used == g_prof.pool.size()) {
        hipEvent_t e;
        hipError_t err = hipEventCreate(&e);
        if (err != hipSuccess) return err;
        g_prof.pool.push_back(e);
    }
    return hipEventRecord(g_prof.pool[g_prof.used++], s);
}
}  // namespace

thread_local int g_draft_path = 0;
int draft_path_option() { return g_draft_path; }
thread_local int g_barrier_spin = 0;
int barrier_spin_option() { return g_barrier_spin; }

bool profiling_enabled() { return g_prof.on; }
hipError_t profile_begin(hipStream_t s) { return g_prof.on ? record(s) : hipSuccess; }
hipError_t profile_end(hipStream_t s) { return g_prof.on ? record(s) : hipSuccess; }

}  // namespace dspark

extern "C" {

size_t dspark_workspace_size(const dspark_dims* dims, int which) {
    if (check_dims(dims) != DSPARK_OK) return 0;
    if (which == DSPARK_CALL_DRAFT) return dspark::draft_layout(*dims).total;
    if (which == DSPARK_CALL_LOSS) return dspark::loss_layout(*dims).total;
    if (which == DSPARK_CALL_LOSS_BACKWARD) return dspark::bwd_layout(*dims).total;
    if (which == DSPARK_CALL_VERIFY) return dspark::verify_layout(*dims).total;
    return 0;
}

dspark_status dspark_draft_block(const dspark_dims* dims, const void* U, const void* h,
                                 const int32_t* anchor, const void* W1, const void* W2,
                                 const void* w_conf, const void* W_rnn,
                                 const float* temperature, uint64_t seed, uint64_t offset,
                                 int32_t* tokens, float* logp, float* conf, float* survival,
                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
    dspark_status s = check_dims(dims);
    if (s != DSPARK_OK) return s;
    const char* missing = !U ? "U" : !h ? "h" : !anchor ? "anchor" : !W1 ? "W1" : !W2 ? "W2"
                        : !w_conf ? "w_conf" : !temperature ? "temperature" : !tokens ? "tokens"
                        : !conf ? "conf" : !survival ? "survival" : !workspace ? "workspace"
                        : (dims->head == DSPARK_HEAD_RNN && !W_rnn) ? "W_rnn" : nullptr;
    if (missing) return fail(DSPARK_EINVAL, "required pointer %s is NULL", missing);
    if (!aligned(workspace, 256)) return fail(DSPARK_EINVAL, "workspace is not 256-byte aligned");
    const size_t need = dspark::draft_layout(*dims).total;
    if (workspace_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, need);
    dspark_dims d = *dims;
    const size_t esz = d.dtype == DSPARK_BF16 ? 2 : 4;
    if (!aligned(U, esz) || !aligned(h, esz) || !aligned(W1, esz) || !aligned(W2, esz) ||
        !aligned(w_conf, esz) || (W_rnn && !aligned(W_rnn, esz)))
        return fail(DSPARK_EINVAL, "a tensor is not aligned to its element size");
    if (dspark::mfma_path_ok(d) && (!aligned(U, 16) || !aligned(W2, 16)))
        return fail(DSPARK_EUNSUPPORTED, "bf16 U and W2 must be 16-byte aligned");

    dspark::DraftArgs a{};
    a.dims = d;
    a.U = U; a.h = h; a.W1 = W1; a.W2 = W2; a.w_conf = w_conf; a.W_rnn = W_rnn;
    a.anchor = anchor; a.temperature = temperature; a.seed = seed; a.offset = offset;
    a.tokens = tokens; a.logp = logp; a.conf = conf; a.survival = survival;
    a.ws = static_cast<char*>(workspace);
    a.stream = static_cast<hipStream_t>(hip_stream);
    const hipError_t e = dspark::launch_draft(a);
    if (e == hipErrorNotSupported)
        return fail(DSPARK_EUNSUPPORTED, "the single-launch path does not fit this problem on this device");
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

dspark_status dspark_draft_block_noalloc(const dspark_dims* dims, const void* U, const void* h,
                                         const int32_t* anchor, const void* W1, const void* W2,
                                         const void* w_conf, const void* W_rnn,
                                         const float* temperature, uint64_t seed, uint64_t offset,
                                         int32_t* tokens, float* logp, float* conf, float* survival,
                                         void* hip_stream) {
    dspark_status s = check_dims(dims);
    if (s != DSPARK_OK) return s;
    const size_t need = dspark::draft_layout(*dims).total;
    if (need > dspark::kDraftScratchBytes)
        return fail(DSPARK_EWORKSPACE,
                    "this problem needs %zu bytes of scratch; the built-in scratch holds %zu "
                    "(use dspark_draft_block with a workspace)",
                    need, dspark::kDraftScratchBytes);
    void* ws = nullptr;
    const hipError_t e = dspark::draft_scratch(&ws);
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "scratch lookup failed: %s", hipGetErrorString(e));
    return dspark_draft_block(dims, U, h, anchor, W1, W2, w_conf, W_rnn, temperature, seed, offset, tokens, logp,
                              conf, survival, ws, dspark::kDraftScratchBytes, hip_stream);
}

dspark_status dspark_block_loss(const dspark_dims* dims, const void* U, const void* T_logits,
                                const void* h, const int32_t* anchor, const int32_t* labels,
                                const void* W1, const void* W2, const void* w_conf,
                                const float* alpha, const float* pos_weight,
                                float* loss4, float* c_star, float* conf,
                                void* dlogits, int32_t dlogits_dtype, float* dW2,
                                float* dconf_logit,
                                void* workspace, size_t workspace_bytes, void* hip_stream) {
    dspark_status s = check_dims(dims);
    if (s != DSPARK_OK) return s;
    if (dims->head != DSPARK_HEAD_MARKOV)
        return fail(DSPARK_EUNSUPPORTED, "the training objective is built for the Markov head only");
    const char* missing = !U ? "U" : !T_logits ? "T_logits" : !h ? "h" : !anchor ? "anchor"
                        : !labels ? "labels" : !W1 ? "W1" : !W2 ? "W2" : !w_conf ? "w_conf"
                        : !loss4 ? "loss4" : !c_star ? "c_star" : !workspace ? "workspace" : nullptr;
    if (missing) return fail(DSPARK_EINVAL, "required pointer %s is NULL", missing);
    if (dW2 && !dlogits) return fail(DSPARK_EINVAL, "dW2 is computed from dlogits: pass dlogits too");
    if (dlogits && dlogits_dtype != DSPARK_F32 && dlogits_dtype != DSPARK_BF16)
        return fail(DSPARK_EINVAL, "dlogits_dtype = %d is neither DSPARK_F32 nor DSPARK_BF16", dlogits_dtype);
    if (!aligned(workspace, 256)) return fail(DSPARK_EINVAL, "workspace is not 256-byte aligned");
    const size_t need = dspark::loss_layout(*dims).total;
    if (workspace_bytes < need)
        return fail(DSPARK_EWORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, need);
    const size_t esz = dims->dtype == DSPARK_BF16 ? 2 : 4;
    if (!aligned(U, esz) || !aligned(T_logits, esz) || !aligned(h, esz) || !aligned(W1, esz) ||
        !aligned(W2, esz) || !aligned(w_conf, esz) || (dlogits && !aligned(dlogits, 4)) ||
        (dW2 && !aligned(dW2, 4)))
        return fail(DSPARK_EINVAL, "a tensor is not aligned to its element size");
    if (dspark::loss_mfma_ok(*dims) &&
        (!aligned(U, 16) || !aligned(T_logits, 16) || !aligned(W2, 16) ||
         (dlogits && !aligned(dlogits, 16)) || (dW2 && !aligned(dW2, 16))))
        return fail(DSPARK_EUNSUPPORTED, "bf16 U, T_logits, W2, dlogits and dW2 must be 16-byte aligned");

    dspark::LossArgs a{};
    a.dims = *dims;
    a.U = U; a.T_logits = T_logits; a.h = h; a.W1 = W1; a.W2 = W2; a.w_conf = w_conf;
    a.anchor = anchor; a.labels = labels;
    const float defaults[3] = {0.1f, 0.9f, 1.0f};  // Eq 12
    for (int q = 0; q < 3; ++q) a.alpha[q] = alpha ? alpha[q] : defaults[q];
    for (int k = 0; k < dims->gamma; ++k)
        a.pos_weight[k] = pos_weight ? pos_weight[k]
                                     : static_cast<float>(exp(-static_cast<double>(k) / dims->gamma));
    a.loss4 = loss4; a.c_star = c_star; a.conf = conf; a.dconf_logit = dconf_logit; a.dW2 = dW2;
    a.dlogits = dlogits; a.dlogits_dtype = dlogits_dtype;
    a.ws = static_cast<char*>(workspace);
    a.stream = static_cast<hipStream_t>(hip_stream);
    const hipError_t e = dspark::launch_loss(a);
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

dspark_status dspark_block_loss_backward(const dspark_dims* dims, const void* dlogits,
                                         int32_t dlogits_dtype, const float* dconf_logit,
                                         const void* h, const int32_t* anchor,
                                         const int32_t* labels, const void* W1, const void* W2,
                                         const void* w_conf, float* dW1, float* dw_conf, float* dh,
                                         void* workspace, size_t workspace_bytes,
                                         void* hip_stream) {
    dspark_status s = check_dims(dims);
    if (s != DSPARK_OK) return s;
    if (dims->head != DSPARK_HEAD_MARKOV)
        return fail(DSPARK_EUNSUPPORTED, "the training objective is built for the Markov head only");
    const char* missing = !anchor ? "anchor" : !labels ? "labels" : !W1 ? "W1" : !W2 ? "W2"
                        : !w_conf ? "w_conf" : !workspace ? "workspace"
                        : (dW1 && !dlogits) ? "dlogits (needed for dW1)"
                        : ((dw_conf || dh) && !dconf_logit) ? "dconf_logit (needed for dw_conf and dh)"
                        : (dw_conf && !h) ? "h (needed for dw_conf)" : nullptr;
    if (missing) return fail(DSPARK_EINVAL, "required pointer %s is NULL", missing);
    if (dlogits && dlogits_dtype != DSPARK_F32 && dlogits_dtype != DSPARK_BF16)
        return fail(DSPARK_EINVAL, "dlogits_dtype = %d is neither DSPARK_F32 nor DSPARK_BF16", dlogits_dtype);
    if (!aligned(workspace, 256)) return fail(DSPARK_EINVAL, "workspace is not 256-byte aligned");
    const dspark::BwdLayout L = dspark::bwd_layout(*dims);
    if (workspace_bytes < L.total)
        return fail(DSPARK_EWORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, L.total);
    const size_t esz = dims->dtype == DSPARK_BF16 ? 2 : 4;
    const size_t dzsz = dlogits_dtype == DSPARK_BF16 ? 2 : 4;
    if ((h && !aligned(h, esz)) || !aligned(W1, esz) || !aligned(W2, esz) || !aligned(w_conf, esz) ||
        (dlogits && !aligned(dlogits, dzsz)) || (dconf_logit && !aligned(dconf_logit, 4)) ||
        (dW1 && !aligned(dW1, 4)) || (dw_conf && !aligned(dw_conf, 4)) || (dh && !aligned(dh, 4)))
        return fail(DSPARK_EINVAL, "a tensor is not aligned to its element size");
    if (L.mfma && dW1 && (!aligned(W2, 16) || !aligned(dlogits, 16)))
        return fail(DSPARK_EUNSUPPORTED, "bf16 W2 and dlogits must be 16-byte aligned");

    dspark::BwdArgs a{};
    a.dims = *dims;
    a.dz = dlogits; a.dz_dtype = dlogits_dtype; a.dA = dconf_logit;
    a.h = h; a.W1 = W1; a.W2 = W2; a.w_conf = w_conf; a.anchor = anchor; a.labels = labels;
    a.dW1 = dW1; a.dw_conf = dw_conf; a.dh = dh;
    a.ws = static_cast<char*>(workspace);
    a.stream = static_cast<hipStream_t>(hip_stream);
    const hipError_t e = dspark::launch_loss_backward(a);
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

dspark_status dspark_verify_block(const dspark_dims* dims, const void* U, const int32_t* anchor,
                                  const void* W1, const void* W2, const void* T_logits,
                                  const int32_t* tokens, const float* logp, const float* survival,
                                  const float* temperature, float threshold, uint64_t seed,
                                  uint64_t offset, int32_t* n_keep, int32_t* n_accept,
                                  int32_t* next_token, float* accept_prob, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
    dspark_status s = check_dims(dims);
    if (s != DSPARK_OK) return s;
    if (dims->head != DSPARK_HEAD_MARKOV)
        return fail(DSPARK_EUNSUPPORTED, "verification is built for the Markov head only");
    const char* missing = !U ? "U" : !anchor ? "anchor" : !W1 ? "W1" : !W2 ? "W2"
                        : !T_logits ? "T_logits" : !tokens ? "tokens" : !logp ? "logp"
                        : !survival ? "survival" : !temperature ? "temperature"
                        : !n_keep ? "n_keep" : !n_accept ? "n_accept" : !next_token ? "next_token"
                        : !workspace ? "workspace" : nullptr;
    if (missing) return fail(DSPARK_EINVAL, "required pointer %s is NULL", missing);
    if (isnan(threshold)) return fail(DSPARK_EINVAL, "threshold is NaN");
    if (!aligned(workspace, 256)) return fail(DSPARK_EINVAL, "workspace is not 256-byte aligned");
    const dspark::VerifyLayout L = dspark::verify_layout(*dims);
    if (workspace_bytes < L.total)
        return fail(DSPARK_EWORKSPACE, "workspace has %zu bytes, the call needs %zu", workspace_bytes, L.total);
    const size_t esz = dims->dtype == DSPARK_BF16 ? 2 : 4;
    if (!aligned(U, esz) || !aligned(W1, esz) || !aligned(W2, esz) || !aligned(T_logits, esz) ||
        !aligned(logp, 4) || !aligned(survival, 4) || !aligned(temperature, 4) ||
        (accept_prob && !aligned(accept_prob, 4)))
        return fail(DSPARK_EINVAL, "a tensor is not aligned to its element size");
    if (L.mfma && (!aligned(U, 16) || !aligned(W2, 16)))
        return fail(DSPARK_EUNSUPPORTED, "bf16 U and W2 must be 16-byte aligned");

    dspark::VerifyArgs a{};
    a.dims = *dims;
    a.U = U; a.W1 = W1; a.W2 = W2; a.T_logits = T_logits;
    a.anchor = anchor; a.tokens = tokens; a.logp = logp; a.survival = survival;
    a.temperature = temperature; a.threshold = threshold; a.seed = seed; a.offset = offset;
    a.n_keep = n_keep; a.n_accept = n_accept; a.next_token = next_token; a.accept_prob = accept_prob;
    a.ws = static_cast<char*>(workspace);
    a.stream = static_cast<hipStream_t>(hip_stream);
    const hipError_t e = dspark::launch_verify(a);
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

dspark_status dspark_sts_calibrate(int32_t N, int32_t gamma, const float* conf_logit,
                                   const int32_t* accepted, const float* grid, int32_t G,
                                   int32_t bins, float* temperature, float* ece_before,
                                   float* ece_after) {
    if (N < 1 || gamma < 1) return fail(DSPARK_EINVAL, "N = %d, gamma = %d: both must be >= 1", N, gamma);
    if (!conf_logit || !accepted || !temperature)
        return fail(DSPARK_EINVAL, "conf_logit, accepted and temperature must not be NULL");
    std::vector<double> g;
    if (grid) {
        if (G < 1) return fail(DSPARK_EINVAL, "grid has %d entries", G);
        for (int i = 0; i < G; ++i) {
            if (!(grid[i] > 0.0f)) return fail(DSPARK_EINVAL, "grid[%d] = %g is not positive", i, grid[i]);
            g.push_back(static_cast<double>(grid[i]));
        }
    } else {
        g = dspark::sts_default_grid();
    }
    for (int n = 0; n < N; ++n)
        if (accepted[n] < 0 || accepted[n] > gamma)
            return fail(DSPARK_EINVAL, "accepted[%d] = %d is outside 0..gamma", n, accepted[n]);
    dspark::sts_calibrate(N, gamma, conf_logit, accepted, g, bins > 0 ? bins : 15, temperature, ece_before,
                          ece_after);
    return ok();
}

dspark_status dspark_schedule_prefixes(int32_t R, int32_t gamma, const float* survival,
                                       const float* sps, int32_t T, int32_t* length,
                                       float* theta) {
    if (R < 1 || gamma < 0) return fail(DSPARK_EINVAL, "R = %d, gamma = %d", R, gamma);
    if ((gamma > 0 && !survival) || !sps || !length)
        return fail(DSPARK_EINVAL, "survival, sps and length must not be NULL");
    if (static_cast<int64_t>(T) < static_cast<int64_t>(R) * (gamma + 1))
        return fail(DSPARK_EINVAL, "sps covers %d tokens, a full batch is %lld", T,
                    static_cast<long long>(R) * (gamma + 1));
    const double t = dspark::schedule_prefixes(R, gamma, survival, sps, length);
    if (theta) *theta = static_cast<float>(t);
    return ok();
}

dspark_status dspark_noise(uint64_t seed, uint64_t offset, uint32_t c1, uint32_t c2, int32_t v0, int32_t n,
                           const uint32_t* words_in, uint32_t* words, float* gumbel, float* gumbel_log2,
                           void* hip_stream) {
    if (n < 0 || v0 < 0 || static_cast<int64_t>(v0) + n > (int64_t(1) << 31))
        return fail(DSPARK_EINVAL, "v0 = %d, n = %d: need v0 >= 0, n >= 0 and v0 + n <= 2^31", v0, n);
    if (n == 0) return ok();
    const hipError_t e = dspark::launch_noise(seed, offset, c1, c2, static_cast<uint32_t>(v0), n, words_in, words,
                                              gumbel, gumbel_log2, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

dspark_status dspark_read_device_error(const dspark_dims* dims, const void* workspace,
                                       int32_t* code, void* hip_stream) {
    dspark_status s = check_dims(dims);
    if (s != DSPARK_OK) return s;
    if (!workspace || !code) return fail(DSPARK_EINVAL, "workspace and code must not be NULL");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    hipError_t e = hipStreamSynchronize(st);
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "stream synchronisation failed: %s", hipGetErrorString(e));
    const int n = dims->B;
    std::string flags(sizeof(int32_t) * n, '\0');
    e = hipMemcpy(&flags[0], workspace, sizeof(int32_t) * n, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return fail(DSPARK_EDEVICE, "reading the error flags failed: %s", hipGetErrorString(e));
    int32_t count = 0;
    bool timed_out = false;
    for (int i = 0; i < n; ++i) {
        int32_t f;
        memcpy(&f, &flags[sizeof(int32_t) * i], sizeof f);
        count += f != 0;
        timed_out |= f == 2;
    }
    *code = count;
    if (timed_out)
        return fail(DSPARK_EDEVICE,
                    "a grid barrier of the single-launch drafting kernel gave up waiting (other work may hold "
                    "compute units); every block of the call is invalid");
    return ok();
}

dspark_status dspark_set_option(int option, int value) {
    if (option == DSPARK_OPT_DRAFT_PATH) {
        if (value < 0 || value > 2) return fail(DSPARK_EINVAL, "draft path %d is not 0, 1 or 2", value);
        dspark::g_draft_path = value;
        return ok();
    }
    if (option == DSPARK_OPT_BARRIER_SPIN) {
        if (value < -1) return fail(DSPARK_EINVAL, "barrier spin %d is below -1", value);
        dspark::g_barrier_spin = value;
        return ok();
    }
    return fail(DSPARK_EINVAL, "unknown option %d", option);
}

dspark_status dspark_profile_enable(int enable) {
    dspark::g_prof.on = enable != 0;
    return ok();
}

dspark_status dspark_profile_read(float* kernel_ms, int32_t* launches) {
    if (!kernel_ms || !launches) return fail(DSPARK_EINVAL, "kernel_ms and launches must not be NULL");
    auto& P = dspark::g_prof;
    float total = 0.0f;
    const size_t pairs = P.used / 2;
    for (size_t i = 0; i < pairs; ++i) {
        hipError_t e = hipEventSynchronize(P.pool[2 * i + 1]);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, P.pool[2 * i], P.pool[2 * i + 1]);
        if (e != hipSuccess) {
            P.used = 0;
            return fail(DSPARK_EDEVICE, "profiling event failed: %s", hipGetErrorString(e));
        }
        total += ms;
    }
    P.used = 0;
    *kernel_ms = total;
    *launches = static_cast<int32_t>(pairs);
    return ok();
}

dspark_status dspark_profile_read_each(float* kernel_ms, int32_t capacity, int32_t* launches) {
    if (!launches || capacity < 0 || (capacity > 0 && !kernel_ms))
        return fail(DSPARK_EINVAL, "launches must not be NULL, kernel_ms must hold capacity entries");
    auto& P = dspark::g_prof;
    const size_t pairs = P.used / 2;
    if (pairs > static_cast<size_t>(capacity)) {
        *launches = static_cast<int32_t>(pairs);
        return fail(DSPARK_EINVAL, "%zu timed launches, capacity %d", pairs, capacity);
    }
    for (size_t i = 0; i < pairs; ++i) {
        hipError_t e = hipEventSynchronize(P.pool[2 * i + 1]);
        float ms = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, P.pool[2 * i], P.pool[2 * i + 1]);
        if (e != hipSuccess) {
            P.used = 0;
            return fail(DSPARK_EDEVICE, "profiling event failed: %s", hipGetErrorString(e));
        }
        kernel_ms[i] = ms;
    }
    P.used = 0;
    *launches = static_cast<int32_t>(pairs);
    return ok();
}

const char* dspark_draft_kernel_name(const dspark_dims* dims) {
    if (check_dims(dims) != DSPARK_OK) return "";
    return dspark::draft_kernel_name(*dims);
}

const char* dspark_last_error(void) { return g_last_error.c_str(); }

int dspark_version(void) { return DSPARK_VERSION; }

}  // extern "C"
