// Host-side post-draft stages: Sequential Temperature Scaling of the
// confidence head and the hardware-aware prefix scheduler.  Plain C++ on
// host arrays (no device work); the C ABI is in include/dspark.h.
//
// STS (dormouse "DSpark - paper verification", section 1, the transcription
// of the paper's post-hoc calibration; bowenzhou "DSpark：既要猜得连贯，也要
// 把验证算力花在刀刃上", "设计"): the survival of a k-token prefix is the
// product of the conditional confidences, and STS fits one temperature per
// position, left to right, by a 1-D grid search that minimises the ECE of
// that product with the positions before it held fixed.
//
// Scheduler (bowenzhou, "设计"; Meridian "Phase-Conditioned Speculative
// Decoding", section 3): choose each request's verified prefix so that
// expected accepted tokens per cycle times the engine's steps/s at the
// resulting batch is largest, comparing the value of one more verified
// token by its prefix survival and keeping every request's choice a prefix.
//
#include "internal.h"

#include <math.h>

#include <algorithm>
#include <queue>
#include <vector>

namespace dspark {

namespace {

double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

// Expected calibration error of predictions p against 0/1 outcomes o over
// `bins` equal-width bins of [0, 1] (a prediction of exactly 1 falls in the
// last bin): sum over bins of (bin size / n) |mean p - mean o|.
double ece(const std::vector<double>& p, const std::vector<double>& o, int bins) {
    std::vector<double> sp(bins, 0.0), so(bins, 0.0);
    std::vector<int64_t> cnt(bins, 0);
    for (size_t i = 0; i < p.size(); ++i) {
        const int b = std::min(bins - 1, std::max(0, static_cast<int>(p[i] * bins)));
        sp[b] += p[i];
        so[b] += o[i];
        ++cnt[b];
    }
    double e = 0.0;
    for (int b = 0; b < bins; ++b)
        if (cnt[b] > 0) e += fabs(sp[b] - so[b]);
    return e / static_cast<double>(p.size());
}

}  // namespace

std::vector<double> sts_default_grid() {
    // 201 temperatures, geometric from 0.05 to 20; the middle one is 1.
    std::vector<double> g(201);
    for (int i = 0; i < 201; ++i) g[i] = 0.05 * pow(400.0, i / 200.0);
    g[100] = 1.0;
    return g;
}

void sts_calibrate(int N, int gamma, const float* logit, const int32_t* accepted,
                   const std::vector<double>& grid, int bins, float* temperature, float* ece_before,
                   float* ece_after) {
    std::vector<double> prev(N, 1.0), raw(N, 1.0), p(N), o(N);
    for (int k = 0; k < gamma; ++k) {
        for (int n = 0; n < N; ++n) o[n] = accepted[n] > k ? 1.0 : 0.0;  // prefix of k + 1 survived
        if (ece_before) {
            for (int n = 0; n < N; ++n) p[n] = raw[n] * sigmoid(static_cast<double>(logit[static_cast<int64_t>(n) * gamma + k]));
            ece_before[k] = static_cast<float>(ece(p, o, bins));
        }
        for (int n = 0; n < N; ++n) raw[n] *= sigmoid(static_cast<double>(logit[static_cast<int64_t>(n) * gamma + k]));
        size_t best = 0;
        double best_e = INFINITY;
        for (size_t gi = 0; gi < grid.size(); ++gi) {
            for (int n = 0; n < N; ++n)
                p[n] = prev[n] * sigmoid(static_cast<double>(logit[static_cast<int64_t>(n) * gamma + k]) / grid[gi]);
            const double e = ece(p, o, bins);
            if (e < best_e) {  // strict: the first grid point wins a tie
                best_e = e;
                best = gi;
            }
        }
        temperature[k] = static_cast<float>(grid[best]);
        if (ece_after) ece_after[k] = static_cast<float>(best_e);
        for (int n = 0; n < N; ++n)
            prev[n] *= sigmoid(static_cast<double>(logit[static_cast<int64_t>(n) * gamma + k]) / grid[best]);
    }
}

double schedule_prefixes(int R, int gamma, const float* survival, const float* sps,
                         int32_t* length) {
    // candidate = the next position of a request; larger survival first,
    // then lower request, so that equal values are taken in a fixed order
    struct Cand {
        double v;
        int r, k;
    };
    auto worse = [](const Cand& a, const Cand& b) { return a.v < b.v || (a.v == b.v && a.r > b.r); };
    std::priority_queue<Cand, std::vector<Cand>, decltype(worse)> heap(worse);
    for (int r = 0; r < R; ++r)
        if (gamma > 0) heap.push(Cand{static_cast<double>(survival[static_cast<int64_t>(r) * gamma]), r, 0});
    std::vector<int> order;
    order.reserve(static_cast<size_t>(R) * gamma);
    double sum = 0.0;
    // n = 0: every request verifies its bonus position only
    double best = static_cast<double>(R) * sps[R];
    size_t best_n = 0;
    while (!heap.empty()) {
        const Cand c = heap.top();
        heap.pop();
        order.push_back(c.r);
        sum += c.v;
        if (c.k + 1 < gamma)
            heap.push(Cand{static_cast<double>(survival[static_cast<int64_t>(c.r) * gamma + c.k + 1]), c.r, c.k + 1});
        const double theta = (static_cast<double>(R) + sum) * sps[R + order.size()];
        if (theta > best) {
            best = theta;
            best_n = order.size();
        }
    }
    for (int r = 0; r < R; ++r) length[r] = 0;
    for (size_t i = 0; i < best_n; ++i) ++length[order[i]];
    return best;
}

}  // namespace dspark
