"""CPU reference ("oracle") for the host-side post-draft stages.  TEST
INFRASTRUCTURE ONLY (tests, smoke check, benchmark CPU baseline); the product
path never calls it and it shares no code with the library.

Plain Python and numpy, float64, written from the pages:
  - Sequential Temperature Scaling: dormouse "DSpark - paper verification",
    section 1 (post-hoc calibration paragraph); bowenzhou "设计".  The
    prefix survival is the product of the conditional confidences; one
    temperature per position is fitted left to right by a 1-D grid search
    on the ECE of that product, earlier positions held fixed.
  - prefix scheduler: bowenzhou "设计"; Meridian "Phase-Conditioned
    Speculative Decoding", section 3: maximise expected accepted tokens per
    cycle times steps/s at the resulting batch, every request's choice a
    prefix.
  - depth planner: Meridian section 6, Theta(g) = tau(a, g) / cycle cost.
Readings where the pages leave a detail open: the ECE uses 15 equal-width
bins over [0, 1]; the default temperature grid is 201 geometric points in
[0.05, 20] with 1 in the middle; the scheduler's batch size counts every
request's bonus position.
"""
from __future__ import annotations

import itertools

import numpy as np


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-np.asarray(x, np.float64)))


def default_grid() -> np.ndarray:
    g = 0.05 * 400.0 ** (np.arange(201) / 200.0)
    g[100] = 1.0
    return g


def ece(p, o, bins: int = 15) -> float:
    """Expected calibration error with `bins` equal-width bins of [0, 1]:
    sum over bins of |sum of p - sum of o| / n (p = 1 goes to the last bin)."""
    p = np.asarray(p, np.float64)
    o = np.asarray(o, np.float64)
    total = 0.0
    for b in range(bins):
        lo, hi = b / bins, (b + 1) / bins
        sel = (p >= lo) & ((p < hi) | (b == bins - 1))
        if sel.any():
            total += abs(p[sel].sum() - o[sel].sum())
    return total / len(p)


def sts_calibrate(conf_logit, accepted, grid=None, bins: int = 15) -> dict:
    """Temperatures [gamma] fitted left to right; ECE of the raw and the
    calibrated survival product at every position."""
    a = np.asarray(conf_logit, np.float64)
    acc = np.asarray(accepted)
    N, gamma = a.shape
    grid = default_grid() if grid is None else np.asarray(grid, np.float64)
    temps, before, after = [], [], []
    prefix = np.ones(N)
    for k in range(gamma):
        outcome = (acc > k).astype(np.float64)     # the prefix of k + 1 tokens survived
        raw = np.prod(sigmoid(a[:, :k + 1]), axis=1)
        before.append(ece(raw, outcome, bins))
        errs = [ece(prefix * sigmoid(a[:, k] / t), outcome, bins) for t in grid]
        best = int(np.argmin(errs))               # first minimum
        temps.append(grid[best])
        after.append(errs[best])
        prefix = prefix * sigmoid(a[:, k] / grid[best])
    return dict(temperature=np.array(temps), ece_before=np.array(before), ece_after=np.array(after))


def theta(lengths, survival, sps) -> float:
    """(R + expected accepted drafted tokens) * sps[R + sum lengths]."""
    s = np.asarray(survival, np.float64)
    R = s.shape[0]
    tau = R + sum(s[r, :l].sum() for r, l in enumerate(lengths))
    return tau * float(sps[R + int(np.sum(lengths))])


def schedule_prefixes(survival, sps) -> dict:
    """Greedy by survival (ties: lower request), the best prefix count."""
    s = np.asarray(survival, np.float64)
    R, gamma = s.shape
    nxt = [0] * R
    order = []
    while True:
        cand = [(s[r, nxt[r]], -r) for r in range(R) if nxt[r] < gamma]
        if not cand:
            break
        v, neg_r = max(cand)
        order.append(-neg_r)
        nxt[-neg_r] += 1
    best_n, best_t = 0, theta([0] * R, s, sps)
    lengths = [0] * R
    for n, r in enumerate(order, start=1):
        lengths[r] += 1
        t = theta(lengths, s, sps)
        if t > best_t:
            best_n, best_t = n, t
    out = [0] * R
    for r in order[:best_n]:
        out[r] += 1
    return dict(length=np.array(out), theta=best_t)


def schedule_brute_force(survival, sps) -> dict:
    """Every combination of prefix lengths (tiny problems only)."""
    s = np.asarray(survival, np.float64)
    R, gamma = s.shape
    best, arg = -np.inf, None
    for ls in itertools.product(range(gamma + 1), repeat=R):
        t = theta(ls, s, sps)
        if t > best:
            best, arg = t, ls
    return dict(length=np.array(arg), theta=best)
