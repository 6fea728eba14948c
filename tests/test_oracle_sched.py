"""Pins of the oracle's host-side post-draft stages (oracle/sched.py).

  - ECE: hand-computed values for constant predictions and a two-bin case;
  - STS: on synthetic blocks whose outcomes are drawn from known conditional
    probabilities, logits scaled by s are calibrated back to temperature s
    (and already calibrated logits keep temperature 1), position by position;
    at the first position the calibrated ECE never exceeds the raw one;
  - scheduler: equals exhaustive search over every prefix-length combination
    on small batches with survivals that decrease along each request; a flat
    steps/s curve verifies every drafted token, a steep one none.
"""
import numpy as np

from oracle import sched


def test_ece_hand_values():
    assert sched.ece([0.7] * 10, [0] * 10) == 0.7
    assert abs(sched.ece([0.7] * 10, [1] * 7 + [0] * 3)) < 1e-15
    # two bins: {0.05, 0.05} with outcomes {0, 1}, {0.95, 0.95} with {1, 1}
    e = sched.ece([0.05, 0.05, 0.95, 0.95], [0, 1, 1, 1], bins=10)
    assert abs(e - (abs(0.1 - 1) + abs(1.9 - 2)) / 4) < 1e-15


def synthetic_blocks(N, gamma, seed, scale):
    rng = np.random.default_rng(seed)
    z = rng.normal(1.0, 1.5, size=(N, gamma))
    c = 1.0 / (1.0 + np.exp(-z))
    u = rng.random((N, gamma))
    ok = u < c
    accepted = np.where(ok.all(axis=1), gamma, np.argmin(ok, axis=1))
    return scale * z, accepted


def test_sts_recovers_the_scale():
    for scale in (1.0, 2.5, 0.5):
        logit, acc = synthetic_blocks(40000, 4, seed=int(scale * 10), scale=scale)
        out = sched.sts_calibrate(logit, acc)
        assert np.all(np.abs(np.log(out["temperature"] / scale)) < np.log(1.2)), (scale, out["temperature"])
        assert out["ece_after"][0] <= out["ece_before"][0] + 1e-15
        assert np.all(out["ece_after"] < 0.02)
        if scale != 1.0:
            assert out["ece_before"][0] > 0.03


def test_scheduler_equals_exhaustive_search():
    rng = np.random.default_rng(3)
    for trial in range(40):
        R, gamma = 3, 3
        s = np.sort(rng.random((R, gamma)), axis=1)[:, ::-1].copy()  # decreasing along the block
        T = R * (gamma + 1)
        # steps/s falling with batch size at a random rate
        sps = 100.0 / (1.0 + rng.random() * 0.3 * np.arange(T + 1))
        g = sched.schedule_prefixes(s, sps)
        b = sched.schedule_brute_force(s, sps)
        assert abs(g["theta"] - b["theta"]) <= 1e-12 * b["theta"], trial


def test_scheduler_extremes():
    s = np.array([[0.9, 0.5, 0.1], [0.8, 0.7, 0.6]])
    flat = np.full(9, 50.0)
    assert list(sched.schedule_prefixes(s, flat)["length"]) == [3, 3]
    steep = np.concatenate([[50.0] * 3, [1.0] * 6])  # any extra token costs almost everything
    assert list(sched.schedule_prefixes(s, steep)["length"]) == [0, 0]
