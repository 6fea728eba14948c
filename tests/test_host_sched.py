"""The library's host-side post-draft stages (STS and the prefix scheduler;
C ABI, host arrays, no GPU work) against the oracle.

Every test runs twice: once in the CPU suite, and once more marked `gpu`, so
that the GPU run on the MI355X host exercises the same library build there
too (the stages run on the host cores of the GPU machine in a deployment)."""
import numpy as np
import pytest

from oracle import sched


@pytest.fixture(scope="module", params=["host", pytest.param("gpu-host", marks=pytest.mark.gpu)])
def lib(request):
    from semi_autoregressive_draft_markov_amd import binding
    binding.load()
    return binding


def blocks(N, gamma, seed, scale):
    rng = np.random.default_rng(seed)
    z = rng.normal(0.8, 1.5, size=(N, gamma))
    ok = rng.random((N, gamma)) < 1.0 / (1.0 + np.exp(-z))
    acc = np.where(ok.all(axis=1), gamma, np.argmin(ok, axis=1)).astype(np.int32)
    return (scale * z).astype(np.float32), acc


@pytest.mark.parametrize("scale,bins", [(1.0, 15), (2.2, 15), (0.6, 10)])
def test_sts_matches_oracle(lib, scale, bins):
    logit, acc = blocks(6000, 5, seed=int(scale * 7), scale=scale)
    t, eb, ea = lib.dspark_sts_calibrate(logit, acc, bins=bins)
    ref = sched.sts_calibrate(logit.astype(np.float64), acc, bins=bins)
    assert np.allclose(eb, ref["ece_before"], rtol=1e-5, atol=1e-7)
    assert np.allclose(ea, ref["ece_after"], rtol=1e-5, atol=1e-7)
    assert np.allclose(t, ref["temperature"], rtol=1e-6)


def test_sts_custom_grid_and_errors(lib):
    from semi_autoregressive_draft_markov_amd.binding import DsparkError
    logit, acc = blocks(500, 3, seed=9, scale=1.5)
    grid = [0.5, 1.0, 1.5, 2.0]
    t, _, ea = lib.dspark_sts_calibrate(logit, acc, grid=grid)
    ref = sched.sts_calibrate(logit.astype(np.float64), acc, grid=grid)
    assert np.allclose(t, ref["temperature"]) and np.allclose(ea, ref["ece_after"], rtol=1e-5)
    with pytest.raises(DsparkError):
        lib.dspark_sts_calibrate(logit, acc, grid=[1.0, -1.0])
    with pytest.raises(DsparkError):
        lib.dspark_sts_calibrate(logit, np.full(500, 4, np.int32))


def test_scheduler_matches_oracle(lib):
    rng = np.random.default_rng(11)
    for trial in range(20):
        R, gamma = int(rng.integers(1, 40)), int(rng.integers(1, 9))
        c = rng.random((R, gamma)) ** 0.3
        s = np.cumprod(c, axis=1).astype(np.float32)  # a survival curve per request
        T = R * (gamma + 1)
        sps = (1000.0 / (1.0 + rng.random() * 0.05 * np.arange(T + 1))).astype(np.float32)
        length, theta = lib.dspark_schedule_prefixes(s, sps)
        ref = sched.schedule_prefixes(s.astype(np.float64), sps.astype(np.float64))
        assert np.array_equal(length, ref["length"]), trial
        assert abs(theta - ref["theta"]) <= 1e-5 * ref["theta"]
