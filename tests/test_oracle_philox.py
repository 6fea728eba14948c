"""Pins for the oracle's random numbers (CPU only).

The pages fix no generator; the reading is Philox4x32-10 (Salmon et al.,
SC'11) with a stated key/counter layout.  Pinned here against an independent
implementation (rocRAND's philox4x32_10 engine, compiled for the host from
its header) and against the Gumbel law's closed-form moments.
"""
import math
import os
import shutil
import subprocess

import numpy as np
import pytest

ROCRAND_PROBE = r"""
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>
// argv: seed subsequence counter01 -> the four 32-bit words of Philox4x32-10
// at counter (counter01 lo, counter01 hi, subsequence lo, subsequence hi),
// key (seed lo, seed hi); rocRAND's offset counts single words, 4 per counter.
int main(int argc, char** argv) {
  for (int a = 1; a + 2 < argc; a += 3) {
    unsigned long long seed = strtoull(argv[a], 0, 0);
    unsigned long long sub = strtoull(argv[a + 1], 0, 0);
    unsigned long long c01 = strtoull(argv[a + 2], 0, 0);
    rocrand_device::philox4x32_10_engine e(seed, sub, 4ull * c01);
    for (int i = 0; i < 4; i++) printf("%u ", e.next());
    printf("\n");
  }
  return 0;
}
"""


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("rocRAND headers / hipcc not available")
    d = tmp_path_factory.mktemp("rocrand")
    src = d / "probe.cpp"
    src.write_text(ROCRAND_PROBE)
    exe = d / "probe"
    subprocess.run([hipcc, "-O1", str(src), "-o", str(exe)], check=True,
                   stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
    return str(exe)


def test_philox_matches_rocrand(oracle_lib, rocrand_probe):
    rng = np.random.default_rng(7)
    # rocRAND takes the word offset 4 * counter01 as a 64-bit count, so counter01 < 2^62
    cases = [(0, 0, 0), (0xFFFFFFFFFFFFFFFF, 0xFFFFFFFFFFFFFFFF, 2**62 - 1)]
    for _ in range(30):
        cases.append(tuple(int(x) for x in rng.integers(0, 2**62, size=3, dtype=np.int64)))
    args = []
    for s, sub, c in cases:
        args += [str(s), str(sub), str(c)]
    out = subprocess.run([rocrand_probe] + args, check=True, capture_output=True, text=True).stdout
    lines = out.strip().splitlines()
    assert len(lines) == len(cases)
    for (s, sub, c), line in zip(cases, lines):
        want = [int(x) for x in line.split()]
        ctr = [c & 0xFFFFFFFF, c >> 32, sub & 0xFFFFFFFF, sub >> 32]
        key = [s & 0xFFFFFFFF, s >> 32]
        got = oracle_lib.philox4x32_10(ctr, key).tolist()
        assert got == want, (s, sub, c)


def test_uniform_is_odd_multiple_of_2pow_minus24(oracle_lib):
    for v in range(0, 64):
        u = oracle_lib.uniform(0, 0, 3, 2, v)
        m = u * 2**24
        assert 0.0 < u < 1.0
        assert m == int(m) and int(m) % 2 == 1


def test_uniform_counter_layout(oracle_lib):
    # element v of block b at step k uses word v % 4 of counter (v/4, k, b, offset)
    seed, offset, b, k = 0x123456789ABCDEF0, 77, 5, 3
    for v in (0, 1, 2, 3, 4, 9, 1023):
        words = oracle_lib.philox4x32_10([v // 4, k, b, offset],
                                         [seed & 0xFFFFFFFF, seed >> 32])
        u = (2 * (int(words[v % 4]) >> 9) + 1) / 2**24
        assert oracle_lib.uniform(seed, offset, b, k, v) == u


def test_gumbel_moments(oracle_lib):
    # standard Gumbel: mean = Euler-Mascheroni constant, variance = pi^2 / 6
    g = np.array([oracle_lib.gumbel(0, 0, b, 0, v) for b in range(50) for v in range(4000)])
    n = g.size
    euler_gamma = 0.5772156649015329
    assert abs(g.mean() - euler_gamma) < 5 * math.sqrt(math.pi**2 / 6 / n)
    assert abs(g.var() - math.pi**2 / 6) < 0.03
    # CDF exp(-exp(-x)) at a few points
    for x in (-1.0, 0.0, 1.0, 3.0):
        emp = (g <= x).mean()
        assert abs(emp - math.exp(-math.exp(-x))) < 5 * math.sqrt(0.25 / n)
