"""Pins for the oracle's Philox4x32-10 and the per-decision uniform.

The oracle's generator is checked against rocRAND's Philox4x32-10 block
function (an independent implementation shipped with ROCm, compiled here as
host code) on random counters and keys, and the uniform mapping against its
definition (exact multiples of 2^-24 in [0, 1)) and a uniformity test.
"""
import os
import shutil
import subprocess

import numpy as np
import pytest
from scipy import stats

from oracle.philox import philox4x32_10, uniform, PURPOSE_DRAFT, PURPOSE_ACCEPT

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_probe(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_philox4x32_10.h"):
        pytest.skip("rocRAND headers / hipcc not available")
    exe = str(tmp_path_factory.mktemp("probe") / "philox_probe")
    subprocess.run([hipcc, "-O1", "-o", exe, os.path.join(HERE, "rocrand_philox_probe.cpp")],
                   check=True, capture_output=True)
    return exe


def test_philox_matches_rocrand(rocrand_probe):
    rng = np.random.default_rng(7)
    n = 20000
    words = rng.integers(0, 2 ** 32, size=(n, 6), dtype=np.uint64)
    words[0] = 0
    words[1] = 0xFFFFFFFF
    inp = "\n".join(" ".join("%x" % int(w) for w in row) for row in words) + "\n"
    out = subprocess.run([rocrand_probe], input=inp, capture_output=True, text=True, check=True).stdout
    ref = np.array([[int(t, 16) for t in line.split()] for line in out.strip().splitlines()], dtype=np.uint64)
    got = np.stack(philox4x32_10(words[:, :4].T, words[:, 4:].T), axis=1)
    assert ref.shape == (n, 4)
    np.testing.assert_array_equal(got, ref)


def test_uniform_grid_and_range():
    u = uniform(0x5EED0005, 3, np.arange(4096), 5, PURPOSE_ACCEPT)
    assert np.all(u >= 0) and np.all(u < 1)
    scaled = u * 2 ** 24
    np.testing.assert_array_equal(scaled, np.floor(scaled))
    assert np.all(u.astype(np.float32).astype(np.float64) == u)   # exact in float32


def test_uniform_addresses_are_distinct_streams():
    a = uniform(1, 0, np.arange(1000), 1, PURPOSE_DRAFT)
    b = uniform(1, 0, np.arange(1000), 1, PURPOSE_ACCEPT)
    c = uniform(1, 1, np.arange(1000), 1, PURPOSE_DRAFT)
    d = uniform(2, 0, np.arange(1000), 1, PURPOSE_DRAFT)
    for other in (b, c, d):
        assert np.mean(a == other) < 0.01


def test_uniform_chi_square():
    r = np.arange(1 << 20)
    u = uniform(12345, 0, r, 3, PURPOSE_DRAFT)
    counts = np.bincount((u * 65536).astype(np.int64), minlength=65536)
    chi2 = ((counts - counts.mean()) ** 2 / counts.mean()).sum()
    pval = stats.chi2.sf(chi2, 65535)
    assert pval > 1e-6
