"""Pins for the oracle's scheduler (Algorithm 1 and its modes).

Printed worked examples (Appendix A numbers; the two-request example), exact
brute force over all prefix-length assignments on tiny inputs, the per-token
admission threshold identity, and the empty-system limit.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle.schedule import (schedule_ref, schedule_async_ref, schedule_bruteforce, survival,
                             SCHED_EARLY_STOP, SCHED_GLOBAL, SCHED_TOPK)

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _appendix_sps(g):
    sps = np.zeros(4)
    for b, v in g["sps_by_batch"].items():
        sps[int(b)] = v
    return sps


@pytest.mark.parametrize("case", ["case_high", "case_low"])
def test_appendix_a(case):
    g = _load("appendix_a.json")
    sps = _appendix_sps(g)
    c = np.array([[g["c1"], g[case]["c2"]]], dtype=np.float32)
    es = schedule_ref(c, sps, SCHED_EARLY_STOP)
    assert es["ell"].tolist() == [g["ell_with_break"]]
    assert es["thetas"][0] == pytest.approx(g["theta0"], rel=1e-6)
    assert es["thetas"][1] == pytest.approx(g["theta1"], rel=1e-6)
    assert len(es["thetas"]) == 2                      # broke at the first drop
    gl = schedule_ref(c, sps, SCHED_GLOBAL)
    assert gl["ell"].tolist() == [g[case]["ell_without_break"]]
    assert float(survival(c)[0, 1]) == pytest.approx(g[case]["a2"], rel=1e-6)
    if g[case]["ell_without_break"] == 2:
        assert gl["theta"] == pytest.approx(g[case]["theta2"], rel=1e-6)
    # Theta of verifying both drafts, evaluated exactly
    best, arg = schedule_bruteforce(c, sps)
    cf = [Fraction(float(v)) for v in c[0]]
    theta2 = (1 + cf[0] + cf[0] * cf[1]) * Fraction(float(sps[3]))
    assert float(theta2) == pytest.approx(g[case]["theta2"], rel=1e-6)
    assert list(arg[0]) == [g[case]["ell_without_break"]]


def test_paperglide_two_request_example():
    g = _load("paperglide_two_request.json")
    c = np.array(g["c"], dtype=np.float32)
    sps = np.array(g["sps_constructed"])
    out = schedule_ref(c, sps, SCHED_EARLY_STOP)
    np.testing.assert_allclose(out["a"], np.array(g["a"]), rtol=1e-6)
    order = [[r + 1, j] for r, j in out["order"]]
    assert order == g["sorted_order_1based"]
    assert out["ell"].tolist() == g["ell"]
    assert int(out["cu_seqlens"][-1]) == g["batch"]
    assert out["theta"] / sps[g["batch"]] == pytest.approx(g["tau_with_anchor_terms"], rel=1e-6)
    assert out["theta"] / sps[g["batch"]] - len(g["ell"]) == pytest.approx(g["tau_printed"], rel=1e-6)
    for mode in (SCHED_GLOBAL,):
        assert schedule_ref(c, sps, mode)["ell"].tolist() == g["ell"]
    best, arg = schedule_bruteforce(c, sps)
    assert [list(a) for a in arg] == [g["ell"]]


def _random_case(rng, R, K):
    c = rng.uniform(0, 1, size=(R, K)).astype(np.float32)
    c[rng.uniform(size=(R, K)) < 0.1] = 1.0
    return c


def _check_against_bruteforce(c, sps, mode):
    out = schedule_ref(c, sps, mode)
    best, arg = schedule_bruteforce(c, sps)
    # a is a float32 product (one rounding per factor) and tau is truncated to
    # 2^-32 per term, so Theta can differ from the exact-rational value at the
    # float32 level
    assert out["theta"] == pytest.approx(float(best), rel=1e-6)
    if tuple(out["ell"].tolist()) not in [tuple(a) for a in arg]:
        # only acceptable if the chosen assignment is within rounding of the max
        R = c.shape[0]
        a = [[Fraction(1)] for _ in range(R)]
        for r in range(R):
            for j in range(c.shape[1]):
                a[r].append(a[r][-1] * Fraction(float(c[r, j])))
        tau = R + sum(sum(a[r][1:out["ell"][r] + 1]) for r in range(R))
        theta = tau * Fraction(float(sps[R + int(out["ell"].sum())]))
        assert abs(float(theta - best)) <= 1e-6 * float(best)


def test_global_equals_bruteforce_any_sps():
    rng = np.random.default_rng(11)
    for _ in range(300):
        R, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        c = _random_case(rng, R, K)
        sps = rng.uniform(0.1, 2.0, size=R * (K + 1) + 1)
        _check_against_bruteforce(c, sps, SCHED_GLOBAL)


def test_early_stop_equals_bruteforce_when_unimodal():
    rng = np.random.default_rng(12)
    for i in range(300):
        R, K = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        c = _random_case(rng, R, K)
        B = np.arange(R * (K + 1) + 1, dtype=np.float64)
        if i % 3 == 0:
            sps = np.full(B.shape, 3.0)                           # flat
        else:
            beta = rng.uniform(0.5, 40.0)
            sps = 1000.0 / (1.0 + B / beta)                       # hyperbolic
        _check_against_bruteforce(c, sps, SCHED_EARLY_STOP)


def test_early_stop_can_stop_below_global_on_a_cliff():
    g = _load("appendix_a.json")
    sps = _appendix_sps(g)
    c = np.array([[g["c1"], g["case_high"]["c2"]]], dtype=np.float32)
    assert schedule_ref(c, sps, SCHED_EARLY_STOP)["theta"] < schedule_ref(c, sps, SCHED_GLOBAL)["theta"]


def test_admission_threshold_identity():
    """Continuing is equivalent to a_n > tau_{n-1} * (SPS(B)/SPS(B+1) - 1)."""
    rng = np.random.default_rng(13)
    checked = 0
    for _ in range(200):
        R, K = int(rng.integers(1, 9)), int(rng.integers(1, 8))
        c = _random_case(rng, R, K)
        sps = np.sort(rng.uniform(0.2, 2.0, size=R * (K + 1) + 1))[::-1].copy()
        out = schedule_ref(c, sps, SCHED_GLOBAL)
        a = survival(c)
        tau = Fraction(R)
        thetas = out["thetas"]
        for n, (r, j) in enumerate(out["order"], start=1):
            B = R + n - 1
            an = Fraction(int(np.floor(np.float64(a[r, j - 1]) * 2 ** 32)), 2 ** 32)
            rises = an > tau * (Fraction(float(sps[B])) / Fraction(float(sps[B + 1])) - 1)
            if abs(float(thetas[n] - thetas[n - 1])) > 1e-12 * abs(float(thetas[n - 1])):
                assert rises == (thetas[n] > thetas[n - 1])
                checked += 1
            tau += an
    assert checked > 500


def test_empty_system_limit_verifies_everything_alive():
    rng = np.random.default_rng(14)
    for _ in range(50):
        R, K = int(rng.integers(1, 30)), int(rng.integers(1, 9))
        c = _random_case(rng, R, K)
        c[rng.uniform(size=(R, K)) < 0.05] = 0.0
        sps = np.full(R * (K + 1) + 1, 5.0)
        out = schedule_ref(c, sps, SCHED_EARLY_STOP)
        expect = (survival(c) > 0).sum(axis=1)
        np.testing.assert_array_equal(out["ell"], expect)


def test_topk_admits_the_first_capacity_candidates_and_prefixes_hold():
    rng = np.random.default_rng(15)
    for _ in range(100):
        R, K = int(rng.integers(1, 20)), int(rng.integers(1, 8))
        c = _random_case(rng, R, K)
        c[rng.uniform(size=(R, K)) < 0.05] = 0.0
        sps = rng.uniform(0.2, 2.0, size=R * (K + 1) + 1)
        cap = int(rng.integers(0, R * K + 3))
        out = schedule_ref(c, sps, SCHED_TOPK, cap)
        n = min(cap, len(out["order"]))
        assert out["n_admitted"] == n == int(out["ell"].sum())
        counts = np.zeros(R, dtype=np.int64)
        for r, j in out["order"][:n]:
            counts[r] += 1
            assert j == counts[r]                      # each request's admitted set is a prefix
        np.testing.assert_array_equal(counts, out["ell"])
        np.testing.assert_array_equal(out["cu_seqlens"], np.concatenate([[0], np.cumsum(1 + out["ell"])]))


def test_invalid_confidence_rejected():
    sps = np.ones(10)
    for bad in (np.nan, -0.1, 1.5):
        with pytest.raises(ValueError):
            schedule_ref(np.array([[0.5, bad]], dtype=np.float32), sps)


def test_empty_batch_admits_nothing():
    """No requests (Algorithm 1 with R = 0): the pool is empty, B = tau = 0, so
    nothing is admitted, the flat layout is [0] and Theta = 0 * SPS(0) = 0;
    the asynchronous variant inherits a zero capacity."""
    sps = np.array([3.0, 2.0])
    for mode in (SCHED_EARLY_STOP, SCHED_GLOBAL, SCHED_TOPK):
        out = schedule_ref(np.zeros((0, 4), dtype=np.float32), sps, mode, 5)
        assert out["ell"].shape == (0,) and out["a"].shape == (0, 4)
        assert list(out["cu_seqlens"]) == [0]
        assert out["n_admitted"] == 0 and out["theta"] == 0.0
    out = schedule_async_ref(np.zeros((0, 4), dtype=np.float32), np.zeros((0, 4), dtype=np.float32), sps)
    assert out["capacity"] == 0 and out["n_admitted"] == 0 and list(out["cu_seqlens"]) == [0]
