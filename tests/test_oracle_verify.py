"""Pins for the oracle's rejection-sampling verification.

* p == q accepts every scheduled draft and emits the bonus sample;
* position-1 acceptance frequency equals sum_v min(p, q) = 1 - TV(p, q);
* the emitted token follows p (chi-square, V = 8, 10^6 trials), and so does the
  bonus token (it follows the next row's p);
* the printed two-token example (p = (0.7, 0.3), q = (0.5, 0.5)): acceptance
  0.8, P(A) = 0.7; a planted mistake (correction drawn from the whole p) must
  give the printed 0.64 and fail the chi-square, showing the test has power;
* E[accepted] = sum_k prod_{i<=k} alpha_i for independent positions;
* greedy verification equals plain argmax matching;
* Appendix A composed: the argmax scheduler (no break) is lossy (P(A) = 0.85),
  the early-stopping scheduler is lossless (P(A) = 0.7);
* end to end: zero bias, p == q and a flat SPS emit K + 1 tokens per request.
"""
import json
import os

import numpy as np
import pytest
from scipy import stats
from scipy.special import logsumexp

import oracle.verify as overify
from oracle.draft import draft_ref
from oracle.schedule import schedule_async_ref, schedule_ref, SCHED_EARLY_STOP, SCHED_GLOBAL
from oracle.step import run_step
from oracle.verify import verify_ref

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _softmax(z):
    return np.exp(z - logsumexp(z))


def _single_position_trials(p_row, q_row, n, seed, step=0):
    """n independent requests, each drafting one token from q and verifying it
    against p (one draft row and one bonus row per request)."""
    V = len(p_row)
    lq, lp = np.log(q_row), np.log(p_row)
    U = np.broadcast_to(lq, (n, 1, V))
    d = draft_ref(U, None, None, np.zeros(n, dtype=np.int64), 1.0, seed, step)
    P = np.broadcast_to(lp, (2 * n, V))
    cu = np.arange(0, 2 * n + 1, 2)
    v = verify_ref(P, cu, U, None, None, np.zeros(n, dtype=np.int64), d["x"], 1.0, seed, step)
    first = np.where(v["n_acc"] >= 1, d["x"][:, 0], v["tok"])
    return d, v, first


def test_p_equals_q_accepts_everything():
    rng = np.random.default_rng(31)
    R, K, V = 20, 5, 50
    D = rng.normal(0, 2, size=(R, K + 1, V))
    x0 = rng.integers(0, V, size=R)
    d = draft_ref(D[:, :K], None, None, x0, 1.0, seed=4, step=2)
    ell = rng.integers(0, K + 1, size=R)
    rows = [D[r, :ell[r] + 1] for r in range(R)]
    P = np.concatenate(rows)
    cu = np.concatenate([[0], np.cumsum(ell + 1)])
    v = verify_ref(P, cu, D[:, :K], None, None, x0, d["x"], 1.0, seed=4, step=2)
    np.testing.assert_array_equal(v["n_acc"], ell)
    assert np.all(v["mode"] == 0)
    assert np.all(v["ratio"][~np.isnan(v["ratio"])] == pytest.approx(1.0, rel=1e-12))


def test_acceptance_equals_one_minus_tv():
    p = _softmax(np.array([0.5, -0.2, 1.3, 0.0, -1.1, 0.7, 0.2, -0.5]))
    q = _softmax(np.array([0.1, 0.4, 0.9, -0.3, -0.2, 0.3, 0.6, -1.0]))
    n = 1_000_000
    d, v, _ = _single_position_trials(p, q, n, seed=101)
    alpha = np.minimum(p, q).sum()
    assert alpha == pytest.approx(1 - 0.5 * np.abs(p - q).sum(), rel=1e-12)
    freq = np.mean(v["n_acc"] == 1)
    sigma = np.sqrt(alpha * (1 - alpha) / n)
    assert abs(freq - alpha) < 5 * sigma


def test_emitted_token_follows_target():
    p = _softmax(np.array([1.5, -0.2, 0.3, 0.0, -1.1, 0.7, 0.2, -2.5]))
    q = _softmax(np.array([-0.4, 0.4, 0.9, 0.8, -0.2, 0.3, 1.6, -1.0]))
    n = 1_000_000
    _, _, first = _single_position_trials(p, q, n, seed=102)
    counts = np.bincount(first, minlength=8)
    assert stats.chisquare(counts, p * n).pvalue > 1e-6


def test_bonus_token_follows_next_target_row():
    n = 1_000_000
    V = 8
    q1 = _softmax(np.linspace(-1, 1, V))
    p2 = _softmax(np.array([0.2, 1.0, -0.5, 0.3, 0.0, -1.0, 0.8, 0.1]))
    U = np.broadcast_to(np.log(q1), (n, 1, V))
    d = draft_ref(U, None, None, np.zeros(n, dtype=np.int64), 1.0, 103, 0)
    P = np.empty((2 * n, V))
    P[0::2] = np.log(q1)          # p_1 == q_1: always accepted
    P[1::2] = np.log(p2)
    cu = np.arange(0, 2 * n + 1, 2)
    v = verify_ref(P, cu, U, None, None, np.zeros(n, dtype=np.int64), d["x"], 1.0, 103, 0)
    assert np.all(v["n_acc"] == 1) and np.all(v["mode"] == 0)
    counts = np.bincount(v["tok"], minlength=V)
    assert stats.chisquare(counts, p2 * n).pvalue > 1e-6


def test_printed_two_token_example_and_planted_mistake(monkeypatch):
    with open(os.path.join(GOLD, "appendix_a.json")) as f:
        g = json.load(f)
    p, q = np.array(g["target"]), np.array(g["draft"])
    n = 1_000_000
    _, v, first = _single_position_trials(p, q, n, seed=104)
    assert np.mean(v["n_acc"] == 1) == pytest.approx(g["acceptance"], abs=5 * np.sqrt(0.16 / n))
    pa = np.mean(first == 0)
    assert pa == pytest.approx(g["output_A_lossless"], abs=5 * np.sqrt(0.21 / n))
    assert stats.chisquare(np.bincount(first, minlength=2), p * n).pvalue > 1e-6
    # planted mistake: correction drawn from the whole target row
    monkeypatch.setattr(overify, "_correction_distribution", lambda pp, qq: pp.copy())
    _, _, bad = _single_position_trials(p, q, n, seed=104)
    assert np.mean(bad == 0) == pytest.approx(g["output_A_if_residual_were_full_target"], abs=5 * np.sqrt(0.23 / n))
    assert stats.chisquare(np.bincount(bad, minlength=2), p * n).pvalue < 1e-6


def test_expected_accepted_length_independent_positions():
    n, K, V = 1_000_000, 3, 8
    rng = np.random.default_rng(32)
    lq = rng.normal(0, 1, size=(K, V))
    lp = lq + rng.normal(0, 0.7, size=(K, V))
    lp_bonus = rng.normal(0, 1, size=V)
    U = np.broadcast_to(lq, (n, K, V))
    d = draft_ref(U, None, None, np.zeros(n, dtype=np.int64), 1.0, 105, 0)
    P = np.broadcast_to(np.vstack([lp, lp_bonus[None]]), (n, K + 1, V)).reshape(n * (K + 1), V)
    cu = np.arange(0, n * (K + 1) + 1, K + 1)
    v = verify_ref(P, cu, U, None, None, np.zeros(n, dtype=np.int64), d["x"], 1.0, 105, 0)
    alphas = [np.minimum(_softmax(lp[k]), _softmax(lq[k])).sum() for k in range(K)]
    expect = sum(np.prod(alphas[:k + 1]) for k in range(K))
    sd = v["n_acc"].std()
    assert abs(v["n_acc"].mean() - expect) < 5 * sd / np.sqrt(n)


def test_greedy_is_argmax_matching():
    rng = np.random.default_rng(33)
    R, K, V = 30, 4, 6
    D = rng.integers(-2, 3, size=(R, K, V)).astype(np.float64)
    T_rows = rng.integers(-2, 3, size=(R, K + 1, V)).astype(np.float64)
    x0 = rng.integers(0, V, size=R)
    x = np.argmax(D, axis=2)
    x[rng.uniform(size=(R, K)) < 0.3] = 0
    ell = rng.integers(0, K + 1, size=R)
    P = np.concatenate([T_rows[r, :ell[r] + 1] for r in range(R)])
    cu = np.concatenate([[0], np.cumsum(ell + 1)])
    v = verify_ref(P, cu, D, None, None, x0, x, 0.0, 9, 0)
    for r in range(R):
        n = 0
        while n < ell[r] and int(np.argmax(T_rows[r, n])) == x[r, n]:
            n += 1
        assert v["n_acc"][r] == n
        assert v["tok"][r] == int(np.argmax(T_rows[r, n]))


@pytest.mark.parametrize("mode,expect_key", [(SCHED_GLOBAL, "output_A_without_break"),
                                             (SCHED_EARLY_STOP, "output_A_lossless")])
def test_appendix_a_composed_monte_carlo(mode, expect_key):
    with open(os.path.join(GOLD, "appendix_a.json")) as f:
        g = json.load(f)
    sps = np.zeros(4)
    for b, val in g["sps_by_batch"].items():
        sps[int(b)] = val
    p, q = np.array(g["target"]), np.array(g["draft"])
    trials = 20000
    U = np.broadcast_to(np.log(q), (trials, 2, 2))
    d = draft_ref(U, None, None, np.zeros(trials, dtype=np.int64), 1.0, 106, 0)
    outs = np.empty(trials, dtype=np.int64)
    for t in range(trials):
        # the confidence of position 2 depends on the sampled x_1
        c2 = g["case_high"]["c2"] if d["x"][t, 0] == 0 else g["case_low"]["c2"]
        s = schedule_ref(np.array([[g["c1"], c2]], dtype=np.float32), sps, mode)
        ell = int(s["ell"][0])
        P = np.broadcast_to(np.log(p), (ell + 1, 2))
        v = verify_ref(P, [0, ell + 1], U[t:t + 1], None, None, [0], d["x"][t:t + 1], 1.0, 106, t + 1)
        outs[t] = d["x"][t, 0] if v["n_acc"][0] >= 1 else v["tok"][0]
    pa = np.mean(outs == 0)
    assert pa == pytest.approx(g[expect_key], abs=5 * np.sqrt(0.25 / trials))


def test_appendix_a_async_capacity_monte_carlo():
    """The same composed experiment with the asynchronous scheduler: the
    capacity comes from the no-break search over the confidences of an
    earlier, independent block (two steps back), the current block takes its
    top-capacity candidates.  The capacity then cannot see x_1, so the first
    emitted token is A with the target's probability 0.7, although the no-break
    search itself is used (it gives 0.85 when run on the current block)."""
    with open(os.path.join(GOLD, "appendix_a.json")) as f:
        g = json.load(f)
    sps = np.zeros(4)
    for b, val in g["sps_by_batch"].items():
        sps[int(b)] = val
    p, q = np.array(g["target"]), np.array(g["draft"])
    c2_of = lambda x1: g["case_high"]["c2"] if x1 == 0 else g["case_low"]["c2"]
    trials = 20000
    U = np.broadcast_to(np.log(q), (trials, 2, 2))
    d = draft_ref(U, None, None, np.zeros(trials, dtype=np.int64), 1.0, 107, 0)
    old = draft_ref(U, None, None, np.zeros(trials, dtype=np.int64), 1.0, 108, 0)   # the block two steps back
    outs = np.empty(trials, dtype=np.int64)
    caps = np.empty(trials, dtype=np.int64)
    for t in range(trials):
        c_now = np.array([[g["c1"], c2_of(d["x"][t, 0])]], dtype=np.float32)
        c_old = np.array([[g["c1"], c2_of(old["x"][t, 0])]], dtype=np.float32)
        s = schedule_async_ref(c_now, c_old, sps)
        caps[t] = s["capacity"]
        ell = int(s["ell"][0])
        P = np.broadcast_to(np.log(p), (ell + 1, 2))
        v = verify_ref(P, [0, ell + 1], U[t:t + 1], None, None, [0], d["x"][t:t + 1], 1.0, 107, t + 1)
        outs[t] = d["x"][t, 0] if v["n_acc"][0] >= 1 else v["tok"][0]
    # both capacities occur (2 after an old x_1 = A, 0 after B)
    assert set(np.unique(caps)) == {0, 2}
    pa = np.mean(outs == 0)
    assert pa == pytest.approx(g["output_A_lossless"], abs=5 * np.sqrt(0.21 / trials))


def test_end_to_end_zero_bias_equal_distributions_flat_sps():
    rng = np.random.default_rng(34)
    R, K, V = 12, 5, 40
    T = rng.normal(0, 2, size=(R, K + 1, V))
    x0 = rng.integers(0, V, size=R)
    c = rng.uniform(0.3, 1.0, size=(R, K)).astype(np.float32)
    sps = np.full(R * (K + 1) + 1, 2.0)
    out = run_step(T[:, :K], None, None, x0, c, sps, lambda r, n: T[r, :n], 1.0, 8, 0)
    assert np.all(out["schedule"]["ell"] == K)
    assert np.all(out["verify"]["n_acc"] == K)
    assert np.all(out["verify"]["mode"] == 0)
