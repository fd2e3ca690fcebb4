"""Pins for the confidence head, the ECE and STS.

The head is pinned through the Markov-embedding index it gathers (an
embedding table that encodes each token's id), the ECE by hand-worked bins,
and STS by a synthetic held-out set drawn from a known calibrated model:
the fit must recover the temperatures that generated the survival labels.
"""
import numpy as np
import pytest

from oracle.confidence import confidence_head_ref, confidence_logits_ref, ece_ref, sts_fit_ref


def test_head_gathers_the_previous_token_embedding():
    """W1 row v = (v, 1): with w_e = (1, 0) the logit is the previous token's
    id, the anchor at position 1 and x_{k-1} after it; h and w_h add a known
    constant."""
    V, R, K, d = 50, 3, 4, 6
    W1 = np.stack([np.arange(V, dtype=np.float64), np.ones(V)], axis=1)
    x0 = np.array([7, 20, 41])
    x = np.array([[3, 9, 11, 2], [0, 49, 5, 6], [8, 8, 8, 8]])
    H = np.ones((R, K, d))
    w_h = np.full(d, 0.5)
    z = confidence_logits_ref(H, w_h, np.array([1.0, 0.0]), -2.0, W1, x0, x)
    prev = np.array([[7, 3, 9, 11], [20, 0, 49, 5], [41, 8, 8, 8]])
    np.testing.assert_array_equal(z, prev + 0.5 * d - 2.0)


def test_head_values_and_temperature_order():
    rng = np.random.default_rng(5)
    R, K, d, r, V = 40, 5, 16, 8, 30
    H = rng.normal(size=(R, K, d))
    W1 = rng.normal(size=(V, r))
    x0 = rng.integers(0, V, size=R)
    x = rng.integers(0, V, size=(R, K))
    w_h, w_e = rng.normal(size=d), rng.normal(size=r)
    c = confidence_head_ref(H, w_h, w_e, 0.3, W1, x0, x)
    assert np.all((c > 0) & (c < 1))
    # sigmoid(0) = 1/2 and sigmoid(-z) = 1 - sigmoid(z)
    zero = confidence_head_ref(np.zeros((1, 1, d)), w_h, None, 0.0, None, [0], [[0]])
    assert zero[0, 0] == 0.5
    neg = confidence_head_ref(-H, w_h, None, 0.0, None, x0, x)
    np.testing.assert_allclose(neg, 1 - confidence_head_ref(H, w_h, None, 0.0, None, x0, x), atol=1e-15)
    # temperature scaling keeps every position's ranking of requests
    T = np.array([0.3, 0.7, 1.0, 2.5, 9.0])
    cT = confidence_head_ref(H, w_h, w_e, 0.3, W1, x0, x, T)
    for k in range(K):
        np.testing.assert_array_equal(np.argsort(cT[:, k], kind="stable"), np.argsort(c[:, k], kind="stable"))
    # a very large temperature flattens everything to one half
    big = confidence_head_ref(H, w_h, w_e, 0.3, W1, x0, x, np.full(K, 1e9))
    np.testing.assert_allclose(big, 0.5, atol=1e-7)


def test_ece_hand_worked():
    # two bins of 0.5: [0.1, 0.2 | labels 0, 1] and [0.8, 0.9, 0.7 | labels 1, 1, 0]
    pred = np.array([0.1, 0.2, 0.8, 0.9, 0.7])
    lab = np.array([0, 1, 1, 1, 0])
    expect = 2 / 5 * abs(0.5 - 0.15) + 3 / 5 * abs(2 / 3 - 0.8)
    assert ece_ref(pred, lab, 2) == pytest.approx(expect, abs=1e-15)
    # a prediction of exactly 1 falls in the last bin; perfect calibration has zero error
    assert ece_ref([1.0, 1.0, 0.0], [1, 1, 0], 4) == 0.0
    # a single bin: |mean label - mean prediction|
    assert ece_ref(pred, lab, 1) == pytest.approx(abs(lab.mean() - pred.mean()), abs=1e-15)
    # a sample with no prediction (NaN) is in no bin but counts in the total:
    # the hand-worked sums over 6 samples instead of 5
    pn = np.append(pred, np.nan)
    ln = np.append(lab, 1)
    assert ece_ref(pn, ln, 2) == pytest.approx(expect * 5 / 6, abs=1e-15)


def test_sts_recovers_generating_temperatures():
    """Held-out set from a known model: the true conditional acceptance at
    position k is sigmoid(logit / T*_k); prefix survival is drawn left to
    right.  STS with the cumulative-product ECE recovers T*."""
    rng = np.random.default_rng(11)
    N, K = 60000, 4
    T_true = np.array([2.0, 1.5, 0.8, 1.2])
    logits = rng.normal(1.5, 2.0, size=(N, K))
    p_cond = 1.0 / (1.0 + np.exp(-logits / T_true))
    alive = np.ones(N, dtype=bool)
    survived = np.zeros((N, K))
    for k in range(K):
        alive &= rng.uniform(size=N) < p_cond[:, k]
        survived[:, k] = alive
    grid = np.exp(np.linspace(np.log(0.25), np.log(4.0), 121))
    T, ece = sts_fit_ref(logits, survived, grid, n_bins=15)
    np.testing.assert_allclose(T, T_true, rtol=0.12)
    assert np.all(ece < 0.02)
    # an already calibrated head fits temperatures near 1
    T1, _ = sts_fit_ref(logits / T_true, survived, grid, n_bins=15)
    np.testing.assert_allclose(T1, 1.0, rtol=0.12)
