"""Pins for the analytic acceptance label c* = 1 - 1/2 ||q - p||_1.

Each test fixes the oracle against something other than its own formula: the
pages' printed two-token example, the acceptance frequency of the verifier's
sampled decisions, a closed form for two point-mass-like distributions, and
the greedy limit.
"""
import json
import os

import numpy as np
import pytest

from oracle.draft import draft_ref
from oracle.label import acceptance_label_ref
from oracle.verify import verify_ref

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_printed_two_token_example():
    """The pages' example: target (0.7, 0.3), draft (0.5, 0.5), acceptance 0.8."""
    with open(os.path.join(GOLD, "appendix_a.json")) as f:
        g = json.load(f)
    p, q = np.array(g["target"]), np.array(g["draft"])
    c = acceptance_label_ref(np.log(p)[None, None], np.log(q)[None, None], None, None, [0], [[0]], 1.0)
    assert c[0, 0] == pytest.approx(g["acceptance"], abs=1e-12)


def test_equals_acceptance_frequency_of_the_verifier():
    """c*_{r,1} is the probability that verification accepts position 1: the
    fraction of accepted first positions over many seeded draws matches it
    (Markov bias on, so q depends on the anchor through W1 W2)."""
    rng = np.random.default_rng(41)
    R, V, r = 4000, 12, 4
    base_p = rng.normal(0, 1.5, size=V)
    base_d = base_p + rng.normal(0, 1.0, size=V)
    U = np.broadcast_to(base_d, (R, 1, V)).copy()
    W1 = rng.normal(0, 0.4, size=(V, r))
    W2 = rng.normal(0, 0.4, size=(r, V))
    x0 = np.full(R, 3)
    P = np.broadcast_to(base_p, (R, 1, V)).copy()
    d = draft_ref(U, W1, W2, x0, 1.0, 55, 0)
    c = acceptance_label_ref(P, U, W1, W2, x0, d["x"], 1.0)
    assert np.allclose(c, c[0, 0])
    # one scheduled draft per request: its judging row, then a bonus row
    flat = np.stack([P[:, 0, :], np.zeros((R, V))], axis=1).reshape(2 * R, V)
    v = verify_ref(flat, np.arange(0, 2 * R + 1, 2), U, W1, W2, x0, d["x"], 1.0, 55, 0)
    freq = np.mean(v["n_acc"] >= 1)
    assert freq == pytest.approx(c[0, 0], abs=5 * np.sqrt(0.25 / R))


def test_closed_form_shifted_logits():
    """Two distributions that differ only in one logit: p = softmax(0, .., 0)
    and q = the same with logit 0 raised by s.  Then
    sum_v min(p, q) = (V - 1) / (V - 1 + e^s) + 1 / V for s > 0."""
    V, s = 9, 1.7
    P = np.zeros((1, 1, V))
    D = np.zeros((1, 1, V))
    D[0, 0, 0] = s
    c = acceptance_label_ref(P, D, None, None, [0], [[0]], 1.0)
    assert c[0, 0] == pytest.approx((V - 1) / (V - 1 + np.exp(s)) + 1.0 / V, rel=1e-12)


def test_identity_temperature_and_greedy_limit():
    rng = np.random.default_rng(2)
    R, K, V = 5, 3, 30
    D = rng.normal(0, 2, size=(R, K, V))
    x = np.argmax(D, axis=2)
    # identical distributions accept with probability 1 at any temperature
    for T in (0.5, 1.0, 3.0):
        assert np.allclose(acceptance_label_ref(D, D, None, None, np.zeros(R, int), x, T), 1.0)
    # greedy: 1 exactly where the target's argmax is the drafted token
    P = D.copy()
    P[1, 2] = -P[1, 2]
    c = acceptance_label_ref(P, D, None, None, np.zeros(R, int), x, 0.0)
    expect = (np.argmax(P, axis=2) == x).astype(float)
    np.testing.assert_array_equal(c, expect)
    assert c[1, 2] == 0.0 and c.sum() == R * K - 1
