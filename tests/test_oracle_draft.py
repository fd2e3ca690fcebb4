"""Pins for the oracle's sequential Markov-head drafter.

* zero Markov bias reduces to the independent per-position sampler (a plain
  scalar loop over the inverse CDF, written separately in the oracle);
* a constructed deterministic chain whose tokens have a closed form pins the
  gather index, the anchor at position 1 and the left-to-right dependency;
* chi-square of the drawn token against softmax(U) on V = 8, 10^6 draws;
* greedy mode equals a plain first-argmax loop;
* q(x) and the log-normaliser agree with scipy's logsumexp.
"""
import numpy as np
import pytest
from scipy import stats
from scipy.special import logsumexp

from oracle.draft import draft_ref, independent_draft_ref


@pytest.mark.parametrize("temperature", [1.0, 0.7, 0.0])
def test_zero_bias_reduces_to_independent_sampler(temperature):
    rng = np.random.default_rng(21)
    B, K, V, r = 5, 4, 12, 4
    U = rng.normal(0, 2, size=(B, K, V))
    x0 = rng.integers(0, V, size=B)
    W1 = rng.normal(0, 1, size=(V, r))
    W2 = np.zeros((r, V))
    a = draft_ref(U, W1, W2, x0, temperature, seed=99, step=3)["x"]
    b = draft_ref(U, None, None, x0, temperature, seed=99, step=3)["x"]
    c = independent_draft_ref(U, temperature, seed=99, step=3)
    np.testing.assert_array_equal(a, c)
    np.testing.assert_array_equal(b, c)


def test_markov_chain_closed_form():
    """V = r = 8, W1 = lam*Q, W2 = lam*Pi (permutation matrices), U = 0.

    B(prev, v) = lam^2 * (Q Pi)[prev, v], so with lam^2 = 50 every draw is the
    successor sigma(prev) = the column of the 1 in row prev of Q Pi, except with
    probability about 7 e^-50.  Hence x_k = sigma^k(x_0)."""
    V = 8
    rng = np.random.default_rng(22)
    q_perm = rng.permutation(V)
    pi_perm = rng.permutation(V)
    Q = np.eye(V)[q_perm]            # Q[i, q_perm[i]] = 1
    Pi = np.eye(V)[pi_perm]
    lam = np.sqrt(50.0)
    W1, W2 = lam * Q, lam * Pi
    succ = lambda t: pi_perm[q_perm[t]]
    K = 7
    x0 = np.arange(V)
    out = draft_ref(np.zeros((V, K, V)), W1, W2, x0, 1.0, seed=5, step=0)
    expect = np.zeros((V, K), dtype=np.int64)
    for b in range(V):
        t = x0[b]
        for k in range(K):
            t = succ(t)
            expect[b, k] = t
    np.testing.assert_array_equal(out["x"], expect)
    assert np.all(out["q_tok"] > 1 - 1e-15)
    # the transposed factor would walk the inverse permutation instead
    back = draft_ref(np.zeros((V, K, V)), W1, W2.T.copy(), x0, 1.0, seed=5, step=0)["x"]
    assert not np.array_equal(back, expect)


def test_draw_follows_softmax_chi_square():
    n = 1_000_000
    V = 8
    row = np.array([0.3, -1.0, 2.0, 0.0, 1.1, -0.4, 0.9, -2.5])
    q = np.exp(row - logsumexp(row))
    U = np.broadcast_to(row, (n, 1, V))
    x = draft_ref(U, None, None, np.zeros(n, dtype=np.int64), 1.0, seed=77, step=0)["x"][:, 0]
    counts = np.bincount(x, minlength=V)
    chi2, pval = stats.chisquare(counts, q * n)
    assert pval > 1e-6


def test_greedy_is_first_argmax_of_biased_logits():
    rng = np.random.default_rng(23)
    B, K, V, r = 6, 5, 20, 3
    U = np.round(rng.normal(0, 1, size=(B, K, V)))      # many exact ties
    W1 = np.round(rng.normal(0, 1, size=(V, r)))
    W2 = np.round(rng.normal(0, 1, size=(r, V)))
    x0 = rng.integers(0, V, size=B)
    out = draft_ref(U, W1, W2, x0, 0.0, seed=1, step=0)
    for b in range(B):
        prev = x0[b]
        for k in range(K):
            vals = [U[b, k, v] + sum(W1[prev, i] * W2[i, v] for i in range(r)) for v in range(V)]
            best = max(vals)
            expect = vals.index(best)
            assert out["x"][b, k] == expect
            assert out["q_tok"][b, k] == 1.0
            prev = expect


def test_probabilities_and_normaliser():
    rng = np.random.default_rng(24)
    B, K, V, r = 4, 3, 50, 8
    U = rng.normal(0, 3, size=(B, K, V))
    W1 = rng.normal(0, 0.3, size=(V, r))
    W2 = rng.normal(0, 0.3, size=(r, V))
    x0 = rng.integers(0, V, size=B)
    T = 0.8
    out = draft_ref(U, W1, W2, x0, T, seed=3, step=1)
    for b in range(B):
        prev = x0[b]
        for k in range(K):
            z = (U[b, k] + W1[prev] @ W2) / T
            assert out["lse"][b, k] == pytest.approx(logsumexp(z), rel=1e-12)
            assert out["q_tok"][b, k] == pytest.approx(np.exp(z[out["x"][b, k]] - logsumexp(z)), rel=1e-10)
            prev = out["x"][b, k]
    # temperature only rescales the logits
    a = draft_ref(U, None, None, x0, 2.0, seed=3, step=1)
    b2 = draft_ref(U / 2.0, None, None, x0, 1.0, seed=3, step=1)
    np.testing.assert_array_equal(a["x"], b2["x"])
