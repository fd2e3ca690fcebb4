"""Confidence head and Sequential Temperature Scaling (STS).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes:
  * the head (DSpark paper, section 3.2.1, Confidence Head; "Speculative
    decoding, from zero to DSpark", section 8, The confidence head): one
    linear projection of the backbone hidden state h_{r,k} and the Markov
    embedding W1[x_{r,k-1}] of the previous token, then a sigmoid:
        c_{r,k} = sigmoid((w_h . h_{r,k} + w_e . W1[x_{r,k-1}] + b) / T_k)
    with x_{r,0} the anchor and T_k the position's STS temperature (1 before
    calibration).  The paper's equation is lost in the copy we have; the
    blog's description (single linear projection + sigmoid over the two
    inputs) is what is implemented, the temperature dividing the logit as in
    temperature scaling;
  * STS (DSpark paper, section 3.2.1, Post-hoc Calibration; "Speculative
    decoding, from zero to DSpark", Appendix A5): on held-out data, walking
    k = 1..K left to right, T_k is the grid value minimising the expected
    calibration error of the cumulative product a_k = prod_{i<=k} c_i against
    the observed prefix survival (positions 1..k all accepted), with
    T_1..T_{k-1} already fixed.

Readings where the pages leave a step open: the ECE (Naeini et al., 2015)
uses n_bins equal-width bins on [0, 1], the last one closed, each bin
weighted by its share of samples; the grid is given by the caller; equal
ECE values keep the first grid value.
"""

import numpy as np


def _sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    e = np.exp(z[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def confidence_logits_ref(H, w_h, w_e, bias, W1, x0, x):
    """H [R, K, d]; w_h [d]; w_e [r] (or None with W1 None); W1 [V, r];
    x0 [R]; x [R, K].  Returns the head's logits [R, K] before temperature."""
    H = np.asarray(H, dtype=np.float64)
    R, K, _ = H.shape
    z = H @ np.asarray(w_h, dtype=np.float64) + float(bias)
    if W1 is not None and w_e is not None and np.asarray(W1).shape[1] > 0:
        W1 = np.asarray(W1, dtype=np.float64)
        x = np.asarray(x, dtype=np.int64)
        prev = np.concatenate([np.asarray(x0, dtype=np.int64)[:, None], x[:, :K - 1]], axis=1)
        z = z + W1[prev] @ np.asarray(w_e, dtype=np.float64)
    return z


def confidence_head_ref(H, w_h, w_e, bias, W1, x0, x, temperatures=None):
    z = confidence_logits_ref(H, w_h, w_e, bias, W1, x0, x)
    T = np.ones(z.shape[1]) if temperatures is None else np.asarray(temperatures, dtype=np.float64)
    return _sigmoid(z / T[None, :])


def ece_ref(pred, label, n_bins):
    """Expected calibration error of predictions in [0, 1] against 0/1 labels.
    A sample without a prediction (NaN, from a NaN logit) falls in no bin but
    still counts in the sample total."""
    pred = np.asarray(pred, dtype=np.float64)
    label = np.asarray(label, dtype=np.float64)
    b = np.full(pred.shape, -1, dtype=np.int64)
    ok = ~np.isnan(pred)
    b[ok] = np.minimum((pred[ok] * n_bins).astype(np.int64), n_bins - 1)
    total = 0.0
    for i in range(n_bins):
        m = b == i
        if m.any():
            total += m.sum() / pred.size * abs(label[m].mean() - pred[m].mean())
    return total


def sts_fit_ref(logits, survived, grid, n_bins=10):
    """logits [N, K] (the head's logits on held-out data); survived [N, K]
    (1 where positions 1..k were all accepted); grid [G] candidate
    temperatures.  Returns (T [K], ece [K] at the chosen temperatures)."""
    logits = np.asarray(logits, dtype=np.float64)
    survived = np.asarray(survived, dtype=np.float64)
    grid = np.asarray(grid, dtype=np.float64)
    N, K = logits.shape
    prod = np.ones(N)
    T = np.empty(K)
    best_ece = np.empty(K)
    for k in range(K):
        errs = [ece_ref(prod * _sigmoid(logits[:, k] / t), survived[:, k], n_bins) for t in grid]
        g = int(np.argmin(errs))                 # first minimum
        T[k], best_ece[k] = grid[g], errs[g]
        prod = prod * _sigmoid(logits[:, k] / T[k])
    return T, best_ece
