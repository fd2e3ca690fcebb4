"""Analytic per-position acceptance probability (the confidence head's label).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark paper, section 3.2.1, Confidence Head: the label is
the per-step acceptance rate fixed by the total variation distance between
the draft and target distributions, and section 3.3 on the TV loss;
"Speculative decoding, from zero to DSpark", section 2 and Appendix A4):

  c*_{r,k} = 1 - 1/2 * || q_{r,k} - p_{r,k} ||_1 = sum_v min(q_{r,k}(v), p_{r,k}(v))

with q_{r,k} the Markov drafter's distribution at position k (base logits
plus the bias W1[x_{r,k-1}] W2 from the drafted previous token, x_{r,0} the
anchor) and p_{r,k} = softmax(t_{r,k} / T) the target distribution that judges
position k.  It is the probability that position k is accepted given the
earlier positions were.

Reading where the pages leave a step open: at T = 0 both distributions are
the point masses on their first argmax, so c* is 1 when the target's argmax
equals the drafted token x_{r,k} (the drafter's argmax) and 0 otherwise.
"""

import numpy as np


def _softmax_rows(z):
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    return w / w.sum(axis=1, keepdims=True)


def acceptance_label_ref(P, D, W1, W2, x0, x, temperature, O=None):
    """P: [R, K, V] target logits (row (r, k) judges draft position k+1);
    D: [R, K, V] draft base logits; W1 [V, r], W2 [r, V] or None; x0 [R];
    x [R, K] drafted tokens; O [R, K, r] or None (drafts of the RNN head: the
    bias of position k is O[r, k] @ W2 and W1 is not used).  Returns c* [R, K]
    (float64)."""
    P = np.asarray(P, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    x = np.asarray(x, dtype=np.int64)
    x0 = np.asarray(x0, dtype=np.int64)
    R, K, V = D.shape
    if O is not None:
        O = np.asarray(O, dtype=np.float64)
        W2 = np.asarray(W2, dtype=np.float64)
        have_bias = False
    else:
        have_bias = W1 is not None and W2 is not None and np.asarray(W1).shape[1] > 0
    if have_bias:
        W1 = np.asarray(W1, dtype=np.float64)
        W2 = np.asarray(W2, dtype=np.float64)
    out = np.empty((R, K))
    for k in range(K):
        prev = x0 if k == 0 else x[:, k - 1]
        if O is not None:
            z = D[:, k, :] + O[:, k, :] @ W2
        else:
            z = D[:, k, :] + (W1[prev] @ W2 if have_bias else 0.0)
        t = P[:, k, :]
        if temperature == 0:
            out[:, k] = (np.argmax(t, axis=1) == x[:, k]).astype(np.float64)
            continue
        q = _softmax_rows(z / temperature)
        p = _softmax_rows(t / temperature)
        out[:, k] = np.minimum(p, q).sum(axis=1)
    return out
