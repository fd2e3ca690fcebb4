"""RNN-head drafter: the sequential stage with a recurrent state.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark paper, section 3.1, "Sequential stage", the "RNN
head" paragraph; "Speculative decoding, from zero to DSpark", section 6, on
carrying the whole in-block prefix instead of the last token): a state
s_k in R^r accumulates the prefix of the block.  At position k the head forms
the input

  z_k = [s_{k-1}; W1[x_{k-1}]; h_k]        (length 2r + d, s_0 = 0)

and applies one linear map W in R^{3r x (2r+d)} whose rows split, in order,
into the gate, candidate and output parts W_g, W_c, W_o.

The page's update equation did not survive extraction.  Reading adopted, a
plain GRU-style gated update with no additive bias (the page names only the
three matrices):

  g_k  = sigmoid(W_g z_k)
  c~_k = tanh(W_c z_k)
  o_k  = W_o z_k
  s_k  = (1 - g_k) * s_{k-1} + g_k * c~_k

and the output part stands where the Markov head has its embedding W1[x_{k-1}],
in front of the same logit projection W2:

  p_k(v | x_0, x_<k) = softmax_v( (U_k(v) + o_k . W2[:, v]) / T ).

With W_o = [0 | I | 0] the head is the Markov head exactly.  Sampling is the
Markov drafter's: an inverse-CDF draw with the uniform of (r, k, DRAFT), or the
first argmax when T = 0.  float64 throughout.
"""

import numpy as np

from .draft import _inverse_cdf, _first_argmax_and_gap
from .philox import uniform, PURPOSE_DRAFT


def _sigmoid(v):
    out = np.empty_like(v)
    pos = v >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-v[pos]))
    ev = np.exp(v[~pos])
    out[~pos] = ev / (1.0 + ev)
    return out


def rnn_cell_ref(s_prev, e_prev, h, W):
    """One gated update for a batch of rows.

    s_prev: [n, r] state s_{k-1}; e_prev: [n, r] embedding W1[x_{k-1}];
    h: [n, d] backbone hidden state h_k; W: [3r, 2r + d].
    Returns (s_k [n, r], o_k [n, r])."""
    s_prev = np.asarray(s_prev, dtype=np.float64)
    r = s_prev.shape[1]
    z = np.concatenate([s_prev, np.asarray(e_prev, dtype=np.float64), np.asarray(h, dtype=np.float64)], axis=1)
    pre = z @ np.asarray(W, dtype=np.float64).T          # [n, 3r] = W z_k per row
    g = _sigmoid(pre[:, :r])
    cand = np.tanh(pre[:, r:2 * r])
    o = pre[:, 2 * r:]
    s = (1.0 - g) * s_prev + g * cand
    return s, o


def rnn_draft_ref(U, H, W, W1, W2, x0, temperature, seed, step, request_ids=None):
    """Draft K tokens per request with the RNN head.

    U: [B, K, V] base logits; H: [B, K, d] backbone hidden states (h_k at
    [:, k-1]); W: [3r, 2r + d] (gate rows, candidate rows, output rows);
    W1: [V, r]; W2: [r, V]; x0: [B] anchors.  Returns the Markov drafter's
    dict (x, q_tok, lse, margin) plus O [B, K, r] (the output parts o_k, which
    verification needs to rebuild q) and S [B, K, r] (the states s_k).
    An anchor or drawn token outside [0, V) has no embedding: that request's
    remaining positions get x = -1 and NaN probabilities.
    """
    U = np.asarray(U, dtype=np.float64)
    H = np.asarray(H, dtype=np.float64)
    W1 = np.asarray(W1, dtype=np.float64)
    W2 = np.asarray(W2, dtype=np.float64)
    B, K, V = U.shape
    r = W1.shape[1]
    x0 = np.asarray(x0, dtype=np.int64)
    x = np.zeros((B, K), dtype=np.int64)
    q_tok = np.zeros((B, K))
    lse = np.zeros((B, K))
    margin = np.zeros((B, K))
    O = np.zeros((B, K, r))
    S = np.zeros((B, K, r))
    s = np.zeros((B, r))                                   # s_0 = 0
    rows = np.arange(B)
    requests = rows if request_ids is None else np.asarray(request_ids, dtype=np.int64)
    dead = np.zeros(B, dtype=bool)
    for k in range(1, K + 1):                              # left to right over the block
        prev = x0 if k == 1 else x[:, k - 2]
        dead |= (prev < 0) | (prev >= V)
        e = np.where(dead[:, None], 0.0, W1[np.clip(prev, 0, V - 1)])
        s, o = rnn_cell_ref(s, e, H[:, k - 1, :], W)
        O[:, k - 1] = o
        S[:, k - 1] = s
        logits = U[:, k - 1, :] + o @ W2
        if temperature == 0:
            tok, gap = _first_argmax_and_gap(logits)
            q_tok[:, k - 1] = 1.0
            lse[:, k - 1] = logits[rows, tok]
            margin[:, k - 1] = gap
        else:
            z = logits / temperature
            m = z.max(axis=1)
            w = np.exp(z - m[:, None])
            tot = w.sum(axis=1)
            q = w / tot[:, None]
            u = uniform(seed, step, requests, k, PURPOSE_DRAFT)
            tok, mg = _inverse_cdf(q, u)
            q_tok[:, k - 1] = q[rows, tok]
            lse[:, k - 1] = m + np.log(tot)
            margin[:, k - 1] = mg
        x[:, k - 1] = np.where(dead, -1, tok)
        q_tok[dead, k - 1] = np.nan
        lse[dead, k - 1] = np.nan
    return {"x": x, "q_tok": q_tok, "lse": lse, "margin": margin, "O": O, "S": S}
