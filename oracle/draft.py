"""Sequential Markov-head drafter (the semi-autoregressive sequential stage).

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark paper, section 3.1, "Sequential stage" and "Markov
head"; restated in "Speculative decoding, from zero to DSpark", section 6 and
Appendix A4):

  p_k(v | x_0, x_<k) = softmax_v( U_k(v) + B(x_{k-1}, v) ),
  B(x_{k-1}, .)      = W1[x_{k-1}, :] @ W2,   W1 in R^{V x r}, W2 in R^{r x V},

sampled left to right for k = 1..K, the anchor x_0 being the previous round's
final token.  The bias is applied at every position, the first one included,
where it is looked up from the anchor (reading adopted where the page's toy
example is garbled).  Temperature T > 0 divides the biased logits; T = 0 is
greedy (first argmax).  Each draw is an inverse-CDF draw in ascending token id
with the uniform of (r, k, DRAFT); the exact probability q_k(x_k) and the
log-normaliser are kept, since verification needs exact draft probabilities
(DSpark paper, section 6, Related Work, the parallel-generation paragraph:
the sequential correction stays local so per-token probabilities remain exact).

All arithmetic is float64 on float64 inputs (bf16 and fp32 inputs convert
exactly).
"""

import numpy as np

from .philox import uniform, PURPOSE_DRAFT


def _inverse_cdf(prob, u):
    """Index of the first v with cdf[v] > u, per row, and the decision margin.

    prob: [n, V] rows summing to ~1; u: [n].  If rounding leaves u above the
    whole cdf, the last index with positive mass is taken.  The margin is the
    distance from u to the nearer cdf boundary of the chosen bin.
    """
    cdf = np.cumsum(prob, axis=1)
    idx = (cdf <= u[:, None]).sum(axis=1)
    V = prob.shape[1]
    over = idx >= V
    if np.any(over):
        for i in np.nonzero(over)[0]:
            idx[i] = np.nonzero(prob[i] > 0)[0][-1]
    rows = np.arange(prob.shape[0])
    upper = cdf[rows, idx]
    lower = np.where(idx > 0, cdf[rows, np.maximum(idx - 1, 0)], 0.0)
    margin = np.minimum(np.abs(upper - u), np.abs(u - lower))
    return idx, margin


def _first_argmax_and_gap(z):
    """First argmax per row and the gap to the best other entry (greedy margin)."""
    idx = np.argmax(z, axis=1)
    rows = np.arange(z.shape[0])
    best = z[rows, idx]
    other = z.copy()
    other[rows, idx] = -np.inf
    gap = best - other.max(axis=1) if z.shape[1] > 1 else np.full(z.shape[0], np.inf)
    return idx, gap


def draft_ref(U, W1, W2, x0, temperature, seed, step, request_ids=None):
    """Draft K tokens per request with the Markov head.

    U: [B, K, V] base logits; W1: [V, r] or None; W2: [r, V] or None (r = 0,
    no Markov head); x0: [B] anchors; temperature: float (0 = greedy);
    request_ids: the requests' indices in their batch, which address their
    uniforms (default 0..B-1; a subset of a batch passes its own indices).
    Returns dict with x [B, K] int64, q_tok [B, K] (q_k(x_k); 1 when greedy),
    lse [B, K] (log sum_v exp(z_k(v)); the max biased logit when greedy) and
    margin [B, K] (distance of the uniform from the chosen CDF bin's edges, or
    the top-2 logit gap when greedy).
    """
    U = np.asarray(U, dtype=np.float64)
    B, K, V = U.shape
    x0 = np.asarray(x0, dtype=np.int64)
    have_bias = W1 is not None and W2 is not None and np.asarray(W1).shape[1] > 0
    if have_bias:
        W1 = np.asarray(W1, dtype=np.float64)
        W2 = np.asarray(W2, dtype=np.float64)
    x = np.zeros((B, K), dtype=np.int64)
    q_tok = np.zeros((B, K))
    lse = np.zeros((B, K))
    margin = np.zeros((B, K))
    rows = np.arange(B)
    requests = rows if request_ids is None else np.asarray(request_ids, dtype=np.int64)
    for k in range(1, K + 1):                       # left to right over the block
        prev = x0 if k == 1 else x[:, k - 2]
        logits = U[:, k - 1, :].copy()
        if have_bias:
            logits += W1[prev, :] @ W2              # B(x_{k-1}, .) for every request
        if temperature == 0:
            tok, gap = _first_argmax_and_gap(logits)
            x[:, k - 1] = tok
            q_tok[:, k - 1] = 1.0
            lse[:, k - 1] = logits[rows, tok]
            margin[:, k - 1] = gap
            continue
        z = logits / temperature
        m = z.max(axis=1)
        w = np.exp(z - m[:, None])
        s = w.sum(axis=1)
        q = w / s[:, None]
        u = uniform(seed, step, requests, k, PURPOSE_DRAFT)
        tok, mg = _inverse_cdf(q, u)
        x[:, k - 1] = tok
        q_tok[:, k - 1] = q[rows, tok]
        lse[:, k - 1] = m + np.log(s)
        margin[:, k - 1] = mg
    return {"x": x, "q_tok": q_tok, "lse": lse, "margin": margin}


def independent_draft_ref(U, temperature, seed, step):
    """The parallel drafter with no sequential head: position k sampled from
    softmax(U_k / T) alone, with the same uniforms.  With a zero Markov bias the
    sequential drafter must reduce to exactly this (DSpark paper, section 3.1:
    the backbone alone predicts each position independently)."""
    U = np.asarray(U, dtype=np.float64)
    B, K, V = U.shape
    x = np.zeros((B, K), dtype=np.int64)
    for k in range(1, K + 1):
        for b in range(B):
            row = U[b, k - 1]
            if temperature == 0:
                x[b, k - 1] = int(np.argmax(row))
                continue
            u = float(uniform(seed, step, b, k, PURPOSE_DRAFT))
            top = max(row) / temperature
            weights = [np.exp(val / temperature - top) for val in row]
            total = sum(weights)
            acc = 0.0
            choice = V - 1
            for v, wv in enumerate(weights):
                acc += wv / total
                if acc > u:
                    choice = v
                    break
            x[b, k - 1] = choice
    return x
