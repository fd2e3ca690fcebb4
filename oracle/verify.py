"""Rejection-sampling verification over the flattened variable-length batch.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark paper, section 2.1; "Speculative decoding, from zero
to DSpark", section 2 and Appendix A1; the five-step verification routine in
the glean.smartcoder article):

  for each request r, walking its scheduled prefix left to right, j = 1..l_r:
      p_j = softmax(target logits of flat row cu[r] + j - 1 / T)
      q_j = the draft distribution of position j (Markov head, recomputed from
            the factored inputs, as the drafter defined it)
      accept x_j with probability min(1, p_j(x_j) / q_j(x_j)):
            u = uniform(r, j, ACCEPT); accept iff u < p_j(x_j) / q_j(x_j)
      at the first rejection: sample the correction from
            norm(max(0, p_j - q_j)) with uniform(r, j, RESAMPLE); stop
  if all l_r drafts survive: sample the bonus token from p_{l_r + 1}
      (flat row cu[r] + l_r) with uniform(r, l_r + 1, RESAMPLE).
  Emitted tokens: x_1..x_{n_acc}, then the correction or bonus token.

A request with l_r = 0 still sends its anchor row and gets one token back
("Speculative decoding, from zero to DSpark", section 8, the two +1 terms).

Readings where the pages leave a step open:
  * strict test u < ratio with u in [0, 1) gives probability min(1, ratio);
  * q_j(x_j) = 0 can only come from underflow: the draft is then accepted;
  * a residual mass of zero (possible only through rounding, since the
    rejection probability equals it) falls back to sampling from p_j;
  * T = 0 is greedy verification: accept iff the first argmax of the target
    row equals x_j; the correction or bonus token is that first argmax.
"""

import numpy as np

from .philox import uniform, PURPOSE_ACCEPT, PURPOSE_RESAMPLE


def _softmax(z):
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    return w / w.sum(axis=1, keepdims=True)


def _correction_distribution(p, q):
    """Unnormalised residual max(0, p - q) (Appendix A1 of the blog post)."""
    return np.maximum(p - q, 0.0)


def _inverse_cdf_unnormalised(w, u):
    """First v with cumsum(w)[v] > u * sum(w), per row; margin relative to sum."""
    cdf = np.cumsum(w, axis=1)
    total = cdf[:, -1]
    target = u * total
    idx = (cdf <= target[:, None]).sum(axis=1)
    V = w.shape[1]
    for i in np.nonzero(idx >= V)[0]:
        idx[i] = np.nonzero(w[i] > 0)[0][-1]
    rows = np.arange(w.shape[0])
    upper = cdf[rows, idx]
    lower = np.where(idx > 0, cdf[rows, np.maximum(idx - 1, 0)], 0.0)
    margin = np.minimum(np.abs(upper - target), np.abs(target - lower)) / total
    return idx, margin


def _top2_gap(z, idx):
    rows = np.arange(z.shape[0])
    other = z.copy()
    other[rows, idx] = -np.inf
    return z[rows, idx] - other.max(axis=1)


def verify_ref(P, cu_seqlens, D, W1, W2, x0, x, temperature, seed, step, request_ids=None, O=None):
    """Verify every request's scheduled prefix.

    P: [N, V] flat target logits (request r owns rows cu[r] .. cu[r+1]-1);
    cu_seqlens: [R+1]; D: [R, K, V] draft base logits; W1 [V, r] / W2 [r, V]
    or None; x0: [R] anchors; x: [R, K] draft tokens; temperature (0 = greedy);
    request_ids: the requests' indices in their batch, which address their
    uniforms (default 0..R-1); O: [R, K, r] or None.  With O (drafts of the
    RNN head) the draft row of position j carries the bias O[r, j-1] @ W2, the
    head's output part in place of the Markov embedding, and W1 is not used.

    Returns dict: n_acc [R], tok [R] (correction or bonus token), mode [R]
    (0 = bonus, 1 = correction), p_x / q_x / ratio [R, K] (NaN where a position
    was not examined), accept_margin [R, K] (|u - ratio|, or the target's top-2
    logit gap when greedy; NaN where not examined), sample_margin [R].
    """
    P = np.asarray(P, dtype=np.float64)
    D = np.asarray(D, dtype=np.float64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    x = np.asarray(x, dtype=np.int64)
    x0 = np.asarray(x0, dtype=np.int64)
    R, K, V = D.shape
    if O is not None:
        O = np.asarray(O, dtype=np.float64)
        have_bias = True
    else:
        have_bias = W1 is not None and W2 is not None and np.asarray(W1).shape[1] > 0
    if have_bias:
        if O is None:
            W1 = np.asarray(W1, dtype=np.float64)
        W2 = np.asarray(W2, dtype=np.float64)
    ell = cu[1:] - cu[:-1] - 1
    if np.any(ell < 0) or np.any(ell > K) or cu[0] != 0 or cu[-1] != P.shape[0]:
        raise ValueError("inconsistent cu_seqlens")
    greedy = temperature == 0
    ids = np.arange(R) if request_ids is None else np.asarray(request_ids, dtype=np.int64)

    n_acc = np.full(R, -1, dtype=np.int64)
    tok = np.full(R, -1, dtype=np.int64)
    mode = np.full(R, -1, dtype=np.int64)
    p_x = np.full((R, K), np.nan)
    q_x = np.full((R, K), np.nan)
    ratio_out = np.full((R, K), np.nan)
    accept_margin = np.full((R, K), np.nan)
    sample_margin = np.full(R, np.nan)

    alive = np.ones(R, dtype=bool)
    for j in range(1, K + 1):                        # left to right
        rs = np.nonzero(alive & (ell >= j))[0]
        if rs.size == 0:
            continue
        t_rows = P[cu[rs] + j - 1]
        xj = x[rs, j - 1]
        if greedy:
            top = np.argmax(t_rows, axis=1)
            gap = _top2_gap(t_rows, top)
            accepted = top == xj
            accept_margin[rs, j - 1] = gap
            rej = rs[~accepted]
            n_acc[rej] = j - 1
            tok[rej] = top[~accepted]
            mode[rej] = 1
            sample_margin[rej] = gap[~accepted]
            alive[rej] = False
            continue
        p = _softmax(t_rows / temperature)
        base = D[rs, j - 1, :].copy()
        if O is not None:
            base += O[rs, j - 1, :] @ W2
        elif have_bias:
            prev = x0[rs] if j == 1 else x[rs, j - 2]
            base += W1[prev, :] @ W2
        q = _softmax(base / temperature)
        rows = np.arange(rs.size)
        pj, qj = p[rows, xj], q[rows, xj]
        with np.errstate(divide="ignore", invalid="ignore"):
            ratio = np.where(qj > 0, pj / qj, np.inf)
        u = uniform(seed, step, ids[rs], j, PURPOSE_ACCEPT)
        accepted = u < ratio
        p_x[rs, j - 1], q_x[rs, j - 1], ratio_out[rs, j - 1] = pj, qj, ratio
        accept_margin[rs, j - 1] = np.abs(u - ratio)
        if np.all(accepted):
            continue
        sel = ~accepted
        rej = rs[sel]
        resid = _correction_distribution(p[sel], q[sel])
        zero = resid.sum(axis=1) <= 0
        resid[zero] = p[sel][zero]
        u2 = uniform(seed, step, ids[rej], j, PURPOSE_RESAMPLE)
        y, mg = _inverse_cdf_unnormalised(resid, u2)
        n_acc[rej] = j - 1
        tok[rej] = y
        mode[rej] = 1
        sample_margin[rej] = mg
        alive[rej] = False

    rs = np.nonzero(alive)[0]                        # whole prefix survived
    if rs.size:
        rows_bonus = P[cu[rs] + ell[rs]]
        n_acc[rs] = ell[rs]
        mode[rs] = 0
        if greedy:
            top = np.argmax(rows_bonus, axis=1)
            tok[rs] = top
            sample_margin[rs] = _top2_gap(rows_bonus, top)
        else:
            p = _softmax(rows_bonus / temperature)
            u2 = uniform(seed, step, ids[rs], ell[rs] + 1, PURPOSE_RESAMPLE)
            y, mg = _inverse_cdf_unnormalised(p, u2)
            tok[rs] = y
            sample_margin[rs] = mg
    return {"n_acc": n_acc, "tok": tok, "mode": mode, "p_x": p_x, "q_x": q_x,
            "ratio": ratio_out, "accept_margin": accept_margin,
            "sample_margin": sample_margin}
