"""Hardware-aware prefix scheduler (Algorithm 1) and its section-5.2 modes.

TEST INFRASTRUCTURE ONLY (see the package docstring).

What it computes (DSpark paper, section 3.2.2 and Algorithm 1; the Paperglide
reader's clean restatement of the algorithm; "Speculative decoding, from zero
to DSpark", section 8):

  a_{r,j} = prod_{i<=j} c_{r,i}                       (prefix survival)
  E       = {(r, j) : a_{r,j} > 0}, sorted by a descending
  start   : l_r = 0, B = R, tau = R, Theta_best = R * SPS(R)
  for each (r, j) in sorted order:
      l_r = j; B += 1; tau += a_{r,j}; Theta = tau * SPS(B)
      if Theta > Theta_best: Theta_best = Theta; l* = l
      else: break                                     (EARLY_STOP)

Modes:
  EARLY_STOP -- Algorithm 1 exactly (the break keeps admission non-anticipating,
                DSpark paper, section 3.2.2 and Appendix A).
  GLOBAL     -- the same walk without the break; the best Theta over the whole
                sorted path, the earliest one on ties (section 5.2: the
                unconstrained search used once capacity comes from old data).
  TOPK       -- admit exactly the first min(capacity, |E|) candidates
                (section 5.2: dynamic top-K with a capacity fixed in advance).

Readings where the pages leave a step open:
  * a is the float32 product taken left to right, one rounding per factor.
  * Ties in a are broken by position j ascending, then request r ascending
    (position-first keeps each request's admitted set a prefix).
  * tau is carried in int64 fixed point with 2^-32 resolution: each admitted
    a adds floor(a * 2^32); Theta = float64(tau) * 2^-32 * SPS[B].  The sum is
    exact and order-free, so a parallel scan reproduces this loop bit for bit.
  * SPS is a table indexed by the verify batch size B (tokens), steps/s.
  * c must lie in [0, 1]; c = 0 removes that position and all later ones.
"""

import numpy as np
from fractions import Fraction
import itertools

SCHED_EARLY_STOP = 0
SCHED_GLOBAL = 1
SCHED_TOPK = 2

_FIX = 1 << 32


def survival(c):
    """a[r, j] = c[r, 0] * ... * c[r, j], float32, one rounding per factor."""
    c = np.asarray(c, dtype=np.float32)
    R, K = c.shape
    a = np.zeros((R, K), dtype=np.float32)
    for r in range(R):
        acc = np.float32(1.0)
        for j in range(K):
            acc = np.float32(acc * c[r, j])
            a[r, j] = acc
    return a


def schedule_ref(c, sps, mode=SCHED_EARLY_STOP, capacity=0):
    """Run the scheduler.  c: [R, K] in [0, 1]; sps: table with len > R*(K+1).

    Returns dict: a [R, K] float32, ell [R] int64, cu_seqlens [R+1] int64,
    n_admitted int, theta float (Theta of the chosen admission count),
    order [list of (r, j)] the sorted candidate pool, thetas [n_c + 1] the Theta
    of every prefix of that pool that was evaluated.
    """
    c = np.asarray(c, dtype=np.float32)
    if np.any(~np.isfinite(c)) or np.any(c < 0) or np.any(c > 1):
        raise ValueError("confidence outside [0, 1]")
    sps = np.asarray(sps, dtype=np.float64)
    R, K = c.shape
    if len(sps) <= R * (K + 1):
        raise ValueError("SPS table too short")
    a = survival(c)
    pool = [(float(a[r, j]), j + 1, r) for r in range(R) for j in range(K) if a[r, j] > 0]
    pool.sort(key=lambda t: (-t[0], t[1], t[2]))

    ell = [0] * R
    batch = R
    tau_q = R * _FIX
    theta_best = float(tau_q) * 2.0 ** -32 * sps[batch]
    ell_star = list(ell)
    n_star = 0
    thetas = [theta_best]
    limit = len(pool) if mode != SCHED_TOPK else min(max(int(capacity), 0), len(pool))
    for n, (a_val, j, r) in enumerate(pool[:limit], start=1):
        ell[r] = j
        batch += 1
        tau_q += int(np.floor(np.float64(a_val) * _FIX))
        theta = float(tau_q) * 2.0 ** -32 * sps[batch]
        thetas.append(theta)
        if mode == SCHED_TOPK:
            theta_best, ell_star, n_star = theta, list(ell), n
        elif theta > theta_best:
            theta_best, ell_star, n_star = theta, list(ell), n
        elif mode == SCHED_EARLY_STOP:
            break
    ell_star = np.asarray(ell_star, dtype=np.int64)
    cu = np.zeros(R + 1, dtype=np.int64)
    cu[1:] = np.cumsum(1 + ell_star)
    return {"a": a, "ell": ell_star, "cu_seqlens": cu, "n_admitted": int(n_star),
            "theta": float(theta_best), "order": [(r, j) for (_, j, r) in pool],
            "thetas": np.asarray(thetas)}


def schedule_async_ref(c_now, c_old, sps):
    """Asynchronous capacity (DSpark paper, section 5.2; "Speculative decoding,
    from zero to DSpark", section 9): the number of tokens the next pass can
    verify is fixed beforehand by the no-break (GLOBAL) search over
    confidences from two steps earlier; the current step then admits the
    top-capacity candidates of its fresh survival values (TOPK).  The
    capacity never depends on the current block's tokens, which is what makes
    the no-break search lossless here."""
    capacity = schedule_ref(c_old, sps, SCHED_GLOBAL)["n_admitted"]
    out = schedule_ref(c_now, sps, SCHED_TOPK, capacity)
    out["capacity"] = int(capacity)
    return out


def schedule_bruteforce(c, sps):
    """Exhaustive search over every (l_1..l_R) in {0..K}^R, exact rationals.

    tau = sum_r (1 + sum_{j<=l_r} a_{r,j}) with a the exact product of the
    (float32) confidences, B = sum_r (1 + l_r), Theta = tau * SPS[B].
    Returns (best Theta as Fraction, list of all maximising l tuples).
    Tiny R and K only: (K+1)^R assignments.
    """
    c = np.asarray(c, dtype=np.float32)
    R, K = c.shape
    cf = [[Fraction(float(c[r, j])) for j in range(K)] for r in range(R)]
    prefix = []
    for r in range(R):
        row = [Fraction(0)]
        prod = Fraction(1)
        for j in range(K):
            prod *= cf[r][j]
            row.append(row[-1] + prod)
        prefix.append(row)
    spsf = [Fraction(float(s)) for s in np.asarray(sps, dtype=np.float64)]
    best = None
    arg = []
    for ell in itertools.product(range(K + 1), repeat=R):
        tau = R + sum(prefix[r][ell[r]] for r in range(R))
        batch = R + sum(ell)
        theta = tau * spsf[batch]
        if best is None or theta > best:
            best, arg = theta, [ell]
        elif theta == best:
            arg.append(ell)
    return best, arg
