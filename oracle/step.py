"""One whole draft -> schedule -> verify step, composed from the oracle parts.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Order of a decoding round ("Speculative decoding, from zero to DSpark",
sections 2, 6, 8; DSpark paper, Figure 1 caption): the sequential head drafts
K tokens from the anchor, the scheduler picks each request's verify length
from the confidences and SPS(B), the target pass produces one logit row per
verify token (flattened, request-major), and rejection sampling emits the
accepted prefix plus one correction or bonus token.

The target pass itself is outside the method: ``target_rows(r, n)`` returns
the n = 1 + l_r target logit rows of request r.
"""

import numpy as np

from .draft import draft_ref
from .schedule import schedule_ref, SCHED_EARLY_STOP
from .verify import verify_ref


def run_step(U, W1, W2, x0, c, sps, target_rows, temperature, seed, step,
             mode=SCHED_EARLY_STOP, capacity=0):
    d = draft_ref(U, W1, W2, x0, temperature, seed, step)
    s = schedule_ref(c, sps, mode, capacity)
    R = len(x0)
    rows = [np.asarray(target_rows(r, 1 + int(s["ell"][r])), dtype=np.float64) for r in range(R)]
    P = np.concatenate(rows, axis=0)
    v = verify_ref(P, s["cu_seqlens"], U, W1, W2, x0, d["x"], temperature, seed, step)
    return {"draft": d, "schedule": s, "verify": v}
