"""Philox4x32-10 counter-based generator and the per-decision uniform.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix no generator; the method only needs one independent uniform per
random decision.  This module follows the published description of Philox
(Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy as 1, 2, 3",
SC'11): a 4x32-bit counter, a 2x32-bit key, ten rounds, each round two 32x32->64
multiplications whose high and low halves are mixed with the other two counter
words and the round key, the key advanced by two Weyl constants between rounds.

Decision address (one uniform per decision, independent of thread order and of
schedule outcomes):
  key     = (seed mod 2^32, seed >> 32)
  counter = (step mod 2^32, step >> 32, request index r, (position << 2) | purpose)
  u       = (first output word >> 8) * 2^-24, an exact float32 value in [0, 1).

Purposes: DRAFT (the draft sample at position k), ACCEPT (the min(1, p/q) test
at position j), RESAMPLE (the correction or bonus sample at position j).
"""

import numpy as np

PURPOSE_DRAFT = 0
PURPOSE_ACCEPT = 1
PURPOSE_RESAMPLE = 2

_MASK32 = np.uint64(0xFFFFFFFF)
_MUL0 = np.uint64(0xD2511F53)
_MUL1 = np.uint64(0xCD9E8D57)
_WEYL0 = np.uint64(0x9E3779B9)
_WEYL1 = np.uint64(0xBB67AE85)


def philox4x32_10(counter, key):
    """Ten Philox4x32 rounds.

    counter: 4 arrays (or scalars) of 32-bit words (x0, x1, x2, x3);
    key: 2 arrays (or scalars) of 32-bit words (k0, k1).
    Returns a list of 4 uint64 arrays holding the 32-bit output words.
    """
    x0, x1, x2, x3 = (np.asarray(w, dtype=np.uint64) & _MASK32 for w in counter)
    k0, k1 = (np.asarray(w, dtype=np.uint64) & _MASK32 for w in key)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + _WEYL0) & _MASK32
            k1 = (k1 + _WEYL1) & _MASK32
        prod0 = _MUL0 * x0          # < 2^64, exact in uint64
        prod1 = _MUL1 * x2
        hi0, lo0 = prod0 >> np.uint64(32), prod0 & _MASK32
        hi1, lo1 = prod1 >> np.uint64(32), prod1 & _MASK32
        x0, x1, x2, x3 = hi1 ^ x1 ^ k0, lo1, hi0 ^ x3 ^ k1, lo0
    return [x0, x1, x2, x3]


def uniform(seed, step, r, position, purpose):
    """The uniform in [0, 1) that drives decision (r, position, purpose) of `step`.

    r and position may be integer arrays (broadcast together); returns float64.
    """
    seed = int(seed)
    step = int(step)
    r = np.asarray(r, dtype=np.uint64)
    position = np.asarray(position, dtype=np.uint64)
    r, position = np.broadcast_arrays(r, position)
    word3 = (position << np.uint64(2)) | np.uint64(purpose)
    out = philox4x32_10(
        (np.full(r.shape, step & 0xFFFFFFFF, dtype=np.uint64),
         np.full(r.shape, (step >> 32) & 0xFFFFFFFF, dtype=np.uint64),
         r, word3),
        (np.uint64(seed & 0xFFFFFFFF), np.uint64((seed >> 32) & 0xFFFFFFFF)),
    )
    return (out[0] >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
