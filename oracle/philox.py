"""Philox4x32-10, written from its published definition.

Source: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, section 3 (the Philox S-P network).

The sampler configuration on the pages asks for Philox noise keyed per step
("gumbel-max at temperature 1.0 (Philox, seed per step)"); the pages fix neither
the variant nor the counter layout, so this module fixes Philox4x32 with 10
rounds and ``sampler.py`` fixes the counter layout.

A Philox4x32 round maps a 4-word counter (c0, c1, c2, c3) under a 2-word key
(k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with the paper's multipliers M0 = 0xD2511F53, M1 = 0xCD9E8D57; between rounds
the key advances by the Weyl constants (0x9E3779B9, 0xBB67AE85) modulo 2^32.
The first round uses the key as given.

Test infrastructure only (see the package docstring).
"""

import numpy as np

_MASK = np.uint64(0xFFFFFFFF)
_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = np.uint64(0x9E3779B9)
_W1 = np.uint64(0xBB67AE85)
ROUNDS = 10


def philox4x32(ctr, key, rounds=ROUNDS):
    """Return the four output words for counter ``ctr`` under ``key``.

    ``ctr`` is a sequence of four integer arrays (broadcastable, values < 2^32),
    ``key`` a sequence of two.  Returns a tuple of four uint32 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK for c in ctr)
    k0, k1 = (np.asarray(k, dtype=np.uint64) & _MASK for k in key)
    for r in range(rounds):
        if r:
            k0 = (k0 + _W0) & _MASK
            k1 = (k1 + _W1) & _MASK
        p0 = c0 * _M0          # exact: a 32x32-bit product fits in 64 bits
        p1 = c2 * _M1
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(np.asarray(w, dtype=np.uint32) for w in (c0, c1, c2, c3))


def seed_key(seed):
    """Split a 64-bit seed into the 2-word key (low word, high word)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32
