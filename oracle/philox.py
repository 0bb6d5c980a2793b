"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py): nothing on the product path imports this.

Source of the definition: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel Random
Numbers: As Easy as 1, 2, 3", SC'11, section on the Philox family.  Philox4x32 keeps four 32-bit
counter words and a two-word key.  One round multiplies counter words 0 and 2 by two fixed odd
multipliers, keeps the high and low halves of the 64-bit products, and mixes them with the other
two words and the key; the key is advanced by two fixed Weyl constants between rounds.  Ten rounds
are the recommended, crush-resistant variant.

The pages name only a ``generator`` argument (diffusers DiffusionGemmaPipeline docs,
``__call__`` parameters), so which generator drives the sampler is a reading: this one, with the
counter layout fixed in ``oracle/sampler.py``.
"""
import numpy as np

# multipliers and Weyl key increments of Philox4x32 (SC'11, Philox section)
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85

_MASK32 = np.uint64(0xFFFFFFFF)


def _mulhilo(a, b):
    """64-bit product of two 32-bit words, split into (hi, lo)."""
    p = np.uint64(a) * b.astype(np.uint64)
    return (p >> np.uint64(32)).astype(np.uint32), (p & _MASK32).astype(np.uint32)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply Philox4x32 with 10 rounds to counters (c0..c3) under key (k0, k1).

    Every argument is broadcast to a common shape of uint32 words; returns four uint32 arrays.
    """
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint32) for c in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 = int(k0) & 0xFFFFFFFF
    k1 = int(k1) & 0xFFFFFFFF
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + PHILOX_W0) & 0xFFFFFFFF
            k1 = (k1 + PHILOX_W1) & 0xFFFFFFFF
        hi0, lo0 = _mulhilo(PHILOX_M0, c0)
        hi1, lo1 = _mulhilo(PHILOX_M1, c2)
        n0 = hi1 ^ c1 ^ np.uint32(k0)
        n1 = lo1
        n2 = hi0 ^ c3 ^ np.uint32(k1)
        n3 = lo0
        c0, c1, c2, c3 = n0, n1, n2, n3
    return c0, c1, c2, c3


def seed_key(seed):
    """Split a 64-bit seed into the two key words (low word first)."""
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    return seed & 0xFFFFFFFF, seed >> 32
