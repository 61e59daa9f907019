"""Philox4x32-10 counter-based generator, vectorised over numpy uint64 lanes.

Definition: Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3" (SC'11), the Philox-4x32 bijection with 10 rounds. One round maps
a 4-word counter (c0, c1, c2, c3) under a 2-word key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

where hi/lo are the upper/lower 32 bits of the 64-bit product; between rounds
the key is bumped by the Weyl constants (W0, W1) modulo 2^32.

The paper under study only asks that the sample indicators be independent
Bernoulli(r_i) draws ("Verify Before You Fetch", §4.1); this generator is the
one the library fixes so that the sample is reproducible from
(seed, layer, head, token) alone. Pinned by the published known-answer
vectors of Philox4x32-10 (tests/golden/philox_kat.json) and statistically
(uniformity, avalanche, bijectivity, Bernoulli frequencies).
"""

import numpy as np

MASK32 = np.uint64(0xFFFFFFFF)
M0 = np.uint64(0xD2511F53)
M1 = np.uint64(0xCD9E8D57)
W0 = 0x9E3779B9
W1 = 0xBB67AE85


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Return the four 32-bit output words (as uint64 arrays) for the counters.

    ``c0..c3`` are integer arrays (broadcastable) holding 32-bit values;
    ``k0, k1`` are Python ints (32-bit key words).
    """
    c0 = np.asarray(c0, dtype=np.uint64) & MASK32
    c1 = np.asarray(c1, dtype=np.uint64) & MASK32
    c2 = np.asarray(c2, dtype=np.uint64) & MASK32
    c3 = np.asarray(c3, dtype=np.uint64) & MASK32
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    ka, kb = int(k0) & 0xFFFFFFFF, int(k1) & 0xFFFFFFFF
    for _ in range(10):
        p0 = M0 * c0
        p1 = M1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ np.uint64(ka), lo1,
                          hi0 ^ c3 ^ np.uint64(kb), lo0)
        ka = (ka + W0) & 0xFFFFFFFF
        kb = (kb + W1) & 0xFFFFFFFF
    return c0, c1, c2, c3


def uniform24(seed, token, head, layer):
    """Uniform draw on the 2^-24 grid in [0, 1) for each token.

    Key = (seed low word, seed high word); counter = (token, head, layer, 0).
    The top 24 bits of the first output word give u = (x0 >> 8) * 2^-24,
    which is exactly representable in float32 and float64.
    """
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    x0, _, _, _ = philox4x32_10(token, head, layer, 0,
                                seed & 0xFFFFFFFF, seed >> 32)
    return (x0 >> np.uint64(8)).astype(np.float64) * 2.0 ** -24
