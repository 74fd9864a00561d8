"""Philox4x32-10 counter-based generator and the per-element 16-bit draw.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages say only that the backward re-quantization uses hardware-accelerated
stochastic rounding ("Inkling 2 Small uses four-bit training ...", section
"Stochastic rounding across transposes"). The random numbers here come from a
counter-based generator keyed by a seed and the element's index, so that any
two implementations agree bit for bit.

Generator: Philox4x32 with 10 rounds, as published by Salmon, Moraes, Dror and
Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3" (SC'11). One round maps the
counter (c0, c1, c2, c3) with key (k0, k1) to

    (hi(M1*c2) ^ c1 ^ k0,  lo(M1*c2),  hi(M0*c0) ^ c3 ^ k1,  lo(M0*c0))

with 64-bit products of 32-bit words, M0 = 0xD2511F53, M1 = 0xCD9E8D57; the key
is bumped by (0x9E3779B9, 0xBB67AE85) mod 2^32 between rounds.

Element mapping (a reading; the pages give none):
    key     = (seed mod 2^32, seed >> 32)
    counter = (q mod 2^32, q >> 32, tag, 0)   with q = idx >> 3
    u16     = 16-bit half (idx & 1) of output word ((idx & 7) >> 1),
              the low half first
so one generator call serves 8 consecutive elements of an output buffer.
"""

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Ten Philox rounds on arrays of 32-bit words; returns four uint32 arrays."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK32 for c in (c0, c1, c2, c3))
    k0 = np.asarray(k0, dtype=np.uint64) & _MASK32
    k1 = np.asarray(k1, dtype=np.uint64) & _MASK32
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
            k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
        p0 = m0 * c0                      # < 2^64, exact in uint64
        p1 = m1 * c2
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c0, c1, c2, c3 = (hi1 ^ c1 ^ k0) & _MASK32, lo1, (hi0 ^ c3 ^ k1) & _MASK32, lo0
    return tuple(c.astype(np.uint32) for c in (c0, c1, c2, c3))


def uniform16(seed, tag, idx):
    """16-bit uniform draw for each linear element index ``idx`` (int array)."""
    idx = np.asarray(idx, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    q = idx >> np.uint64(3)
    words = philox4x32_10(q & _MASK32, q >> np.uint64(32),
                          np.full_like(q, int(tag) & 0xFFFFFFFF), np.zeros_like(q),
                          seed & 0xFFFFFFFF, seed >> 32)
    w = np.stack(words, axis=0).astype(np.uint32)           # [4, ...]
    sel = ((idx & np.uint64(7)) >> np.uint64(1)).astype(np.int64)
    half = (idx & np.uint64(1)).astype(np.uint32)
    word = np.take_along_axis(w, sel[None, ...], axis=0)[0]
    return ((word >> (half * np.uint32(16))) & np.uint32(0xFFFF)).astype(np.uint32)


def uniform16_range(seed, tag, start, count):
    """Draws for the consecutive indices start .. start+count-1.

    Same values as ``uniform16(seed, tag, np.arange(start, start+count))``;
    the generator runs once per group of 8 indices instead of once per index.
    """
    start = int(start)
    count = int(count)
    if count <= 0:
        return np.zeros(0, dtype=np.uint32)
    q0 = start >> 3
    q1 = (start + count - 1) >> 3
    q = np.arange(q0, q1 + 1, dtype=np.uint64)
    seed = int(seed) & 0xFFFFFFFFFFFFFFFF
    words = philox4x32_10(q & _MASK32, q >> np.uint64(32),
                          np.full_like(q, int(tag) & 0xFFFFFFFF), np.zeros_like(q),
                          seed & 0xFFFFFFFF, seed >> 32)
    w = np.stack(words, axis=1).astype(np.uint32)            # [nq, 4]
    u = np.empty((q.shape[0], 8), dtype=np.uint32)
    u[:, 0::2] = w & np.uint32(0xFFFF)                        # low half first
    u[:, 1::2] = w >> np.uint32(16)
    u = u.reshape(-1)
    off = start - (q0 << 3)
    return u[off:off + count]
