"""Philox4x32-10 counter-based generator, written from its published definition.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Reference: J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel
Random Numbers: As Easy as 1, 2, 3", SC'11.  Philox-4x32 keeps a 128-bit
counter (four 32-bit words) and a 64-bit key (two words).  One round:

    (hi0, lo0) = 64-bit product  M0 * c0
    (hi1, lo1) = 64-bit product  M1 * c2
    c' = (hi1 ^ c1 ^ k0,  lo1,  hi0 ^ c3 ^ k1,  lo0)

and between rounds the key is advanced by the Weyl constants
(k0 += W0, k1 += W1, modulo 2^32).  The "-10" variant applies ten rounds;
the first uses the caller's key unmodified.

The noise draws on the pages (one t ~ U(0,1) for each sequence on the
LLaDA-8B-MDLM-LoRA card, Training table; uniform-token noise in the diffusiongemma card,
Finetuning notes) fix only distributions.  Realising them with this counter
generator makes every draw a pure function of (seed, index, stream tag), so a
GPU implementation can reproduce them bit for bit.
"""

import numpy as np

# Round multipliers and Weyl key increments of Philox-4x32 (SC'11, section 5).
PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9  # golden ratio, 2^32 * (sqrt(5)-1)/2
PHILOX_W1 = 0xBB67AE85  # 2^32 * (sqrt(3)-1)

_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Apply ten Philox-4x32 rounds to counters (c0..c3) under key (k0, k1).

    All arguments are broadcastable integer arrays (or scalars) holding values
    in [0, 2^32).  Returns a tuple of four uint32 arrays, the output words.
    Arithmetic is carried in uint64 so each 32x32 product is exact.
    """
    c0, c1, c2, c3, k0, k1 = np.broadcast_arrays(
        *[np.asarray(a, dtype=np.uint64) for a in (c0, c1, c2, c3, k0, k1)]
    )
    c0, c1, c2, c3 = c0.copy(), c1.copy(), c2.copy(), c3.copy()
    k0, k1 = k0.copy(), k1.copy()
    m0 = np.uint64(PHILOX_M0)
    m1 = np.uint64(PHILOX_M1)
    w0 = np.uint64(PHILOX_W0)
    w1 = np.uint64(PHILOX_W1)
    s32 = np.uint64(32)
    for rnd in range(10):
        if rnd > 0:
            k0 = (k0 + w0) & _MASK32
            k1 = (k1 + w1) & _MASK32
        p0 = m0 * c0
        p1 = m1 * c2
        hi0, lo0 = p0 >> s32, p0 & _MASK32
        hi1, lo1 = p1 >> s32, p1 & _MASK32
        c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return tuple(x.astype(np.uint32) for x in (c0, c1, c2, c3))
