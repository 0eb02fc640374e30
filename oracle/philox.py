"""Philox4x32 counter-based random numbers, pure Python -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark may import this module; it shares no code
with the HIP path.

Philox4x32-R is defined in J. K. Salmon, M. A. Moraes, R. O. Dror and D. E. Shaw, "Parallel
random numbers: as easy as 1, 2, 3" (SC '11): a 128-bit counter (four 32-bit words) is
transformed by R rounds keyed by a 64-bit key (two words).  One round multiplies counter words
0 and 2 by the constants 0xD2511F53 and 0xCD9E8D57 into 64-bit products, and the new counter is
(hi(c2 M1) ^ c1 ^ k0, lo(c2 M1), hi(c0 M0) ^ c3 ^ k1, lo(c0 M0)); the key is then bumped by the
Weyl constants (0x9E3779B9, 0xBB67AE85).  The attention dropout contract uses R = 10, the
paper's recommended count.
"""

from __future__ import annotations

M0, M1 = 0xD2511F53, 0xCD9E8D57
W0, W1 = 0x9E3779B9, 0xBB67AE85
MASK32 = 0xFFFFFFFF


def philox4x32(counter, key, rounds: int = 10):
    """Philox4x32-`rounds` of one 128-bit counter (4 ints) under a 64-bit key (2 ints)."""
    c0, c1, c2, c3 = (int(x) & MASK32 for x in counter)
    k0, k1 = (int(x) & MASK32 for x in key)
    for _ in range(rounds):
        p0 = M0 * c0
        p1 = M1 * c2
        c0, c1, c2, c3 = ((p1 >> 32) ^ c1 ^ k0) & MASK32, p1 & MASK32, ((p0 >> 32) ^ c3 ^ k1) & MASK32, p0 & MASK32
        k0 = (k0 + W0) & MASK32
        k1 = (k1 + W1) & MASK32
    return c0, c1, c2, c3
