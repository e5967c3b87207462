"""Counter-based random bits for attention dropout (CPU, test infrastructure).

TEST INFRASTRUCTURE ONLY: imported by tests and the smoke check, never by the
library. The GPU kernels implement the same generator on their own.

The pages name dropout only as a branch that a correct implementation must
cover ("Flash Attention algorithm design and I/O optimisation", answer on
verification). The random bits come from Philox4x32-10, the counter-based
generator of Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as easy
as 1, 2, 3" (SC 2011), written here from its definition: a 128-bit counter
and a 64-bit key; ten rounds, each multiplying counter words 0 and 2 by two
fixed 32-bit constants, crossing the high halves into the other words with
the key, then bumping the key by two Weyl constants.

How the bits are used (the same reading on both sides):
  * Element (i, j) of the attention of (batch b, head h) belongs to the 4x4
    block (i >> 2, j >> 2). One Philox call with counter
    (j >> 2, i >> 2, b * H + h, offset) and key (seed mod 2^32, seed >> 32)
    returns four 32-bit words; word (i & 3) holds the block's row, and byte
    (j & 3) of it (bits 8 (j & 3) .. 8 (j & 3) + 7) is element (i, j)'s byte.
  * The element is dropped when its byte is below thr = floor(256 p + 0.5):
    the dropout probability is rounded to a multiple of 1/256, and the kept
    probabilities are scaled by 1 / (1 - thr / 256).
"""

import math

import numpy as np

PHILOX_M0 = 0xD2511F53
PHILOX_M1 = 0xCD9E8D57
PHILOX_W0 = 0x9E3779B9
PHILOX_W1 = 0xBB67AE85
_MASK32 = np.uint64(0xFFFFFFFF)


def philox4x32_10(c0, c1, c2, c3, k0, k1):
    """Philox4x32 with 10 rounds on arrays of counters (broadcast); returns
    the four output words as uint64 arrays holding 32-bit values."""
    c = [np.asarray(x, dtype=np.uint64) & _MASK32 for x in (c0, c1, c2, c3)]
    k0 = np.uint64(int(k0) & 0xFFFFFFFF)
    k1 = np.uint64(int(k1) & 0xFFFFFFFF)
    m0, m1 = np.uint64(PHILOX_M0), np.uint64(PHILOX_M1)
    for _ in range(10):
        p0 = m0 * c[0]                     # 64-bit products of 32-bit values
        p1 = m1 * c[2]
        hi0, lo0 = p0 >> np.uint64(32), p0 & _MASK32
        hi1, lo1 = p1 >> np.uint64(32), p1 & _MASK32
        c = [hi1 ^ c[1] ^ k0, lo1, hi0 ^ c[3] ^ k1, lo0]
        k0 = (k0 + np.uint64(PHILOX_W0)) & _MASK32
        k1 = (k1 + np.uint64(PHILOX_W1)) & _MASK32
    return c


def dropout_threshold(p):
    """Byte threshold of dropout probability p (0 <= p < 1): an element is
    dropped when its byte is below floor(256 p + 0.5)."""
    if not 0.0 <= p < 1.0:
        raise ValueError("dropout probability must be in [0, 1)")
    return int(math.floor(float(np.float32(p)) * 256.0 + 0.5))


def keep_mask(bh, rows, cols, p, seed, offset):
    """Keep decisions for the attention of flattened (batch, head) index bh:
    bool [len(rows), len(cols)] for query positions `rows` and key positions
    `cols`."""
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    thr = dropout_threshold(p)
    seed = int(seed)
    words = philox4x32_10((cols >> 2)[None, :], (rows >> 2)[:, None], bh, int(offset),
                          seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF)
    w = np.stack(np.broadcast_arrays(*words))          # [4, rows, cols]
    word = np.take_along_axis(w, (rows & 3)[None, :, None].repeat(len(cols), axis=2), axis=0)[0]
    byte = (word >> (np.uint64(8) * (cols & 3).astype(np.uint64))[None, :]) & np.uint64(0xFF)
    return byte >= np.uint64(thr)
