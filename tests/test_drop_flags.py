"""The byte arithmetic behind the dropout keep masks of the kernels (no GPU).

A Philox word holds the random bytes of four elements; an element is kept
when its byte is at least thr = floor(256 p + 0.5) (0 <= thr <= 255 at every
entry point). The kernels decide all four bytes of a word at once: with t4 =
thr in every byte and c4 = 0x80808080 - (t4 & 0x7f7f7f7f), bit 7 of each byte
of majority(x, NOT t4, (x & 0x7f7f7f7f) + c4) is that byte's decision (one
add and one three-input bit operation). v_perm then spreads a byte's flag
over a 16-bit half (bf16 pair operands) or a whole word (fp32 values), with
the selectors 8 .. 11, which copy bit 15 or bit 31 of either source into a
byte. Both steps are checked here, exhaustively over bytes and thresholds,
against the plain comparison; the v_perm model follows the instruction's
published definition (selector bytes 0 .. 3 pick bytes of the second source,
4 .. 7 of the first, 8 .. 11 sign-extend bits 15 and 31 of the second and of
the first, 12 gives 0x00). The GPU parity tests check the same masks on the
device, bit for bit against the oracle's keep decisions."""

import numpy as np

M7 = 0x7F7F7F7F


def keep_flags4(x, thr):
    """Bit 7 of byte k set when byte k of x >= thr (x: uint32 array)."""
    t4 = np.uint32(thr * 0x01010101)
    c4 = np.uint32((0x80808080 - (int(t4) & M7)) & 0xFFFFFFFF)
    d = (x & np.uint32(M7)) + c4  # no byte carries into the next
    nt = ~t4
    return (x & nt) | (x & d) | (nt & d)


def v_perm(s0, s1, sel):
    src = [(int(s1) >> (8 * i)) & 0xFF for i in range(4)] + [(int(s0) >> (8 * i)) & 0xFF for i in range(4)]
    out = 0
    for i in range(4):
        b = (sel >> (8 * i)) & 0xFF
        if b < 8:
            v = src[b]
        elif b < 12:
            v = 0xFF if (src[2 * (b - 8) + 1] >> 7) & 1 else 0x00
        elif b == 12:
            v = 0x00
        else:
            v = 0xFF
        out |= v << (8 * i)
    return out


def keep_mask_pair(g, q):
    return v_perm((g << 8) & 0xFFFFFFFF, g, 0x09090B0B if q else 0x08080A0A)


def keep_mask_elem(g, k):
    sel = (0x0A0A0A0A, 0x08080808, 0x0B0B0B0B, 0x09090909)[k]
    return v_perm((g << 8) & 0xFFFFFFFF, g, sel)


def test_every_byte_and_threshold():
    x = np.arange(256, dtype=np.uint32)
    for thr in range(256):
        f = keep_flags4(x, thr)
        np.testing.assert_array_equal((f >> 7) & 1, (x >= thr).astype(np.uint32), err_msg=f"thr {thr}")


def test_whole_words_no_carry_between_bytes():
    rng = np.random.default_rng(11)
    words = rng.integers(0, 2 ** 32, size=1 << 16, dtype=np.uint64).astype(np.uint32)
    # Bytes at the edges of every threshold's range, in every position.
    edge = np.array([0x00, 0x01, 0x7F, 0x80, 0x81, 0xFE, 0xFF], dtype=np.uint32)
    combos = np.stack(np.meshgrid(edge, edge, edge, edge, indexing="ij"), -1).reshape(-1, 4)
    words = np.concatenate([words, combos[:, 0] | combos[:, 1] << 8 | combos[:, 2] << 16 | combos[:, 3] << 24])
    for thr in (0, 1, 2, 64, 127, 128, 129, 200, 254, 255):
        f = keep_flags4(words, thr)
        for k in range(4):
            byte = (words >> (8 * k)) & 0xFF
            np.testing.assert_array_equal((f >> (8 * k + 7)) & 1, (byte >= thr).astype(np.uint32),
                                          err_msg=f"thr {thr} byte {k}")


def test_masks_from_flags():
    # Every pattern of four flags, with the bits below bit 7 of each byte
    # set arbitrarily (keep_flags4 leaves them undefined).
    rng = np.random.default_rng(5)
    for pattern in range(16):
        for _ in range(8):
            junk = int(rng.integers(0, 2 ** 32)) & M7
            g = junk | sum(((pattern >> k) & 1) << (8 * k + 7) for k in range(4))
            kept = [(pattern >> k) & 1 for k in range(4)]
            for q in range(2):
                want = (0xFFFF if kept[2 * q] else 0) | ((0xFFFF if kept[2 * q + 1] else 0) << 16)
                assert keep_mask_pair(g, q) == want, (pattern, q)
            for k in range(4):
                assert keep_mask_elem(g, k) == (0xFFFFFFFF if kept[k] else 0), (pattern, k)


def test_mutant_without_top_bit_term_fails():
    # Dropping the top-bit term (reading bit 7 of the biased sum alone) is
    # wrong exactly where the top bits of the byte and thr differ.
    x = np.arange(256, dtype=np.uint32)
    thr = 100
    t4 = thr * 0x01010101
    d = (x & np.uint32(M7)) + np.uint32(0x80808080 - (t4 & M7))
    assert not np.array_equal((d >> 7) & 1, (x >= thr).astype(np.uint32))
