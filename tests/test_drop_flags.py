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
the first, 12 gives 0x00). The byte transpose's selectors and the LDS
layout of the quad transpose are checked the same way (the transpose, the
area's bounds, alignment and banks). The GPU parity tests check the same
masks on the device, bit for bit against the oracle's keep decisions."""

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


# The quad transpose of the Philox words goes through a per-wave LDS area:
# lane L stores its word e at word 80 e + L, lane 4 q + s reads the four
# words from 80 s + 4 q. The layout constants are restated here from the
# kernel source and checked for the transpose, the bounds of the area
# (kQuadXWords words), the 16-byte alignment of the reads, and bank
# conflicts (64 banks of 4 bytes; 16-byte reads served 16 lanes at a time).
QUAD_X_WORDS = 3 * 80 + 64


def test_quad_transpose_layout():
    area = {}
    for lane in range(64):
        for e in range(4):
            addr = 80 * e + lane
            assert 0 <= addr < QUAD_X_WORDS
            assert addr not in area
            area[addr] = (lane, e)  # word e of lane `lane`
    for lane in range(64):
        q, s = lane >> 2, lane & 3
        base = 80 * s + 4 * q
        assert base % 4 == 0 and base + 3 < QUAD_X_WORDS  # 16-byte aligned, in bounds
        got = [area[base + m] for m in range(4)]
        # column s of the quad: word s of lanes 4q + 0 .. 4q + 3, in order
        assert got == [(4 * q + m, s) for m in range(4)]
    for e in range(4):  # each store instruction: 64 lanes, distinct banks
        assert len({(80 * e + lane) % 64 for lane in range(64)}) == 64
    for first in range(0, 64, 16):  # each 16-lane phase of the 16-byte read
        banks = [(80 * (l & 3) + 4 * (l >> 2) + m) % 64 for l in range(first, first + 16)
                 for m in range(4)]
        assert len(set(banks)) == 64


def byte_transpose(x):
    a = v_perm(x[1], x[0], 0x05010400)
    b = v_perm(x[1], x[0], 0x07030602)
    c = v_perm(x[3], x[2], 0x05010400)
    d = v_perm(x[3], x[2], 0x07030602)
    return [v_perm(c, a, 0x05040100), v_perm(c, a, 0x07060302),
            v_perm(d, b, 0x05040100), v_perm(d, b, 0x07060302)]


def test_byte_transpose_selectors():
    rng = np.random.default_rng(9)
    for _ in range(200):
        x = [int(v) for v in rng.integers(0, 2 ** 32, size=4)]
        out = byte_transpose(x)
        for t in range(4):
            for w in range(4):
                assert (out[t] >> (8 * w)) & 0xFF == (x[w] >> (8 * t)) & 0xFF
