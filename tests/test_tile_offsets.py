"""Host-side check of the address identities the attention kernel's tile
loads rely on (CPU only; no device code runs here).

The kernel stages a 128-token block as two half tiles of 64 rows; a wave of
lane L stages rows 16w + 4i + L/16 of each half at physical 16-byte chunk
L % 16. Instead of one offset register per load it keeps one lane offset and
derives the others:
* a row's token offset is linear in the bits of its slot index when the
  chunk sides are powers of two, so slot(16w + 4i + r) = slot(16w + r) +
  slot(4i), and the upper half is the lower one plus slot(64);
* the K swizzle (logical chunk = physical ^ swap23(row & 15)) then reduces to
  an XOR of the lane offset with 64 * sb(i), sb swapping the two bits of i;
  the V swizzle (physical ^ 4 (row & 3)) does not depend on i.
This test recomputes every offset directly from those definitions for all
36 chunk shapes of 128 tokens and checks the derived form.
"""

import itertools


def swap23(m):
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


def slot(j, ct, ch, cw, H, W):
    iw, r2 = j % cw, j // cw
    return ((r2 // ch) * H + r2 % ch) * W + iw


def chunk_shapes():
    sides = [1 << e for e in range(8)]
    return [(ct, ch, 128 // (ct * ch)) for ct, ch in itertools.product(sides, sides)
            if 128 % (ct * ch) == 0]


def test_all_chunk_shapes_are_counted():
    assert len(chunk_shapes()) == 36


def test_tile_offsets_from_one_lane_offset():
    sb64 = [0, 128, 64, 192]
    for ct, ch, cw in chunk_shapes():
        H, W = ch * 3, cw * 5  # any grid the chunk divides
        half = slot(64, ct, ch, cw, H, W) * 256
        rows_s = [slot(4 * i, ct, ch, cw, H, W) * 256 for i in range(4)]
        for w in range(4):
            for lane in range(64):
                r = lane >> 4
                base = slot(16 * w + r, ct, ch, cw, H, W) * 256
                k0 = base + (((lane & 15) ^ r) << 4)
                v0 = base + (((lane & 15) ^ (4 * r)) << 4)
                vx = 80 * r
                assert v0 == k0 ^ vx
                for h in range(2):
                    for i in range(4):
                        row = 64 * h + 16 * w + 4 * i + r
                        rowoff = slot(row, ct, ch, cw, H, W) * 256
                        k_direct = rowoff + (((lane & 15) ^ swap23(row & 15)) << 4)
                        v_direct = rowoff + (((lane & 15) ^ (4 * (row & 3))) << 4)
                        assert (k0 ^ sb64[i]) + rows_s[i] + h * half == k_direct
                        assert v0 + rows_s[i] + h * half == v_direct


def key_chunk_shapes():
    """Power-of-two key chunks of 64 to 1024 tokens."""
    sides = [1 << e for e in range(11)]
    return [(a, b, n // (a * b)) for n in (64, 128, 256, 512, 1024)
            for a, b in itertools.product(sides, sides) if n % (a * b) == 0]


def test_key_unit_offsets():
    """Key blocks of 128 * m tokens are walked in units of 128 keys: the token
    of slot 128u + 64h + 16w + 4i + r is the sum of the offsets of slots
    128u, 64h, 16w + r and 4i (the kernel adds the first two on the scalar
    side). Key blocks of 64 tokens use u = h = 0."""
    shapes = key_chunk_shapes()
    assert len(shapes) == 28 + 36 + 45 + 55 + 66  # C(k+2, 2) shapes of 2^k tokens
    for ct, ch, cw in shapes:
        n = ct * ch * cw
        H, W = ch * 3, cw * 2
        for u in range(max(1, n // 128)):
            for h in range(2 if n >= 128 else 1):
                for w in range(4):
                    for i in range(4):
                        for r in range(4):
                            j = 128 * u + 64 * h + 16 * w + 4 * i + r
                            parts = (slot(128 * u, ct, ch, cw, H, W) + slot(64 * h, ct, ch, cw, H, W)
                                     + slot(16 * w + r, ct, ch, cw, H, W) + slot(4 * i, ct, ch, cw, H, W))
                            assert slot(j, ct, ch, cw, H, W) == parts


def test_score_register_key_order():
    """Accumulator value i of lane (n, gs) of a 32x32 MFMA output holds row
    8 (i/4) + 4 gs + i%4; the K rows are read in swap23 order, so that value
    holds key swap23(row) of the sub-tile. The partial-block mask computes
    that key as 16 (i/8) + 8 gs + i%8 (plus 32 per sub-tile): the two agree,
    and a lane pair (gs = 0, 1) covers each of the 32 keys once."""
    for tl in range(2):
        seen = []
        for gs in range(2):
            for i in range(16):
                row = 8 * (i // 4) + 4 * gs + i % 4
                key = 32 * tl + swap23(row)
                assert key == 32 * tl + 16 * (i >> 3) + 8 * gs + (i & 7)
                seen.append(key)
        assert sorted(seen) == list(range(32 * tl, 32 * tl + 32))


def test_key_slot_bits():
    """With power-of-two key chunk sides, slot j of a key block has
    iw = j & (cw-1), ih = (j >> log2 cw) & (ch-1), it = j >> log2(cw ch), the
    same (t, h, w) offsets as the division form of the slot order."""
    for ctk, chk, cwk in [(2, 4, 8), (4, 8, 8), (8, 8, 16), (1, 8, 128), (16, 8, 8)]:
        lw, lh = cwk.bit_length() - 1, chk.bit_length() - 1
        for j in range(ctk * chk * cwk):
            assert (j & (cwk - 1), (j >> lw) & (chk - 1), j >> (lw + lh)) == (
                j % cwk, (j // cwk) % chk, j // (cwk * chk))
