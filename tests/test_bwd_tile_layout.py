"""Host-side check of the LDS layout the backward kernels rely on (CPU only;
no device code runs here).

A 128-row tile (a block of Q, K, V or dO, 256 bytes per row) is stored with
16-byte chunk c of row r at physical chunk c ^ f(r), f(r) = 4 (r % 4) +
(r // 4) % 4, and is read two ways:
* row operands of the 32x32x16 MFMA: lane (n, gs) reads row 32t + swap23(n),
  channels 16s + 8gs .. +7, at t*8192 + (ra ^ 32s);
* transposing reads (ds_read_b64_tr_b16): lane l reads 8 bytes of row
  16k + 8gs + (l%16)//4 (+4 for the second read) at channels
  32u + 16((l//16)%2) + 4(l%4) .. +3, at (16k)*256 + (ta ^ 64u) and
  (16k+4)*256 + (ta ^ 64u ^ 16).
Tiles are written by direct-to-LDS loads: load i of wave w, lane L, writes
physical chunk L%16 of row 32w + 4i + L//16 from global byte
(ld ^ 16 (i%4)) + origin*256 + slot(4i)*256.

This test recomputes every address from the kernel's per-lane formulas and
checks, for all 36 chunk shapes, that each read meets the intended logical
element, and that the reads are free of LDS bank conflicts (64 banks of 4
bytes): 16 lanes of a 16-byte read, or 32 lanes of an 8-byte read, touch 64
distinct banks.
"""

import itertools


def swap23(m):
    return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1)


def slot(j, ct, ch, cw, H, W):
    iw, r2 = j % cw, j // cw
    return ((r2 // ch) * H + r2 % ch) * W + iw


def f(row):
    return 4 * (row % 4) + (row // 4) % 4


def chunk_shapes():
    sides = [1 << e for e in range(8)]
    return [(ct, ch, 128 // (ct * ch)) for ct, ch in itertools.product(sides, sides)
            if 128 % (ct * ch) == 0]


def lane_ra(lane):
    n, gs = lane & 31, lane >> 5
    f_row = ((n & 3) << 2) | ((n >> 3) & 1) | (((n >> 2) & 1) << 1)
    return swap23(n) * 256 + 16 * (gs ^ f_row)


def lane_ta(lane):
    gs = lane >> 5
    jj = lane & 15
    q4, hb, c1 = jj >> 2, (lane >> 4) & 1, (jj & 3) >> 1
    return (8 * gs + q4) * 256 + 64 * q4 + 16 * ((2 * hb + c1) ^ (2 * gs)) + 8 * (jj & 1)


def logical(byte):
    """(row, logical byte within the row) of an LDS byte address of a tile."""
    row, within = divmod(byte, 256)
    phys, off = divmod(within, 16)
    return row, 16 * (phys ^ f(row)) + off


def test_swizzle_is_a_permutation_per_row():
    for row in range(128):
        assert sorted((c ^ f(row)) for c in range(16)) == list(range(16))


def test_tile_loads_place_every_chunk():
    for ct, ch, cw in chunk_shapes():
        H, W = ch * 3, cw * 5
        origin = slot(0, ct, ch, cw, H, W) + 7 * W  # any block origin
        seen = {}
        for w in range(4):
            for lane in range(64):
                r = lane >> 4
                ld = slot(32 * w + r, ct, ch, cw, H, W) * 256 + (((lane & 15) ^ (r << 2)) << 4)
                for i in range(8):
                    g = (ld ^ (16 * (i & 3))) + origin * 256 + slot(4 * i, ct, ch, cw, H, W) * 256
                    row = 32 * w + 4 * i + r
                    token, gbyte = divmod(g, 256)
                    assert token == origin + slot(row, ct, ch, cw, H, W)
                    lds = row * 256 + 16 * (lane & 15)
                    lrow, lbyte = logical(lds)
                    assert lrow == row and lbyte == gbyte
                    seen[(row, gbyte // 16)] = True
        assert len(seen) == 128 * 16


def test_row_operand_reads():
    for t in range(4):
        for s in range(8):
            banks = {}
            for lane in range(64):
                n, gs = lane & 31, lane >> 5
                byte = t * 8192 + (lane_ra(lane) ^ (32 * s))
                row, lbyte = logical(byte)
                assert row == 32 * t + swap23(n)
                assert lbyte == 2 * (16 * s + 8 * gs)
                banks.setdefault(lane // 16, set()).update(
                    ((byte // 4) + b) % 64 for b in range(4))
            assert all(len(b) == 64 for b in banks.values())


def test_transposing_reads():
    for k in range(8):
        for u in range(4):
            groups = {}
            for lane in range(64):
                gs, jj, hb = lane >> 5, lane & 15, (lane >> 4) & 1
                ta = lane_ta(lane)
                for hi, byte in ((0, 16 * k * 256 + (ta ^ (64 * u))),
                                 (1, (16 * k + 4) * 256 + (ta ^ (64 * u) ^ 16))):
                    row, lbyte = logical(byte)
                    assert row == 16 * k + 8 * gs + (jj >> 2) + 4 * hi
                    assert lbyte == 2 * (32 * u + 16 * hb + 4 * (jj & 3))
                    groups.setdefault((hi, lane // 32), set()).update(
                        ((byte // 4) + b) % 64 for b in range(2))
            assert all(len(b) == 64 for b in groups.values())
