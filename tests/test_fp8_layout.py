"""Host model of the fp8 attention kernel's LDS tiles (no GPU).

64-row tiles of E4M3 bytes, row pitch D bytes, 16-byte chunks.  LDS DMA with
row-major lanes: lane i of instruction q carries row q*R + i // CPR (R = 1024
// D rows, CPR = D // 16 chunks) and writes slot i of the instruction's 1 KiB;
the slot at position p of row r holds chunk p ^ swz(r).  K rows hold key
key_of_row(r % 32) + 32 (r // 32), V rows their own key.
  * K fragment (fp8 MFMA A operand, 32 bytes per lane): lane l reads row
    32 kb + l % 32, chunks 4 s + 2 (l // 32) and the next, i.e. dims
    64 s + 32 (l // 32) + 0..31.
  * V fragment (ds_read_b64_tr_b8; within a 16-lane group lane i receives byte
    i % 8 of the chunks addressed by lanes 2 e + i // 8): lane l addresses row
    16 t + 8 (l // 32) + (l % 16) // 2 at dims 32 db + 16 ((l // 16) % 2) +
    8 (l % 2), so it receives V[16 t + 8 (l // 32) + e][32 db + l % 32],
    e = 0..7.
The model checks placement, bounds, quad coalescing of the DMA and the absence
of bank conflicts (64 banks of 4 bytes; 128- and 256-byte phases).
"""

import pytest


def key_of_row(i):
    return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3)


def swz_k(d, r):
    return {256: r & 15, 128: (r >> 1) & 7, 64: (r >> 2) & 3, 32: (r ^ (r >> 3)) & 1}[d]


def swz_v(d, r):
    return {256: (r & 7) << 1, 128: r & 7, 64: ((r >> 2) & 1) << 1, 32: (r ^ (r >> 1)) & 1}[d]


def krow(r):
    return 32 * (r // 32) + key_of_row(r % 32)


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_fp8_tiles(d):
    cpr = d // 16
    rows_per = 1024 // d
    tile = 64 * d
    ks, vs = {}, {}
    for q in range(64 // rows_per):
        for lane in range(64):
            r = q * rows_per + lane // cpr
            p = lane % cpr
            a = q * 1024 + 16 * lane
            assert a == r * d + 16 * p and a + 16 <= tile
            ks[a] = (krow(r), p ^ swz_k(d, r))
            vs[a] = (r, p ^ swz_v(d, r))
        for base in range(0, 64, 4):  # each quad: one aligned 64-byte source segment
            for slot in (ks, vs):
                seg = {(slot[q * 1024 + 16 * (base + j)][0], slot[q * 1024 + 16 * (base + j)][1] // 4)
                       for j in range(4)}
                assert len(seg) == 1 or cpr < 4
    conflicts = 0
    for kb in range(2):
        for s in range(max(1, d // 64)):
            for half in range(2):
                addrs = []
                for lane in range(64):
                    l32, hh = lane & 31, lane >> 5
                    r = 32 * kb + l32
                    # head_dim 32: lane half 1 repeats half 0's reads (its Q half is zero)
                    c = half if d == 32 else 4 * s + 2 * hh + half
                    a = r * d + 16 * (c ^ swz_k(d, r))
                    assert ks[a] == (32 * kb + key_of_row(l32), c) and a + 16 <= tile
                    addrs.append(a)
                for grp in (8, 16):
                    for st in range(0, 64, grp):
                        # lanes reading one address share it (a broadcast, no conflict)
                        distinct = set(addrs[st:st + grp])
                        conflicts += len({(a % 256) // 16 for a in distinct}) != len(distinct)
    for db in range(d // 32):
        for t in range(4):
            addrs = []
            lanes = {}
            for lane in range(64):
                hh, g, i = lane >> 5, (lane >> 4) & 1, lane & 15
                r = 16 * t + 8 * hh + (i >> 1)
                c = 2 * db + g
                a = r * d + 16 * (c ^ swz_v(d, r)) + 8 * (i & 1)
                row, chunk = vs[a - a % 16]
                assert row == r and 16 * chunk + 8 * ((a % 16) // 8) == 32 * db + 16 * g + 8 * (i & 1)
                assert a + 8 <= tile
                addrs.append(a)
                lanes[lane] = (row, 16 * chunk + 8 * ((a % 16) // 8))
            # what each lane receives: byte i % 8 of the chunks of lanes 2 e + i // 8
            for lane in range(64):
                grp0 = lane & ~15
                i = lane & 15
                for e in range(8):
                    row, dim0 = lanes[grp0 + 2 * e + i // 8]
                    assert row == 16 * t + 8 * (lane >> 5) + e
                    assert dim0 + i % 8 == 32 * db + (lane & 31)
            for grp in (16, 32):
                for st in range(0, 64, grp):
                    conflicts += len({(a % 256) // 8 for a in addrs[st:st + grp]}) != grp
    assert conflicts == 0
