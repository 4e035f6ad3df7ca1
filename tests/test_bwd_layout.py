"""Host model of the backward kernels' LDS tiles (no GPU).

The dQ and dK/dV kernels (csrc/attn_bwd.hip) stage 64-row bf16 tiles by LDS
DMA: instruction q of a tile moves R = 64 / (D/8) rows; lane i of it carries
16-byte chunk c = i / R of tile row q*R + ((i % R) ^ rot(c)), read from source
row key_of_row() of that row within its 32-row block; chunk c of row r sits at
byte (r / R) * G + 16 * (c * R + ((r % R) ^ rot(c))).  Two fragment reads use
the tile:
  * row fragments (16 bytes per lane): lane l reads tile row 32*blk + l%32,
    chunk 2*s + l/32, so the MFMA accumulator rows come out in key_of_row
    order;
  * transposed fragments (ds_read_b64_tr_b16, 8 bytes per lane, two per
    operand): lane l addresses natural row 32*blk + 16*tt + 8*(l/32) + 4*hi +
    (l%16)/4 and dims 32*db + 16*((l/16)%2) + 4*(l%4).
This model restates those formulas, checks that every read lands on the row
and dims it must, stays inside the tile, and (for 64 banks of 4 bytes, 128-byte
phases for 16-lane groups of 8-byte reads and 8-lane groups of 16-byte reads,
256-byte phases for twice as many lanes) that no read has a bank conflict.
At head_dim 256 an instruction moves 2 rows and no padding or chunk rotation
of this layout keeps both shapes conflict-free (a host search over paddings of
1024 + 16k bytes and rotations); 1056-byte steps keep the row fragments (two
thirds of the bytes read) conflict-free and leave the transposed fragments
2-way conflicted, which the model pins.
"""

import collections

import pytest


def key_of_row(i):
    return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3)


def layout(d):
    cpr = d // 8
    r = 64 // cpr
    g = 1024 + {2: 32, 4: 64, 8: 128, 16: 0}[r]
    rot = {8: lambda c: 4 * ((c ^ (c >> 1)) & 1), 16: lambda c: 4 * c}.get(r, lambda c: 0)
    at = lambda row, c: (row // r) * g + 16 * (c * r + ((row % r) ^ rot(c)))
    return r, g, rot, at


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_dma_placement_and_fragment_reads(d):
    r, g, rot, at = layout(d)
    ni = 64 // r
    tile = ni * g
    slot = {}
    for q in range(ni):
        for lane in range(64):
            c = lane // r
            row = q * r + ((lane % r) ^ rot(c))
            assert at(row, c) == q * g + 16 * lane
            slot[q * g + 16 * lane] = ((row & ~31) + key_of_row(row & 31), c)
    assert len(slot) == 64 * (d // 8)
    assert max(slot) + 16 <= tile
    conflicts = 0      # row fragments
    tr_ways = collections.Counter()  # transposed fragments: lanes per bank, worst per group
    for blk in range(2):
        for s in range(d // 16):
            addrs = []
            for lane in range(64):
                l32, hh = lane & 31, lane >> 5
                rd = [at(l32, hh), at(l32, 2 + hh)]
                a = rd[s & 1] + (32 * blk // r) * g + 16 * r * 2 * (s & ~1)
                assert slot[a] == (32 * blk + key_of_row(l32), 2 * s + hh)
                addrs.append(a)
            for grp, span in ((8, 128), (16, 256)):
                for st in range(0, 64, grp):
                    conflicts += len({(a % span) // 16 for a in addrs[st:st + grp]}) != grp
        for tt in range(2):
            for db in range(d // 32):
                for hi in range(2):
                    addrs = []
                    for lane in range(64):
                        hh, u = lane >> 5, (lane & 15) >> 2
                        vcc = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
                        a = (at(8 * hi + 4 * hh + u, vcc) + 8 * (lane & 1)
                             + ((32 * blk + 16 * tt) // r) * g + 16 * r * 4 * db)
                        row, c = slot[a - a % 16]
                        assert row == 32 * blk + 16 * tt + 8 * hh + 4 * hi + u
                        assert 8 * c + 4 * ((a % 16) // 8) == 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
                        assert a + 8 <= tile
                        addrs.append(a)
                    for grp, span in ((16, 128), (32, 256)):
                        for st in range(0, 64, grp):
                            n = collections.Counter((a % span) // 8 for a in addrs[st:st + grp])
                            tr_ways[max(n.values())] += 1
    assert conflicts == 0
    if d == 256:
        assert set(tr_ways) == {2}  # every transposed read 2-way, none worse
    else:
        assert set(tr_ways) == {1}
