"""Host model of the paged-attention kernel's LDS tiles (no GPU).

A 32-row tile of K or V is filled by LDS DMA with row-major lanes: lane i of
instruction q carries row q*R + i // CPR (R = 64 // CPR rows, CPR = D // 8
chunks of 16 bytes per row) and writes LDS slot i of the instruction's 1 KiB.
The slot at position p of a row holds global chunk p ^ swz(row), so the four
lanes of every quad read one aligned 64-byte segment of one source row.  K rows
hold key key_of_row(row) (the MFMA accumulator order the P operand needs); V
rows hold their own key.  The model checks that K row fragments (16 bytes per
lane: lane l reads row l % 32, dims 16 s + 8 (l // 32) ..) and V transposed
fragments (ds_read_b64_tr_b16: lane l addresses natural row 16 tt + 8 (l // 32)
+ 4 hi + (l % 16) // 4 and dims 32 db + 16 ((l // 16) % 2) + 4 (l % 4)) land on
the intended data, stay in the tile, and (64 banks of 4 bytes) have no bank
conflicts in 128- or 256-byte phases; and that every DMA quad is one 64-byte
aligned segment.
"""

import pytest


def key_of_row(i):
    return ((i >> 4) << 4) + (((i >> 2) & 1) << 3) + (((i >> 3) & 1) << 2) + (i & 3)


def swz_k(d, row):
    return {256: row & 15, 128: row & 15, 64: (row >> 1) & 7, 32: (row >> 2) & 3}[d]


def swz_v(d, row):
    return {256: (row & 3) << 2, 128: (row & 3) << 2, 64: ((row >> 1) & 1) << 2, 32: 0}[d]


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_row_major_swizzled_tiles(d):
    cpr = d // 8
    r = 64 // cpr
    pitch = 2 * d
    tile = 32 * pitch
    kslot, vslot = {}, {}
    for q in range(32 // r):
        for lane in range(64):
            row = q * r + lane // cpr
            p = lane % cpr
            a = q * 1024 + 16 * lane
            assert a == row * pitch + 16 * p and a + 16 <= tile
            kslot[a] = (key_of_row(row), p ^ swz_k(d, row))
            vslot[a] = (row, p ^ swz_v(d, row))
        # each quad of lanes reads one aligned 64-byte source segment
        for base in range(0, 64, 4):
            for slot, rowmap in ((kslot, key_of_row), (vslot, lambda x: x)):
                srcs = {(slot[q * 1024 + 16 * (base + j)][0], slot[q * 1024 + 16 * (base + j)][1] // 4)
                        for j in range(4)}
                assert len(srcs) == 1
    assert len(kslot) == len(vslot) == 32 * cpr
    conflicts = 0
    for s in range(d // 16):
        addrs = []
        for lane in range(64):
            l32, hh = lane & 31, lane >> 5
            a = l32 * pitch + 16 * ((2 * s + hh) ^ swz_k(d, l32))
            assert kslot[a] == (key_of_row(l32), 2 * s + hh)
            addrs.append(a)
        for grp, span in ((8, 128), (16, 256)):
            for st in range(0, 64, grp):
                conflicts += len({(a % 256) // 16 for a in addrs[st:st + grp]}) != grp
    for tt in range(2):
        for db in range(d // 32):
            for hi in range(2):
                addrs = []
                for lane in range(64):
                    hh, u = lane >> 5, (lane & 15) >> 2
                    k = 16 * tt + 8 * hh + 4 * hi + u
                    c = 4 * db + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1)
                    a = k * pitch + 16 * (c ^ swz_v(d, k)) + 8 * (lane & 1)
                    row, chunk = vslot[a - a % 16]
                    assert row == k
                    assert 8 * chunk + 4 * ((a % 16) // 8) == 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)
                    assert a + 8 <= tile
                    addrs.append(a)
                for grp in (16, 32):
                    for st in range(0, 64, grp):
                        conflicts += len({(a % 256) // 8 for a in addrs[st:st + grp]}) != grp
    assert conflicts == 0


# E4M3 cache tiles: 32 rows of D bytes (CPR = D // 16 chunks), R = 64 // CPR
# rows per DMA instruction (all 32 at head_dim 32, issued once per 16-key
# group).  K fragments are one 16-byte read per MFMA pair (lane l: row l % 32,
# chunk 2 j + l // 32); V fragments are ds_read_b64_tr_b8 (lane l: row
# 16 tt + 8 (l // 32) + (l % 16) // 2, byte 8 ((l % 16) % 2) of chunk
# 2 db + (l // 16) % 2).
def swz_k8(d, r):
    return {256: (r ^ (r >> 1)) & 15, 128: (r ^ (r >> 1)) & 7, 64: (r ^ (r >> 2)) & 3,
            32: ((r >> 2) ^ (r >> 3)) & 1}[d]


def swz_v8(d, r):
    return {256: (r ^ (r >> 1)) & 7, 128: (r ^ (r >> 1)) & 7, 64: (r ^ (r >> 1)) & 3,
            32: (r ^ (r >> 2)) & 1}[d]


@pytest.mark.parametrize("d", [32, 64, 128, 256])
def test_e4m3_tiles(d):
    cpr = d // 16
    r = 64 // cpr
    pitch = d
    tile = 32 * pitch
    kslot, vslot = {}, {}
    for q in range(max(1, 32 // r)):
        for lane in range(64):
            row = q * r + lane // cpr
            p = lane % cpr
            a = q * 1024 + 16 * lane
            assert row < 32 and a == row * pitch + 16 * p and a + 16 <= tile
            # the 16-key group whose page this lane loads from holds its key
            g = row >> 4 if r > 16 else (q * r) >> 4
            assert key_of_row(row) >> 4 == g and row >> 4 == g
            kslot[a] = (key_of_row(row), p ^ swz_k8(d, row))
            vslot[a] = (row, p ^ swz_v8(d, row))
    assert len(set(kslot.values())) == len(set(vslot.values())) == 32 * cpr
    kc = 0
    for j in range(max(1, d // 32)):
        addrs = []
        for lane in range(64):
            l32, hh = lane & 31, lane >> 5
            a = l32 * pitch + 16 * ((2 * j + hh) ^ swz_k8(d, l32))
            assert kslot[a] == (key_of_row(l32), 2 * j + hh)
            addrs.append(a)
        for grp, span in ((8, 128), (16, 256)):
            for st in range(0, 64, grp):
                kc += len({(a % span) // 16 for a in addrs[st:st + grp]}) != grp
    vc = {128: 0, 256: 0}
    for tt in range(2):
        for db in range(d // 32):
            addrs = []
            for lane in range(64):
                hh, vg, vi = lane >> 5, (lane >> 4) & 1, lane & 15
                row = 16 * tt + 8 * hh + (vi >> 1)
                x = swz_v8(d, 8 * hh + (vi >> 1))  # the lane constant the kernel uses
                assert x == swz_v8(d, row)
                c = 2 * db + vg
                a = row * pitch + 8 * (vi & 1) + 16 * (c ^ x)
                assert vslot[a - a % 16] == (row, c) and a + 8 <= tile
                addrs.append(a)
            for grp, span in ((16, 128), (32, 256)):
                for st in range(0, 64, grp):
                    vc[span] += len({(a % span) // 8 for a in addrs[st:st + grp]}) != grp
    assert kc == 0
    if d == 256:
        assert vc[128] == 0 and vc[256] > 0  # 2-way in the 256-byte grouping only
    else:
        assert vc == {128: 0, 256: 0}
