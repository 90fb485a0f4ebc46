"""LDS row layouts of the grouped GEMMs, checked on the CPU.

Operand rows sit in LDS as 16-byte chunks, chunk c of row r at slot
c ^ key(r): rows of 128 bytes use key (r & 7) ^ ((r >> 3) & 1), rows of 64
bytes key (r >> 2) & 3 (csrc/mfma.h, swz128 and swz64).  gfx950's LDS has 64
banks of 4 bytes and serves a 16-byte-per-lane read 16 lanes per clock; a
fragment read takes one logical chunk from rows 32 i + (lane & 31), the two
halves of the wave taking neighbouring chunks.  These tests check that
each key is a permutation of the slots of a row (the direct loads fill slot
p of row r with chunk p ^ key(r), so every chunk lands once and reads back
where it is looked for), and that every 16 lanes of every fragment read hit
16 different 4-bank groups, i.e. the reads are free of bank conflicts.  The
keys they replace ((r & 7), (r >> 1) & 3) fail the second check with 2-way
conflicts, which a bank-conflict counter and a read probe on the GPU showed
at half the LDS's rate.
"""
import pytest


def swz128(r):
    return (r & 7) ^ ((r >> 3) & 1)


def swz64(r):
    return (r >> 2) & 3


def bank_group(row, slot, row_bytes):
    return ((row * row_bytes + 16 * slot) // 16) % 16


def groups_of_read(key, row_bytes, block, chunk_of_half):
    """4-bank groups hit by each 16-lane quarter of one fragment read."""
    quarters = []
    for q0 in range(0, 64, 16):
        g = []
        for lane in range(q0, q0 + 16):
            row = 32 * block + (lane & 31)
            c = chunk_of_half(lane >> 5)
            g.append(bank_group(row, c ^ key(row), row_bytes))
        quarters.append(g)
    return quarters


@pytest.mark.parametrize("key,row_bytes", [(swz128, 128), (swz64, 64)])
def test_key_permutes_the_slots_of_each_row(key, row_bytes):
    n = row_bytes // 16
    for r in range(512):
        assert sorted(c ^ key(r) for c in range(n)) == list(range(n))


def test_fragment_reads_of_128_byte_rows_are_conflict_free():
    # sub-step q of a 64-K step: the two halves take chunks 2 q and 2 q + 1
    for block in range(8):
        for q in range(4):
            for g in groups_of_read(swz128, 128, block, lambda h: 2 * q + h):
                assert len(set(g)) == 16


def test_fragment_reads_of_64_byte_rows_are_conflict_free():
    # K half h of a 32-K stage: the halves of the wave take chunks 2 h, 2 h + 1
    for block in range(8):
        for h in range(2):
            for g in groups_of_read(swz64, 64, block, lambda kg: 2 * h + kg):
                assert len(set(g)) == 16


def test_the_replaced_keys_conflict():
    old128 = lambda r: r & 7
    old64 = lambda r: (r >> 1) & 3
    g128 = groups_of_read(old128, 128, 0, lambda h: h)[0]
    g64 = groups_of_read(old64, 64, 0, lambda h: h)[0]
    assert len(set(g128)) == 8 and len(set(g64)) == 8  # two lanes per group: 2-way conflicts


def test_key_of_a_fragment_row_is_that_of_its_lane():
    for i in range(16):
        for f in range(32):
            assert swz128(32 * i + f) == swz128(f) and swz64(32 * i + f) == swz64(f)


def test_staged_gate_up_rows_cover_the_tile_once_and_read_back_conflict_free():
    """The gate/up epilogue's tile-wide staging (csrc/mfma.h,
    store_gateup_staged): 256 rows of 256 bytes, chunk c of row t at
    c ^ (t % 16).  Wave (wm, wn) writes 8 bytes per lane of rows
    wm * 128 + 32 i + (lane & 31), chunk 4 wn + g, half lane >> 5; wave w
    reads back rows 32 w + 4 j + (lane >> 4), chunk lane & 15.  Every byte of
    the tile is written exactly once, and read back exactly once, from where
    it was written; each 16-lane quarter of a read-back hits 16 different
    4-bank groups."""
    RB = 256
    owner = {}
    for wm in range(2):
        for wn in range(4):
            for i in range(4):
                for g in range(4):
                    for lane in range(64):
                        t = wm * 128 + i * 32 + (lane & 31)
                        c = wn * 4 + g
                        addr = t * RB + ((c ^ (t & 15)) << 4) + (lane >> 5) * 8
                        for b in range(8):
                            assert addr + b not in owner
                            owner[addr + b] = (t, c, lane >> 5, b)
    assert len(owner) == 256 * RB
    read = set()
    for w in range(8):
        for j in range(8):
            quarters = {}
            for lane in range(64):
                t = w * 32 + 4 * j + (lane >> 4)
                c = lane & 15
                addr = t * RB + ((c ^ (t & 15)) << 4)
                for b in range(16):
                    tt, cc, half, bb = owner[addr + b]
                    assert (tt, cc, 8 * half + bb) == (t, c, b)   # the bytes of chunk c of row t
                    assert addr + b not in read
                    read.add(addr + b)
                quarters.setdefault(lane // 16, []).append((addr // 16) % 16)
            for q in quarters.values():
                assert len(set(q)) == 16
    assert len(read) == 256 * RB
