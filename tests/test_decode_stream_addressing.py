"""The persistent decode kernel's work walk and addresses, modelled on the CPU.

decode_stream_kernel (csrc/experts.hip) has each of G workgroups walk units
b', b' + G, ... (b' = xcd_contiguous(b, G), so each XCD's workgroups start on
adjacent units) of (token tile of at most 16 rows, 32 weight rows: 8 per wave),
in steps of 4 K-quarters of 64, with a ring of 6 LDS stages that its direct
global->LDS loads fill 5 steps ahead and that runs on from one unit into the
next.  These tests restate its cursors and its address arithmetic integer
for integer and check, for routings with empty experts, experts of more than
16 rows, K not a multiple of 256 and output widths of several units:
  - the stage each step is read from holds that step's loads, of the unit the
    compute cursor is on, and a load never targets a stage that a step still
    to be read occupies;
  - every 16-byte load stays inside its operand (the expert's [NOUT, K]
    weight matrix, the token buffer), each lane reading its own row, with no
    negative or 32-bit-overflowing token offset;
  - LDS destinations and fragment reads stay inside the 144 KB ring and the
    stage's regions;
  - every K quarter of every output is multiplied exactly once, and every
    (row, output) of every expert is stored exactly once.
"""
import numpy as np
import pytest

ROWB, NS = 128, 6
TQ = 16 * ROWB            # token rows of one quarter
TOK = 4 * TQ
WQ = 8 * ROWB             # a wave's rows of one quarter
STAGE = TOK + 4 * 4 * WQ  # 24 KB
U32 = 1 << 32


def swz128(r):
    return (r & 7) ^ ((r >> 3) & 1)


def tile_list(counts, BM=16):
    offs = np.concatenate([[0], np.cumsum(counts)])
    tiles = []
    for e, c in enumerate(counts):
        for r in range(int(offs[e]), int(offs[e + 1]), BM):
            tiles.append((e, r, min(r + BM, int(offs[e + 1]))))
    return tiles


def walk(b, G, U, nk):
    """Per iteration g the slot the one issue writes and the (unit, step) it
    loads, and the compute's slot and (unit, step); the prologue's issues
    first.  The issue cursor stops at the last step and repeats it."""
    nu = (U - 1 - b) // G + 1
    iu = is_ = 0
    slot_issue = 0
    lds = {}
    log = []

    def issue():
        nonlocal iu, is_, slot_issue
        lds[slot_issue] = (iu, is_)
        s = slot_issue
        slot_issue = 0 if slot_issue == NS - 1 else slot_issue + 1
        if is_ + 1 < nk:
            is_ += 1
        elif iu + 1 < nu:
            is_ = 0
            iu += 1
        return s

    for _ in range(NS - 1):
        issue()
    slot = 0
    cj = cs = 0
    for g in range(nu * nk):
        live = {(slot + d) % NS for d in range(NS - 1)}   # steps g .. g + NS - 2
        s = issue()
        assert s not in live
        assert lds[slot] == (cj, cs), (g, slot, lds[slot], (cj, cs))
        log.append((cj, cs))
        slot = 0 if slot == NS - 1 else slot + 1
        cs += 1
        if cs == nk:
            cs = 0
            cj += 1
    assert cj == nu
    return log


@pytest.mark.parametrize("nk", [1, 2, 3, 5, 6, 16, 64])
@pytest.mark.parametrize("U,G", [(1, 256), (5, 3), (10944, 256), (300, 256), (64, 7)])
def test_ring_holds_each_step_when_it_is_read(nk, U, G):
    for b in range(0, min(G, U), max(1, min(G, U) // 16)):
        log = walk(b, G, U, nk)
        assert len(log) == ((U - 1 - b) // G + 1) * nk


def check_units(gateup, counts, NOUT, K, a_rows, x_rows):
    tiles = tile_list(counts)
    UN = 16 if gateup else 32
    WN = UN // 4
    n_units = (NOUT + UN - 1) // UN
    nq = K // 64
    nk = (nq + 3) // 4
    nrows = int(sum(counts))
    stored = np.zeros((nrows, NOUT), np.int64)
    E = len(counts)
    for u in range(len(tiles) * n_units):
        mi = u // n_units
        e, r0, r1 = tiles[mi]
        n0 = (u - mi * n_units) * UN
        src = [min(a_rows[min(r0 + t, r1 - 1)], x_rows - 1) if a_rows is not None else min(r0 + t, r1 - 1)
               for t in range(16)]
        for wid in range(4):
            quarters = np.zeros((8, nq), np.int64)   # (wave row, quarter) multiplied
            for lane in range(64):
                row_l = lane >> 3
                mat = 1 if (gateup and row_l >= 4) else 0
                mrow = min(n0 + WN * wid + ((row_l & 3) if gateup else row_l), NOUT - 1)
                chunk = ((lane & 7) ^ swz128(row_l)) << 4
                for h in range(2):
                    toff = src[8 * h + row_l] * K * 2 + (((lane & 7) ^ swz128(8 * h + row_l)) << 4)
                    assert 0 <= toff < U32
                for is_ in range(nk):
                    for q in range(4):
                        qq = min(4 * is_ + q, nq - 1)
                        addr = (e * NOUT + mrow) * K * 2 + chunk + qq * ROWB
                        assert e * NOUT * K * 2 <= addr and addr + 16 <= (e + 1) * NOUT * K * 2
                        assert addr // (K * 2) == e * NOUT + mrow            # the lane's own row
                        dst = (NS - 1) * STAGE + TOK + (4 * wid + q) * WQ + 16 * lane
                        assert TOK <= dst - (NS - 1) * STAGE and dst + 16 <= NS * STAGE <= 160 * 1024
                    qt = min(4 * is_ + wid, nq - 1)
                    for h in range(2):
                        toff = src[8 * h + row_l] * K * 2 + (((lane & 7) ^ swz128(8 * h + row_l)) << 4)
                        assert toff + qt * ROWB + 16 <= x_rows * K * 2
                        dst = wid * TQ + h * 1024 + 16 * lane
                        assert dst + 16 <= TOK
            # fragment reads and the quarters each step multiplies
            for lane in range(64):
                kg = lane >> 4
                fw = TOK + 4 * wid * WQ + (lane & 7) * ROWB
                ft = (lane & 15) * ROWB
                for cs in range(nk):
                    qv = min(nq - 4 * cs, 4)
                    for q in range(4):
                        if q >= qv:
                            continue
                        for h in range(2):
                            c = 4 * h + kg
                            assert fw + q * WQ + ((c ^ swz128(lane & 7)) << 4) + 16 <= TOK + (4 * wid + 4) * WQ
                            assert q * TQ + ft + ((c ^ swz128(lane & 15)) << 4) + 16 <= (q + 1) * TQ
                        if lane == 0:
                            quarters[:, 4 * cs + q] += 1
            assert (quarters == 1).all()
            # epilogue
            col0 = n0 + WN * wid
            for lane in range(64):
                grow = r0 + (lane & 15)
                if gateup:
                    if lane < 16 and grow < r1 and col0 < NOUT:
                        assert col0 + 4 <= NOUT
                        stored[grow, col0:col0 + 4] += 1
                else:
                    col = col0 + 4 * (lane >> 4)
                    if lane < 32 and grow < r1 and col < NOUT:
                        assert col + 4 <= NOUT
                        stored[grow, col:col + 4] += 1
    assert (stored == 1).all()


@pytest.mark.parametrize("gateup", [True, False])
@pytest.mark.parametrize("NOUT,K", [(192, 256), (64, 64), (448, 192), (320, 640), (128, 1536)])
def test_decode_units_stay_in_their_buffers(gateup, NOUT, K):
    rng = np.random.default_rng(NOUT + K + gateup)
    counts = [0, 1, 15, 16, 17, 40, 0, 5]
    N = sum(counts)
    x_rows = 40
    a_rows = [int(v) for v in rng.integers(0, x_rows, N)]
    check_units(gateup, counts, NOUT, K, a_rows, x_rows)
    check_units(gateup, counts, NOUT, K, None, N)


def xcd_contiguous(bid, n):
    q, rem = n // 8, n % 8
    xcd, loc = bid % 8, bid // 8
    return (xcd * (q + 1) if xcd < rem else rem * (q + 1) + (xcd - rem) * q) + loc


@pytest.mark.parametrize("G", [1, 7, 8, 9, 80, 255, 256, 304])
def test_workgroup_numbering_is_a_permutation_contiguous_per_xcd(G):
    """Workgroup b runs on XCD b % 8 and walks units from xcd_contiguous(b, G):
    every unit start is taken once, and each XCD's starts are one run."""
    ids = [xcd_contiguous(b, G) for b in range(G)]
    assert sorted(ids) == list(range(G))
    for x in range(8):
        mine = sorted(ids[b] for b in range(x, G, 8))
        assert mine == list(range(mine[0], mine[0] + len(mine))) if mine else True


def test_decode_shape():
    """The benchmark's decode shape: T=32, k=8, E=128, H=4096, I=1536; its
    tile list and the walk of the first and last workgroup."""
    rng = np.random.default_rng(3)
    counts = np.bincount(rng.integers(0, 128, 256), minlength=128)
    tiles = tile_list(counts)
    assert all(r1 - r0 <= 16 for _, r0, r1 in tiles)
    for n_units, nk in ((1536 // 16, 4096 // 256), (4096 // 32, 1536 // 256)):
        U = len(tiles) * n_units
        walk(0, 256, U, nk)
        walk(255, 256, U, nk)
