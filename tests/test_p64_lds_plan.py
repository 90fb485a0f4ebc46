"""The LDS plan of the persistent 64-K grouped GEMM, checked on the CPU.

grouped_gemm_pipe64_kernel (csrc/experts.hip) keeps 160 KB of LDS as five
32 KB slots: token slots 0-1 at [0, 64 KB), weight slots 0-2 at
[64 KB, 160 KB); step kt's token rows go to token slot kt % 2 and its weight
rows to weight slot kt % 3.  Each wave's DMA piece j of an operand fills
1 KB at wid * 4 KB + j KB of the slot.  Between two tiles the kernel:
  - stages the finished tile's outputs in weight slots 1-2
    ([96 KB, 160 KB)): the gate/up product tile-wide, 256 rows of 256 bytes;
    the down product per wave, 8 KB a wave, in two rounds of 64 rows;
  - meanwhile loads the next tile's token rows of steps 0 and 1 and weight
    rows of step 0, then, after a barrier that follows every wave's staged
    reads, its weight rows of step 1 and the first quarter of step 2.
These tests restate that plan and check that the pieces loaded during the
epilogue never touch the staging region, that the staging stays inside it
(each output element staged and read back once, by the wave that wrote
it), and that the vmcnt waits the kernel counts for an ordinary prologue
also hold for a prefetched one: vector loads complete in issue order, and
the stores between them may complete in any order.
"""
import pytest

KB = 1024
SLOT = 32 * KB
NA, NB = 2, 3
LPO, BQ = 4, 1          # DMA pieces per wave and operand step; weight pieces per sub-step
STAGE = (NA + 1) * SLOT  # weight slot 1


def piece_bytes(op, kt, wid, j):
    """LDS byte range [lo, hi) that wave wid's piece j of step kt fills."""
    base = wid * LPO * KB + j * KB
    if op == "A":
        lo = (kt % NA) * SLOT + base
    else:
        lo = NA * SLOT + (kt % NB) * SLOT + base
    return lo, lo + KB


def test_slots_tile_the_lds():
    spans = sorted(piece_bytes(op, kt, w, j) for op, n in (("A", NA), ("B", NB)) for kt in range(n)
                   for w in range(8) for j in range(LPO))
    assert spans[0][0] == 0 and spans[-1][1] == 160 * KB
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 == b0


@pytest.mark.parametrize("wid", range(8))
def test_prefetched_pieces_miss_the_staging_region(wid):
    before = [("A", 0, j) for j in range(LPO)] + [("B", 0, j) for j in range(LPO)] + [("A", 1, j) for j in range(LPO)]
    after = [("B", 1, j) for j in range(LPO)] + [("B", 2, j) for j in range(BQ)]
    for op, kt, j in before:
        lo, hi = piece_bytes(op, kt, wid, j)
        assert hi <= STAGE or lo >= STAGE + 2 * SLOT
    for op, kt, j in after:
        lo, hi = piece_bytes(op, kt, wid, j)
        assert STAGE <= lo and hi <= STAGE + 2 * SLOT


def test_gate_up_staging_fits_the_two_slots():
    RB = 256
    hi = max(t * RB + ((c ^ (t & 15)) << 4) + 16 for t in range(256) for c in range(16))
    assert STAGE + hi <= 160 * KB


@pytest.mark.parametrize("wid", range(8))
def test_down_staging_in_two_rounds(wid):
    """store_tile32_staged<.., MB=4, NB=2, WTM=128, WTN=64, ROUNDS=2>: per
    round, lane (frow, half) writes 8 bytes of row ib * 32 + frow (round-local,
    ib < 2) at chunk (col / 8) ^ ((t / 2) % 8) of 128-byte rows, then reads
    back chunk c = lane % 8 of row t0 + lane / 8 and stores it to output row
    wm * 128 + rd * 64 + t.  Every output element of the wave's 128 x 64 block
    goes through the wave's 8 KB region once, to its own row and column."""
    RB, CPR, RPS, MBR, WTR = 128, 8, 2, 2, 64
    region = STAGE + wid * 8 * KB
    assert region + 8 * KB <= 160 * KB
    stored = {}
    for rd in range(2):
        owner = {}
        for ib in range(MBR):
            for lane in range(64):
                frow, half = lane & 31, lane >> 5
                t = ib * 32 + frow
                sw = (t // RPS) % CPR
                for g in range(4):
                    for f in range(2):
                        col = f * 32 + g * 8 + half * 4
                        addr = t * RB + (((col >> 3) ^ sw) << 4) + half * 8
                        assert 0 <= addr and addr + 8 <= 8 * KB
                        for b in range(8):
                            assert addr + b not in owner
                            # bytes 2k, 2k+1 hold column col + k of block row i = rd * MBR + ib
                            owner[addr + b] = ((rd * MBR + ib) * 32 + frow, col + b // 2)
        for lane in range(64):
            c, rr = lane % CPR, lane // CPR
            for t0 in range(0, WTR, 64 // CPR):
                t = t0 + rr
                addr = t * RB + ((c ^ ((t // RPS) % CPR)) << 4)
                row = rd * WTR + t
                for b in range(16):
                    r_, col_ = owner[addr + b]
                    assert (r_, col_) == (row, c * 8 + b // 2)
                    stored[(r_, col_, b % 2)] = stored.get((r_, col_, b % 2), 0) + 1
    assert len(stored) == 128 * 64 * 2 and set(stored.values()) == {1}


def landed_ok(order, n_wait, targets):
    """With vmcnt <= n_wait, are all pieces named in `targets` complete, in
    every state reachable when loads ('L') complete in issue order and
    stores ('S') in any order?  Stores are interchangeable here, so a state
    is a completed prefix of the loads plus a number of completed stores."""
    loads = [name for k, name in order if k == "L"]
    n_st = sum(1 for k, _ in order if k == "S")
    for done_loads in range(len(loads) + 1):
        for done_st in range(n_st + 1):
            if len(order) - done_loads - done_st > n_wait:
                continue
            if any(name in targets for name in loads[done_loads:]):
                return False
    return True


def pieces(name, n):
    return [("L", name)] * n


@pytest.mark.parametrize("n_stores", [0, 1, 4, 8, 16])
def test_tile_start_wait_holds_for_a_prefetched_tile(n_stores):
    """The tile start waits for vmcnt <= 2 LPO + BQ and then needs A0 and
    B0: true for the ordinary prologue (A0 B0 B1 A1 B2q) and for the
    prefetched one (A0 B0 A1, the epilogue's stores, B1 B2q)."""
    N = 2 * LPO + BQ
    plain = pieces("A0", LPO) + pieces("B0", LPO) + pieces("B1", LPO) + pieces("A1", LPO) + pieces("B2", BQ)
    pre = (pieces("A0", LPO) + pieces("B0", LPO) + pieces("A1", LPO) + [("S", "st")] * n_stores +
           pieces("B1", LPO) + pieces("B2", BQ))
    assert landed_ok(plain, N, {"A0", "B0"})
    assert landed_ok(pre, N, {"A0", "B0"})
    # a wait that allowed one more piece in flight would not be enough
    assert not landed_ok(plain, N + 1, {"B0"})
    assert not landed_ok(pre, N + 1, {"B0"})


@pytest.mark.parametrize("n_stores", [0, 8, 16])
def test_first_step_wait_holds_for_a_prefetched_tile(n_stores):
    """Step 0 waits for vmcnt <= LPO before its barrier and needs step 1's
    token and weight rows (A1, B1); after them only B2 goes out: its first
    quarter with the prologue, the other three in sub-steps 0-2."""
    pre = (pieces("A0", LPO) + pieces("B0", LPO) + pieces("A1", LPO) + [("S", "st")] * n_stores +
           pieces("B1", LPO) + pieces("B2", BQ) + pieces("B2", 3 * BQ))
    assert landed_ok(pre, LPO, {"A0", "B0", "A1", "B1"})
    assert not landed_ok(pre, LPO + 1, {"B1"})
