"""The grouped GEMMs' work decomposition, modelled on the CPU.

The expert products walk a list of (expert, row range) token tiles that one
workgroup builds on the device from expert_offsets, and map each workgroup
id to one (token tile, weight tile) pair, group by group, in runs per XCD
(csrc/experts.hip build_tiles_kernel, csrc/tiles.h tile_of_block).  With
stream tiles enabled, an expert's last tile, when it holds at most SR rows
(a whole small expert, or the rows past its full tiles), is a stream tile
(flagged in bit 30 of its expert field); the others hold BM rows.
These tests restate both in Python, integer for integer, and check on random
routings -- Zipf-skewed, uniform, empty experts, one hot expert -- that
every row of every expert lies in exactly one token tile of at most BM (or
SR) rows, that the host's bound on the list length holds, and that the
launched grid computes every (token tile, weight tile) pair exactly once --
both the grid of one workgroup per pair and the persistent grid of the
64-K kernel, whose workgroups claim tiles with atomic adds on one word per
XCD (csrc/tiles.h, claimed tiles), under random interleavings of the claims.
Section 5 of the ruDNN user guide requires the dispatch to drop no token; a
hole or a double count here would drop or double rows.
"""
import numpy as np
import pytest

MAX_TILE_BITS = 26
STREAM_FLAG = 1 << 30


def max_mtiles(N, E, BM, SR=0):
    """The host's bound on the list length.  Without stream tiles each expert
    adds at most one partial tile; with them an expert of at most SR rows
    adds one tile and a larger one ceil(c / BM) <= 1 + floor(c / BM)."""
    if N <= 0:
        return 0
    if SR:
        return min(N, E + N // BM)
    return min((N + E * (BM - 1)) // BM, N)


def build_tiles(offsets, E, N, BM, max_tiles, G, SR=0):
    """build_tiles_kernel: per expert, in ascending expert order,
    ceil(rows / BM) tiles split into ceil(n / G) groups of near-equal size
    (the first n % ng groups one tile larger); each tile records its group's
    first tile (26 bits) and size (6 bits).  The last tile is a stream tile
    when it holds 1..SR rows (SR < BM)."""
    assert SR < BM
    tiles = []
    t = 0
    for e in range(E):
        b = min(int(offsets[e]), N)
        en = max(min(int(offsets[e + 1]), N), b)
        n = (en - b + BM - 1) // BM
        ng = (n + G - 1) // G
        sz = n // ng if ng else 0
        big = n % ng if ng else 0
        for j in range(n):
            if j < big * (sz + 1):
                first = j // (sz + 1) * (sz + 1)
                gm = sz + 1
            else:
                first = big * (sz + 1) + (j - big * (sz + 1)) // sz * sz
                gm = sz
            r = b + j * BM
            re = min(r + BM, en)
            flag = STREAM_FLAG if re - r <= SR else 0
            if t < max_tiles:
                tiles.append((e | flag, r, re, (t - j + first) | (gm << MAX_TILE_BITS)))
            t += 1
    return tiles, min(t, max_tiles)


def xcd_run(x, live):
    q, rem = live // 8, live % 8
    return (x * (q + 1) if x < rem else rem * (q + 1) + (x - rem) * q), q + (1 if x < rem else 0)


def tile_of_block(bid, nblocks, n_tiles, m_tiles, tiles):
    live = min(nblocks, m_tiles * n_tiles)
    if bid >= live:
        return None
    xcd, loc = bid % 8, bid // 8
    return tile_of_id(xcd_run(xcd, live)[0] + loc, n_tiles, m_tiles, tiles)


def tile_of_id(pid, n_tiles, m_tiles, tiles):
    g = tiles[pid // n_tiles][3]
    first_m = g & ((1 << MAX_TILE_BITS) - 1)
    gm = max(1, min(g >> MAX_TILE_BITS, m_tiles - first_m))
    in_group = pid - first_m * n_tiles
    return first_m + in_group % gm, in_group // gm


def routing_counts(rng, kind, E, N):
    if kind == "zipf":
        w = np.arange(1, E + 1, dtype=np.float64) ** -rng.uniform(0.5, 1.6)
        return rng.multinomial(N, w / w.sum())
    if kind == "uniform":
        return rng.multinomial(N, np.full(E, 1.0 / E))
    if kind == "holes":
        w = rng.random(E) * (rng.random(E) < 0.4)
        if w.sum() == 0:
            w[rng.integers(E)] = 1.0
        return rng.multinomial(N, w / w.sum())
    c = np.zeros(E, np.int64)  # one hot expert
    c[rng.integers(E)] = N
    return c


def check_cover(counts, BM, G, n_tiles, SR=0):
    E = len(counts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    N = int(offsets[-1])
    mt = max_mtiles(N, E, BM, SR)
    # the bound holds without truncation: build with room to spare
    tiles, count = build_tiles(offsets, E, N, BM, mt + 10 ** 6, G, SR)
    assert count == len(tiles) <= mt
    # token tiles: every row of every expert exactly once, in its own expert;
    # a stream tile is an expert's last and holds 1..SR rows, the others
    # hold BM rows, or fewer in an expert's last tile when that is over SR
    seen = np.zeros(N, np.int64)
    for x, r0, r1, _ in tiles:
        e = x & ~STREAM_FLAG
        assert offsets[e] <= r0 < r1 <= offsets[e + 1]
        assert (r0 - offsets[e]) % BM == 0
        if x & STREAM_FLAG:
            assert SR and r1 == offsets[e + 1] and r1 - r0 <= SR
        else:
            assert r1 - r0 == BM or (r1 == offsets[e + 1] and r1 - r0 > SR)
        seen[r0:r1] += 1
    assert (seen == 1).all()
    # groups: consecutive tiles of one expert (its stream tile among them), at most G of them
    for m, (x, _, _, g) in enumerate(tiles):
        first, gm = g & ((1 << MAX_TILE_BITS) - 1), g >> MAX_TILE_BITS
        assert 1 <= gm <= G and first <= m < first + gm
        assert all(tiles[i][0] & ~STREAM_FLAG == x & ~STREAM_FLAG for i in range(first, min(first + gm, count)))
    # the launched grid: every (token tile, weight tile) pair exactly once
    nblocks = mt * n_tiles
    hits = np.zeros((max(count, 1), n_tiles), np.int64)
    for b in range(nblocks):
        r = tile_of_block(b, nblocks, n_tiles, count, tiles)
        if r is not None:
            hits[r] += 1
    assert (hits[:count] == 1).all()
    for seed in range(2):
        claimed = claim_walk(count, n_tiles, nblocks, int(np.random.default_rng(seed).choice([1, 5, 8, 37, 256])),
                             np.random.default_rng(seed + N))
        hits = np.zeros((max(count, 1), n_tiles), np.int64)
        for pid in claimed:
            hits[tile_of_id(pid, n_tiles, count, tiles)] += 1
        assert (hits[:count] == 1).all()


def claim_walk(m_tiles, n_tiles, nblocks, cus, rng):
    """The persistent launch: min(nblocks, cus) workgroups, workgroup b on XCD
    b % 8, each claiming from the front of its XCD's run (one 64-bit word per
    XCD: front claims add 1, back claims 2^32) until that run is used up,
    then from the backs of the other runs, nearest XCD first, and ending when
    all are used up.  Every atomic add is one step, and the steps of all
    workgroups interleave at random.  Returns the logical ids claimed."""
    live = min(nblocks, m_tiles * n_tiles)
    grid = min(nblocks, cus)
    words = [0] * 8
    claimed = []

    def workgroup(b):
        x = b % 8
        while True:
            old = words[x]
            words[x] += 1
            yield
            start, ln = xcd_run(x, live)
            f, bk = old & 0xFFFFFFFF, old >> 32
            if f + bk < ln:
                claimed.append(start + f)
                continue
            for d in range(1, 8):
                v = (x + d) % 8
                start, ln = xcd_run(v, live)
                if ln == 0:
                    continue
                old = words[v]
                words[v] += 1 << 32
                yield
                f, bk = old & 0xFFFFFFFF, old >> 32
                if f + bk < ln:
                    claimed.append(start + ln - 1 - bk)
                    break
            else:
                return

    active = [workgroup(b) for b in range(grid)]
    while active:
        i = int(rng.integers(len(active)))
        try:
            next(active[i])
        except StopIteration:
            active.pop(i)
    assert sorted(claimed) == list(range(live)), "each logical id claimed exactly once"
    return claimed


@pytest.mark.parametrize("live,cus", [(0, 256), (1, 256), (7, 3), (9, 256), (300, 8), (2409, 256), (5000, 256),
                                      (64, 1), (100, 13)])
def test_claims_take_every_id_once(live, cus):
    """Claim words alone, on id ranges of every size against grids of 1 to
    256 workgroups, including XCDs with no workgroup and runs of length 0."""
    for seed in range(6):
        claim_walk(live, 1, live, cus, np.random.default_rng(seed))


@pytest.mark.parametrize("G", range(1, 9))
@pytest.mark.parametrize("kind", ["zipf", "uniform", "holes", "hot"])
def test_tiles_cover_every_row_and_pair_once(G, kind):
    rng = np.random.default_rng(100 * G + len(kind))
    for _ in range(12):
        E = int(rng.choice([1, 3, 8, 64, 256]))
        N = int(rng.integers(0, 6000))
        BM = int(rng.choice([16, 128, 256]))
        n_tiles = int(rng.integers(1, 20))
        check_cover(routing_counts(rng, kind, E, N), BM, G, n_tiles)


@pytest.mark.parametrize("kind", ["zipf", "uniform", "holes", "hot"])
def test_stream_and_block_tiles_cover_every_row_and_pair_once(kind):
    """The 64-K kernel's list: 256-row tiles, and a stream tile for an
    expert's last tile of at most 64 rows."""
    rng = np.random.default_rng(300 + len(kind))
    for _ in range(40):
        E = int(rng.choice([1, 3, 8, 64, 128, 256]))
        N = int(rng.integers(0, 9000))
        check_cover(routing_counts(rng, kind, E, N), 256, 8, int(rng.integers(1, 20)), SR=64)


def test_stream_bound_is_tight_and_holds_at_the_edges():
    """Experts of exactly SR and SR+1 rows, and of 257 rows (two tiles each,
    where the bound E + N / 256 is reached exactly)."""
    for c in (1, 63, 64, 65, 255, 256, 257, 511, 512, 513):
        for E in (1, 7, 100):
            check_cover(np.full(E, c), 256, 8, 3, SR=64)
    counts = np.full(100, 257)
    offsets = np.concatenate([[0], np.cumsum(counts)])
    tiles, count = build_tiles(offsets, 100, int(offsets[-1]), 256, 10 ** 6, 8, 64)
    assert count == max_mtiles(int(offsets[-1]), 100, 256, 64) == 200


def test_prefill_and_skewed_shapes():
    """The benchmark's shapes: 49152 rows over 64 experts (11 and 8 weight
    tiles), 65536 rows over 256 Zipf-skewed experts (16 and 28), with and
    without stream tiles."""
    rng = np.random.default_rng(7)
    for SR in (0, 64):
        check_cover(routing_counts(rng, "uniform", 64, 49152), 256, 8, 11, SR=SR)
        check_cover(routing_counts(rng, "uniform", 64, 49152), 256, 8, 8, SR=SR)
        w = np.arange(1, 257, dtype=np.float64) ** -2.2
        c = rng.multinomial(65536, w / w.sum())
        check_cover(c, 256, 8, 16, SR=SR)
        check_cover(c, 256, 8, 28, SR=SR)


def test_short_last_tiles_become_stream_tiles():
    """769 rows: three 256-row tiles and a stream tile of one row, in the
    expert's group; 64 rows: one stream tile; 321 rows: 256 + a stream tile
    of 65 rows is not allowed, so a 65-row block tile."""
    offsets = np.array([0, 769, 833, 1154])
    tiles, count = build_tiles(offsets, 3, 1154, 256, 100, 8, 64)
    assert [(x & ~STREAM_FLAG, bool(x & STREAM_FLAG), r0, r1) for x, r0, r1, _ in tiles] == [
        (0, False, 0, 256), (0, False, 256, 512), (0, False, 512, 768), (0, True, 768, 769),
        (1, True, 769, 833),
        (2, False, 833, 1089), (2, False, 1089, 1154)]
    assert [(g & ((1 << MAX_TILE_BITS) - 1), g >> MAX_TILE_BITS) for *_, g in tiles] == [
        (0, 4), (0, 4), (0, 4), (0, 4), (4, 1), (5, 2), (5, 2)]


def test_group_bits_hold_the_largest_list():
    # the host refuses lists of 2^26 tiles or more; 6 bits hold sizes up to 63
    assert max_mtiles((1 << 31) - 1, 4096, 128) < (1 << MAX_TILE_BITS)
