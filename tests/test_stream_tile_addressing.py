"""Address arithmetic of the 64-K kernel's stream tiles, modelled on the CPU.

A stream tile (csrc/experts.hip, stream_tile) has each of its 8 waves load
32 weight rows of one expert's matrix and 8 of its 64 token rows by direct
global->LDS loads: a wave-uniform base address plus a 32-bit per-lane byte
offset.  These tests restate that arithmetic integer for integer and check,
for every weight tile, wave, lane, load and K step, that each 16-byte load
stays inside the expert's [NOUT, K] matrix (or the token buffer), that no
per-lane offset is negative before its cast to 32 bits, that every LDS
destination and fragment read lies inside the 160 KB ring, and that the
epilogue's 4-wide stores stay inside the output row.  A last weight tile that
NOUT does not fill (NOUT not a multiple of the tile width) once gave waves a
base row past the matrix and a negative offset; the model pins the clamp.
"""
import numpy as np
import pytest

ROWB = 128                  # bytes per row per 64-K step
TOK = 64 * ROWB             # token rows of a stage
STAGE = TOK + 256 * ROWB    # 40 KB
NS = 4
LDS = 160 * 1024
U32 = 1 << 32


def swz128(r):
    return (r & 7) ^ ((r >> 3) & 1)


def weight_offsets(gateup, n0, NOUT, K, wid, lane, j):
    """(base row of the piece, per-lane byte offset before the 32-bit cast,
    the matrix row the lane loads) for weight piece j of wave wid."""
    wi0 = n0 + (16 if gateup else 32) * wid
    row_l = lane >> 3
    brow = 8 * j + row_l
    mrow0 = min(wi0 + (8 * (j & 1) if gateup else 8 * j), NOUT - 1)
    mrow = min(mrow0 + row_l, NOUT - 1)
    off = (mrow - mrow0) * K * 2 + (((lane & 7) ^ swz128(brow)) << 4)
    return mrow0, off, mrow


def check_tile(gateup, NOUT, K, n_idx, r0, r1, x_rows):
    n0 = n_idx * (128 if gateup else 256)
    nk = K // 64
    lanes = np.arange(64)
    for wid in range(8):
        for j in range(4):
            for lane in lanes:
                mrow0, off, mrow = weight_offsets(gateup, n0, NOUT, K, wid, int(lane), j)
                assert 0 <= mrow0 < NOUT and 0 <= off < U32
                for ks in (0, nk - 1):
                    addr = mrow0 * K * 2 + off + ks * ROWB
                    assert 0 <= addr and addr + 16 <= NOUT * K * 2
                    assert (addr - mrow * K * 2) // (K * 2) == 0   # the lane's own row
            # LDS destination of the piece (lane l at +16 l)
            dst = (NS - 1) * STAGE + TOK + wid * 4096 + j * 1024
            assert dst + 1024 <= LDS
        # token piece: rows 8 wid + row_l of the slots, clamped to the tile
        for lane in lanes:
            trow = 8 * wid + (lane >> 3)
            row = min(r0 + trow, r1 - 1)
            assert 0 <= row < x_rows
            off = row * K * 2 + (((lane & 7) ^ swz128(trow)) << 4)
            assert off + (nk - 1) * ROWB + 16 <= x_rows * K * 2 and off < U32
        assert (NS - 1) * STAGE + wid * 1024 + 1024 <= TOK + (NS - 1) * STAGE
        # fragment reads: own weight rows and both token blocks
        for lane in lanes:
            frow, kg = lane & 31, lane >> 5
            for q in range(4):
                c = ((2 * q + kg) ^ swz128(frow)) << 4
                assert TOK + wid * 4096 + frow * ROWB + c + 16 <= STAGE
                assert (32 + frow) * ROWB + c + 16 <= TOK
        # epilogue columns: a 4-wide store that starts inside the row ends inside it
        wi0 = n0 + (16 if gateup else 32) * wid
        for g in range(2 if gateup else 4):
            for kg in (0, 1):
                col = wi0 + 8 * g + 4 * kg
                if col < NOUT:
                    assert col + 4 <= NOUT


@pytest.mark.parametrize("gateup", [True, False])
@pytest.mark.parametrize("NOUT,K", [(192, 256), (64, 64), (448, 192), (1536, 4096), (4096, 1536), (320, 640),
                                    (2048, 7168), (1408, 2048)])
def test_stream_tile_loads_stay_in_their_buffers(gateup, NOUT, K):
    tile = 128 if gateup else 256
    n_tiles = (NOUT + tile - 1) // tile
    x_rows = 1000
    for n_idx in range(n_tiles):
        for r0, r1 in ((0, 1), (0, 64), (936, 1000), (999, 1000), (500, 537)):
            check_tile(gateup, NOUT, K, n_idx, r0, r1, x_rows)


def test_unclamped_base_row_would_leave_the_matrix():
    """The fault the clamp fixes: with NOUT = 192 the second gate/up tile's
    waves 4-7 start past row 191, and without the clamp their lane offsets
    are negative and wrap to about 4 GiB."""
    n0, NOUT, K = 128, 192, 256
    for wid in range(4, 8):
        wi0 = n0 + 16 * wid
        mrow0 = wi0                       # unclamped base row
        mrow = min(mrow0, NOUT - 1)
        assert mrow0 >= NOUT and (mrow - mrow0) * K * 2 < 0
        clamped, off, _ = weight_offsets(True, n0, NOUT, K, wid, 0, 0)
        assert clamped == NOUT - 1 and 0 <= off < U32
