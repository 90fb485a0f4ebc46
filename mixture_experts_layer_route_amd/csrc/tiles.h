// tiles.h -- the per-expert M-tile list of the grouped GEMMs and the
// workgroup -> tile order, shared by experts.hip and train.hip.
#pragma once

#include "moe_internal.h"

namespace moe {

#ifndef MOE_GROUP_M
#define MOE_GROUP_M 8
#endif
constexpr int kGroupM = MOE_GROUP_M;
static_assert(kGroupM >= 1 && kGroupM < 64, "group size is packed in 6 bits");
constexpr int64_t kMaxTiles = int64_t(1) << 26;  // tile index packed in 26 bits

// An expert with 1..stream_rows rows gets a single stream tile (its whole row
// range), marked by this bit in the tile's expert field; the others get
// BM-row tiles.  stream_rows = 0: BM-row tiles only.
constexpr int kStreamTileFlag = 1 << 30;

// Upper bound of the M-tiles that N rows over E experts produce: BM-row
// tiles only (each expert adds at most one partial tile), or with stream
// tiles (an expert of 1..stream_rows rows adds one, a larger one
// ceil(c / BM) <= 1 + floor(c / BM)), so at most E + floor(N / BM).
int64_t max_mtiles(int64_t N, int64_t E, int BM, int stream_rows = 0);
// Writes the (expert, row_begin, row_end, group) M-tile list for
// expert_offsets into tiles (at most max_tiles entries) and its length into
// *count, in one workgroup on stream s.
hipError_t launch_build_tiles(const uint32_t* offsets, int E, int64_t N, int BM, int64_t max_tiles, int4* tiles,
                              uint32_t* count, hipStream_t s, int stream_rows = 0);

// ------------------------------------------------------------------ tile order
// Workgroup id -> logical id: the hardware hands workgroup b of a launch to
// XCD b % 8, and this gives each XCD a contiguous run of the ids [0, n)
// (the first n % 8 XCDs one more), a permutation of [0, n).
__device__ __forceinline__ int xcd_contiguous(int bid, int n) {
    const int q = n / 8, rem = n % 8;
    const int xcd = bid % 8, loc = bid / 8;
    return (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + loc;
}

// Workgroup b -> (token tile, weight tile).  The grid is sized for the most
// token tiles the routing could produce; only the first m_tiles (the count the
// tile-list kernel wrote) exist.  The hardware hands workgroup b to XCD b % 8,
// so the live workgroups are the first m_tiles * n_tiles ids, which every XCD
// shares evenly; their ids are remapped to give each XCD a contiguous run of
// logical tiles.  The run is walked group by group -- a group is a few token
// tiles of ONE expert (at most kGroupM), taken token tile first, then weight
// tile -- so the ~32 workgroups an XCD runs at once share that expert's weight
// tiles and the group's token tiles in the XCD's L2.  A group of g token tiles
// starting at tile f owns logical ids [f * n_tiles, (f + g) * n_tiles), so id
// p belongs to the group recorded with token tile p / n_tiles.  Returns false
// for a workgroup with no tile.
__device__ __forceinline__ bool tile_of_block(int bid, int nblocks, int n_tiles, int m_tiles,
                                              const int4* __restrict__ tiles, int* m_idx, int* n_idx) {
    const int live = min(nblocks, m_tiles * n_tiles);
    if (bid >= live) return false;
    const int pid = xcd_contiguous(bid, live);
    const uint32_t g = (uint32_t)tiles[pid / n_tiles].w;
    const int first_m = (int)(g & 0x3ffffffu);  // 26 bits of first tile, 6 of group size
    const int gm = max(1, min((int)(g >> 26), m_tiles - first_m));
    const int in_group = pid - first_m * n_tiles;
    *m_idx = first_m + in_group % gm;
    *n_idx = in_group / gm;
    return true;
}

// Source row of product row r: r itself, or (fused gather) the token row
// a_rows[r], clamped into the token buffer.
__device__ __forceinline__ int64_t src_row(const uint32_t* __restrict__ a_rows, int a_nrows, int r) {
    return a_rows ? (int64_t)min(a_rows[r], (uint32_t)(a_nrows - 1)) : (int64_t)r;
}

}  // namespace moe
