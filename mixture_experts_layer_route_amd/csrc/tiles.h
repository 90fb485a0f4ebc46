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

// An expert's rows are cut into BM-row tiles; its last tile, when it holds
// 1..stream_rows rows (a whole small expert, or the rows past its full
// tiles), is a stream tile, marked by this bit in the tile's expert field.
// stream_rows = 0: BM-row tiles only.  (stream_rows < BM.)
constexpr int kStreamTileFlag = 1 << 30;

// Upper bound of the M-tiles that N rows over E experts produce: BM-row
// tiles only (each expert adds at most one partial tile), or with stream
// tiles (an expert of 1..stream_rows rows adds one, a larger one
// ceil(c / BM) <= 1 + floor(c / BM)), so at most E + floor(N / BM).
int64_t max_mtiles(int64_t N, int64_t E, int BM, int stream_rows = 0);
// Writes the (expert, row_begin, row_end, group) M-tile list for
// expert_offsets into tiles (at most max_tiles entries) and its length into
// *count, in one workgroup on stream s; clears the n_queues claim words at
// queues (below), if any.
hipError_t launch_build_tiles(const uint32_t* offsets, int E, int64_t N, int BM, int64_t max_tiles, int4* tiles,
                              uint32_t* count, hipStream_t s, int stream_rows = 0,
                              unsigned long long* queues = nullptr, int n_queues = 0);

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
// for a workgroup with no tile.  tile_of_id is the id -> tile half.
__device__ __forceinline__ void tile_of_id(int pid, int n_tiles, int m_tiles, const int4* __restrict__ tiles,
                                           int* m_idx, int* n_idx) {
    const uint32_t g = (uint32_t)tiles[pid / n_tiles].w;
    const int first_m = (int)(g & 0x3ffffffu);  // 26 bits of first tile, 6 of group size
    const int gm = max(1, min((int)(g >> 26), m_tiles - first_m));
    const int in_group = pid - first_m * n_tiles;
    *m_idx = first_m + in_group % gm;
    *n_idx = in_group / gm;
}
__device__ __forceinline__ bool tile_of_block(int bid, int nblocks, int n_tiles, int m_tiles,
                                              const int4* __restrict__ tiles, int* m_idx, int* n_idx) {
    const int live = min(nblocks, m_tiles * n_tiles);
    if (bid >= live) return false;
    tile_of_id(xcd_contiguous(bid, live), n_tiles, m_tiles, tiles, m_idx, n_idx);
    return true;
}

// ------------------------------------------------------------------ claimed tiles
// A persistent launch (one workgroup per CU) claims logical tile ids at run
// time instead of deriving one from its workgroup id.  XCD x owns the run of
// ids that xcd_contiguous gives it, [start, start + len), and a 64-bit word
// q[x] counts the claims made on that run: the low half those taken from its
// front (by the XCD's own workgroups, in order, so they keep the group walk
// above), the high half those taken from its back (by workgroups of other
// XCDs once their own run is used up).  A claim is one atomic add on the
// word; it succeeds when the front and back counts it returns sum to less
// than len, and then takes the id its own count names.  Each id is thus
// claimed at most once, and every id is claimed before the last workgroup
// finds all eight runs used up.  The tile-list kernel of the same call
// clears the words.
constexpr int kXcds = 8;
struct XcdRun {
    int start, len;
};
__device__ __forceinline__ XcdRun xcd_run(int x, int live) {
    const int q = live / kXcds, rem = live % kXcds;
    return {x < rem ? x * (q + 1) : rem * (q + 1) + (x - rem) * q, q + (x < rem ? 1 : 0)};
}
// The id a front claim on XCD x's run got, from the word the atomic returned; -1: none left.
__device__ __forceinline__ int front_claim(unsigned long long old, int x, int live) {
    const XcdRun r = xcd_run(x, live);
    const uint64_t f = old & 0xffffffffu, b = old >> 32;
    return f + b < (uint64_t)r.len ? r.start + (int)f : -1;
}
// Back claims on the other XCDs' runs, nearest first; -1 when all are used up.
__device__ __forceinline__ int steal_claim(unsigned long long* q, int x, int live) {
    for (int d = 1; d < kXcds; ++d) {
        const int v = (x + d) % kXcds;
        const XcdRun r = xcd_run(v, live);
        if (r.len == 0) continue;
        const unsigned long long old = atomicAdd(q + v, 1ull << 32);
        const uint64_t f = old & 0xffffffffu, b = old >> 32;
        if (f + b < (uint64_t)r.len) return r.start + r.len - 1 - (int)b;
    }
    return -1;
}
// Source row of product row r: r itself, or (fused gather) the token row
// a_rows[r], clamped into the token buffer.
__device__ __forceinline__ int64_t src_row(const uint32_t* __restrict__ a_rows, int a_nrows, int r) {
    return a_rows ? (int64_t)min(a_rows[r], (uint32_t)(a_nrows - 1)) : (int64_t)r;
}

}  // namespace moe
