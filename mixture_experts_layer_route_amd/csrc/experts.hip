// experts.hip -- SwiGLU experts as two grouped GEMMs on CDNA4 matrix cores.
//
// Follows the ruDNN User Guide, section 5 "Expert weights and dispatch"
// (gate and up are [E,I,H], down is [E,H,I], no bias) and the SwiGLU FFN of
// tiny-llm deep dive 5 (ops.rs, "SiLU" block):
//     y = down_e (silu(gate_e x) * up_e x),   silu(z) = z / (1 + exp(-z)).
//
// Both products are "NT" GEMMs: the dispatched rows x (K = H contiguous) and
// the weight rows (also K contiguous) feed the MFMA A and B operands with the
// same per-lane K slice, so no transposition is ever needed.
//   gate/up:  h[r, i] = silu(sum_h x[r,h] gate[e,i,h]) * (sum_h x[r,h] up[e,i,h])
//             -- one workgroup tile holds matching gate and up rows, so the
//             SiLU*mul epilogue is register-local and h is written once, in
//             the weight dtype.
//   down:     y[r, c] = sum_i h[r,i] down[e,c,i]
//
// Row source: row r of the products is either row r of a dispatched copy, or
// (fused gather) token row x[token_of_row[r]] read in place, so the forward
// needs no dispatched copy of the tokens.
//
// Work list: a one-workgroup kernel turns expert_offsets into a list of
// (expert, row_begin, row_end) M-tiles in ascending expert order, on the
// device, so no host sync is needed.  Each XCD walks a contiguous run of the
// live (M-tile, weight tile) pairs, group by group of one expert's tiles:
// the 64-K kernel's persistent workgroups claim them at run time (and take
// tiles off other XCDs' runs once their own is used up), the other kernels
// get one workgroup per pair from a grid sized for the most M-tiles any
// routing could produce.
//
// Four kernels:
//   decode_stream_kernel (bf16/f16, H and I multiples of 64, experts of a
//     few rows each): one persistent workgroup per CU streams units of 32
//     weight rows against token tiles of at most 16 rows, each wave walking
//     8 weight rows 128 bytes per load (the HBM read pattern measured
//     fastest), through an LDS ring that runs on from unit to unit.
//   grouped_gemm_pipe64_kernel (bf16/f16, H and I multiples of 64; the
//     default for prefill-sized batches): one persistent workgroup per CU
//     claiming 256x256 tiles, 8 waves of 32x32x16 MFMAs; 64-element K steps
//     filled by direct global->LDS loads into two token-row slots and three
//     weight-row slots of 32 KB, the weight rows issued about two steps
//     ahead, a quarter per 16-K sub-step, and the token rows one step ahead,
//     in the last sub-step of a step; epilogues staged through LDS while the
//     next tile's first steps load.  An expert of at most 64 rows, and in
//     the gate/up product an expert's last rows past its full tiles when at
//     most 64, run as a stream tile of 64 token slots.
//   grouped_gemm_pipe_kernel (bf16/f16, K a multiple of 32 but not of 64, or
//     a row-operand buffer of 4 GiB or more, which the 64-K kernel's 32-bit
//     offsets cannot span): 256x256 tiles on
//     8 waves of 32x32x16 MFMAs; 32-element K stages filled by direct
//     global->LDS loads in a 4-stage ring, issued three stages ahead and
//     interleaved with the MFMAs and the next fragment reads.
//   grouped_gemm_kernel (f32, other K, and a 16-row tile for few-row experts
//     there): 128-byte K slices staged through registers into padded LDS,
//     double buffered, 16x16 MFMAs.
// FP32 accumulation throughout.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "mfma.h"
#include "tiles.h"

namespace moe {
namespace {

// ------------------------------------------------------------------ tile list
// offsets are clamped to [0, N] and to be non-decreasing per expert, so even
// a corrupt offsets array cannot send a tile outside the row buffers; at most
// max_tiles entries are written.
__device__ uint32_t block_exclusive_scan_1024(uint32_t v, uint32_t* total) {
    __shared__ uint32_t wsum[16];
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) wsum[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        uint32_t s = (lane < 16) ? wsum[lane] : 0u;
        s = wave_inclusive_scan(s);
        if (lane < 16) wsum[lane] = s;
    }
    __syncthreads();
    const uint32_t prefix = wid ? wsum[wid - 1] : 0u;
    *total = wsum[15];
    __syncthreads();
    return prefix + inc - v;
}

__global__ __launch_bounds__(1024) void build_tiles_kernel(const uint32_t* __restrict__ offsets, int E,
                                                           uint32_t N, int BM, uint32_t stream_rows,
                                                           uint32_t max_tiles, int4* __restrict__ tiles,
                                                           uint32_t* __restrict__ count,
                                                           unsigned long long* __restrict__ queues, int n_queues) {
    if ((int)threadIdx.x < n_queues) queues[threadIdx.x] = 0;
    const int per = (E + 1023) / 1024;
    const int e0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const uint32_t b = min(offsets[e], N);
            const uint32_t en = max(min(offsets[e + 1], N), b);
            local += (en - b + BM - 1) / BM;
        }
    }
    uint32_t total;
    uint32_t t = block_exclusive_scan_1024(local, &total);
    for (int i = 0; i < per; ++i) {
        const int e = e0 + i;
        if (e < E) {
            const uint32_t b = min(offsets[e], N);
            const uint32_t en = max(min(offsets[e + 1], N), b);
            // the expert's M-tiles are split into ceil(n / kGroupM) groups of
            // near-equal size; each tile records its group (first tile, size).
            // Its last tile, when it holds at most stream_rows rows (a whole
            // small expert, or the rows past its full tiles), is a stream
            // tile; in the expert's group it reads the weight tiles while the
            // others have them in L2.
            const uint32_t n = (en - b + BM - 1) / BM;
            const uint32_t ng = (n + kGroupM - 1) / kGroupM;
            const uint32_t sz = ng ? n / ng : 0, big = ng ? n % ng : 0;  // `big` groups of sz+1
            for (uint32_t j = 0; j < n; ++j, ++t) {
                uint32_t first, gm;
                if (j < big * (sz + 1)) {
                    first = j / (sz + 1) * (sz + 1);
                    gm = sz + 1;
                } else {
                    first = big * (sz + 1) + (j - big * (sz + 1)) / sz * sz;
                    gm = sz;
                }
                const uint32_t r = b + j * BM, re = min(r + BM, en);
                const int flag = re - r <= stream_rows ? kStreamTileFlag : 0;  // only the last can be short
                if (t < max_tiles) tiles[t] = make_int4(e | flag, (int)r, (int)re, (int)((t - j + first) | (gm << 26)));
            }
        }
    }
    if (threadIdx.x == 0) *count = min(total, max_tiles);
}


// ------------------------------------------------------------------ grouped GEMM



// MFMA operand roles: the weight rows are the A operand (16 rows of the
// output's columns) and the token rows the B operand, so the 16x16 result
// fragment leaves lane l holding token (l % 16) and four consecutive output
// columns 4 (l / 16) + 0..3 -- one 8-byte (bf16/f16) or 16-byte (f32) store.
template <typename DT, bool GATEUP, int BM, int BNB, int WGM, int WGN>
__global__ __launch_bounds__(WGM* WGN* kWave) void grouped_gemm_kernel(
    const typename DT::storage* __restrict__ A,   // [rows, K] token rows
    const typename DT::storage* __restrict__ B0,  // [E, NOUT, K]  (gate or down)
    const typename DT::storage* __restrict__ B1,  // [E, NOUT, K]  (up; GATEUP only)
    typename DT::storage* __restrict__ C,         // [rows, NOUT]
    float* __restrict__ gu,                       // [rows, 2 NOUT] g | u (GATEUP) or null
    const uint32_t* __restrict__ a_rows, int a_nrows, const int4* __restrict__ tiles,
    const uint32_t* __restrict__ tile_count, int K, int NOUT,
    int n_tiles, int nblocks) {
    using S = typename DT::storage;
    constexpr int NT = WGM * WGN * kWave;
    constexpr int ROWB = 128;                 // K bytes per row per pipeline stage
    constexpr int LDS_STRIDE = ROWB + 16;     // padded row stride (bytes)
    constexpr int CPR = ROWB / 16;            // 16-byte chunks per row per stage
    constexpr int A_CHUNKS = BM * CPR, B_CHUNKS = BNB * CPR;
    constexpr int A_CH = (A_CHUNKS + NT - 1) / NT;
    constexpr int B_CH = (B_CHUNKS + NT - 1) / NT;
    constexpr int BN_OUT = GATEUP ? BNB / 2 : BNB;
    constexpr int WTM = BM / WGM;             // token rows per wave
    constexpr int MF = WTM / 16;              // 16-row token fragments per wave
    constexpr int NF = BNB / WGN / 16;        // 16-row weight fragments per wave
    constexpr int WCN = BN_OUT / WGN;         // output columns per wave
    constexpr int STAGE = (BM + BNB) * LDS_STRIDE;
    static_assert(NT % CPR == 0, "chunk column must be fixed per thread");
    static_assert(WTM % 16 == 0 && (BNB / WGN) % 16 == 0, "wave tile must be whole fragments");
    static_assert(!GATEUP || NF % 2 == 0, "gate and up fragments pair up");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    int m_idx, n_idx;
    if (!tile_of_block(blockIdx.x, nblocks, n_tiles, (int)*tile_count, tiles, &m_idx, &n_idx)) return;
    const int4 tl = tiles[m_idx];
    const int e = tl.x, r0 = tl.y, r1 = tl.z;
    const int n0 = n_idx * BN_OUT;
    const int tid = threadIdx.x;
    const int kbytes = K * (int)sizeof(S);
    const int my_ch = tid % CPR;

    const char* a_src[A_CH];
    int a_lds[A_CH];
#pragma unroll
    for (int i = 0; i < A_CH; ++i) {
        const int c = tid + i * NT;
        const int row = min(c / CPR, BM - 1);
        const int grow = min(r0 + row, r1 - 1);
        a_src[i] = (const char*)(A + src_row(a_rows, a_nrows, grow) * K) + my_ch * 16;
        a_lds[i] = row * LDS_STRIDE + my_ch * 16;
    }
    const char* b_src[B_CH];
    int b_lds[B_CH];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) {
        const int c = tid + i * NT;
        const int row = min(c / CPR, BNB - 1);
        const S* base;
        if (GATEUP) {
            const int nrow = min(n0 + (row % BN_OUT), NOUT - 1);
            base = (row < BN_OUT ? B0 : B1) + ((int64_t)e * NOUT + nrow) * K;
        } else {
            const int nrow = min(n0 + row, NOUT - 1);
            base = B0 + ((int64_t)e * NOUT + nrow) * K;
        }
        b_src[i] = (const char*)base + my_ch * 16;
        b_lds[i] = BM * LDS_STRIDE + row * LDS_STRIDE + my_ch * 16;
    }

    uint4 ra[A_CH], rb[B_CH];
    // Loads never branch on K: a chunk past K reads a valid address (step 0's)
    // and is zeroed when it is written to LDS, once it has arrived.  (Zeroing
    // it at the load made the compiler clear the register and load into it
    // under a mask, and wait for each load before issuing the next: two
    // memory round trips per step.)
    auto gload = [&](int kt) {
        const int kb = kt * ROWB;
        const int off = kb + my_ch * 16 < kbytes ? kb : 0;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            if (A_CHUNKS % NT == 0 || tid + i * NT < A_CHUNKS) ra[i] = *(const uint4*)(a_src[i] + off);
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            if (B_CHUNKS % NT == 0 || tid + i * NT < B_CHUNKS) rb[i] = *(const uint4*)(b_src[i] + off);
    };
    auto lstore = [&](int st, int kt) {
        unsigned char* base = smem + st * STAGE;
        // a select per 32-bit word: a select of whole uint4 values would
        // pick between their addresses and move the arrays to scratch
        const uint32_t keep = kt * ROWB + my_ch * 16 < kbytes ? ~0u : 0u;
        auto masked = [keep](const uint4& v) {
            return make_uint4(v.x & keep, v.y & keep, v.z & keep, v.w & keep);
        };
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            if (A_CHUNKS % NT == 0 || tid + i * NT < A_CHUNKS) *(uint4*)(base + a_lds[i]) = masked(ra[i]);
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            if (B_CHUNKS % NT == 0 || tid + i * NT < B_CHUNKS) *(uint4*)(base + b_lds[i]) = masked(rb[i]);
    };

    const int lane = lane_id(), wid = tid / kWave;
    const int wm = wid / WGN, wn = wid % WGN;
    int fa[MF], fb[NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) fa[i] = (wm * WTM + i * 16 + (lane & 15)) * LDS_STRIDE + (lane >> 4) * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
        int brow;
        if (GATEUP)
            brow = (f < NF / 2) ? wn * WCN + f * 16 : BN_OUT + wn * WCN + (f - NF / 2) * 16;
        else
            brow = wn * (BNB / WGN) + f * 16;
        fb[f] = BM * LDS_STRIDE + (brow + (lane & 15)) * LDS_STRIDE + (lane >> 4) * 16;
    }

    f32x4_t acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = (kbytes + ROWB - 1) / ROWB;
    gload(0);
    lstore(0, 0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) gload(kt + 1);
        const unsigned char* base = smem + st * STAGE;
#pragma unroll
        for (int kk = 0; kk < ROWB / 64; ++kk) {
            uint4 av[MF], bv[NF];
#pragma unroll
            for (int i = 0; i < MF; ++i) av[i] = *(const uint4*)(base + fa[i] + kk * 64);
#pragma unroll
            for (int f = 0; f < NF; ++f) bv[f] = *(const uint4*)(base + fb[f] + kk * 64);
#pragma unroll
            for (int i = 0; i < MF; ++i)
#pragma unroll
                for (int f = 0; f < NF; ++f) acc[i][f] = mma<DT>::run(bv[f], av[i], acc[i][f]);
        }
        if (kt + 1 < nk) lstore(st ^ 1, kt + 1);
        __syncthreads();
    }

    // epilogue: lane holds token (lane % 16) of each token fragment and
    // output columns 4 (lane / 16) + 0..3 of each weight fragment
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const int grow = r0 + wm * WTM + i * 16 + (lane & 15);
        if (grow >= r1) continue;
        S* crow = C + (int64_t)grow * NOUT;
        if (GATEUP) {
#pragma unroll
            for (int f = 0; f < NF / 2; ++f) {
                const int col = n0 + wn * WCN + f * 16 + (lane >> 4) * 4;
                if (col < NOUT) {
                    float v[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = silu_mul(acc[i][f][r], acc[i][f + NF / 2][r]);
                    store4<DT>::run(crow + col, v);
                    if (gu) {
                        const float g4[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
                        const float u4[4] = {acc[i][f + NF / 2][0], acc[i][f + NF / 2][1], acc[i][f + NF / 2][2],
                                             acc[i][f + NF / 2][3]};
                        save_preact(gu, grow, NOUT, col, g4, u4);
                    }
                }
            }
        } else {
#pragma unroll
            for (int f = 0; f < NF; ++f) {
                const int col = n0 + wn * WCN + f * 16 + (lane >> 4) * 4;
                if (col < NOUT) {
                    float v[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
                    store4<DT>::run(crow + col, v);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ pipelined grouped GEMM (16-bit)
// The large-tile kernel for bf16/f16: a 256-token x 256-weight-row workgroup
// tile, a ring of 4 LDS stages of 32 K-elements each, filled by direct
// global->LDS loads (global_load_lds_dwordx4: each wave instruction writes
// 1 KB of LDS, lane l at +16 l), issued three stages ahead.  Every LDS row is
// 64 bytes; the 16-byte chunk c of row r sits at chunk c ^ swz64(r), so
// the 16 rows a fragment read touches spread over all banks.  While the
// matrix cores work on step k, the wave reads the fragments of step k+1 into
// a second register set; one barrier per step publishes the next stage.
// Requires K % 32 == 0 (no tail handling: loads never leave the rows).
#ifndef MOE_P_STAGES
#define MOE_P_STAGES 4
#endif
#ifndef MOE_P_BK64
#define MOE_P_BK64 1
#endif
#ifndef MOE_P64_WM
#define MOE_P64_WM 2   // waves along token rows of the 64-K kernel's tile
#define MOE_P64_WN 4   // waves along weight rows
#endif
#ifndef MOE_P_BN
#define MOE_P_BN 256
#endif
constexpr int kPipeBM = 256, kPipeBN = MOE_P_BN, kPipeBK = 32, kPipeStages = MOE_P_STAGES;
constexpr int kPipeAhead = kPipeStages - 1;  // K steps of DMA in flight ahead of the reads


// Epilogue of the 32x32-block kernels: lane holds token (lane % 32) of each
// token block and output columns 8 (r / 4) + 4 (lane / 32) + (r % 4) of each
// weight block; gate/up pairs go through SiLU*mul, rows past r1 and columns
// past NOUT are not written.
template <typename DT, bool GATEUP, int MB, int NB, int WTM, int WTN, int WCN>
__device__ __forceinline__ void store_tile32(const f32x16_t (&acc)[MB][NB], typename DT::storage* __restrict__ C,
                                             float* __restrict__ gu, int r0, int r1, int n0, int wm, int wn,
                                             int NOUT, int lane) {
    using S = typename DT::storage;
    const int frow = lane & 31;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int grow = r0 + wm * WTM + i * 32 + frow;
        if (grow >= r1) continue;
        S* crow = C + (int64_t)grow * NOUT;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int cb = g * 8 + (lane >> 5) * 4;
            if (GATEUP) {
#pragma unroll
                for (int f = 0; f < NB / 2; ++f) {
                    const int col = n0 + wn * WCN + f * 32 + cb;
                    if (col < NOUT) {
                        float v[4];
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            v[r] = silu_mul(acc[i][f][g * 4 + r], acc[i][f + NB / 2][g * 4 + r]);
                        store4<DT>::run(crow + col, v);
                        if (gu) {
                            float g4[4], u4[4];
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                g4[r] = acc[i][f][g * 4 + r];
                                u4[r] = acc[i][f + NB / 2][g * 4 + r];
                            }
                            save_preact(gu, grow, NOUT, col, g4, u4);
                        }
                    }
                }
            } else {
#pragma unroll
                for (int f = 0; f < NB; ++f) {
                    const int col = n0 + wn * WTN + f * 32 + cb;
                    if (col < NOUT) {
                        float v[4] = {acc[i][f][g * 4], acc[i][f][g * 4 + 1], acc[i][f][g * 4 + 2],
                                      acc[i][f][g * 4 + 3]};
                        store4<DT>::run(crow + col, v);
                    }
                }
            }
        }
    }
}

// The training forward's FP32 pre-activations of the gate/up product (g at
// columns [0, I) of a row of gu, u at [I, 2I)), staged through LDS: per
// round of RR token rows (32 or 64) each wave writes its RR x 32 g and u
// values into its own RR * 256 bytes (128-byte rows, g rows then u rows,
// 16-byte chunk c of row t at c ^ ((t / 2) % 8)), then reads them back a
// chunk per lane, so a store instruction writes 8 whole 128-byte row
// segments instead of 16 bytes of 32 rows.
template <int MB, int NB, int WTM, int WCN, int RR = 64>
__device__ __forceinline__ void save_preact_staged(const f32x16_t (&acc)[MB][NB], float* __restrict__ gu, int r0,
                                                   int r1, int n0, int wm, int wn, int I, int lane,
                                                   unsigned char* stage) {
    static_assert(WCN == 32 && NB == 2, "one gate and one up block of 32 columns per wave");
    static_assert((RR == 32 || RR == 64) && (MB * 32) % RR == 0, "rounds of whole 32-row blocks");
    constexpr int BPR = RR / 32, UOFF = RR * 128;  // blocks per round; offset of the u rows
    asm volatile("" : "+v"(lane));  // keeps the addresses out of the K loop
    const int frow = lane & 31, kg = lane >> 5;
    const int c = lane & 7, rr = lane >> 3;
    const int col = n0 + wn * WCN + 4 * c;
#pragma unroll
    for (int h = 0; h < MB / BPR; ++h) {
#pragma unroll
        for (int ii = 0; ii < BPR; ++ii) {
            const int t = 32 * ii + frow, sw = (t >> 1) & 7;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const f32x16_t& ga = acc[BPR * h + ii][0];
                const f32x16_t& ua = acc[BPR * h + ii][1];
                const int a = t * 128 + (((2 * g + kg) ^ sw) << 4);
                *(float4*)(stage + a) = make_float4(ga[4 * g], ga[4 * g + 1], ga[4 * g + 2], ga[4 * g + 3]);
                *(float4*)(stage + UOFF + a) = make_float4(ua[4 * g], ua[4 * g + 1], ua[4 * g + 2], ua[4 * g + 3]);
            }
        }
        wait_lgkm0();
#pragma unroll
        for (int t0 = 0; t0 < RR; t0 += 8) {
            const int t = t0 + rr;
            const int a = t * 128 + ((c ^ ((t >> 1) & 7)) << 4);
            const float4 g4 = *(const float4*)(stage + a);
            const float4 u4 = *(const float4*)(stage + UOFF + a);
            const int grow = r0 + wm * WTM + RR * h + t;
            if (grow < r1 && col < I) {
                float* p = gu + (int64_t)grow * 2 * I + col;
                *(float4*)p = g4;
                *(float4*)(p + I) = u4;
            }
        }
        wait_lgkm0();  // read back before the next round rewrites the region
    }
}

#ifndef MOE_P_MINB
#define MOE_P_MINB 1   // workgroups per CU the register budget must allow
#endif
template <typename DT, bool GATEUP, int WGM, int WGN>
__global__ __launch_bounds__(WGM* WGN* kWave, MOE_P_MINB) void grouped_gemm_pipe_kernel(
    const typename DT::storage* __restrict__ A, const typename DT::storage* __restrict__ B0,
    const typename DT::storage* __restrict__ B1, typename DT::storage* __restrict__ C, float* __restrict__ gu,
    const uint32_t* __restrict__ a_rows, int a_nrows, const int4* __restrict__ tiles,
    const uint32_t* __restrict__ tile_count, int K, int NOUT, int n_tiles,
    int nblocks) {
    using S = typename DT::storage;
    constexpr int NW = WGM * WGN;
    constexpr int ROWB = kPipeBK * 2;                      // 64 bytes per row per stage
    constexpr int STAGE = (kPipeBM + kPipeBN) * ROWB;      // 32 KB
    constexpr int LPW = (kPipeBM + kPipeBN) * ROWB / 1024 / NW;  // 1 KB loads per wave per stage
    constexpr int BN_OUT = GATEUP ? kPipeBN / 2 : kPipeBN;
    constexpr int WTM = kPipeBM / WGM, WTN = kPipeBN / WGN;
    constexpr int MB = WTM / 32, NB = WTN / 32;            // 32x32 blocks per wave
    constexpr int WCN = BN_OUT / WGN;
    static_assert(!GATEUP || NB % 2 == 0, "gate and up blocks pair up");

    constexpr int NSTAGE = kPipeStages;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NSTAGE * STAGE];

    int m_idx, n_idx;
    if (!tile_of_block(blockIdx.x, nblocks, n_tiles, (int)*tile_count, tiles, &m_idx, &n_idx)) return;
    const int4 tl = tiles[m_idx];
    const int e = tl.x, r0 = tl.y, r1 = tl.z;
    const int n0 = n_idx * BN_OUT;
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const int wm = wid / WGN, wn = wid % WGN;

    // global sources of this lane's LDS-DMA chunks (one per load instruction)
    const char* src[LPW];
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
        const int row = (wid * LPW + j) * 16 + (lane >> 2);  // stage row 0..511
        const int lc = (lane & 3) ^ swz64(row);              // logical chunk for this physical slot
        const S* p;
        if (row < kPipeBM) {
            p = A + src_row(a_rows, a_nrows, min(r0 + row, r1 - 1)) * K;
        } else {
            const int w = row - kPipeBM;
            if (GATEUP)
                p = (w < BN_OUT ? B0 : B1) + ((int64_t)e * NOUT + min(n0 + (w % BN_OUT), NOUT - 1)) * K;
            else
                p = B0 + ((int64_t)e * NOUT + min(n0 + w, NOUT - 1)) * K;
        }
        src[j] = (const char*)p + lc * 16;
    }
    const int nk = K / kPipeBK;
    const uint32_t smem_base = lds_offset(smem) + wid * LPW * 1024;
    // fragment rows; the swizzle term depends only on the lane for every block
    const int frow = lane & 31;
    const int sw0 = (((lane >> 5) + 0) ^ swz64(frow)) * 16;  // K half 0 of a stage
    const int sw1 = (((lane >> 5) + 2) ^ swz64(frow)) * 16;  // K half 1
    const int fa0 = (wm * WTM + frow) * ROWB;
    int fb[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
        int brow;
        if (GATEUP)
            brow = (f < NB / 2) ? wn * WCN + f * 32 : BN_OUT + wn * WCN + (f - NB / 2) * 32;
        else
            brow = wn * WTN + f * 32;
        fb[f] = (kPipeBM + brow + frow) * ROWB;
    }

    // Token blocks of 32 rows that lie wholly past the tile's last row are
    // skipped (wave-uniform): the last tile of an expert is often nearly
    // empty, and its MFMAs would otherwise cost as much as a full tile.
    const int rows_live = __builtin_amdgcn_readfirstlane(r1 - r0) - __builtin_amdgcn_readfirstlane(wm) * WTM;
    f32x16_t acc[MB][NB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int f = 0; f < NB; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;

    uint4 av[2][MB], bv[2][NB];
    auto read_frags = [&](int kt, int half, int set) {
        const unsigned char* base = smem + (kt % NSTAGE) * STAGE + (half ? sw1 : sw0);
#pragma unroll
        for (int i = 0; i < MB; ++i) av[set][i] = *(const uint4*)(base + fa0 + i * 32 * ROWB);
#pragma unroll
        for (int f = 0; f < NB; ++f) bv[set][f] = *(const uint4*)(base + fb[f]);
    };
    {
        // DMA of one 1 KB piece j of K step kt; steps past the end re-load the
        // last step into a stage nobody reads again, so every count is static
        auto issue_part = [&](int kt, int j) {
            const int ks = min(kt, nk - 1);
            lds_dma16(src[j] + ks * ROWB, smem_base + (kt % NSTAGE) * STAGE + j * 1024);
        };
        static_assert(LPW % 2 == 0 && LPW / 2 <= MB * NB, "DMA pieces spread over the MFMAs");
        // One fragment read (r < MB: token block r, else weight block r - MB).
        auto read_one = [&](int kt, int half, int set, int r) {
            const unsigned char* base = smem + (kt % NSTAGE) * STAGE + (half ? sw1 : sw0);
            if (r < MB)
                av[set][r] = *(const uint4*)(base + fa0 + r * 32 * ROWB);
            else
                bv[set][r - MB] = *(const uint4*)(base + fb[r - MB]);
        };
        // The MFMAs of one K half (operands in `set`), with the fragment reads
        // of the next K half (rkt, rhalf) into the other set spread over the
        // first half of the MFMAs and the DMA pieces [j0, j0 + LPW/2) of step
        // dkt over the second half.  Issue is in order, so a burst of reads or
        // DMAs would hold the MFMAs behind a full queue; one or two per MFMA
        // keep the matrix pipe fed while the reads still land a quarter stage
        // before their use.  The fences pin this order against the scheduler.
        // `full` (a std::bool_constant) says every token block of the wave
        // holds live rows, so the common case carries no per-MFMA branch.
        // `nd` (a std::integral_constant) is the number of DMA pieces, issued
        // by calling dma(d) for d = 0 .. nd-1.
        auto compute_mix = [&](auto full, auto nd, int set, int rkt, int rhalf, auto&& dma) {
            constexpr int NM = MB * NB, NR = MB + NB, ND = decltype(nd)::value, H1 = NM / 2, H2 = NM - NM / 2;
#pragma unroll
            for (int m = 0; m < NM; ++m) {
                const int i = m / NB, f = m % NB;
                if (decltype(full)::value || i * 32 < rows_live)
                    acc[i][f] = mma32<DT>::run(bv[set][f], av[set][i], acc[i][f]);
                if (m < H1) {
#pragma unroll
                    for (int r = (m * NR) / H1; r < ((m + 1) * NR) / H1; ++r) read_one(rkt, rhalf, set ^ 1, r);
                } else {
                    const int q = m - H1;
#pragma unroll
                    for (int d = (q * ND) / H2; d < ((q + 1) * ND) / H2; ++d) dma(d);
                }
                sched_fence();
            }
        };
        using half_dma = std::integral_constant<int, LPW / 2>;
#pragma unroll
        for (int p = 0; p < kPipeAhead; ++p)
#pragma unroll
            for (int j = 0; j < LPW; ++j) issue_part(p, j);
        wait_vm<(kPipeAhead - 1) * LPW>();  // stage 0 landed
        barrier_lds();
        read_frags(0, 0, 0);
        // Per K step: multiply the first K half while reading the second half
        // and starting half of the DMA of step kt+3; publish stage kt+1; then
        // multiply the second half while reading the first half of step kt+1
        // and starting the rest of the DMA.
        auto main_loop = [&](auto full) {
            for (int kt = 0; kt < nk; ++kt) {
                // the first half's fragments were read a whole K half ago; an
                // explicit wait here lets the compiler see the counter at zero,
                // so the half's MFMAs do not wait on the reads issued next
                wait_lgkm0();
                compute_mix(full, half_dma{}, 0, kt, 1, [&](int d) { issue_part(kt + kPipeAhead, d); });
                // stage kt+1 landed; step kt+2 and half of kt+3 may be in
                // flight.  This wave's reads of stage kt complete before the
                // barrier, so the stage can be refilled once every wave has
                // passed it.
                wait_vm<(kPipeAhead - 2) * LPW + LPW / 2>();
                wait_lgkm0();
                barrier_lds();
                compute_mix(full, half_dma{}, 1, kt + 1, 0, [&](int d) { issue_part(kt + kPipeAhead, LPW / 2 + d); });
            }
        };
        if (rows_live >= MB * 32)
            main_loop(std::true_type{});
        else
            main_loop(std::false_type{});
        wait_vm<0>();
    }

    store_tile32<DT, GATEUP, MB, NB, WTM, WTN, WCN>(acc, C, gu, r0, r1, n0, wm, wn, NOUT, lane);
}

// ------------------------------------------------------------------ stream tiles
// An expert's last token tile, when it holds at most kStreamRows rows (a
// whole small expert, or the rows past its full tiles), runs as a stream
// tile: its rows (64 token slots) against 256 weight rows, on the 64-K
// kernel's workgroup of 8 waves and 160 KB of LDS.  Such a product is a
// stream of weight rows
// (each is used by a few tokens only), so the tile is built for bytes in
// flight: a ring of 4 stages of 40 KB (64 token rows and 256 weight rows of
// 128 bytes, chunk c of row r at c ^ swz128(r)), filled by direct global->LDS
// loads issued 3 steps ahead, 120 KB in flight per CU.
//   Each wave owns 32 weight rows -- it loads them and only it reads them --
// and one 32x32 MFMA block of them: for gate/up, rows 0-15 are gate rows
// i0..i0+15 and rows 16-31 the up rows of the same i, so every lane holds
// matching g and u (result rows 8 (r / 4) + 4 (lane / 32) + r % 4) and the
// SiLU*mul stays in registers; for down, 32 output columns.  Each wave also
// loads 8 of the 64 token rows, which all waves read: one barrier per step
// publishes them and frees the stage read a step before.
constexpr int kStreamRows = 64;
constexpr int kStreamStages = 4;

template <typename DT, bool GATEUP>
__device__ __forceinline__ void stream_tile(const typename DT::storage* __restrict__ A,
                                            const typename DT::storage* __restrict__ B0,
                                            const typename DT::storage* __restrict__ B1,
                                            typename DT::storage* __restrict__ C, float* __restrict__ gu,
                                            const uint32_t* __restrict__ a_rows, int a_nrows, int e, int r0, int r1,
                                            int n0, int K, int NOUT, int wid, int lane, unsigned char* smem) {
    using S = typename DT::storage;
    constexpr int ROWB = 128;                                     // bytes per row per 64-K step
    constexpr int TOK = kStreamRows * ROWB;                       // 8 KB of token rows per stage
    constexpr int STAGE = TOK + 256 * ROWB;                       // 40 KB
    constexpr int NS = kStreamStages, AHEAD = NS - 1;
    constexpr int PIECES = 5;                                     // 1 KB DMA pieces per wave and step
    static_assert(NS * STAGE <= 160 * 1024, "the ring fits the LDS");
    const int nk = K / 64;
    // this wave's 32 weight rows: gate/up rows of i in [wi0, wi0 + 16), or
    // down rows (output columns) [wi0, wi0 + 32)
    const int wi0 = n0 + (GATEUP ? 16 : 32) * wid;
    const int row_l = lane >> 3;                                  // row of this lane within a piece
    // weight pieces j = 0..3: rows 8 j + row_l of the block; gate/up blocks
    // take gate rows for j < 2 and up rows for j >= 2.  Rows past the
    // matrix's last row (a last weight tile that NOUT does not fill) read
    // that last row; the piece's base row is clamped the same way, so the
    // lane offset from it is never negative.
    const char* wbase[4];
    uint32_t woff[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int brow = 8 * j + row_l;                           // block row 0..31
        const S* m = (GATEUP && j >= 2) ? B1 : B0;
        const int mrow0 = min(wi0 + (GATEUP ? 8 * (j & 1) : 8 * j), NOUT - 1);  // base row of the piece
        const int mrow = min(mrow0 + row_l, NOUT - 1);
        wbase[j] = (const char*)(m + ((int64_t)e * NOUT + mrow0) * K);
        woff[j] = (uint32_t)((int64_t)(mrow - mrow0) * K * (int64_t)sizeof(S)) + (((lane & 7) ^ swz128(brow)) << 4);
    }
    // token piece: rows 8 wid + row_l of the 64 token slots, clamped to the
    // tile's last row (slots past it are computed but never stored)
    const int trow = 8 * wid + row_l;
    const uint32_t toff = (uint32_t)(src_row(a_rows, a_nrows, min(r0 + trow, r1 - 1)) * K * (int64_t)sizeof(S)) +
                          (((lane & 7) ^ swz128(trow)) << 4);
    const uint32_t lds0 = lds_offset(smem);
    auto issue = [&](int kt) {
        const int ks = min(kt, nk - 1);                           // past the end: re-load the last step
        const uint32_t st = lds0 + (kt % NS) * STAGE;
        lds_dma16_so((const char*)A + ks * ROWB, toff, st + wid * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) lds_dma16_so(wbase[j] + ks * ROWB, woff[j], st + TOK + wid * 4096 + j * 1024);
    };
    const int frow = lane & 31, kg = lane >> 5;
    f32x16_t acc[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[b][r] = 0.0f;
#pragma unroll
    for (int p = 0; p < AHEAD; ++p) issue(p);
    for (int kt = 0; kt < nk; ++kt) {
        // step kt landed (only the pieces of kt+1 and kt+2 may be in flight);
        // after the barrier every wave's token rows of kt are in, and every
        // wave is done with the stage of kt-1, which the loads of kt+3 reuse
        wait_vm<(AHEAD - 1) * PIECES>();
        barrier_lds();
        issue(kt + AHEAD);
        const unsigned char* st = smem + (kt % NS) * STAGE;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int c = ((2 * q + kg) ^ swz128(frow)) << 4;
            const uint4 w = *(const uint4*)(st + TOK + wid * 4096 + frow * ROWB + c);
            const uint4 t0 = *(const uint4*)(st + frow * ROWB + c);
            const uint4 t1 = *(const uint4*)(st + (32 + frow) * ROWB + c);
            acc[0] = mma32<DT>::run(w, t0, acc[0]);
            acc[1] = mma32<DT>::run(w, t1, acc[1]);
        }
    }
    wait_vm<0>();
    // lane: token slot 32 b + frow; block rows 8 g + 4 kg + 0..3 in acc[b][4 g ..]
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int grow = r0 + 32 * b + frow;
        if (grow >= r1) continue;
        S* crow = C + (int64_t)grow * NOUT;
        if constexpr (GATEUP) {
#pragma unroll
            for (int g = 0; g < 2; ++g) {                         // gate rows 8 g + 4 kg + 0..3, up rows 16 + ...
                const int col = wi0 + 8 * g + 4 * kg;
                if (col < NOUT) {
                    float v[4], g4[4], u4[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        g4[r] = acc[b][4 * g + r];
                        u4[r] = acc[b][8 + 4 * g + r];
                        v[r] = silu_mul(g4[r], u4[r]);
                    }
                    store4<DT>::run(crow + col, v);
                    if (gu) save_preact(gu, grow, NOUT, col, g4, u4);
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int col = wi0 + 8 * g + 4 * kg;
                if (col < NOUT) {
                    const float v[4] = {acc[b][4 * g], acc[b][4 * g + 1], acc[b][4 * g + 2], acc[b][4 * g + 3]};
                    store4<DT>::run(crow + col, v);
                }
            }
        }
    }
}

// ------------------------------------------------------------------ decode stream kernel
// For batches whose experts own a few rows each (decode), where the products
// are a stream of weight rows that each serve a handful of tokens, so the
// kernel is built around the HBM read pattern.  Measured on this chip with
// direct global->LDS loads: a wave whose loads in flight spread over 32 rows
// of an 8 KB-pitch matrix streams at 5.2 TB/s in all (8 rows x 128 B or
// 1 row x 1 KB per load alike), over 16 rows at 5.5-5.8, and over 8 rows --
// walking them 128 bytes per load -- at 6.2-6.4, above a contiguous stream
// (6.1).  So each wave owns 8 weight rows, one 1 KB load (8 rows x 128 B)
// per 64 K.
//   One persistent workgroup of 4 waves per CU walks units of (a token tile
// of at most 16 rows, 32 weight rows): workgroup b of G takes units b,
// b + G, ...  A unit's K runs in steps of 256 (4 quarters of 64): per step
// each wave loads its 8 rows' 4 quarters and 2 of the 8 token pieces (16
// token rows x one quarter half), 6 loads of 1 KB; the ring of 6 stages of
// 24 KB (LDS rows of 128 bytes, chunk c of row r at c ^ swz128(r)) runs on
// from one unit into the next, so the stream never drains between units,
// and the ~40 units per workgroup at decode size keep the launch's tail
// short.  Each XCD's workgroups take adjacent units.  For gate/up a wave's
// rows are gate rows i0 .. i0 + 3 and the up rows of the same i; for down,
// 8 output columns.
//   16x16x32 MFMAs take the wave's 8 rows twice (rows 8-15 repeat 0-7) as
// the first operand and the 16 token slots as the second; lanes 0-31 then
// hold the 8 rows of one token each.  The waits on the vector-memory
// counter are counted by hand (6 loads per wave and step), so every other
// memory read here is a scalar load (the unit's tile, the token row
// indices), which that counter does not see; the loads past a workgroup's
// last step re-load that step into the stage the ring has just freed,
// keeping the count of loads per step fixed.  A last step past K (K a
// multiple of 64 but not of 256) loads its missing quarters from the last
// valid one and skips their MFMAs.
#ifndef MOE_DEC_ROWS
#define MOE_DEC_ROWS 16
#define MOE_DEC_STAGES 6
#endif
constexpr int kDecRows = MOE_DEC_ROWS, kDecWaveRows = 8, kDecStages = MOE_DEC_STAGES, kDecWaves = 4;
// The host takes this kernel when no expert can own more than kStreamRows
// rows, or when the experts own at most kDecMeanRows rows on average: then
// even an expert that owns every row costs at most N / kDecRows extra
// passes over its weights, E + N / kDecRows <= 1.25 E expert matrices read
// in all, against E for kernels with taller tiles.
constexpr int kDecMeanRows = 4;

// Scalar loads of values the whole wave shares.
__device__ __forceinline__ uint32_t sload_u32(const uint32_t* p) {
    uint32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return v;
}
// Eight scalar loads with one wait: p[i0], ..., p[i7].
__device__ __forceinline__ void sload8(const uint32_t* p, const int (&i)[8], uint32_t (&v)[8]) {
    asm volatile(
        "s_load_dword %0, %8, 0x0\n\ts_load_dword %1, %9, 0x0\n\t"
        "s_load_dword %2, %10, 0x0\n\ts_load_dword %3, %11, 0x0\n\t"
        "s_load_dword %4, %12, 0x0\n\ts_load_dword %5, %13, 0x0\n\t"
        "s_load_dword %6, %14, 0x0\n\ts_load_dword %7, %15, 0x0\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&s"(v[0]), "=&s"(v[1]), "=&s"(v[2]), "=&s"(v[3]), "=&s"(v[4]), "=&s"(v[5]), "=&s"(v[6]), "=&s"(v[7])
        : "s"(p + i[0]), "s"(p + i[1]), "s"(p + i[2]), "s"(p + i[3]), "s"(p + i[4]), "s"(p + i[5]), "s"(p + i[6]),
          "s"(p + i[7])
        : "memory");
}
__device__ __forceinline__ int4 sload_int4(const int4* p) {
    typedef int v4i_t __attribute__((ext_vector_type(4)));
    v4i_t v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p) : "memory");
    return make_int4(v.x, v.y, v.z, v.w);
}

template <typename DT, bool GATEUP>
__global__ __launch_bounds__(kDecWaves* kWave, 1) void decode_stream_kernel(
    const typename DT::storage* __restrict__ A, const typename DT::storage* __restrict__ B0,
    const typename DT::storage* __restrict__ B1, typename DT::storage* __restrict__ C, float* __restrict__ gu,
    const uint32_t* __restrict__ a_rows, int a_nrows, const int4* __restrict__ tiles,
    const uint32_t* __restrict__ tile_count, int K, int NOUT, int n_units) {
    using S = typename DT::storage;
    constexpr int ROWB = 128;                                  // bytes per row per quarter (64 K)
    constexpr int TQ = kDecRows * ROWB;                        // 2 KB: the token rows of one quarter
    constexpr int TOK = 4 * TQ;                                // 8 KB of token rows per stage
    constexpr int WQ = kDecWaveRows * ROWB;                    // 1 KB: a wave's rows of one quarter
    constexpr int STAGE = TOK + kDecWaves * 4 * WQ;            // 24 KB
    constexpr int TPW = kDecRows / 8;                          // token loads per wave and step
    constexpr int NS = kDecStages, PIECES = 4 + TPW;           // 1 KB loads per wave and step
    constexpr int UN = GATEUP ? kDecWaves * kDecWaveRows / 2 : kDecWaves * kDecWaveRows;  // outputs per unit
    constexpr int WN = UN / kDecWaves;                         // outputs per wave
    static_assert(NS * STAGE <= 160 * 1024 && (NS - 2) * PIECES < 64, "ring fits the LDS and the counter");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NS * STAGE];

    const int lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    // units b, b + G, ... of workgroup b, numbered so that the ~32
    // workgroups of each XCD stream adjacent units (adjacent weight rows):
    // measured 4.6% faster on decode gate/up than consecutive workgroups on
    // adjacent units, which spreads every XCD's rows over the whole window
    const int G = (int)gridDim.x, b = xcd_contiguous((int)blockIdx.x, (int)gridDim.x);
    const int U = (int)sload_u32(tile_count) * n_units;
    if (b >= U) return;
    const int nu = (U - 1 - b) / G + 1;                        // this workgroup's units
    const int nq = K / 64, nk = (nq + 3) / 4;                  // quarters, steps of 4 quarters
    const int row_l = lane >> 3;                               // row of this lane within a 1 KB load

    // the unit's tile: expert, token rows [r0, r1), first output
    auto unit_tile = [&](int j, int& e, int& r0, int& r1, int& n0) __attribute__((always_inline)) {
        const int u = b + j * G;
        const int mi = u / n_units;
        const int4 tl = sload_int4(tiles + mi);
        e = tl.x;
        r0 = tl.y;
        r1 = tl.z;
        n0 = (u - mi * n_units) * UN;
    };

    // ---- issue cursor: unit iu, step is; the addressing of unit iu
    int iu = 0, is = 0;
    const char* wptr = nullptr;                                // this lane's weight row, chunk included
    uint32_t toff[TPW];                                        // token slots 8 h + row_l
    auto set_unit = [&](int j) __attribute__((always_inline)) {
        int e, r0, r1, n0;
        unit_tile(j, e, r0, r1, n0);
        // gate/up: lanes 0-31 read gate rows i0 + row_l, lanes 32-63 up rows
        // i0 + row_l - 4; down: output rows n0 + 8 wid + row_l.  Rows past the
        // matrix's last row read that row (their outputs are not stored).
        const S* m = (GATEUP && row_l >= 4) ? B1 : B0;
        const int mrow = min(n0 + WN * wid + (GATEUP ? (row_l & 3) : row_l), NOUT - 1);
        wptr = (const char*)(m + ((int64_t)e * NOUT + mrow) * K) + (((lane & 7) ^ swz128(row_l)) << 4);
        // token slots 8 h + row_l, clamped to the tile's last row (slots past
        // it are computed but never stored); the wave reads the source rows
        // of its 16 slots with scalar loads and each lane keeps its own
        uint32_t src[TPW];
#pragma unroll
        for (int h = 0; h < TPW; ++h) {
            src[h] = 0;
            int rows[8];
            uint32_t v[8];
#pragma unroll
            for (int t = 0; t < 8; ++t) v[t] = rows[t] = __builtin_amdgcn_readfirstlane(min(r0 + 8 * h + t, r1 - 1));
            if (a_rows) {
                sload8(a_rows, rows, v);
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = min(v[t], (uint32_t)(a_nrows - 1));
            }
#pragma unroll
            for (int t = 0; t < 8; ++t)
                if (row_l == t) src[h] = v[t];
        }
#pragma unroll
        for (int h = 0; h < TPW; ++h)
            toff[h] = (uint32_t)((int64_t)src[h] * K * (int64_t)sizeof(S)) + (((lane & 7) ^ swz128(8 * h + row_l)) << 4);
    };
    const uint32_t lds0 = lds_offset(smem);
    int slot_issue = 0;                                        // stage of the next loads
    auto issue = [&]() __attribute__((always_inline)) {
        const uint32_t st = lds0 + slot_issue * STAGE;
        // token quarter wid (both halves of the 16 slots), then the wave's
        // rows, quarter by quarter; quarters past K repeat the last one
        const int qt = min(4 * is + wid, nq - 1);
#pragma unroll
        for (int h = 0; h < TPW; ++h) lds_dma16_so((const char*)A + qt * ROWB, toff[h], st + wid * TQ + h * 1024);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            lds_dma16(wptr + min(4 * is + q, nq - 1) * ROWB, st + TOK + (4 * wid + q) * WQ);
        slot_issue = slot_issue == NS - 1 ? 0 : slot_issue + 1;
        // advance, except past the last step, which later loads repeat
        if (is + 1 < nk) {
            ++is;
        } else if (iu + 1 < nu) {
            is = 0;
            set_unit(++iu);
        }
    };

    set_unit(0);
#pragma unroll 1
    for (int p = 0; p < NS - 1; ++p) issue();

    // fragments: weight row (lane & 7) of the wave's block, token slot
    // (lane & 15); K group lane / 16 of each 32-K half of a quarter
    const int kg = lane >> 4;
    const int fw = TOK + 4 * wid * WQ + (lane & 7) * ROWB, ft = (lane & (kDecRows - 1)) * ROWB;
    const int sw_w = swz128(lane & 7), sw_t = swz128(lane & (kDecRows - 1));
    f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
    int cj = 0, cs = 0, slot = 0;                              // compute cursor
#pragma unroll 1
    for (int g = 0, total = nu * nk; g < total; ++g) {
        // step g landed (only the loads of the next NS - 2 steps may be in
        // flight); after the barrier every wave's token rows of step g are
        // in, and every wave is done with the stage of step g - 1, which the
        // loads issued now reuse
        wait_vm<(NS - 2) * PIECES>();
        barrier_lds();
        issue();
        const unsigned char* st = smem + slot * STAGE;
        const int qv = min(nq - 4 * cs, 4);                    // valid quarters of this step
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (q < qv) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c = 4 * h + kg;
                    const uint4 w = *(const uint4*)(st + fw + q * WQ + ((c ^ sw_w) << 4));
                    const uint4 t = *(const uint4*)(st + q * TQ + ft + ((c ^ sw_t) << 4));
                    acc = mma<DT>::run(w, t, acc);
                }
            }
        }
        slot = slot == NS - 1 ? 0 : slot + 1;
        if (++cs < nk) continue;
        // the unit's last step: lane l holds token slot l % 16 and block rows
        // 4 (l / 16) + 0..3 (rows 8-15, lanes 32-63, repeat rows 0-7)
        int e, r0, r1, n0;
        unit_tile(cj, e, r0, r1, n0);
        const int col0 = n0 + WN * wid;
        const int grow = (lane & 15) < kDecRows ? r0 + (lane & 15) : r1;
        if constexpr (GATEUP) {
            // gate rows 0-3 in lanes 0-15, the up rows of the same i in 16-31
            float u4[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) u4[r] = __shfl_down(acc[r], 16);
            if (lane < 16 && grow < r1 && col0 < NOUT) {
                const float g4[4] = {acc[0], acc[1], acc[2], acc[3]};
                float v[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) v[r] = silu_mul(g4[r], u4[r]);
                store4<DT>::run(C + (int64_t)grow * NOUT + col0, v);
                if (gu) save_preact(gu, grow, NOUT, col0, g4, u4);
            }
        } else {
            const int col = col0 + 4 * kg;
            if (lane < 32 && grow < r1 && col < NOUT) {
                const float v[4] = {acc[0], acc[1], acc[2], acc[3]};
                store4<DT>::run(C + (int64_t)grow * NOUT + col, v);
            }
        }
        acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
        cs = 0;
        ++cj;
    }
    // the repeated loads of the last steps land before the workgroup ends
    wait_vm<0>();
}

// ------------------------------------------------------------------ pipelined grouped GEMM, 64-wide K stages
// The same 256x256 tile and 8 waves of 128x64 as above, with 64-element K
// stages: every LDS row holds 128 bytes (one whole cache line of each operand
// row per stage, chunk c of row r at c ^ swz128(r)), so each DMA instruction
// moves 8 rows x 128 bytes, and one barrier covers 64 K instead of 32.
// The token rows and the weight rows have rings of their own in the 160 KB
// of LDS: 2 slots of 32 KB for the tokens, 3 for the weights, so the weight
// tiles -- the operand L2 shares least -- are requested two steps ahead.
// A step runs as four 16-K sub-steps; the fragments of the next sub-step are
// read during the current one.  The barrier sits between sub-steps 2 and 3
// of step kt: by then every wave has read all of step kt and landed its DMA
// of step kt+1, so sub-step 3 reads the first fragments of kt+1 and starts
// the DMA of the token rows of kt+2 and of a quarter of the weight rows of
// kt+3 into the slots step kt leaves; the other weight rows of kt+3 follow,
// a quarter per sub-step, over sub-steps 0-2 of step kt+1.  Requires
// K % 64 == 0.
//   The launch is persistent: one workgroup per CU claims tiles (tiles.h,
// claimed tiles) until every XCD's run is used up, so an XCD whose run holds
// cheap tiles (stream tiles, an expert's few last rows) takes tiles off the
// back of the others' runs instead of idling.  Thread 0 makes the claim for
// the next tile as the K loop ends, and hands it to the other waves through
// LDS word 0 between two barriers.  The next tile's token rows of steps 0
// and 1 and weight rows of step 0 then go out before the current tile's
// epilogue, which stages its outputs in the other two slots, so the new
// tile's first step does not wait on memory.
constexpr int kP64SlotsA = 2, kP64SlotsB = 3;
template <typename DT, bool GATEUP, int WGM, int WGN>
__global__ __launch_bounds__(WGM* WGN* kWave, 1) void grouped_gemm_pipe64_kernel(
    const typename DT::storage* __restrict__ A, const typename DT::storage* __restrict__ B0,
    const typename DT::storage* __restrict__ B1, typename DT::storage* __restrict__ C, float* __restrict__ gu,
    const uint32_t* __restrict__ a_rows, int a_nrows, const int4* __restrict__ tiles,
    const uint32_t* __restrict__ tile_count, int K, int NOUT, int n_tiles, int nblocks,
    unsigned long long* __restrict__ queues) {
    using S = typename DT::storage;
    constexpr int NW = WGM * WGN;
    constexpr int ROWB = 128;                                   // bytes per row per step
    constexpr int SLOT = kPipeBM * ROWB;                        // 32 KB: one operand, one step
    static_assert(kPipeBN == kPipeBM, "both operand tiles are 256 rows");
    constexpr int NA = kP64SlotsA, NB_ = kP64SlotsB;
    constexpr int LPO = SLOT / 1024 / NW;                       // 4 pieces of 8 rows per wave per operand
    constexpr int BN_OUT = GATEUP ? kPipeBN / 2 : kPipeBN;
    constexpr int WTM = kPipeBM / WGM, WTN = kPipeBN / WGN;
    constexpr int MB = WTM / 32, NB = WTN / 32;
    constexpr int WCN = BN_OUT / WGN;
    constexpr int NM = MB * NB, NR = MB + NB;                   // MFMAs and fragment reads per sub-step
    static_assert(!GATEUP || NB % 2 == 0, "gate and up blocks pair up");
    static_assert(LPO + LPO / 4 <= 2 * NM, "at most two DMA pieces per MFMA of a sub-step");
    static_assert(NA == 2 && NB_ == 3, "the vmcnt waits below are counted for 2 token and 3 weight slots");
    static_assert(GATEUP || NW * WTM * WTN * 2 <= (NA + NB_) * SLOT, "the staged outputs fit the LDS");
    static_assert(!GATEUP || NW * 8192 <= 2 * SLOT, "the staged pre-activations fit the staging slots");
    static_assert(NW * kWave <= 512, "one workgroup of at most 8 waves");
    __shared__ __attribute__((aligned(1024))) unsigned char smem[(NA + NB_) * SLOT];

    // the wave id is wave-uniform: in a scalar register the DMA's LDS
    // addresses are scalar arithmetic, with no per-piece readfirstlane
    const int lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int wm = wid / WGN, wn = wid % WGN;
    const int live_m = (int)*tile_count;
    const int nk = K / 64;

    const int xcd = blockIdx.x % kXcds, live = min(nblocks, live_m * n_tiles);
    // The epilogue stages its outputs in weight slots 1 and 2 (64 KB), so the
    // next tile's token rows of steps 0 and 1 and weight rows of step 0 can
    // land in the other three slots meanwhile.
    unsigned char* const stage = smem + (NA + 1) * SLOT;
    // (an LDS pointer: through a generic one the word's accesses would be
    // flat instructions, whose waits also drain every load and store)
    volatile __attribute__((address_space(3))) int* const claim_word =
        (volatile __attribute__((address_space(3))) int*)smem;
    // thread 0 finishes a claim (the front word `old` returned, else the
    // other runs' backs) and hands it to every wave through LDS word 0,
    // which no wave touches between the first and the last barrier here
    auto publish_claim = [&](unsigned long long old) {
        wait_lgkm0();
        barrier_lds();
        if (threadIdx.x == 0) {
            int p = front_claim(old, xcd, live);
            if (p < 0) p = steal_claim(queues, xcd, live);
            *claim_word = p;
        }
        wait_lgkm0();
        barrier_lds();
        const int p = __builtin_amdgcn_readfirstlane(*claim_word);
        wait_lgkm0();
        barrier_lds();
        return p;
    };
    int e, r0, r1, n0;
    // DMA piece j of this wave, per operand: rows (wid * LPO + j) * 8 + lane / 8
    // of the operand tile, the lane's 16-byte physical slot (lane & 7) holding
    // logical chunk slot ^ swz128(row).  Each piece is addressed as a
    // wave-uniform base in scalar registers (the token buffer, or the weight
    // matrix's rows of this tile), advanced a step at a time, plus a 32-bit
    // per-lane offset; the host only picks this kernel when every offset fits
    // 32 bits.  (64-bit per-lane addresses cost a vector add per piece and
    // step: 2-3% of the product's time.)
    const char* basb[LPO];
    uint32_t voffa[LPO], voffb[LPO];
    auto setup = [&](int4 tl, int ni) {
        e = tl.x & ~kStreamTileFlag;
        r0 = tl.y;
        r1 = tl.z;
        n0 = ni * BN_OUT;
        // the token rows of the pieces, looked up together
        static_assert(LPO == 4, "four token-row lookups per lane");
        int srow[LPO];
#pragma unroll
        for (int j = 0; j < LPO; ++j) srow[j] = min(r0 + (wid * LPO + j) * 8 + (lane >> 3), r1 - 1);
        if (a_rows) {
            uint32_t v[4];
#pragma unroll
            for (int j = 0; j < LPO; ++j) v[j] = (uint32_t)srow[j] * 4u;
            load4_u32(a_rows, v);
#pragma unroll
            for (int j = 0; j < LPO; ++j) srow[j] = (int)min(v[j], (uint32_t)(a_nrows - 1));
        }
#pragma unroll
        for (int j = 0; j < LPO; ++j) {
            const int prow0 = (wid * LPO + j) * 8;  // first row of the piece (wave-uniform)
            const int row = prow0 + (lane >> 3);
            const int lc = (lane & 7) ^ swz128(row);
            voffa[j] = (uint32_t)((int64_t)srow[j] * K * (int64_t)sizeof(S)) + lc * 16;
            const S* m = (GATEUP && prow0 >= BN_OUT) ? B1 : B0;
            basb[j] = (const char*)(m + ((int64_t)e * NOUT + n0) * K);
            const int brow = GATEUP ? row % BN_OUT : row;
            voffb[j] = (uint32_t)((int64_t)(min(n0 + brow, NOUT - 1) - n0) * K * (int64_t)sizeof(S)) + lc * 16;
        }
    };
    const uint32_t lds_a = lds_offset(smem) + wid * LPO * 1024;
    const uint32_t lds_b = lds_a + NA * SLOT;
    // A flagged tile runs as a stream tile in the gate/up product; in the
    // down product only when it is a whole expert (a group of one tile), an
    // expert's leftover rows otherwise taking the 256-row path.  Leftover
    // stream tiles end well before the expert's full tiles of the same weight
    // tile, which drift apart and find the weight tiles in L2 less often:
    // measured at prefill, the down product then reads 12% more from HBM and
    // is no faster, gate/up reads 35% more and is 1% faster.
    auto streams = [&](int4 tl) { return (tl.x & kStreamTileFlag) && (GATEUP || ((uint32_t)tl.w >> 26) == 1); };
    // fragment rows are 32-aligned blocks plus (lane & 31), whose chunk key is that of lane & 31
    const int frow = lane & 31, kg = lane >> 5;
    const int fa0 = (wm * WTM + frow) * ROWB;
    int fb[NB];
#pragma unroll
    for (int f = 0; f < NB; ++f) {
        int brow;
        if (GATEUP)
            brow = (f < NB / 2) ? wn * WCN + f * 32 : BN_OUT + wn * WCN + (f - NB / 2) * 32;
        else
            brow = wn * WTN + f * 32;
        fb[f] = NA * SLOT + (brow + frow) * ROWB;
    }
    int csw[4];  // byte offset of sub-step q's chunk in this lane's rows
#pragma unroll
    for (int q = 0; q < 4; ++q) csw[q] = ((2 * q + kg) ^ swz128(frow)) * 16;

    f32x16_t acc[MB][NB];
    uint4 av[2][MB], bv[2][NB];
    auto read_one = [&](int kt, int q, int set, int r) {
        if (r < MB)
            av[set][r] = *(const uint4*)(smem + (kt % NA) * SLOT + csw[q] + fa0 + r * 32 * ROWB);
        else
            bv[set][r - MB] = *(const uint4*)(smem + (kt % NB_) * SLOT + csw[q] + fb[r - MB]);
    };
    // a step past the end (the first weight rows of one, from the loop's
    // third-last step, or a K of at most 128's in the prologue) re-loads the
    // last step into a slot nobody reads again
    auto dma_a = [&](int kt, int j) {
        lds_dma16_so((const char*)A + min(kt, nk - 1) * ROWB, voffa[j], lds_a + (kt % NA) * SLOT + j * 1024);
    };
    auto dma_b = [&](int kt, int j) {
        lds_dma16_so(basb[j] + min(kt, nk - 1) * ROWB, voffb[j], lds_b + (kt % NB_) * SLOT + j * 1024);
    };
    // Weight rows of step kt+2 go out a quarter step (BQ pieces) per sub-step,
    // from sub-step 3 of step kt-1 to sub-step 2 of step kt, into the slot the
    // barrier of step kt-1 freed; token rows of step kt+2 go out whole in
    // sub-step 3 of step kt, the first moment their slot is free.  Spreading
    // the weight rows keeps the DMA issue of a step from queueing up behind
    // one sub-step.  Before step 0 the pieces that schedule would have issued
    // go out in its order: A0 B0 B1 A1 B2[0, BQ).
    constexpr int BQ = LPO / 4;
    static_assert(LPO % 4 == 0, "weight-row pieces spread over four sub-steps");
    auto prologue_dma = [&]() {
#pragma unroll
        for (int j = 0; j < LPO; ++j) dma_a(0, j);
#pragma unroll
        for (int j = 0; j < LPO; ++j) dma_b(0, j);
#pragma unroll
        for (int j = 0; j < LPO; ++j) dma_b(1, j);
#pragma unroll
        for (int j = 0; j < LPO; ++j) dma_a(1, j);
#pragma unroll
        for (int j = 0; j < BQ; ++j) dma_b(2, j);
    };
    constexpr int kPrologueAfter0 = 2 * LPO + BQ;  // pieces issued after B0
    // the MFMAs of sub-step (set), the reads of the next sub-step (rkt, rq)
    // into the other set over the first half of them, and `nd` DMA pieces
    // spread over all of them (over the second half only measured 1-2%
    // slower on the down product)
    int rows_live = 0;
    auto substep = [&](auto full, auto nd, int set, int rkt, int rq, auto&& dma) {
        constexpr int ND = decltype(nd)::value, H1 = NM / 2;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int i = m / NB, f = m % NB;
            if (decltype(full)::value || i * 32 < rows_live)
                acc[i][f] = mma32<DT>::run(bv[set][f], av[set][i], acc[i][f]);
            if (m < H1) {
#pragma unroll
                for (int r = (m * NR) / H1; r < ((m + 1) * NR) / H1; ++r) read_one(rkt, rq, set ^ 1, r);
            }
#pragma unroll
            for (int d = (m * ND) / NM; d < ((m + 1) * ND) / NM; ++d) dma(d);
            sched_fence();
        }
    };
    using q_dma = std::integral_constant<int, BQ>;
    using q3_dma = std::integral_constant<int, LPO + BQ>;
    using no_dma = std::integral_constant<int, 0>;
    auto main_loop = [&](auto full) {
        int kt = 0;
        for (; kt < nk - 2; ++kt) {
            wait_lgkm0();
            substep(full, q_dma{}, 0, kt, 1, [&](int d) { dma_b(kt + 2, BQ + d); });
            wait_lgkm0();
            substep(full, q_dma{}, 1, kt, 2, [&](int d) { dma_b(kt + 2, 2 * BQ + d); });
            wait_lgkm0();
            substep(full, q_dma{}, 0, kt, 3, [&](int d) { dma_b(kt + 2, 3 * BQ + d); });
            // step kt+1 landed: its weight rows all went out before its token
            // rows, and only the LPO weight-row pieces of kt+2 after them.
            // The reads of step kt complete before the barrier, so its slots
            // can be refilled once every wave has passed it.
            wait_vm<LPO>();
            wait_lgkm0();
            barrier_lds();
            // token rows of kt+2, then the first weight rows of kt+3
            substep(full, q3_dma{}, 1, kt + 1, 0,
                    [&](int d) { if (d < LPO) dma_a(kt + 2, d); else dma_b(kt + 3, d - LPO); });
        }
        // The last two steps load nothing: after the token rows of the last
        // step only BQ pieces went out (the first weight rows of the step
        // past the end, from the loop above, or of step 2, from the prologue).
        for (; kt < nk; ++kt) {
            wait_lgkm0();
            substep(full, no_dma{}, 0, kt, 1, [](int) {});
            wait_lgkm0();
            substep(full, no_dma{}, 1, kt, 2, [](int) {});
            wait_lgkm0();
            substep(full, no_dma{}, 0, kt, 3, [](int) {});
            wait_vm<BQ>();
            wait_lgkm0();
            barrier_lds();
            substep(full, no_dma{}, 1, kt + 1, 0, [](int) {});
        }
    };

    int pid = publish_claim(threadIdx.x == 0 ? atomicAdd(queues + xcd, 1ull) : 0ull);
    bool pre = false;  // pid's token rows of steps 0-1 and weight rows of step 0 are in flight
    while (pid >= 0) {
        bool streamed = false;
        if (!pre) {
            int m_idx, n_idx;
            tile_of_id(pid, n_tiles, live_m, tiles, &m_idx, &n_idx);
            const int4 tl = tiles[m_idx];
            if (streams(tl)) {
                static_assert(NW == 8, "a stream tile runs on 8 waves of 32 weight rows");
                stream_tile<DT, GATEUP>(A, B0, B1, C, gu, a_rows, a_nrows, tl.x & ~kStreamTileFlag, tl.y, tl.z,
                                        n_idx * BN_OUT, K, NOUT, wid, lane, smem);
                pid = publish_claim(threadIdx.x == 0 ? atomicAdd(queues + xcd, 1ull) : 0ull);
                streamed = true;
            } else {
                setup(tl, n_idx);
                prologue_dma();
            }
        }
        if (!streamed) {
            rows_live = __builtin_amdgcn_readfirstlane(r1 - r0) - __builtin_amdgcn_readfirstlane(wm) * WTM;
#pragma unroll
            for (int i = 0; i < MB; ++i)
#pragma unroll
                for (int f = 0; f < NB; ++f)
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;
            // the loads complete in order, so at most 2 LPO + BQ pieces still
            // in flight means A0 and B0 landed: after B0 went out either
            // B1 A1 B2[0, BQ), or (a prefetched tile) A1, the previous
            // epilogue's stores, B1 B2[0, BQ); the stores only make the wait
            // stricter
            wait_vm<kPrologueAfter0>();
            barrier_lds();
#pragma unroll
            for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r);
            if (rows_live >= MB * 32)
                main_loop(std::true_type{});
            else
                main_loop(std::false_type{});
            // every DMA of this tile landed and every wave finished its reads:
            // the LDS is free to stage the outputs.  The claim goes out before
            // that wait, which thus also covers it: a wait the compiler placed
            // at its use would count only the stores it issued after it, and
            // so would also wait for the next tile's loads below.
            unsigned long long next = 0;
            if (threadIdx.x == 0) next = atomicAdd(queues + xcd, 1ull);
            wait_vm0_known();
            wait_lgkm0();
            barrier_lds();
            const int nxt = publish_claim(next);
            const int t_r0 = r0, t_r1 = r1, t_n0 = n0;
            // the next tile's first loads, into token slots 0 and 1 and weight
            // slot 0; its weight rows of step 1 and first ones of step 2 go
            // into the staging slots once every wave has read them back
            pre = false;
            if (nxt >= 0) {
                int m_idx, n_idx;
                tile_of_id(nxt, n_tiles, live_m, tiles, &m_idx, &n_idx);
                const int4 tl = tiles[m_idx];
                if (!streams(tl)) {
                    setup(tl, n_idx);
#pragma unroll
                    for (int j = 0; j < LPO; ++j) dma_a(0, j);
#pragma unroll
                    for (int j = 0; j < LPO; ++j) dma_b(0, j);
#pragma unroll
                    for (int j = 0; j < LPO; ++j) dma_a(1, j);
                    pre = true;
                }
            }
            if constexpr (GATEUP) {
                constexpr bool staged_gu = WCN == 32 && NB == 2;
                static_assert(staged_gu && NW == 8, "h is staged tile-wide: 8 waves of 32 h columns");
                store_gateup_staged<DT, MB, WTM>(acc, C, t_r0, t_r1, t_n0, wm, wn, wid, NOUT, lane, stage);
                if (gu) {
                    // every wave has read its h rows back before the region is
                    // reused: 8 KB per wave, in rounds of 32 rows
                    wait_lgkm0();
                    barrier_lds();
                    static_assert(NW * 32 * 256 == 2 * SLOT, "rounds of 32 rows in the two staging slots");
                    save_preact_staged<MB, NB, WTM, WCN, 32>(acc, gu, t_r0, t_r1, t_n0, wm, wn, NOUT, lane,
                                                             stage + wid * (32 * 256));
                }
            } else if constexpr (WTN == 64) {
                // two rounds of 8 KB per wave
                static_assert(NW * WTM * WTN * (int)sizeof(S) / 2 == 2 * SLOT, "two rounds in two slots");
                store_tile32_staged<DT, MB, NB, WTM, WTN, 2>(acc, C, t_r0, t_r1, t_n0, wm, wn, NOUT, lane,
                                                             stage + wid * (WTM * WTN * (int)sizeof(S) / 2));
            } else {
                store_tile32<DT, GATEUP, MB, NB, WTM, WTN, WCN>(acc, C, nullptr, t_r0, t_r1, t_n0, wm, wn, NOUT,
                                                                lane);
            }
            // every wave has read its staged outputs back before the slots are
            // refilled
            wait_lgkm0();
            barrier_lds();
            if (pre) {
#pragma unroll
                for (int j = 0; j < LPO; ++j) dma_b(1, j);
#pragma unroll
                for (int j = 0; j < BQ; ++j) dma_b(2, j);
            }
            pid = nxt;
        }
    }
}

template <typename DT, bool GATEUP, int BM, int BNB, int WGM, int WGN>
hipError_t launch_gemm(const void* A, const uint32_t* a_rows, int64_t a_nrows, const void* B0, const void* B1,
                       void* C, float* gu, const int4* tiles, const uint32_t* count, int64_t mt, int K, int NOUT,
                       hipStream_t s) {
    using S = typename DT::storage;
    constexpr int BN_OUT = GATEUP ? BNB / 2 : BNB;
    const int n_tiles = (NOUT + BN_OUT - 1) / BN_OUT;
    const int64_t nb = mt * n_tiles;
    if (nb == 0) return hipSuccess;
    if (nb > 0x7fffffff) return hipErrorInvalidValue;
    grouped_gemm_kernel<DT, GATEUP, BM, BNB, WGM, WGN><<<(unsigned)nb, WGM * WGN * kWave, 0, s>>>(
        (const S*)A, (const S*)B0, (const S*)B1, (S*)C, gu, a_rows, (int)a_nrows, tiles, count, K, NOUT, n_tiles,
        (int)nb);
    return hipGetLastError();
}

template <typename DT, bool GATEUP, int WGM, int WGN>
hipError_t launch_pipe(const void* A, const uint32_t* a_rows, int64_t a_nrows, const void* B0, const void* B1,
                       void* C, float* gu, const int4* tiles, const uint32_t* count, int64_t mt, int K, int NOUT,
                       hipStream_t s) {
    using S = typename DT::storage;
    constexpr int BN_OUT = GATEUP ? kPipeBN / 2 : kPipeBN;
    const int n_tiles = (NOUT + BN_OUT - 1) / BN_OUT;
    const int64_t nb = mt * n_tiles;
    if (nb == 0) return hipSuccess;
    if (nb > 0x7fffffff) return hipErrorInvalidValue;
    grouped_gemm_pipe_kernel<DT, GATEUP, WGM, WGN><<<(unsigned)nb, WGM * WGN * kWave, 0, s>>>(
        (const S*)A, (const S*)B0, (const S*)B1, (S*)C, gu, a_rows, (int)a_nrows, tiles, count, K, NOUT, n_tiles,
        (int)nb);
    return hipGetLastError();
}

// The compute units of the current device, looked up once per device.
hipError_t device_cus(int* n) {
    static std::atomic<int> cached[256];
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev >= 0 && dev < 256 && (*n = cached[dev].load(std::memory_order_relaxed)) > 0) return hipSuccess;
    err = hipDeviceGetAttribute(n, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    if (*n <= 0) return hipErrorInvalidDevice;
    if (dev >= 0 && dev < 256) cached[dev].store(*n, std::memory_order_relaxed);
    return hipSuccess;
}

// One workgroup per CU (the kernel's LDS allows no more), claiming tiles from
// the eight claim words at `queues`, which the tile-list kernel cleared.
template <typename DT, bool GATEUP>
hipError_t launch_pipe64(const void* A, const uint32_t* a_rows, int64_t a_nrows, const void* B0, const void* B1,
                         void* C, float* gu, const int4* tiles, const uint32_t* count, int64_t mt, int K,
                         int NOUT, unsigned long long* queues, hipStream_t s) {
    using S = typename DT::storage;
    constexpr int BN_OUT = GATEUP ? kPipeBN / 2 : kPipeBN;
    const int n_tiles = (NOUT + BN_OUT - 1) / BN_OUT;
    const int64_t nb = mt * n_tiles;
    if (nb == 0) return hipSuccess;
    if (nb > 0x7fffffff) return hipErrorInvalidValue;
    int cus = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    const unsigned grid = (unsigned)std::min<int64_t>(nb, cus);
    grouped_gemm_pipe64_kernel<DT, GATEUP, MOE_P64_WM, MOE_P64_WN><<<grid, MOE_P64_WM * MOE_P64_WN * kWave, 0, s>>>(
        (const S*)A, (const S*)B0, (const S*)B1, (S*)C, gu, a_rows, (int)a_nrows, tiles, count, K, NOUT, n_tiles,
        (int)nb, queues);
    return hipGetLastError();
}


template <typename DT, bool GATEUP>
hipError_t launch_decode(const void* A, const uint32_t* a_rows, int64_t a_nrows, const void* B0, const void* B1,
                         void* C, float* gu, const int4* tiles, const uint32_t* count, int64_t mt, int K, int NOUT,
                         hipStream_t s) {
    using S = typename DT::storage;
    constexpr int UN = GATEUP ? kDecWaves * kDecWaveRows / 2 : kDecWaves * kDecWaveRows;
    const int n_units = (NOUT + UN - 1) / UN;
    const int64_t units = mt * n_units;  // the most the tile list can give
    if (units == 0) return hipSuccess;
    if (units > 0x7fffffff) return hipErrorInvalidValue;
    int cus = 0;
    hipError_t err = device_cus(&cus);
    if (err != hipSuccess) return err;
    const unsigned grid = (unsigned)std::min<int64_t>(units, cus);
    decode_stream_kernel<DT, GATEUP><<<grid, kDecWaves * kWave, 0, s>>>(
        (const S*)A, (const S*)B0, (const S*)B1, (S*)C, gu, a_rows, (int)a_nrows, tiles, count, K, NOUT, n_units);
    return hipGetLastError();
}

#ifndef MOE_P_WM
#define MOE_P_WM 2   // waves along token rows of the pipelined tile
#define MOE_P_WN 4   // waves along weight rows
#endif

// The register-staged kernel's two tile shapes (f32, and 16-bit types whose
// K extents are not multiples of 64): a large tile for experts that own many
// rows, and a 16-row tile for experts that own a handful of rows each.
#ifndef MOE_L_BM
#define MOE_L_BM 128   // rows of the large tile
#define MOE_L_BN 128   // weight rows of the large tile
#define MOE_L_WM 2     // waves along rows
#define MOE_L_WN 2     // waves along weight rows
#endif
#ifndef MOE_S_BN
#define MOE_S_BN 256   // weight rows of the 16-row tile
#define MOE_S_WN 4
#endif
constexpr int kSmallBM = 16;

// The tile list's 256-byte header: the count at byte 0, the 64-K kernels'
// claim words (8 per product) from byte 64.
constexpr int kTileQueueOffset = 64;
static_assert(kTileQueueOffset + 2 * kXcds * 8 <= 256, "the claim words fit the header");

template <typename DT>
hipError_t launch_typed(const ExpertsArgs& a, hipStream_t s, ExpertsPart part) {
    const int H = (int)a.H, I = (int)a.I;
    int4* tiles = (int4*)((char*)a.tiles + 256);
    uint32_t* count = (uint32_t*)a.tiles;
    const int64_t cap = ((int64_t)experts_tile_bytes(a.N, a.E) - 256) / 16;  // entries the workspace holds
    // 16-bit types with both K extents multiples of 64, and row operands
    // that span less than 4 GiB (the kernels address a row as a scalar base
    // plus a 32-bit per-lane offset), take one of two kernels:
    //   - the decode stream kernel, when no expert can hold more than
    //     kStreamRows rows (a token picks an expert at most once, so an
    //     expert holds at most T rows when the rows are read through
    //     token_of_row) or the experts hold at most kDecMeanRows rows on
    //     average: a weight stream in the HBM read pattern measured fastest
    //     (decode gate/up 480 us against 495 for the 16-row register-staged
    //     kernel and ~510 for stream tiles);
    //   - otherwise the 64-K kernel, which picks each expert's tile on the
    //     device: a stream tile for an expert of at most kStreamRows rows,
    //     256-row tiles for the others.
    const int64_t x_rows = a.x_rows ? a.x_nrows : a.N, esz = (int64_t)sizeof(typename DT::storage);
    const bool fits32 = x_rows * a.H * esz < (int64_t(1) << 32) - 256 && a.N * a.I * esz < (int64_t(1) << 32) - 256;
    const int64_t max_expert_rows = a.x_rows ? std::min(a.N, a.x_nrows) : a.N;
    const bool k64 = esz == 2 && MOE_P_BK64 && a.H % 64 == 0 && a.I % 64 == 0 && fits32;
    if (k64 && (max_expert_rows <= kStreamRows || a.N <= kDecMeanRows * (int64_t)a.E)) {
        // decode-sized: the persistent stream kernel on token tiles of at
        // most kDecRows rows
        const int64_t mt = max_mtiles(a.N, a.E, kDecRows);
        if (mt > cap) return hipErrorInvalidValue;
        hipError_t err = launch_build_tiles(a.offsets, a.E, a.N, kDecRows, mt, tiles, count, s);
        if (err != hipSuccess) return err;
        if constexpr (sizeof(typename DT::storage) == 2) {
            if (part != kDown) {
                err = launch_decode<DT, true>(a.x, a.x_rows, a.x_nrows, a.gate, a.up, a.h, a.gu, tiles, count, mt, H, I, s);
                if (err != hipSuccess) return err;
            }
            if (part != kGateUp)
                err = launch_decode<DT, false>(a.h, nullptr, 0, a.down, nullptr, a.y, nullptr, tiles, count, mt, I, H, s);
        }
        return err;
    }
    if (k64) {
        // the claim words of the two products, in the list's header
        unsigned long long* queues = (unsigned long long*)((char*)a.tiles + kTileQueueOffset);
        const int64_t mt = max_mtiles(a.N, a.E, kPipeBM, kStreamRows);
        if (mt > cap) return hipErrorInvalidValue;
        hipError_t err =
            launch_build_tiles(a.offsets, a.E, a.N, kPipeBM, mt, tiles, count, s, kStreamRows, queues, 2 * kXcds);
        if (err != hipSuccess) return err;
        if constexpr (sizeof(typename DT::storage) == 2) {
            if (part != kDown) {
                err = launch_pipe64<DT, true>(a.x, a.x_rows, a.x_nrows, a.gate, a.up, a.h, a.gu, tiles, count, mt, H, I,
                                              queues, s);
                if (err != hipSuccess) return err;
            }
            if (part != kGateUp)
                err = launch_pipe64<DT, false>(a.h, nullptr, 0, a.down, nullptr, a.y, nullptr, tiles, count, mt, I, H,
                                               queues + kXcds, s);
        }
        return err;
    }
    // Otherwise (f32, K not a multiple of 64, or larger operands) one tile
    // height for every expert: 16 rows when the experts own few rows on
    // average (or none can own more than kStreamRows), else
    // the pipelined 32-K kernel (16-bit, K extents multiples of 32) or the
    // register-staged kernel.
    const bool small = a.N < 64 * (int64_t)a.E || max_expert_rows <= kStreamRows;
    const bool pipe = !small && esz == 2 && a.H % kPipeBK == 0 && a.I % kPipeBK == 0;
    const int BM = small ? kSmallBM : (pipe ? kPipeBM : MOE_L_BM);
    const int64_t mt = max_mtiles(a.N, a.E, BM);
    if (mt > cap) return hipErrorInvalidValue;
    hipError_t err = launch_build_tiles(a.offsets, a.E, a.N, BM, mt, tiles, count, s);
    if (err != hipSuccess) return err;
    if (pipe) {
        if constexpr (sizeof(typename DT::storage) == 2) {
            if (part != kDown) {
                err = launch_pipe<DT, true, MOE_P_WM, MOE_P_WN>(a.x, a.x_rows, a.x_nrows, a.gate, a.up, a.h, a.gu, tiles, count, mt, H, I, s);
                if (err != hipSuccess) return err;
            }
            if (part != kGateUp)
                err = launch_pipe<DT, false, MOE_P_WM, MOE_P_WN>(a.h, nullptr, 0, a.down, nullptr, a.y, nullptr, tiles, count, mt, I, H, s);
        }
        return err;
    }
    if (part != kDown) {
        err = small ? launch_gemm<DT, true, 16, MOE_S_BN, 1, MOE_S_WN>(a.x, a.x_rows, a.x_nrows, a.gate, a.up, a.h, a.gu, tiles, count, mt, H, I, s)
                    : launch_gemm<DT, true, MOE_L_BM, MOE_L_BN, MOE_L_WM, MOE_L_WN>(a.x, a.x_rows, a.x_nrows, a.gate, a.up, a.h, a.gu, tiles, count, mt, H, I, s);
        if (err != hipSuccess) return err;
    }
    if (part != kGateUp) {
        err = small ? launch_gemm<DT, false, 16, MOE_S_BN, 1, MOE_S_WN>(a.h, nullptr, 0, a.down, nullptr, a.y, nullptr, tiles, count, mt, I, H, s)
                    : launch_gemm<DT, false, MOE_L_BM, MOE_L_BN, MOE_L_WM, MOE_L_WN>(a.h, nullptr, 0, a.down, nullptr, a.y, nullptr, tiles, count, mt, I, H, s);
    }
    return err;
}

}  // namespace

int64_t max_mtiles(int64_t N, int64_t E, int BM, int stream_rows) {
    if (N <= 0) return 0;
    const int64_t bound = stream_rows > 0 ? E + N / BM : (N + E * (BM - 1)) / BM;
    return bound < N ? bound : N;
}

hipError_t launch_build_tiles(const uint32_t* offsets, int E, int64_t N, int BM, int64_t max_tiles, int4* tiles,
                              uint32_t* count, hipStream_t s, int stream_rows, unsigned long long* queues,
                              int n_queues) {
    if (max_tiles >= kMaxTiles || N >= (int64_t)0xFFFFFFFF || stream_rows < 0 || (stream_rows && stream_rows >= BM))
        return hipErrorInvalidValue;
    if (n_queues < 0 || n_queues > 1024 || (n_queues > 0 && !queues)) return hipErrorInvalidValue;
    build_tiles_kernel<<<1, 1024, 0, s>>>(offsets, E, (uint32_t)N, BM, (uint32_t)stream_rows, (uint32_t)max_tiles,
                                          tiles, count, queues, n_queues);
    return hipGetLastError();
}

// the largest list of any tile policy the expert products use
size_t experts_tile_bytes(int64_t N, int64_t E) {
    const int64_t a = std::max(max_mtiles(N, E, kSmallBM), max_mtiles(N, E, kDecRows)),
                  b = max_mtiles(N, E, kPipeBM, kStreamRows);
    return 256 + 16 * (size_t)(a > b ? a : b);
}

hipError_t launch_experts(const ExpertsArgs& a, hipStream_t s, ExpertsPart part) {
    if (a.N == 0) return hipSuccess;
    switch (a.dtype) {
    case MOE_F32: return launch_typed<f32_t>(a, s, part);
    case MOE_F16: return launch_typed<f16_t>(a, s, part);
    case MOE_BF16: return launch_typed<bf16_t>(a, s, part);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
