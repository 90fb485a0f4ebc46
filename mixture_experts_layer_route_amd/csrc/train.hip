// train.hip -- first-order training of the experts stage and the backward of
// the combine and dispatch steps on CDNA4.
//
// Follows the RUDA ruDNN library guide, section 12 (first-order MoE
// training): the combine backward gives the expert-output gradient and FP32
// weight gradients; the experts backward gives the dispatched-row gradient
// and FP32 dgate, dup and ddown; the dispatch backward adds each token's
// row gradients without applying the routing weights again.
//
// Experts backward.  For the rows r of expert e, with the saved FP32
// pre-activations g = gate_e x, u = up_e x and the stored activation
// h = silu(g) u (weight dtype), from dy (rows x H):
//   dh      = dy down_e                       rows x I    product DH, K = H
//   du      = dh silu(g)                      in DH's epilogue, FP32,
//   dg      = dh u silu'(g)                   stored in the weight dtype as
//             silu'(g) = s (1 + g (1 - s)),   dgu = [dg | du] (rows x 2I)
//             s = 1 / (1 + exp(-g))
//   dx      = dgu [gate_e ; up_e]             rows x H    product DX, K = 2I
//   [dgate_e ; dup_e] = dgu^T x               2I x H      product DWGU, K = rows
//   ddown_e = dy^T h                          H x I       product DWD,  K = rows
// FP32 accumulation throughout; dgate, dup and ddown are written in FP32.
//
// Operand layouts.  The MFMA takes, per lane, 8 (16-bit) or 4 (f32)
// consecutive K values of one output row or column.  The forward products
// have K contiguous in memory for both operands; here only the DH and DX row
// operands (dy, dgu) do.  The others -- down_e, gate_e, up_e read along
// their first index, and every operand of the weight gradients, whose K runs
// over dispatched rows -- are K-outer: contiguous along the output index.
//
// Two kernels:
//   train_pipe2_kernel (bf16/f16, enough rows per expert): 128 x 256 tiles
//     on 4 waves of 32x32x16 MFMAs, 32-K steps loaded straight into LDS by
//     global_load_lds in a 64 KB ring, so two workgroups share a CU and one
//     computes while the other stores; K-outer operands land in their
//     natural layout and are read with the gfx950 LDS transpose read
//     ds_read_b64_tr_b16;
//   train_gemm_kernel (f32, and few rows per expert): 128 x 128 tiles on 4
//     waves of 16x16 MFMAs; K-outer operands are staged through registers,
//     each thread transposing 4 K-rows x 16 bytes before writing K-runs to
//     LDS, double buffered.
// Both walk the forward's per-expert row-tile list for DH and DX, and
// (expert, row tile, column tile) over all experts for the weight gradients;
// an expert without rows gets zero gradients.
#include <algorithm>
#include <type_traits>

#include "mfma.h"
#include "tiles.h"

namespace moe {
namespace {

enum TrainProduct { kDH = 0, kDX = 1, kDWGU = 2, kDWD = 3 };

struct TrainGemm {
    const void* a;            // DH, DWD: dy [N,H]; DX, DWGU: dgu [N,2I]
    const void* b0;           // DH: down [E,H,I]; DX: gate [E,I,H]; DWGU: x rows; DWD: h [N,I]
    const void* b1;           // DX: up [E,I,H]
    const uint32_t* b_rows;   // DWGU: token_of_row (x holds b_nrows token rows) or null
    int b_nrows;
    const float* gu;          // DH: saved g | u [N,2I]
    void* c0;                 // DH: dgu; DX: dx [N,H]; DWGU: dgate; DWD: ddown
    void* c1;                 // DWGU: dup
    const int4* tiles;        // DH, DX: row-tile list and its length
    const uint32_t* tile_count;
    const uint32_t* offsets;  // DWGU, DWD: expert_offsets [E+1]
    int N, H, I;
    int n_tiles;              // output column tiles
    int m_tiles;              // DWGU, DWD: output row tiles per expert
    int nblocks;
};

constexpr int kTBM = 128, kTBN = 128, kTThreads = 256;
constexpr int kTStride = 144;  // LDS bytes per operand row: 128 of K + 16 of padding
constexpr int kTStage = (kTBM + kTBN) * kTStride;


// 4 K-rows of V values each (w[j] = 16 bytes of K-row j) -> V K-runs of 4
// values (out[i] = values (i, K-rows 0..3), the lower K-row in the lower bits).
template <int ES> struct transpose4;
template <> struct transpose4<2> {
    static __device__ __forceinline__ void run(const uint4 (&w)[4], uint2 (&out)[8]) {
        const uint32_t* r0 = (const uint32_t*)&w[0];
        const uint32_t* r1 = (const uint32_t*)&w[1];
        const uint32_t* r2 = (const uint32_t*)&w[2];
        const uint32_t* r3 = (const uint32_t*)&w[3];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            out[2 * p].x = (r0[p] & 0xffffu) | (r1[p] << 16);
            out[2 * p].y = (r2[p] & 0xffffu) | (r3[p] << 16);
            out[2 * p + 1].x = (r0[p] >> 16) | (r1[p] & 0xffff0000u);
            out[2 * p + 1].y = (r2[p] >> 16) | (r3[p] & 0xffff0000u);
        }
    }
};
template <> struct transpose4<4> {
    static __device__ __forceinline__ void run(const uint4 (&w)[4], uint4 (&out)[4]) {
        out[0] = make_uint4(w[0].x, w[1].x, w[2].x, w[3].x);
        out[1] = make_uint4(w[0].y, w[1].y, w[2].y, w[3].y);
        out[2] = make_uint4(w[0].z, w[1].z, w[2].z, w[3].z);
        out[3] = make_uint4(w[0].w, w[1].w, w[2].w, w[3].w);
    }
};

template <typename DT, int MODE>
__global__ __launch_bounds__(kTThreads, 2) void train_gemm_kernel(TrainGemm p) {
    using S = typename DT::storage;
    constexpr int ES = (int)sizeof(S);
    constexpr int KS = 128 / ES;   // K values per stage
    constexpr int V = 16 / ES;     // values per 16-byte vector
    constexpr int KQ = KS / 4;     // K-outer: 4-row groups per stage
    constexpr bool A_KOUTER = MODE == kDWGU || MODE == kDWD;
    constexpr int MF = 4, NF = 4;  // 16-row fragments per wave and side

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * kTStage];

    const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
    const int wm = wid / 2, wn = wid % 2;
    const int64_t I2 = 2 * (int64_t)p.I;

    // ---- this workgroup's tile: expert e, output rows [m0, m1), columns
    // [n0, n0 + 128), K range [kb, ke)
    int e, m0, m1, n0, kb, ke, ncols, lda;
    if constexpr (MODE == kDH || MODE == kDX) {
        int mi, ni;
        if (!tile_of_block(blockIdx.x, p.nblocks, p.n_tiles, (int)*p.tile_count, p.tiles, &mi, &ni)) return;
        const int4 tl = p.tiles[mi];
        e = tl.x;
        m0 = tl.y;
        m1 = tl.z;
        n0 = ni * kTBN;
        kb = 0;
        ke = MODE == kDH ? p.H : 2 * p.I;
        ncols = MODE == kDH ? p.I : p.H;
        lda = ke;
    } else {
        const int pid = xcd_contiguous(blockIdx.x, p.nblocks);
        const int per = p.m_tiles * p.n_tiles;
        e = pid / per;
        const int rem = pid - e * per;
        const int mrows = MODE == kDWGU ? 2 * p.I : p.H;
        m0 = (rem % p.m_tiles) * kTBM;
        m1 = min(m0 + kTBM, mrows);
        n0 = (rem / p.m_tiles) * kTBN;
        kb = (int)min(p.offsets[e], (uint32_t)p.N);
        ke = max((int)min(p.offsets[e + 1], (uint32_t)p.N), kb);
        ncols = MODE == kDWGU ? p.H : p.I;
        lda = mrows;
    }
    const S* A = (const S*)p.a;

    // ---- K-outer row pointers: row k of the N-side operand (B), or of the
    // M-side operand (A) of the weight gradients
    auto b_row = [&](int k) -> const S* {
        if constexpr (MODE == kDH) {
            return (const S*)p.b0 + ((int64_t)e * p.H + k) * p.I;
        } else if constexpr (MODE == kDX) {
            return k < p.I ? (const S*)p.b0 + ((int64_t)e * p.I + k) * p.H
                           : (const S*)p.b1 + ((int64_t)e * p.I + (k - p.I)) * p.H;
        } else if constexpr (MODE == kDWGU) {
            return (const S*)p.b0 + src_row(p.b_rows, p.b_nrows, k) * p.H;
        } else {
            return (const S*)p.b0 + (int64_t)k * p.I;
        }
    };

    // ---- staging registers
    uint4 ra[4], rb[4];
    // K-contiguous M side (DH, DX): thread -> 16-byte chunk (tid % 8) of rows
    // tid / 8 + 32 j
    const int kc_ch = tid % 8, kc_row = tid / 8;
    // K-outer operands: thread -> K-rows 4 (tid % KQ) + 0..3, values
    // V (tid / KQ) + 0..V-1 of the 128 output rows/columns
    const int ko_q = tid % KQ, ko_c = (tid / KQ) * V;

    auto load_kouter = [&](uint4 (&r)[4], int kbase, int cbase, int climit, bool is_a) {
        const int col = cbase + ko_c < climit ? cbase + ko_c : 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int k = kbase + ko_q * 4 + j;
            const bool kin = k < ke;
            const int kk = kin ? k : ke - 1;
            const S* row;
            if constexpr (A_KOUTER) {
                row = is_a ? A + (int64_t)kk * lda : b_row(kk);
            } else {
                row = b_row(kk);
            }
            const uint4 v = *(const uint4*)(row + col);
            r[j] = kin ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto load_kcontig = [&](uint4 (&r)[4], int kbase) {
        const int k = kbase + kc_ch * V;
        const bool kin = k < ke;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int row = min(m0 + kc_row + 32 * j, m1 - 1);
            const uint4 v = *(const uint4*)(A + (int64_t)row * lda + (kin ? k : 0));
            r[j] = kin ? v : make_uint4(0, 0, 0, 0);
        }
    };
    auto gload = [&](int kbase) {
        if constexpr (A_KOUTER)
            load_kouter(ra, kbase, m0, m1, true);
        else
            load_kcontig(ra, kbase);
        load_kouter(rb, kbase, n0, ncols, false);
    };
    auto store_kouter = [&](unsigned char* base, const uint4 (&r)[4]) {
        if constexpr (ES == 2) {
            uint2 t[8];
            transpose4<2>::run(r, t);
#pragma unroll
            for (int i = 0; i < 8; ++i) *(uint2*)(base + (ko_c + i) * kTStride + ko_q * 8) = t[i];
        } else {
            uint4 t[4];
            transpose4<4>::run(r, t);
#pragma unroll
            for (int i = 0; i < 4; ++i) *(uint4*)(base + (ko_c + i) * kTStride + ko_q * 16) = t[i];
        }
    };
    auto lstore = [&](int st) {
        unsigned char* base = smem + st * kTStage;
        if constexpr (A_KOUTER) {
            store_kouter(base, ra);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) *(uint4*)(base + (kc_row + 32 * j) * kTStride + kc_ch * 16) = ra[j];
        }
        store_kouter(base + kTBM * kTStride, rb);
    };

    int fa[MF], fb[NF];
#pragma unroll
    for (int i = 0; i < MF; ++i) fa[i] = (wm * 64 + i * 16 + (lane & 15)) * kTStride + (lane >> 4) * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) fb[f] = (kTBM + wn * 64 + f * 16 + (lane & 15)) * kTStride + (lane >> 4) * 16;

    f32x4_t acc[MF][NF];
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int f = 0; f < NF; ++f) acc[i][f] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const int nk = (ke - kb + KS - 1) / KS;
    if (nk > 0) {
        gload(kb);
        lstore(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) gload(kb + (kt + 1) * KS);
        const unsigned char* base = smem + st * kTStage;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
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
        if (kt + 1 < nk) lstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue: lane holds output row (lane % 16) of each M fragment and
    // columns 4 (lane / 16) + 0..3 of each N fragment
#pragma unroll
    for (int i = 0; i < MF; ++i) {
        const int m = m0 + wm * 64 + i * 16 + (lane & 15);
        if (m >= m1) continue;
#pragma unroll
        for (int f = 0; f < NF; ++f) {
            const int col = n0 + wn * 64 + f * 16 + (lane >> 4) * 4;
            if (col >= ncols) continue;
            if constexpr (MODE == kDH) {
                const float* gr = p.gu + (int64_t)m * I2 + col;
                const float4 g4 = *(const float4*)gr;
                const float4 u4 = *(const float4*)(gr + p.I);
                const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, uv[4] = {u4.x, u4.y, u4.z, u4.w};
                float dg[4], du[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dh = acc[i][f][r];
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[r]));
                    du[r] = dh * (gv[r] * sg);
                    dg[r] = dh * uv[r] * (sg * (1.0f + gv[r] * (1.0f - sg)));
                }
                S* out = (S*)p.c0 + (int64_t)m * I2 + col;
                store4<DT>::run(out, dg);
                store4<DT>::run(out + p.I, du);
            } else if constexpr (MODE == kDX) {
                const float v[4] = {acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]};
                store4<DT>::run((S*)p.c0 + (int64_t)m * p.H + col, v);
            } else {
                float* out;
                if constexpr (MODE == kDWGU)
                    out = m < p.I ? (float*)p.c0 + ((int64_t)e * p.I + m) * p.H + col
                                  : (float*)p.c1 + ((int64_t)e * p.I + (m - p.I)) * p.H + col;
                else
                    out = (float*)p.c0 + ((int64_t)e * p.H + m) * p.I + col;
                *(float4*)out = make_float4(acc[i][f][0], acc[i][f][1], acc[i][f][2], acc[i][f][3]);
            }
        }
    }
}

template <typename DT, int MODE>
hipError_t launch_train_gemm(TrainGemm p, int64_t blocks, hipStream_t s) {
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    p.nblocks = (int)blocks;
    train_gemm_kernel<DT, MODE><<<(unsigned)blocks, kTThreads, 0, s>>>(p);
    return hipGetLastError();
}


// ------------------------------------------------------------------ LDS transpose read
// A K-outer operand lands in LDS in its natural layout (K-rows of
// consecutive output indices) and is read with ds_read_b64_tr_b16: within
// each 16-lane group, lane s gives the address of 4 values (K-row k0 + s / 4,
// columns n0 + 4 (s % 4) .. + 3) and receives column n0 + s's values of
// K-rows k0 .. k0 + 3.  Two such reads give a lane the 8 consecutive K values
// of one operand row that a 32x32x16 MFMA takes.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 lds_read_tr16(const unsigned char* p) {
    const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16*)(const __attribute__((address_space(3))) void*)p);
    return __builtin_bit_cast(uint2, v);
}

// keep the first n (0..4) 16-bit values of a 4-value run
__device__ __forceinline__ uint2 keep_first(uint2 v, int n) {
    if (n <= 0) return make_uint2(0, 0);
    if (n == 1) return make_uint2(v.x & 0xffffu, 0);
    if (n == 2) return make_uint2(v.x, 0);
    if (n == 3) return make_uint2(v.x, v.y & 0xffffu);
    return v;
}

// ------------------------------------------------------------------ pipelined training GEMM (16-bit)
// The four products on 128 x 256 tiles of 4 waves (each 128 x 64, 32x32x16
// MFMAs) with 32-K steps in a 64 KB ring (two row-operand slots of 8 KB,
// three column-operand slots of 16 KB), so two workgroups share a CU and one
// computes while the other stores its tile.  Layouts per slot:
//   K-contiguous row operand: 128 rows x 64 bytes, chunk c of row r at
//     c ^ swz64(r);
//   K-outer row operand (weight gradients): 32 K-rows x 256 bytes (128
//     values), chunk c of K-row r at c ^ (4 (r & 3));
//   K-outer column operand: 32 K-rows x 512 bytes, chunk c at c ^ ((r & 7) << 2).
// K-outer operands are read with the transpose read above; the swizzles put
// the K-rows of one read on distinct banks.  K tails (an expert's last rows,
// K not a multiple of 32): loads are clamped to the last valid K-row or
// chunk, and the fragments of the last step zero every value past the end
// on both operands.
constexpr int kT2BM = 128, kT2BN = 256, kT2Waves = 4;
constexpr int kT2SlotA = 8 * 1024, kT2SlotB = 16 * 1024;
constexpr int kT2SlotsA = 2, kT2SlotsB = 3;
constexpr int kT2LPA = kT2SlotA / 1024 / kT2Waves, kT2LPB = kT2SlotB / 1024 / kT2Waves;  // 2 and 4 pieces

template <typename DT, int MODE>
__global__ __launch_bounds__(kT2Waves* kWave, 2) void train_pipe2_kernel(TrainGemm p) {
    using S = typename DT::storage;
    constexpr bool A_KOUTER = MODE == kDWGU || MODE == kDWD;
    constexpr bool ROWS = MODE == kDH || MODE == kDX;
    constexpr int WTN = 64, MB = 4, NB = 2, NM = MB * NB;
    constexpr int LPA = kT2LPA, LPB = kT2LPB, NA = kT2SlotsA, NB_ = kT2SlotsB;
    constexpr int RA = A_KOUTER ? 2 * MB : MB;
    constexpr int NR = RA + 2 * NB;
    __shared__ __attribute__((aligned(1024))) unsigned char smem[NA * kT2SlotA + NB_ * kT2SlotB];

    // wid = the wave's 64-column group; wave-uniform, so the DMA's LDS
    // addresses are scalar arithmetic
    const int lane = lane_id(), wid = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int64_t I2 = 2 * (int64_t)p.I;
    const S* A = (const S*)p.a;
    const int ncols = (MODE == kDH || MODE == kDWD) ? p.I : p.H;
    const int mrows = MODE == kDWGU ? 2 * p.I : p.H;
    const int lda = MODE == kDH ? p.H : (MODE == kDWD ? p.H : 2 * p.I);

    // ---- tile: expert e, output rows [m0, m1), columns [n0, n0 + 256), K [kb, ke)
    int e, m0, m1, n0, kb, ke;
    if constexpr (ROWS) {
        int mi, ni;
        if (!tile_of_block(blockIdx.x, p.nblocks, p.n_tiles, (int)*p.tile_count, p.tiles, &mi, &ni)) return;
        const int4 tl = p.tiles[mi];
        e = tl.x;
        m0 = tl.y;
        m1 = tl.z;
        n0 = ni * kT2BN;
        kb = 0;
        ke = lda;
    } else {
        const int pid = xcd_contiguous(blockIdx.x, p.nblocks);
        const int per = p.m_tiles * p.n_tiles;
        e = pid / per;
        const int rem = pid - e * per;
        m0 = (rem % p.m_tiles) * kT2BM;
        m1 = min(m0 + kT2BM, mrows);
        n0 = (rem / p.m_tiles) * kT2BN;
        kb = (int)min(p.offsets[e], (uint32_t)p.N);
        ke = max((int)min(p.offsets[e + 1], (uint32_t)p.N), kb);
    }
    e = __builtin_amdgcn_readfirstlane(e);
    m0 = __builtin_amdgcn_readfirstlane(m0);
    m1 = __builtin_amdgcn_readfirstlane(m1);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    kb = __builtin_amdgcn_readfirstlane(kb);
    ke = __builtin_amdgcn_readfirstlane(ke);
    const int nk = (ke - kb + 31) / 32;

    // ---- loads: a wave-uniform base plus a 32-bit byte offset (the launcher
    // keeps offsets below 2^31); steps past the end re-load the last step
    const uint32_t lds_a = lds_offset(smem) + wid * LPA * 1024;
    const uint32_t lds_b = lds_offset(smem) + NA * kT2SlotA + wid * LPB * 1024;
    auto dma_a = [&](int kt, int j) __attribute__((always_inline)) {
        const int s = min(kt, nk - 1);
        const S* base;
        uint32_t off;
        if constexpr (A_KOUTER) {
            // 4 K-rows x 256 bytes per piece
            const int r = (wid * LPA + j) * 4 + (lane >> 4);
            const int c = m0 + 8 * ((lane & 15) ^ (4 * (r & 3)));
            const int k = min(32 * s + r, ke - kb - 1);
            base = A + (int64_t)kb * lda;
            off = (uint32_t)(k * lda + (c < m1 ? c : 0)) * (uint32_t)sizeof(S);
        } else {
            // 16 rows x 64 bytes per piece
            const int row = (wid * LPA + j) * 16 + (lane >> 2);
            const int lc = (lane & 3) ^ swz64(row);
            base = A + (int64_t)m0 * lda;
            off = (uint32_t)(min(row, m1 - m0 - 1) * lda) * (uint32_t)sizeof(S) +
                  (uint32_t)min(64 * s + lc * 16, ke * (int)sizeof(S) - 16);
        }
        lds_dma16_so(base, off, lds_a + (kt % NA) * kT2SlotA + j * 1024);
    };
    auto dma_b = [&](int kt, int j) __attribute__((always_inline)) {
        const int s = min(kt, nk - 1);
        const int r = (wid * LPB + j) * 2 + (lane >> 5);  // 2 K-rows x 512 bytes per piece
        const int c = n0 + 8 * ((lane & 31) ^ ((r & 7) << 2));
        const int col = c < ncols ? c : 0;
        const int k = min(32 * s + r, ke - kb - 1);     // K-row past kb
        const uint32_t lds = lds_b + (kt % NB_) * kT2SlotB + j * 1024;
        const S* base;
        uint32_t off;
        if constexpr (MODE == kDX) {
            // gate rows, then up rows; a piece's two K-rows lie in one tensor (I is even)
            const int kpair = __builtin_amdgcn_readfirstlane(min(32 * s + (wid * LPB + j) * 2, ke - 1));
            const bool in_up = kpair >= p.I;
            base = (const S*)(in_up ? p.b1 : p.b0) + (int64_t)e * p.I * p.H;
            off = (uint32_t)((k - (in_up ? p.I : 0)) * p.H + col) * (uint32_t)sizeof(S);
        } else if constexpr (MODE == kDH) {
            base = (const S*)p.b0 + (int64_t)e * p.H * p.I;
            off = (uint32_t)(k * p.I + col) * (uint32_t)sizeof(S);
        } else if constexpr (MODE == kDWGU) {
            base = (const S*)p.b0 + (int64_t)kb * p.H;
            off = (uint32_t)(k * p.H + col) * (uint32_t)sizeof(S);
        } else {
            base = (const S*)p.b0 + (int64_t)kb * p.I;
            off = (uint32_t)(k * p.I + col) * (uint32_t)sizeof(S);
        }
        lds_dma16_so(base, off, lds);
    };

    // ---- fragment addresses
    const int frow = lane & 31, kg = lane >> 5;
    const int g16 = lane >> 4, s16 = lane & 15;
    // column operand (512-byte K-rows): per (h, block f) at q = 0; q adds 16 K-rows
    int kob[2][NB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int kk = 4 * h + (s16 >> 2);
        const int rowoff = (8 * (g16 >> 1) + kk) * 512 + (2 * (g16 & 1) + ((s16 & 3) >> 1)) * 16 + (s16 & 1) * 8;
#pragma unroll
        for (int f = 0; f < NB; ++f) kob[h][f] = rowoff + 64 * ((2 * wid + f) ^ kk);
    }
    // K-outer row operand (256-byte K-rows): physical chunk 4 (i ^ (s16 / 4)) + 2 (g16 & 1) + (s16 & 3) / 2
    int koa[2][MB];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int rowoff = (8 * (g16 >> 1) + 4 * h + (s16 >> 2)) * 256 + (2 * (g16 & 1) + ((s16 & 3) >> 1)) * 16 +
                           (s16 & 1) * 8;
#pragma unroll
        for (int i = 0; i < MB; ++i) koa[h][i] = rowoff + 64 * (i ^ (s16 >> 2));
    }
    // K-contiguous row operand: row 32 i + frow, logical chunk 2 q + kg
    int kca[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) kca[q] = frow * 64 + (((2 * q + kg) ^ swz64(frow)) * 16);

    f32x16_t acc[MB][NB];
    uint4 av[2][MB], bv[2][NB];
    // MASK: step kt may be the last, partial one; its K values past ke are
    // zeroed (the loads repeat the last valid K-row there)
    auto read_one = [&](int kt, int q, int set, int r, auto mask) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask)::value;
        const int kv = ke - kb - 32 * kt;  // valid K values of step kt (32 or fewer on the last)
        if (r < RA) {
            const unsigned char* base = smem + (kt % NA) * kT2SlotA;
            if constexpr (A_KOUTER) {
                const int i = r >> 1, h = r & 1;
                uint2 v = lds_read_tr16(base + koa[h][i] + q * 16 * 256);
                if (MASK && kv < 32) v = keep_first(v, kv - (16 * q + 8 * (g16 >> 1) + 4 * h));
                if (h == 0) {
                    av[set][i].x = v.x;
                    av[set][i].y = v.y;
                } else {
                    av[set][i].z = v.x;
                    av[set][i].w = v.y;
                }
            } else {
                // rows 32 r + frow keep the chunk key of frow
                uint4 v = *(const uint4*)(base + kca[q] + r * 32 * 64);
                if (MASK && kv < 32 && 16 * q + 8 * kg >= kv) v = make_uint4(0, 0, 0, 0);
                av[set][r] = v;
            }
        } else {
            const int rr = r - RA, f = rr >> 1, h = rr & 1;
            const unsigned char* base = smem + NA * kT2SlotA + (kt % NB_) * kT2SlotB;
            uint2 v = lds_read_tr16(base + kob[h][f] + q * 16 * 512);
            if (MASK && kv < 32) v = keep_first(v, kv - (16 * q + 8 * (g16 >> 1) + 4 * h));
            if (h == 0) {
                bv[set][f].x = v.x;
                bv[set][f].y = v.y;
            } else {
                bv[set][f].z = v.x;
                bv[set][f].w = v.y;
            }
        }
    };
    int rows_live = kT2BM;
    // FULL: every row block of the tile is live (no per-MFMA row check)
    auto substep = [&](auto nd, int set, int rkt, int rq, auto&& dma, auto mask, auto full)
                       __attribute__((always_inline)) {
        constexpr int ND = decltype(nd)::value, H1 = NM / 2, H2 = NM - NM / 2;
#pragma unroll
        for (int m = 0; m < NM; ++m) {
            const int i = m / NB, f = m % NB;
            if (!ROWS || decltype(full)::value || i * 32 < rows_live)
                acc[i][f] = mma32<DT>::run(bv[set][f], av[set][i], acc[i][f]);
            if (m < H1) {
#pragma unroll
                for (int r = (m * NR) / H1; r < ((m + 1) * NR) / H1; ++r) read_one(rkt, rq, set ^ 1, r, mask);
            } else {
                const int q = m - H1;
#pragma unroll
                for (int d = (q * ND) / H2; d < ((q + 1) * ND) / H2; ++d) dma(d);
            }
            sched_fence();
        }
    };
    using no_dma = std::integral_constant<int, 0>;
    using step_dma = std::integral_constant<int, LPA + LPB>;
    auto none = [](int) __attribute__((always_inline)) {};

#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
        for (int f = 0; f < NB; ++f)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][f][r] = 0.0f;
    if (nk > 0) {
        if constexpr (ROWS) rows_live = m1 - m0;
        // issue order A0 B0 A1 B1 B2: step 0 has landed once the pieces after B0 may be in flight
#pragma unroll
        for (int j = 0; j < LPA; ++j) dma_a(0, j);
#pragma unroll
        for (int j = 0; j < LPB; ++j) dma_b(0, j);
#pragma unroll
        for (int j = 0; j < LPA; ++j) dma_a(1, j);
#pragma unroll
        for (int j = 0; j < LPB; ++j) dma_b(1, j);
#pragma unroll
        for (int j = 0; j < LPB; ++j) dma_b(2, j);
        wait_vm<LPA + 2 * LPB>();
        barrier_lds();
        // Step kt reads step kt (second half) and step kt+1 (first half):
        // only the last two steps can touch a partial last step, so the steps
        // before them run without the K-tail masking.
        const bool tail = (ke - kb) % 32 != 0;
        const int nk_plain = tail ? max(nk - 2, 0) : nk;
        auto step = [&](int kt, auto mask, auto full) __attribute__((always_inline)) {
            wait_lgkm0();
            substep(no_dma{}, 0, kt, 1, none, mask, full);
            // step kt+1 landed (only the column operand of kt+2 was issued after
            // it); every wave is done reading step kt once past the barrier
            wait_vm<LPB>();
            wait_lgkm0();
            barrier_lds();
            substep(step_dma{}, 1, kt + 1, 0, [&](int d) __attribute__((always_inline)) {
                if (d < LPA) dma_a(kt + 2, d); else dma_b(kt + 3, d - LPA);
            }, mask, full);
        };
        if (tail && nk == 1) {
#pragma unroll
            for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r, std::true_type{});
        } else {
#pragma unroll
            for (int r = 0; r < NR; ++r) read_one(0, 0, 0, r, std::false_type{});
        }
        int kt = 0;
        if (!ROWS || rows_live >= kT2BM)
            for (; kt < nk_plain; ++kt) step(kt, std::false_type{}, std::true_type{});
        else
            for (; kt < nk_plain; ++kt) step(kt, std::false_type{}, std::false_type{});
        for (; kt < nk; ++kt) step(kt, std::true_type{}, std::false_type{});
        wait_vm<0>();
        wait_lgkm0();
    }

    // ---- epilogue: lane holds output row (lane % 32) of each row block and
    // columns 8 g + 4 (lane / 32) + 0..3 (g = 0..3) of each column block
    if constexpr (MODE == kDWGU || MODE == kDWD) {
        // FP32 weight gradients, staged through LDS: each wave writes 64 of
        // its 128 rows x 64 columns (256-byte rows, 16-byte chunk c of row t
        // at c ^ (t % 16)) into its own 16 KB, then reads them back a chunk
        // per lane, so each store instruction writes 4 whole 256-byte row
        // segments instead of 16 bytes of 32 rows; two rounds.  The barrier
        // makes sure every wave is done with the operand slots first.
        barrier_lds();
        unsigned char* stage = smem + wid * 16384;
        const int c = lane & 15, rr = lane >> 4;
        const int col = n0 + wid * WTN + 4 * c;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
#pragma unroll
            for (int ii = 0; ii < 2; ++ii) {
                const int t = 32 * ii + frow;
#pragma unroll
                for (int f = 0; f < NB; ++f)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x16_t& a = acc[2 * half + ii][f];
                        *(float4*)(stage + t * 256 + (((8 * f + 2 * g + kg) ^ (t & 15)) << 4)) =
                            make_float4(a[4 * g], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]);
                    }
            }
            wait_lgkm0();
#pragma unroll
            for (int t0 = 0; t0 < 64; t0 += 4) {
                const int t = t0 + rr;
                const float4 v = *(const float4*)(stage + t * 256 + ((c ^ (t & 15)) << 4));
                const int m = m0 + 64 * half + t;
                if (m < m1 && col < ncols) {
                    float* out;
                    if constexpr (MODE == kDWGU)
                        out = m < p.I ? (float*)p.c0 + ((int64_t)e * p.I + m) * p.H + col
                                      : (float*)p.c1 + ((int64_t)e * p.I + (m - p.I)) * p.H + col;
                    else
                        out = (float*)p.c0 + ((int64_t)e * p.H + m) * p.I + col;
                    // written once and never read back here: non-temporal
                    // (measured ~1% faster on the experts backward)
                    store_nt16(out, __builtin_bit_cast(uint4, v));
                }
            }
            wait_lgkm0();
        }
        return;
    }
    if constexpr (MODE == kDH) {
        // dg = dh u s (1 + g (1 - s)), du = dh g s from the saved FP32 g, u.
        // Per 32-row block: the block's g and u (32 rows x 64 columns, 256
        // bytes a row each) come into this wave's 16 KB of LDS by direct
        // loads of whole rows (chunk c of row t at c ^ (t % 16)); each lane
        // reads its values back in the MFMA layout, and dg, du go out through
        // the same LDS (128-byte rows, chunk c at c ^ ((t / 2) % 8)) so the
        // stores write whole row segments.
        barrier_lds();
        unsigned char* stage = smem + wid * 16384;
        const uint32_t lds_stage = lds_offset(stage);
        const int c16 = lane & 15, r16 = lane >> 4;  // DMA: 4 rows x 16 chunks per instruction
        const int c8 = lane & 7, r8 = lane >> 3;     // stores: 8 rows x 8 chunks per instruction
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            // g to [0, 8 KB), u to [8 KB, 16 KB)
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                const int t = 4 * d + r16;
                const int m = min(m0 + 32 * i + t, m1 - 1);
                const int col = n0 + wid * WTN + 4 * (c16 ^ (t & 15));
                const uint32_t off = (uint32_t)(m * I2 + (col < ncols ? col : 0)) * 4u;
                lds_dma16_so(p.gu, off, lds_stage + d * 1024);
                lds_dma16_so(p.gu, off + (uint32_t)p.I * 4u, lds_stage + 8192 + d * 1024);
            }
            wait_vm<0>();
            float dg[NB][16], du[NB][16];
#pragma unroll
            for (int f = 0; f < NB; ++f)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ch = 8 * f + 2 * g + kg;
                    const int a = frow * 256 + ((ch ^ (frow & 15)) << 4);
                    const float4 g4 = *(const float4*)(stage + a);
                    const float4 u4 = *(const float4*)(stage + 8192 + a);
                    const float gv[4] = {g4.x, g4.y, g4.z, g4.w}, uv[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float dh = acc[i][f][4 * g + r];
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[r]));
                        du[f][4 * g + r] = dh * (gv[r] * sg);
                        dg[f][4 * g + r] = dh * uv[r] * (sg * (1.0f + gv[r] * (1.0f - sg)));
                    }
                }
            wait_lgkm0();  // the g, u reads are done before the region is rewritten
            // dg to [0, 4 KB), du to [4 KB, 8 KB): row frow, 8-byte half kg of chunk 4 f + g
#pragma unroll
            for (int f = 0; f < NB; ++f)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int a = frow * 128 + (((4 * f + g) ^ ((frow >> 1) & 7)) << 4) + kg * 8;
                    *(uint2*)(stage + a) = make_uint2(fmt<DT>::store2(dg[f][4 * g], dg[f][4 * g + 1]),
                                                      fmt<DT>::store2(dg[f][4 * g + 2], dg[f][4 * g + 3]));
                    *(uint2*)(stage + 4096 + a) = make_uint2(fmt<DT>::store2(du[f][4 * g], du[f][4 * g + 1]),
                                                             fmt<DT>::store2(du[f][4 * g + 2], du[f][4 * g + 3]));
                }
            wait_lgkm0();
            const int col = n0 + wid * WTN + 8 * c8;
#pragma unroll
            for (int t0 = 0; t0 < 32; t0 += 8) {
                const int t = t0 + r8;
                const int a = t * 128 + ((c8 ^ ((t >> 1) & 7)) << 4);
                const uint4 vg = *(const uint4*)(stage + a);
                const uint4 vu = *(const uint4*)(stage + 4096 + a);
                const int m = m0 + 32 * i + t;
                if (m < m1 && col < ncols) {
                    S* out = (S*)p.c0 + (int64_t)m * I2 + col;
                    *(uint4*)out = vg;
                    *(uint4*)(out + p.I) = vu;
                }
            }
            wait_lgkm0();  // read back before the next block's loads land
        }
        return;
    }
    if constexpr (MODE == kDX) {
        // dx rows staged through LDS (each wave's 128 x 64 block in its own
        // 16 KB) so that stores write whole 128-byte row segments
        barrier_lds();
        store_tile32_staged<DT, MB, NB, kT2BM, WTN>(acc, (S*)p.c0, m0, m1, n0, 0, wid, p.H, lane,
                                                    smem + wid * (kT2BM * WTN * (int)sizeof(S)));
        return;
    }
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int m = m0 + 32 * i + frow;
        if (m >= m1) continue;
#pragma unroll
        for (int f = 0; f < NB; ++f) {
            const int cb = n0 + wid * WTN + 32 * f + 4 * kg;
            if constexpr (MODE == kDH) {
                float4 g4[4], u4[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = cb + 8 * g;
                    const float* gr = p.gu + (int64_t)m * I2 + (col < ncols ? col : 0);
                    g4[g] = *(const float4*)gr;
                    u4[g] = *(const float4*)(gr + p.I);
                }
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = cb + 8 * g;
                    if (col >= ncols) continue;
                    const float gv[4] = {g4[g].x, g4[g].y, g4[g].z, g4[g].w};
                    const float uv[4] = {u4[g].x, u4[g].y, u4[g].z, u4[g].w};
                    float dg[4], du[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float dh = acc[i][f][4 * g + r];
                        const float sg = __builtin_amdgcn_rcpf(1.0f + __expf(-gv[r]));
                        du[r] = dh * (gv[r] * sg);
                        dg[r] = dh * uv[r] * (sg * (1.0f + gv[r] * (1.0f - sg)));
                    }
                    S* out = (S*)p.c0 + (int64_t)m * I2 + col;
                    store4<DT>::run(out, dg);
                    store4<DT>::run(out + p.I, du);
                }
            } else {
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = cb + 8 * g;
                    if (col >= ncols) continue;
                    const float v0 = acc[i][f][4 * g], v1 = acc[i][f][4 * g + 1], v2 = acc[i][f][4 * g + 2],
                                v3 = acc[i][f][4 * g + 3];
                    if constexpr (MODE == kDX) {
                        const float v[4] = {v0, v1, v2, v3};
                        store4<DT>::run((S*)p.c0 + (int64_t)m * p.H + col, v);
                    } else {
                        float* out;
                        if constexpr (MODE == kDWGU)
                            out = m < p.I ? (float*)p.c0 + ((int64_t)e * p.I + m) * p.H + col
                                          : (float*)p.c1 + ((int64_t)e * p.I + (m - p.I)) * p.H + col;
                        else
                            out = (float*)p.c0 + ((int64_t)e * p.H + m) * p.I + col;
                        *(float4*)out = make_float4(v0, v1, v2, v3);
                    }
                }
            }
        }
    }
}

template <typename DT, int MODE>
hipError_t launch_train_pipe2(TrainGemm p, int64_t blocks, hipStream_t s) {
    if (blocks == 0) return hipSuccess;
    if (blocks > 0x7fffffff) return hipErrorInvalidValue;
    p.nblocks = (int)blocks;
    train_pipe2_kernel<DT, MODE><<<(unsigned)blocks, kT2Waves * kWave, 0, s>>>(p);
    return hipGetLastError();
}

// rows[r] = x[token_of_row[r]] (the token index clamped into x), one
// wavefront per row, 16-byte chunks, four loads in flight per lane.  A token
// row is read once per slot and stays cached; the gathered rows are written
// once (non-temporal).
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x, const uint32_t* __restrict__ tor,
                                                          int64_t x_rows, int64_t N, int64_t chunks,
                                                          uint4* __restrict__ rows) {
    const int64_t r = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
    if (r >= N) return;
    const int64_t t = min((int64_t)tor[r], x_rows - 1);
    for (int64_t c = lane_id(); c < chunks; c += 4 * kWave) {
        uint4 v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (c + i * kWave < chunks) v[i] = x[t * chunks + c + i * kWave];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (c + i * kWave < chunks) store_nt16(rows + r * chunks + c + i * kWave, v[i]);
    }
}

template <typename DT>
hipError_t experts_backward_typed(const ExpertsBackwardArgs& a, hipStream_t s) {
    const int E = a.E, H = (int)a.H, I = (int)a.I, N = (int)a.N;
    // 16-bit types with enough rows per expert take the pipelined kernel,
    // whose loads use 32-bit byte offsets from a per-tile base
    const int64_t lim = int64_t(1) << 31, es = (int64_t)sizeof(typename DT::storage);
    const bool offsets32 = a.N * 2 * a.I * es < lim && a.N * a.H * es < lim && a.H * a.I * es < lim &&
                           256 * std::max(a.H, 2 * a.I) * es < lim;
    const bool pipe = es == 2 && offsets32 && a.N >= 64 * (int64_t)a.E;
    const int BM = pipe ? kT2BM : kTBM, BN = pipe ? kT2BN : kTBN;
    int4* tiles = (int4*)((char*)a.tiles + 256);
    uint32_t* count = (uint32_t*)a.tiles;
    const int64_t mt = max_mtiles(a.N, a.E, BM);
    hipError_t err = launch_build_tiles(a.offsets, E, a.N, BM, mt, tiles, count, s);
    if (err != hipSuccess) return err;
    auto launch = [&](auto mode, const TrainGemm& q, int64_t blocks) {
        constexpr int M = decltype(mode)::value;
        if constexpr (sizeof(typename DT::storage) == 2) {
            if (pipe) return launch_train_pipe2<DT, M>(q, blocks, s);
        }
        return launch_train_gemm<DT, M>(q, blocks, s);
    };

    TrainGemm p = {};
    p.N = N;
    p.H = H;
    p.I = I;
    p.tiles = tiles;
    p.tile_count = count;
    p.offsets = a.offsets;

    // dh -> dgu = [dg | du]
    p.a = a.dy;
    p.b0 = a.down;
    p.gu = a.gu;
    p.c0 = a.dgu;
    p.n_tiles = (I + BN - 1) / BN;
    err = launch(std::integral_constant<int, kDH>{}, p, mt * p.n_tiles);
    if (err != hipSuccess) return err;

    // dx = dgu [gate ; up]
    p.a = a.dgu;
    p.b0 = a.gate;
    p.b1 = a.up;
    p.c0 = a.dx;
    p.n_tiles = (H + BN - 1) / BN;
    err = launch(std::integral_constant<int, kDX>{}, p, mt * p.n_tiles);
    if (err != hipSuccess) return err;

    // [dgate ; dup] = dgu^T x; the pipelined kernel reads x as contiguous
    // rows, so token rows read through token_of_row are gathered first
    const void* xr = a.x;
    const uint32_t* x_rows = a.x_rows;
    if (pipe && x_rows && N > 0) {
        const int64_t chunks = a.H * (int64_t)sizeof(typename DT::storage) / 16;
        gather_rows_kernel<<<(unsigned)((a.N + 3) / 4), 256, 0, s>>>((const uint4*)a.x, x_rows, a.x_nrows, a.N,
                                                                     chunks, (uint4*)a.xg);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
        xr = a.xg;
        x_rows = nullptr;
    }
    p.a = a.dgu;
    p.b0 = xr;
    p.b1 = nullptr;
    p.b_rows = x_rows;
    p.b_nrows = (int)a.x_nrows;
    p.c0 = a.dgate;
    p.c1 = a.dup;
    p.m_tiles = (2 * I + BM - 1) / BM;
    p.n_tiles = (H + BN - 1) / BN;
    err = launch(std::integral_constant<int, kDWGU>{}, p, (int64_t)E * p.m_tiles * p.n_tiles);
    if (err != hipSuccess) return err;

    // ddown = dy^T h
    p.a = a.dy;
    p.b0 = a.h;
    p.b_rows = nullptr;
    p.b_nrows = 0;
    p.c0 = a.ddown;
    p.c1 = nullptr;
    p.m_tiles = (H + BM - 1) / BM;
    p.n_tiles = (I + BN - 1) / BN;
    return launch(std::integral_constant<int, kDWD>{}, p, (int64_t)E * p.m_tiles * p.n_tiles);
}

// ------------------------------------------------------------------ combine / dispatch backward
// One wavefront per token, 4 tokens per workgroup; lane -> 16-byte column
// chunks c = lane, lane + 64, ... of the token's rows (or single values when
// H is not a whole number of chunks).

// dY[row_j] = w_j g (rounded to the expert dtype), dw_j = <Y[row_j], g> in
// FP32; a token with a slot row >= N gets NaN weight gradients.  One
// workgroup per token: thread -> VEC-column groups c = tid, tid + 256, ...
// of the row.  Slots go in batches of 8: the thread's g values are loaded
// once per batch and its Y loads for the batch's slots go out together.  Each
// dw_j is reduced in a fixed order (the thread's columns in order, a
// butterfly over the wave, then the 4 waves in order), so it does not depend
// on timing.
template <typename DT, typename WT, int VEC>
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const typename DT::storage* __restrict__ Y, int64_t N, const uint32_t* __restrict__ row_of_slot,
    const typename WT::storage* __restrict__ w, const typename DT::storage* __restrict__ g, int k, int64_t H,
    typename DT::storage* __restrict__ dY, float* __restrict__ dw) {
    using S = typename DT::storage;
    constexpr int B = 8, NWAVE = 256 / kWave;
    __shared__ float part[NWAVE][B];
    const int64_t t = blockIdx.x;
    const int tid = threadIdx.x, lane = lane_id(), wid = tid / kWave;
    const uint32_t* rs = row_of_slot + t * k;
    // slot rows and weights are loaded unconditionally, clamped to the last
    // slot, so that each batch's loads go out together
    bool invalid = false;
    for (int j0 = 0; j0 < k; j0 += B) {
        uint32_t r[B];
#pragma unroll
        for (int b = 0; b < B; ++b) r[b] = rs[min(j0 + b, k - 1)];
#pragma unroll
        for (int b = 0; b < B; ++b) invalid |= j0 + b < k && (int64_t)r[b] >= N;
    }
    const S* gt = g + t * H;
    const int64_t chunks = H / VEC;
    for (int j0 = 0; j0 < k; j0 += B) {
        float dot[B], wj[B];
        int64_t row[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int j = min(j0 + b, k - 1);
            const uint32_t rr = rs[j];
            const float wv = fmt<WT>::load(w[t * k + j]);
            dot[b] = 0.0f;
            row[b] = j0 + b < k ? (int64_t)rr : N;  // N: no slot, or a slot past the rows
            wj[b] = row[b] < N ? wv : 0.0f;
        }
        for (int64_t c = tid; c < chunks; c += 256) {
            S gv[VEC], yv[B][VEC];
            if constexpr (VEC * sizeof(S) == 16)
                *(uint4*)gv = *(const uint4*)(gt + c * VEC);
            else
                gv[0] = gt[c];
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (row[b] < N) {
                    if constexpr (VEC * sizeof(S) == 16)
                        *(uint4*)yv[b] = *(const uint4*)(Y + row[b] * H + c * VEC);
                    else
                        yv[b][0] = Y[row[b] * H + c];
                }
            }
#pragma unroll
            for (int b = 0; b < B; ++b) {
                if (row[b] < N) {
                    S ov[VEC];
#pragma unroll
                    for (int v = 0; v < VEC; ++v) {
                        const float gf = fmt<DT>::load(gv[v]);
                        dot[b] = fmaf(fmt<DT>::load(yv[b][v]), gf, dot[b]);
                        ov[v] = fmt<DT>::store(wj[b] * gf);
                    }
                    if constexpr (VEC * sizeof(S) == 16)
                        *(uint4*)(dY + row[b] * H + c * VEC) = *(const uint4*)ov;
                    else
                        dY[row[b] * H + c] = ov[0];
                }
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) dot[b] = wave_sum(dot[b]);
        if (lane == 0) {
#pragma unroll
            for (int b = 0; b < B; ++b) part[wid][b] = dot[b];
        }
        __syncthreads();
        if (tid < B && j0 + tid < k) {
            float sum = part[0][tid];
#pragma unroll
            for (int q = 1; q < NWAVE; ++q) sum += part[q][tid];
            dw[t * k + j0 + tid] = invalid ? __uint_as_float(0x7fc00000u) : sum;
        }
        __syncthreads();
    }
}

// dx[t] = sum_j drows[row_j] in FP32, slot order j = 0..k-1, rounded once; a
// token with a slot row >= N gets a NaN row.  grid (tokens, column chunks):
// thread -> VEC consecutive columns of one token.  The token's k rows are
// wave-uniform and their loads go out in batches of 8 before the adds, so
// the loads of a thread overlap.  Every row of drows is read once and every
// row of dx written once: the 16-byte accesses are non-temporal.
template <typename DT, int VEC>
__global__ __launch_bounds__(256) void dispatch_backward_kernel(const typename DT::storage* __restrict__ drows,
                                                                int64_t N, const uint32_t* __restrict__ row_of_slot,
                                                                int k, int64_t H,
                                                                typename DT::storage* __restrict__ dx) {
    using S = typename DT::storage;
    const int64_t t = blockIdx.x;
    const int64_t c0 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * VEC;
    if (c0 >= H) return;
    const uint32_t* rs = row_of_slot + t * k;
    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
    bool invalid = false;
    constexpr int B = 8;
    for (int j0 = 0; j0 < k; j0 += B) {
        // the batch's rows, loaded unconditionally (slots past k re-read the
        // last one) so that the loads go out together
        uint32_t r[B];
#pragma unroll
        for (int b = 0; b < B; ++b) r[b] = rs[min(j0 + b, k - 1)];
#pragma unroll
        for (int b = 0; b < B; ++b) invalid |= j0 + b < k && (int64_t)r[b] >= N;
        if (invalid) break;
        S vals[B][VEC];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b < k) {
                const S* src = drows + (int64_t)r[b] * H + c0;
                if constexpr (VEC * sizeof(S) == 16)
                    *(uint4*)vals[b] = load_nt16(src);
                else
                    vals[b][0] = *src;
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b < k) {
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] += fmt<DT>::load(vals[b][v]);
            }
        }
    }
    if (invalid) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = __uint_as_float(0x7fc00000u);
    }
    S ov[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) ov[v] = fmt<DT>::store(acc[v]);
    if constexpr (VEC * sizeof(S) == 16)
        store_nt16(dx + t * H + c0, *(const uint4*)ov);
    else
        dx[t * H + c0] = ov[0];
}

bool wide_rows(int64_t H, int es, std::initializer_list<const void*> ptrs) {
    if (H % (16 / es)) return false;
    for (const void* q : ptrs)
        if ((uintptr_t)q % 16) return false;
    return true;
}

template <typename DT, typename WT>
hipError_t combine_backward_typed(const CombineBackwardArgs& a, hipStream_t s) {
    using S = typename DT::storage;
    using W = typename WT::storage;
    constexpr int V16 = 16 / sizeof(S);
    if (a.T > 0x7fffffff) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.T), block(256);
    if (wide_rows(a.H, sizeof(S), {a.y, a.g, a.dy}))
        combine_backward_kernel<DT, WT, V16><<<grid, block, 0, s>>>((const S*)a.y, a.N, a.row_of_slot, (const W*)a.w,
                                                                   (const S*)a.g, a.k, a.H, (S*)a.dy, a.dw);
    else
        combine_backward_kernel<DT, WT, 1><<<grid, block, 0, s>>>((const S*)a.y, a.N, a.row_of_slot, (const W*)a.w,
                                                                 (const S*)a.g, a.k, a.H, (S*)a.dy, a.dw);
    return hipGetLastError();
}

template <typename DT>
hipError_t combine_backward_w(const CombineBackwardArgs& a, hipStream_t s) {
    switch (a.wdtype) {
    case MOE_F32: return combine_backward_typed<DT, f32_t>(a, s);
    case MOE_F16: return combine_backward_typed<DT, f16_t>(a, s);
    case MOE_BF16: return combine_backward_typed<DT, bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <typename DT>
hipError_t dispatch_backward_typed(const DispatchBackwardArgs& a, hipStream_t s) {
    using S = typename DT::storage;
    constexpr int V16 = 16 / sizeof(S);
    const bool wide = wide_rows(a.H, sizeof(S), {a.drows, a.dx});
    const int64_t chunks = ((wide ? a.H / V16 : a.H) + 255) / 256;
    if (a.T > 0x7fffffff || chunks > 65535) return hipErrorInvalidValue;
    if (chunks == 0) return hipSuccess;
    const dim3 grid((unsigned)a.T, (unsigned)chunks), block(256);
    if (wide)
        dispatch_backward_kernel<DT, V16><<<grid, block, 0, s>>>((const S*)a.drows, a.N, a.row_of_slot, a.k, a.H,
                                                                (S*)a.dx);
    else
        dispatch_backward_kernel<DT, 1><<<grid, block, 0, s>>>((const S*)a.drows, a.N, a.row_of_slot, a.k, a.H,
                                                              (S*)a.dx);
    return hipGetLastError();
}

}  // namespace

size_t experts_backward_tile_bytes(int64_t N, int64_t E) { return 256 + 16 * (size_t)max_mtiles(N, E, kTBM); }

hipError_t launch_experts_backward(const ExpertsBackwardArgs& a, hipStream_t s) {
    if (a.E < 1) return hipErrorInvalidValue;
    if ((int64_t)a.E * ((2 * a.I + kTBM - 1) / kTBM) * ((a.H + kTBN - 1) / kTBN) > 0x7fffffff)
        return hipErrorInvalidValue;
    switch (a.dtype) {
    case MOE_F32: return experts_backward_typed<f32_t>(a, s);
    case MOE_F16: return experts_backward_typed<f16_t>(a, s);
    case MOE_BF16: return experts_backward_typed<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    switch (a.dtype) {
    case MOE_F32: return combine_backward_w<f32_t>(a, s);
    case MOE_F16: return combine_backward_w<f16_t>(a, s);
    case MOE_BF16: return combine_backward_w<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_dispatch_backward(const DispatchBackwardArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    switch (a.dtype) {
    case MOE_F32: return dispatch_backward_typed<f32_t>(a, s);
    case MOE_F16: return dispatch_backward_typed<f16_t>(a, s);
    case MOE_BF16: return dispatch_backward_typed<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
