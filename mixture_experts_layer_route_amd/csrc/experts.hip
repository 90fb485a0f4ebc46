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
// Work list: a one-workgroup kernel turns expert_offsets into a list of
// (expert, row_begin, row_end) M-tiles in ascending expert order, on the
// device, so no host sync is needed.  The GEMM grid is sized for the most
// M-tiles any routing could produce; surplus workgroups exit at once.
// Workgroup ids are remapped so each of the 8 XCDs works on a contiguous run
// of tiles (tiles of one expert share A rows and weight rows in that XCD's L2).
//
// Pipeline: 128-byte K slices of A and B are staged in LDS (row stride padded
// by 16 bytes, so the 16 rows a ds_read_b128 touches fall in distinct banks),
// double buffered: the global loads of slice k+1 are in flight while the
// matrix cores work on slice k.  FP32 accumulation throughout.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// One 16-byte operand chunk per lane and per fragment: 8 bf16/f16 values feed
// one 16x16x32 MFMA; 4 f32 values feed four 16x16x4 MFMAs.  A and B always
// take the same K elements in the same register slots, so the products sum
// over exactly the right K indices.
template <typename DT> struct mma;
template <> struct mma<bf16_t> {
    static __device__ __forceinline__ f32x4_t run(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <> struct mma<f16_t> {
    static __device__ __forceinline__ f32x4_t run(uint4 a, uint4 b, f32x4_t c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};
template <> struct mma<f32_t> {
    static __device__ __forceinline__ f32x4_t run(uint4 a, uint4 b, f32x4_t c) {
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
        c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
        return c;
    }
};

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
                                                           uint32_t N, int BM, uint32_t max_tiles,
                                                           int4* __restrict__ tiles,
                                                           uint32_t* __restrict__ count) {
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
            for (uint32_t r = b; r < en; r += BM, ++t)
                if (t < max_tiles) tiles[t] = make_int4(e, (int)r, (int)min(r + BM, en), 0);
        }
    }
    if (threadIdx.x == 0) *count = min(total, max_tiles);
}

// ------------------------------------------------------------------ grouped GEMM
template <typename DT, bool GATEUP, int BM, int BNB, int WGM, int WGN>
__global__ __launch_bounds__(WGM* WGN* kWave) void grouped_gemm_kernel(
    const typename DT::storage* __restrict__ A,   // [rows, K]
    const typename DT::storage* __restrict__ B0,  // [E, NOUT, K]  (gate or down)
    const typename DT::storage* __restrict__ B1,  // [E, NOUT, K]  (up; GATEUP only)
    typename DT::storage* __restrict__ C,         // [rows, NOUT]
    const int4* __restrict__ tiles, const uint32_t* __restrict__ tile_count, int K, int NOUT,
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
    constexpr int WTM = BM / WGM;             // rows per wave
    constexpr int MF = WTM / 16;              // 16-row fragments per wave
    constexpr int NF = BNB / WGN / 16;        // 16-col B fragments per wave
    constexpr int WCN = BN_OUT / WGN;         // output columns per wave
    constexpr int STAGE = (BM + BNB) * LDS_STRIDE;
    static_assert(NT % CPR == 0, "chunk column must be fixed per thread");
    static_assert(WTM % 16 == 0 && (BNB / WGN) % 16 == 0, "wave tile must be whole fragments");
    static_assert(!GATEUP || NF % 2 == 0, "gate and up fragments pair up");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    // XCD-aware remap: hardware hands workgroup b to XCD b % 8; give each XCD
    // a contiguous range of logical tiles.
    const int bid = blockIdx.x;
    const int q = nblocks / 8, rem = nblocks % 8;
    const int xcd = bid % 8, loc = bid / 8;
    const int pid = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + loc;
    const int m_idx = pid / n_tiles, n_idx = pid % n_tiles;
    if (m_idx >= (int)*tile_count) return;
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
        a_src[i] = (const char*)(A + (int64_t)grow * K) + my_ch * 16;
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
    auto gload = [&](int kt) {
        const int kb = kt * ROWB;
        const bool kin = kb + my_ch * 16 < kbytes;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            ra[i] = (kin && (A_CHUNKS % NT == 0 || tid + i * NT < A_CHUNKS))
                        ? *(const uint4*)(a_src[i] + kb) : make_uint4(0, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            rb[i] = (kin && (B_CHUNKS % NT == 0 || tid + i * NT < B_CHUNKS))
                        ? *(const uint4*)(b_src[i] + kb) : make_uint4(0, 0, 0, 0);
    };
    auto lstore = [&](int st) {
        unsigned char* base = smem + st * STAGE;
#pragma unroll
        for (int i = 0; i < A_CH; ++i)
            if (A_CHUNKS % NT == 0 || tid + i * NT < A_CHUNKS) *(uint4*)(base + a_lds[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < B_CH; ++i)
            if (B_CHUNKS % NT == 0 || tid + i * NT < B_CHUNKS) *(uint4*)(base + b_lds[i]) = rb[i];
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
    lstore(0);
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
                for (int f = 0; f < NF; ++f) acc[i][f] = mma<DT>::run(av[i], bv[f], acc[i][f]);
        }
        if (kt + 1 < nk) lstore(st ^ 1);
        __syncthreads();
    }

    // epilogue: lane holds rows 4*(lane/16)+rr, column lane%16 of each fragment
#pragma unroll
    for (int i = 0; i < MF; ++i) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int grow = r0 + wm * WTM + i * 16 + (lane >> 4) * 4 + rr;
            if (grow >= r1) continue;
            S* crow = C + (int64_t)grow * NOUT;
            if (GATEUP) {
#pragma unroll
                for (int f = 0; f < NF / 2; ++f) {
                    const int col = n0 + wn * WCN + f * 16 + (lane & 15);
                    if (col < NOUT) {
                        const float g = acc[i][f][rr], u = acc[i][f + NF / 2][rr];
                        crow[col] = fmt<DT>::store(g / (1.0f + expf(-g)) * u);
                    }
                }
            } else {
#pragma unroll
                for (int f = 0; f < NF; ++f) {
                    const int col = n0 + wn * WCN + f * 16 + (lane & 15);
                    if (col < NOUT) crow[col] = fmt<DT>::store(acc[i][f][rr]);
                }
            }
        }
    }
}

struct GemmShape {
    int BM;
};

int64_t max_mtiles(int64_t N, int64_t E, int BM) {
    if (N <= 0) return 0;
    const int64_t bound = (N + E * (BM - 1)) / BM;
    return bound < N ? bound : N;
}

template <typename DT, bool GATEUP, int BM, int BNB, int WGM, int WGN>
hipError_t launch_gemm(const void* A, const void* B0, const void* B1, void* C, const int4* tiles,
                       const uint32_t* count, int64_t mt, int K, int NOUT, hipStream_t s) {
    using S = typename DT::storage;
    constexpr int BN_OUT = GATEUP ? BNB / 2 : BNB;
    const int n_tiles = (NOUT + BN_OUT - 1) / BN_OUT;
    const int64_t nb = mt * n_tiles;
    if (nb == 0) return hipSuccess;
    if (nb > 0x7fffffff) return hipErrorInvalidValue;
    grouped_gemm_kernel<DT, GATEUP, BM, BNB, WGM, WGN><<<(unsigned)nb, WGM * WGN * kWave, 0, s>>>(
        (const S*)A, (const S*)B0, (const S*)B1, (S*)C, tiles, count, K, NOUT, n_tiles, (int)nb);
    return hipGetLastError();
}

// Two tile shapes: a 128-row tile for experts that own many rows, and a
// 16-row tile for decode-sized batches, where each expert owns a handful of
// rows and the products are a stream of weight rows.
constexpr int kSmallBM = 16;

template <typename DT>
hipError_t launch_typed(const ExpertsArgs& a, hipStream_t s, ExpertsPart part) {
    const bool small = a.N < 64 * (int64_t)a.E;
    const int BM = small ? kSmallBM : 128;
    int4* tiles = (int4*)((char*)a.tiles + 256);
    uint32_t* count = (uint32_t*)a.tiles;
    const int64_t mt = max_mtiles(a.N, a.E, BM);
    build_tiles_kernel<<<1, 1024, 0, s>>>(a.offsets, a.E, (uint32_t)a.N, BM, (uint32_t)mt, tiles, count);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int H = (int)a.H, I = (int)a.I;
    if (part != kDown) {
        err = small ? launch_gemm<DT, true, 16, 256, 1, 4>(a.x, a.gate, a.up, a.h, tiles, count, mt, H, I, s)
                    : launch_gemm<DT, true, 128, 128, 2, 2>(a.x, a.gate, a.up, a.h, tiles, count, mt, H, I, s);
        if (err != hipSuccess) return err;
    }
    if (part != kGateUp) {
        err = small ? launch_gemm<DT, false, 16, 256, 1, 4>(a.h, a.down, nullptr, a.y, tiles, count, mt, I, H, s)
                    : launch_gemm<DT, false, 128, 128, 2, 2>(a.h, a.down, nullptr, a.y, tiles, count, mt, I, H, s);
    }
    return err;
}

}  // namespace

size_t experts_tile_bytes(int64_t N, int64_t E) {
    return 256 + 16 * (size_t)max_mtiles(N, E, kSmallBM);
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
