// mfma.h -- CDNA4 matrix-op wrappers and epilogue helpers shared by the
// grouped-GEMM sources of libmoe.so (experts.hip, train.hip).
#pragma once

#include "moe_internal.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

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

// 32x32x16 matrix op: lane l supplies 8 K-values of row (l % 32) of each
// operand, K group (l / 32); lane l receives column (l % 32) and rows
// 8 (r / 4) + 4 (l / 32) + (r % 4) of the result in register r.
template <typename DT> struct mma32;
template <> struct mma32<bf16_t> {
    static __device__ __forceinline__ f32x16_t run(uint4 a, uint4 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                       __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
    }
};
template <> struct mma32<f16_t> {
    static __device__ __forceinline__ f32x16_t run(uint4 a, uint4 b, f32x16_t c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                      __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
    }
};

// SiLU(g) * u in FP32: exp on the hardware exp2 unit and a hardware
// reciprocal; the product is then rounded to the weight dtype, whose
// precision (bf16/f16), or the f32 tolerance, dwarfs their few-ulp error.
__device__ __forceinline__ float silu_mul(float g, float u) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

template <typename DT> struct store4;
template <> struct store4<f32_t> {
    static __device__ __forceinline__ void run(float* p, const float* v) {
        *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    }
};
template <typename DT> struct store4 {
    static __device__ __forceinline__ void run(uint16_t* p, const float* v) {
        uint2 w;
        w.x = fmt<DT>::store2(v[0], v[1]);
        w.y = fmt<DT>::store2(v[2], v[3]);
        *(uint2*)p = w;
    }
};

// Training forward: the FP32 pre-activations g = gate x (columns [0, I)) and
// u = up x (columns [I, 2I)) of row `row`, four consecutive columns each.
__device__ __forceinline__ void save_preact(float* __restrict__ gu, int64_t row, int I, int col, const float* g,
                                            const float* u) {
    float* p = gu + row * 2 * (int64_t)I + col;
    *(float4*)p = make_float4(g[0], g[1], g[2], g[3]);
    *(float4*)(p + I) = make_float4(u[0], u[1], u[2], u[3]);
}

// ------------------------------------------------------------------ LDS row layout
// Rows of 128 bytes (64 K-values of 16 bits) hold their 16-byte chunk c at
// chunk slot c ^ swz128(r).  gfx950's LDS has 64 banks of 4 bytes and
// serves a 16-byte-per-lane read 16 lanes per clock, so a read is
// conflict-free when its 16 lanes reach 16 different 4-bank groups; row r
// covers groups 8 (r % 2) + 0..7.  The fragment reads of the grouped GEMMs
// take one logical chunk from 16 consecutive rows per 16 lanes: with the key
// r & 7, rows r and r + 8 collide (2-way conflicts, measured at 127 B/clk
// per CU); flipping bit 0 of the key for rows with bit 3 set separates them
// (measured at 254 B/clk, the full 256).  The key of a row 32 i + f is that
// of f.
__device__ __forceinline__ int swz128(int r) { return (r & 7) ^ ((r >> 3) & 1); }
// Rows of 64 bytes (32 K-values) cover groups 4 (r % 4) + 0..3, so the 16
// rows one read takes a chunk from are conflict-free with the key
// (r >> 2) & 3 (with (r >> 1) & 3, rows r and r + 8 collide).  The key of a
// row 32 i + f is that of f.
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

// ------------------------------------------------------------------ LDS pipelines
// The stage ring is driven by hand: the DMA loads, the vmcnt waits and the
// barriers below are the whole ordering protocol of the pipeline, so they
// are written as volatile asm that the compiler neither reorders memory
// around nor pads with waits of its own (it would otherwise drain every DMA
// before each fragment read, since it cannot tell the stages apart).
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// 16 bytes per lane from global address g into LDS at m0 + 16 * lane.
// m0 is written here and nowhere else in these kernels.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}
// The same from a wave-uniform base address plus a 32-bit per-lane byte
// offset (one VGPR per load instead of a 64-bit address).
__device__ __forceinline__ void lds_dma16_so(const void* base, uint32_t voff, uint32_t lds_base) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sb),
                 "s"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory", "m0");
}
// Four 32-bit loads from a wave-uniform base at per-lane byte offsets
// (replaced in place by the values), issued together and waited for once.
// Short of registers, the compiler gives such loads one destination and so
// issues and waits for them one at a time.  The wait drains every vector
// memory operation of the wave, so this goes where none of the hand-counted
// DMA loads can be in flight.
__device__ __forceinline__ void load4_u32(const void* base, uint32_t (&v)[4]) {
    const uint64_t b = (uint64_t)(uintptr_t)base;
    const uint64_t sb = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                        (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
    asm volatile(
        "global_load_dword %0, %0, %4\n\t"
        "global_load_dword %1, %1, %4\n\t"
        "global_load_dword %2, %2, %4\n\t"
        "global_load_dword %3, %3, %4\n\t"
        "s_waitcnt vmcnt(0)"
        : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3])
        : "s"(sb)
        : "memory");
}
#pragma clang diagnostic pop
__device__ __forceinline__ void barrier_lds() { asm volatile("s_barrier" ::: "memory"); }
// Keeps the instruction scheduler from moving anything across this point.
// Placed after the fragment reads of a K half, so they are issued a whole
// K half of MFMAs before their first use instead of being sunk next to it
// (the scheduler otherwise trades that latency slack for fewer registers).
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
template <int N> __device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }
// lgkmcnt(0) through the builtin, so the compiler's own LDS-read tracking
// knows the fragment registers are complete
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// vmcnt(0) through the builtin: every vector memory operation issued so far
// has completed, which the compiler then knows too, so it adds no wait of its
// own (counted without the hand-issued DMA loads) before using a result that
// was pending here
__device__ __forceinline__ void wait_vm0_known() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// An epilogue of 2-byte outputs staged through LDS: each wave
// writes its WTM-token x WTN-column block into its own LDS region (`stage`,
// WTM / ROUNDS * WTN * 2 bytes that no other wave touches before the next
// barrier), row by row, then reads it back a 16-byte chunk per lane, so a
// store instruction writes whole 128-byte row segments of 8 rows instead of
// 8 bytes of 32 rows.  With ROUNDS > 1 the block goes through the region in
// that many rounds of WTM / ROUNDS rows (a wave's LDS operations complete in
// order, so a round's writes never overtake the reads of the one before).
// Staged row t holds its 16-byte chunk c at c ^ ((t / 2) % 8), which spreads
// both the 8-byte writes and the 16-byte reads over all 64 banks.  The lane
// layout is the 32x32 MFMA result's: row (lane % 32) of each 32-row block,
// columns 8 g + 4 (lane / 32) + 0..3 of each 32-column block.
template <typename DT, int MB, int NB, int WTM, int WTN, int ROUNDS = 1>
__device__ __forceinline__ void store_tile32_staged(const f32x16_t (&acc)[MB][NB],
                                                    typename DT::storage* __restrict__ C, int r0, int r1, int n0,
                                                    int wm, int wn, int NOUT, int lane, unsigned char* stage) {
    using S = typename DT::storage;
    constexpr int RB = WTN * 2;     // bytes per staged row
    constexpr int CPR = RB / 16;    // 16-byte chunks per row
    constexpr int RPS = 256 / RB;   // rows per sweep of the 64 banks
    constexpr int MBR = MB / ROUNDS, WTR = WTM / ROUNDS;  // 32-row blocks and rows per round
    static_assert(sizeof(S) == 2 && RB == 128, "2-byte outputs, 64 per wave row");
    static_assert(MB % ROUNDS == 0, "whole 32-row blocks per round");
    // an opaque copy of the lane id keeps the compiler from computing the
    // staging addresses before the K loop and holding them through it
    asm volatile("" : "+v"(lane));
    const int frow = lane & 31, half = lane >> 5;
    constexpr int RPI = 64 / CPR;  // staged rows per store instruction
    const int c = lane % CPR, rr = lane / CPR;
    const int col = n0 + wn * WTN + c * 8;
#pragma unroll
    for (int rd = 0; rd < ROUNDS; ++rd) {
#pragma unroll
        for (int ib = 0; ib < MBR; ++ib) {
            const int i = rd * MBR + ib;
            const int t = ib * 32 + frow;
            const int sw = (t / RPS) % CPR;
#pragma unroll
            for (int g = 0; g < 4; ++g) {
#pragma unroll
                for (int f = 0; f < NB; ++f) {
                    const int col = f * 32 + g * 8 + half * 4;
                    uint2 w;
                    w.x = fmt<DT>::store2(acc[i][f][g * 4], acc[i][f][g * 4 + 1]);
                    w.y = fmt<DT>::store2(acc[i][f][g * 4 + 2], acc[i][f][g * 4 + 3]);
                    *(uint2*)(stage + t * RB + (((col >> 3) ^ sw) << 4) + half * 8) = w;
                }
            }
        }
        wait_lgkm0();
#pragma unroll
        for (int t0 = 0; t0 < WTR; t0 += RPI) {
            const int t = t0 + rr;
            const uint4 v = *(const uint4*)(stage + t * RB + ((c ^ ((t / RPS) % CPR)) << 4));
            const int grow = r0 + wm * WTM + rd * WTR + t;
            if (grow < r1 && col < NOUT) *(uint4*)(C + (int64_t)grow * NOUT + col) = v;
        }
    }
}

// The gate/up epilogue staged through LDS across the whole tile: the tile's
// 256 token rows of h (its 128 columns, 256 bytes a row; 16-byte chunk c of
// row t at c ^ (t % 16)) are written by the 8 waves, each its 128 x 32 part
// after the SiLU*mul, then read back a row chunk per lane after a barrier, so
// each store instruction writes 4 whole 256-byte row segments instead of 16
// bytes of 32 rows.  Needs 64 KB of LDS that no wave reads until the next
// barrier; MB x 32 = WTM token rows and 32 h columns per wave (gate block
// f = 0, up block f = 1).
template <typename DT, int MB, int WTM>
__device__ __forceinline__ void store_gateup_staged(const f32x16_t (&acc)[MB][2], typename DT::storage* __restrict__ C,
                                                    int r0, int r1, int n0, int wm, int wn, int wid, int NOUT,
                                                    int lane, unsigned char* stage) {
    using S = typename DT::storage;
    static_assert(sizeof(S) == 2 && WTM == MB * 32, "2-byte outputs");
    constexpr int RB = 256;  // 128 columns of h per staged row
    asm volatile("" : "+v"(lane));
    const int frow = lane & 31, half = lane >> 5;
#pragma unroll
    for (int i = 0; i < MB; ++i) {
        const int t = wm * WTM + i * 32 + frow;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int c = wn * 4 + g;  // 8 columns wn * 32 + 8 g .. of the tile's 128
            uint2 w;
            w.x = fmt<DT>::store2(silu_mul(acc[i][0][g * 4], acc[i][1][g * 4]),
                                  silu_mul(acc[i][0][g * 4 + 1], acc[i][1][g * 4 + 1]));
            w.y = fmt<DT>::store2(silu_mul(acc[i][0][g * 4 + 2], acc[i][1][g * 4 + 2]),
                                  silu_mul(acc[i][0][g * 4 + 3], acc[i][1][g * 4 + 3]));
            *(uint2*)(stage + t * RB + ((c ^ (t & 15)) << 4) + half * 8) = w;
        }
    }
    wait_lgkm0();
    barrier_lds();
    const int c = lane & 15, rr = lane >> 4;
    const int col = n0 + c * 8;
#pragma unroll
    for (int t0 = 0; t0 < 32; t0 += 4) {
        const int t = wid * 32 + t0 + rr;
        const uint4 v = *(const uint4*)(stage + t * RB + ((c ^ (t & 15)) << 4));
        const int grow = r0 + t;
        if (grow < r1 && col < NOUT) *(uint4*)(C + (int64_t)grow * NOUT + col) = v;
    }
}

}  // namespace moe
