// moe_internal.h -- device helpers and kernel launchers shared by the HIP
// sources of libmoe.so (not installed, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

constexpr uint32_t kInvalidRow = 0xFFFFFFFFu;
constexpr int kWave = 64;

// ------------------------------------------------------------------ formats
// 16-bit floats travel as raw uint16_t.  FP32 -> 16-bit conversions round to
// nearest, ties to even, and keep NaN a (quiet) NaN.  They use gfx950's pair
// conversions (v_cvt_pk_bf16_f32, v_cvt_pk_f16_f32): one instruction per two
// values, checked bit for bit against the written-out rounding
// (u + 0x7fff + ((u >> 16) & 1)) >> 16 with quiet NaN (u >> 16) | 0x40 on
// 16.7M values including ties, denormals and NaN payloads.
struct f32_t { using storage = float; };
struct f16_t { using storage = uint16_t; };
struct bf16_t { using storage = uint16_t; };

typedef float f32x2_cvt_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cvt_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_cvt_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
// a in the low half, b in the high half
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
    const f32x2_cvt_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_cvt_t));
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
    _Float16 h = __builtin_bit_cast(_Float16, b);
    return (float)h;
}

__device__ __forceinline__ uint16_t f32_to_f16(float f) {
    _Float16 h = (_Float16)f;  // v_cvt_f16_f32: nearest even, NaN stays NaN
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
    const f32x2_cvt_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_cvt_t));
}

template <typename DT> struct fmt;
template <> struct fmt<f32_t> {
    static __device__ __forceinline__ float load(float v) { return v; }
    static __device__ __forceinline__ float store(float v) { return v; }
};
template <> struct fmt<f16_t> {
    static __device__ __forceinline__ float load(uint16_t v) { return f16_to_f32(v); }
    static __device__ __forceinline__ uint16_t store(float v) { return f32_to_f16(v); }
    static __device__ __forceinline__ uint32_t store2(float a, float b) { return f32x2_to_f16x2(a, b); }
};
template <> struct fmt<bf16_t> {
    static __device__ __forceinline__ float load(uint16_t v) { return bf16_to_f32(v); }
    static __device__ __forceinline__ uint16_t store(float v) { return f32_to_bf16(v); }
    static __device__ __forceinline__ uint32_t store2(float a, float b) { return f32x2_to_bf16x2(a, b); }
};

// ------------------------------------------------------------------ wave helpers
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Cross-lane moves inside a row of 16 lanes (DPP): swap neighbours, swap
// pairs, mirror within 8 lanes, mirror within 16.  Applied in that order,
// each step pairs every lane with one holding the other half of the lanes
// reduced so far, so a max over the row ends in all 16 lanes; the last two
// steps (across rows) use permutes.  Only order-free reductions (max) use
// this: a sum keeps its xor butterfly so its rounding does not change.
constexpr int kDppSwap1 = 0xB1, kDppSwap2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140;
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppSwap1>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppSwap2>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppHalfMirror>(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_u32<kDppMirror>(__float_as_uint(v))));
    v = fmaxf(v, __shfl_xor(v, 16, kWave));
    v = fmaxf(v, __shfl_xor(v, 32, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t v) {
    const uint64_t o = ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
    return o > v ? o : v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_dpp_u64<kDppSwap1>(v);
    v = max_dpp_u64<kDppSwap2>(v);
    v = max_dpp_u64<kDppHalfMirror>(v);
    v = max_dpp_u64<kDppMirror>(v);
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, m, kWave);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m, kWave);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

// inclusive scan over the 64 lanes of a wave
__device__ __forceinline__ uint32_t wave_inclusive_scan(uint32_t v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        uint32_t y = __shfl_up(v, d, kWave);
        if (lane >= d) v += y;
    }
    return v;
}

// ------------------------------------------------------------------ streaming access
// 16-byte loads and stores with the non-temporal hint (global_load/store ...
// nt), for data a kernel touches exactly once: it streams past the caches
// instead of displacing lines that other rows still reuse.
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
    const u32x4_nt_t v = __builtin_nontemporal_load((const u32x4_nt_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
    const u32x4_nt_t w = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(w, (u32x4_nt_t*)p);
}

// ------------------------------------------------------------------ launchers
// Each returns hipSuccess or the launch error.  Shapes are checked by the
// caller (moe_api.hip) before these run.
struct RouteArgs {
    const void* logits;
    int ldtype;  // moe_dtype of logits and weights
    int64_t T;
    int E, k, renorm;
    uint32_t* idx;
    void* w;
};
hipError_t launch_route(const RouteArgs& a, hipStream_t s);

struct GroupRouteArgs {
    const void* logits;
    int ldtype;         // moe_dtype of logits and weights
    const float* bias;  // [E] FP32 or null
    int64_t T;
    int E, k, groups, selected, top_two, renorm;
    float scale;
    uint32_t* idx;
    void* w;
};
hipError_t launch_route_grouped(const GroupRouteArgs& a, hipStream_t s);

struct DispatchArgs {
    const void* x;
    int64_t T;
    int64_t row_bytes;  // H * element size
    int k, E;
    const uint32_t* idx;
    uint32_t* counts;   // [E] scratch
    uint32_t* rank;     // [T*k] scratch
    uint32_t* offsets;  // [E+1]
    void* dispatched;   // null: write the mapping only, copy no rows
    uint32_t* row_of_slot;
    uint32_t* token_of_row;
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

struct ExpertsArgs {
    int dtype;
    const void* gate;
    const void* up;
    const void* down;
    const void* x;  // [N,H] dispatched rows, or [x_nrows,H] rows picked by x_rows
    const uint32_t* x_rows;  // null, or token_of_row [N]: row r of the products is x[x_rows[r]]
    int64_t x_nrows;
    const uint32_t* offsets;
    void* y;        // [N,H]
    void* h;        // [N,I] workspace
    float* gu;      // null, or [N,2I] FP32: the gate/up product saves g | u (training forward)
    void* tiles;    // tile list workspace
    int64_t N, H, I;
    int E;
};
size_t experts_tile_bytes(int64_t N, int64_t E);
// which products to run: both (the whole experts stage) or one half
enum ExpertsPart { kBoth = 0, kGateUp = 1, kDown = 2 };
hipError_t launch_experts(const ExpertsArgs& a, hipStream_t s, ExpertsPart part = kBoth);

struct CombineArgs {
    const void* y;
    int dtype;
    int64_t N;  // rows of y
    const uint32_t* row_of_slot;
    const void* w;
    int wdtype;
    int64_t T;
    int k;
    int64_t H;
    void* out;
};
hipError_t launch_combine(const CombineArgs& a, hipStream_t s);

// ------------------------------------------------------------------ training
struct RouterWeightArgs {
    const void* logits;
    int ldtype;          // moe_dtype of logits (and of dlogits)
    const void* idx;     // [T,k] U32, I32 or I64
    int idx_dtype;
    const float* gw;     // [T,k] FP32 weight gradients (backward only)
    int64_t T;
    int E, k, scoring, renorm;
    float scale;
    float* w;            // [T,k] FP32 weights (forward only)
    void* dl;            // [T,E] logits gradient (backward only)
};
hipError_t launch_router_weights(const RouterWeightArgs& a, hipStream_t s);
hipError_t launch_router_backward(const RouterWeightArgs& a, hipStream_t s);

struct ExpertsBackwardArgs {
    int dtype;
    const void* gate;
    const void* up;
    const void* down;
    const void* x;           // [N,H] dispatched rows, or [x_nrows,H] token rows picked by x_rows
    const uint32_t* x_rows;  // null, or token_of_row [N]
    int64_t x_nrows;
    const uint32_t* offsets;
    const float* gu;         // [N,2I] saved g | u
    const void* h;           // [N,I] saved activation
    const void* dy;          // [N,H] expert-output gradient
    void* dx;                // [N,H] dispatched-row gradient
    float* dgate;            // [E,I,H]
    float* dup;              // [E,I,H]
    float* ddown;            // [E,H,I]
    void* dgu;               // [N,2I] workspace (weight dtype)
    void* xg;                // [N,H] workspace: token rows gathered through x_rows
    void* tiles;             // tile list workspace
    int64_t N, H, I;
    int E;
};
size_t experts_backward_tile_bytes(int64_t N, int64_t E);
hipError_t launch_experts_backward(const ExpertsBackwardArgs& a, hipStream_t s);

struct CombineBackwardArgs {
    const void* y;       // [N,H] expert outputs
    int dtype;
    int64_t N;
    const uint32_t* row_of_slot;
    const void* w;       // [T,k]
    int wdtype;
    const void* g;       // [T,H] output gradient
    int64_t T;
    int k;
    int64_t H;
    void* dy;            // [N,H]
    float* dw;           // [T,k]
};
hipError_t launch_combine_backward(const CombineBackwardArgs& a, hipStream_t s);

struct DispatchBackwardArgs {
    const void* drows;   // [N,H]
    int dtype;
    int64_t N;
    const uint32_t* row_of_slot;
    int64_t T;
    int k;
    int64_t H;
    void* dx;            // [T,H]
};
hipError_t launch_dispatch_backward(const DispatchBackwardArgs& a, hipStream_t s);

}  // namespace moe
