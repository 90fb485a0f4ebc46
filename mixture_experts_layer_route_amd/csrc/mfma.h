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
        w.x = (uint32_t)fmt<DT>::store(v[0]) | ((uint32_t)fmt<DT>::store(v[1]) << 16);
        w.y = (uint32_t)fmt<DT>::store(v[2]) | ((uint32_t)fmt<DT>::store(v[3]) << 16);
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

}  // namespace moe
