// combine.hip -- weighted combine back into token order.
//
// Follows the ruDNN User Guide, sections 5 and 6: the saved mapping restores
// token order and the expert outputs are merged with the routing weights.
// out[t] = sum_{j<k} w[t,j] * Y[row_of_slot[t*k+j]] in FP32, slots added in
// fixed order j = 0..k-1 (so the result never depends on the row order the
// dispatch atomics produced), rounded once to the output dtype.  A slot whose
// row is out of range (an expert id >= E at dispatch) makes the whole output
// row NaN, with no out-of-bounds access.
//
// One wavefront per token; each lane owns VEC consecutive columns, so every
// row of Y is read with wide coalesced loads.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename DT, typename WT, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const typename DT::storage* __restrict__ Y, int64_t N,
                                                      const uint32_t* __restrict__ row_of_slot,
                                                      const typename WT::storage* __restrict__ w,
                                                      int64_t T, int k, int64_t H,
                                                      typename DT::storage* __restrict__ out) {
    using S = typename DT::storage;
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    bool bad = false;
    for (int j = lane; j < k; j += kWave) bad |= (int64_t)row_of_slot[t * k + j] >= N;
    const bool nan_row = __any(bad);
    S* o = out + t * H;
    for (int64_t c0 = (int64_t)lane * VEC; c0 < H; c0 += (int64_t)kWave * VEC) {
        float acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
        if (!nan_row) {
            for (int j = 0; j < k; ++j) {
                const uint32_t r = row_of_slot[t * k + j];  // wave-uniform, cached
                const float wj = fmt<WT>::load(w[t * k + j]);
                const S* yr = Y + (int64_t)r * H + c0;
                S vals[VEC];
                if constexpr (VEC * sizeof(S) == 16) {
                    *(uint4*)vals = *(const uint4*)yr;
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) vals[v] = yr[v];
                }
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = fmaf(wj, fmt<DT>::load(vals[v]), acc[v]);
            }
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) acc[v] = __uint_as_float(0x7fc00000u);
        }
        S res[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) res[v] = fmt<DT>::store(acc[v]);
        if constexpr (VEC * sizeof(S) == 16) {
            *(uint4*)(o + c0) = *(const uint4*)res;
        } else {
#pragma unroll
            for (int v = 0; v < VEC; ++v) o[c0 + v] = res[v];
        }
    }
}

template <typename DT, typename WT>
hipError_t launch_typed(const CombineArgs& a, hipStream_t s) {
    using S = typename DT::storage;
    using W = typename WT::storage;
    const int wpb = 4;
    const dim3 grid((unsigned)((a.T + wpb - 1) / wpb)), block(wpb * kWave);
    constexpr int V16 = 16 / sizeof(S);
    const uintptr_t al = (uintptr_t)a.y | (uintptr_t)a.out;
    if (a.H % V16 == 0 && al % 16 == 0)
        combine_kernel<DT, WT, V16><<<grid, block, 0, s>>>((const S*)a.y, a.N, a.row_of_slot, (const W*)a.w,
                                                           a.T, a.k, a.H, (S*)a.out);
    else
        combine_kernel<DT, WT, 1><<<grid, block, 0, s>>>((const S*)a.y, a.N, a.row_of_slot, (const W*)a.w,
                                                         a.T, a.k, a.H, (S*)a.out);
    return hipGetLastError();
}

template <typename DT>
hipError_t launch_w(const CombineArgs& a, hipStream_t s) {
    switch (a.wdtype) {
    case MOE_F32: return launch_typed<DT, f32_t>(a, s);
    case MOE_F16: return launch_typed<DT, f16_t>(a, s);
    case MOE_BF16: return launch_typed<DT, bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_combine(const CombineArgs& a, hipStream_t s) {
    if (a.T == 0 || a.H == 0) return hipSuccess;
    switch (a.dtype) {
    case MOE_F32: return launch_w<f32_t>(a, s);
    case MOE_F16: return launch_w<f16_t>(a, s);
    case MOE_BF16: return launch_w<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
