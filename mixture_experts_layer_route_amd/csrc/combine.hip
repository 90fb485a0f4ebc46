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
// Each thread owns VEC consecutive columns of one token, so every row of Y is
// read with wide coalesced loads.  Each row of Y is read once and each output
// row written once, so the 16-byte accesses carry the non-temporal hint
// (15% faster on 235 MB of rows than plain loads and stores).
#include "moe_internal.h"

namespace moe {
namespace {

// grid (tokens, column chunks): thread -> VEC consecutive columns of one
// token.  The token's k rows and weights are wave-uniform; they and the k row
// loads are issued in batches of 8 before their multiply-adds, so the loads
// of one thread overlap instead of forming a chain of round trips.
template <typename DT, typename WT, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const typename DT::storage* __restrict__ Y, int64_t N,
                                                      const uint32_t* __restrict__ row_of_slot,
                                                      const typename WT::storage* __restrict__ w,
                                                      int k, int64_t H,
                                                      typename DT::storage* __restrict__ out) {
    using S = typename DT::storage;
    const int64_t t = blockIdx.x;
    const int64_t c0 = ((int64_t)blockIdx.y * blockDim.x + threadIdx.x) * VEC;
    if (c0 >= H) return;
    const uint32_t* rs = row_of_slot + t * k;
    const typename WT::storage* ws = w + t * k;
    float acc[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] = 0.0f;
    bool nan_row = false;
    constexpr int B = 8;
    for (int j0 = 0; j0 < k; j0 += B) {
        // the batch's rows and weights, loaded unconditionally (slots past
        // k re-read the last one) so that the loads go out together
        uint32_t r[B];
        float wj[B];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            const int j = min(j0 + b, k - 1);
            r[b] = rs[j];
            wj[b] = fmt<WT>::load(ws[j]);
        }
#pragma unroll
        for (int b = 0; b < B; ++b) nan_row |= j0 + b < k && (int64_t)r[b] >= N;
        if (nan_row) break;
        S vals[B][VEC];
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b < k) {
                const S* yr = Y + (int64_t)r[b] * H + c0;
                if constexpr (VEC * sizeof(S) == 16) {
                    *(uint4*)vals[b] = load_nt16(yr);
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) vals[b][v] = yr[v];
                }
            }
        }
#pragma unroll
        for (int b = 0; b < B; ++b) {
            if (j0 + b < k) {  // slots in fixed order j = 0..k-1
#pragma unroll
                for (int v = 0; v < VEC; ++v) acc[v] = fmaf(wj[b], fmt<DT>::load(vals[b][v]), acc[v]);
            }
        }
    }
    if (nan_row) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) acc[v] = __uint_as_float(0x7fc00000u);
    }
    S res[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) res[v] = fmt<DT>::store(acc[v]);
    S* o = out + t * H + c0;
    if constexpr (VEC * sizeof(S) == 16) {
        store_nt16(o, *(const uint4*)res);
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v) o[v] = res[v];
    }
}

template <typename DT, typename WT>
hipError_t launch_typed(const CombineArgs& a, hipStream_t s) {
    using S = typename DT::storage;
    using W = typename WT::storage;
    constexpr int V16 = 16 / sizeof(S);
    const uintptr_t al = (uintptr_t)a.y | (uintptr_t)a.out;
    const bool wide = a.H % V16 == 0 && al % 16 == 0;
    const int64_t chunks = ((wide ? a.H / V16 : a.H) + 255) / 256;
    if (a.T > 0x7fffffff || chunks > 65535) return hipErrorInvalidValue;
    const dim3 block(256);
    if (wide) {
        const dim3 grid((unsigned)a.T, (unsigned)chunks);
        combine_kernel<DT, WT, V16><<<grid, block, 0, s>>>((const S*)a.y, a.N, a.row_of_slot, (const W*)a.w,
                                                           a.k, a.H, (S*)a.out);
    } else {
        const dim3 grid((unsigned)a.T, (unsigned)chunks);
        combine_kernel<DT, WT, 1><<<grid, block, 0, s>>>((const S*)a.y, a.N, a.row_of_slot, (const W*)a.w,
                                                         a.k, a.H, (S*)a.out);
    }
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
