// router_train.hip -- router weights of a fixed selection and their logits
// gradient, one wavefront per token.
//
// Follows the RUDA ruDNN library guide, section 12 (first-order MoE
// training).  For the given [T,k] expert indices (U32, I32 or I64):
//   scores    p_e = softmax(l)_e over all E experts (FP32, max-shifted), or
//             sigmoid(l_e);
//   weights   q_j = p_{idx_j} (a repeated index is gathered again),
//             w_j = scale * q_j / S with S = sum_j q_j (FP32, slot order)
//             when renormalising, else scale * q_j; written in FP32;
//   backward  only the weights of the fixed selection are differentiated:
//             dq_j = scale (gw_j / S - sum_i gw_i q_i / S^2) (or scale gw_j),
//             dp_e = sum of dq_j over the slots with idx_j = e,
//             softmax: dl_e = p_e (dp_e - sum_j q_j dq_j);
//             sigmoid: dl_e = dp_e p_e (1 - p_e);
//             written in the logits dtype.
// An index outside [0, E) makes the token's whole row NaN, with no access
// outside the logits row.
//
// Layout: lane l holds experts l, l+64, ... of the row (as in the routing
// kernel); lane j < k holds slot j, and recomputes its score q_j from the
// logit l_{idx_j} with the wave's max and sum, so q_j is bit-identical to
// p_{idx_j}.  Slot sums are broadcast loops in slot order.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kRouterWaves = 4;  // tokens per workgroup

template <typename IT> struct index_of;
template <> struct index_of<uint32_t> {
    static __device__ __forceinline__ int64_t get(uint32_t v) { return (int64_t)v; }
};
template <> struct index_of<int32_t> {
    static __device__ __forceinline__ int64_t get(int32_t v) { return (int64_t)v; }
};
template <> struct index_of<int64_t> {
    static __device__ __forceinline__ int64_t get(int64_t v) { return v; }
};

__device__ __forceinline__ float sigmoidf(float x) { return 1.0f / (1.0f + expf(-x)); }

// The row's scores for this lane's experts, and the softmax max and sum.
template <typename LT, int EPL>
__device__ __forceinline__ void row_scores(const typename LT::storage* row, int E, int scoring, float (&v)[EPL],
                                           float (&pe)[EPL], float* mx, float* sum) {
    const int lane = lane_id();
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        const float x = fmt<LT>::load(row[min(e, E - 1)]);  // unconditional: the loads go out together
        v[i] = e < E ? x : -INFINITY;
    }
    if (scoring == 0) {
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < EPL; ++i) m = fmaxf(m, v[i]);
        m = wave_max(m);
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            pe[i] = e < E ? expf(v[i] - m) : 0.0f;
            s += pe[i];
        }
        s = wave_sum(s);
#pragma unroll
        for (int i = 0; i < EPL; ++i) pe[i] = pe[i] / s;
        *mx = m;
        *sum = s;
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) pe[i] = sigmoidf(v[i]);
        *mx = 0.0f;
        *sum = 1.0f;
    }
}

// Score of slot lane's expert (lane < k, index valid), as row_scores gives it.
template <typename LT>
__device__ __forceinline__ float slot_score(const typename LT::storage* row, int64_t e, int scoring, float m, float s) {
    const float x = fmt<LT>::load(row[e]);
    return scoring == 0 ? expf(x - m) / s : sigmoidf(x);
}

template <typename LT, typename IT, int EPL>
__global__ __launch_bounds__(kRouterWaves* kWave) void router_weights_kernel(
    const typename LT::storage* __restrict__ logits, const IT* __restrict__ idx, int64_t T, int E, int k,
    int scoring, int renorm, float scale, float* __restrict__ w) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * kRouterWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const typename LT::storage* row = logits + t * (int64_t)E;
    const int64_t my_e = lane < k ? index_of<IT>::get(idx[t * k + lane]) : 0;
    if (__any(lane < k && (my_e < 0 || my_e >= E))) {
        if (lane < k) w[t * k + lane] = __uint_as_float(0x7fc00000u);
        return;
    }
    float v[EPL], pe[EPL], m, s;
    row_scores<LT, EPL>(row, E, scoring, v, pe, &m, &s);
    const float q = lane < k ? slot_score<LT>(row, my_e, scoring, m, s) : 0.0f;
    float S = 0.0f;
    for (int j = 0; j < k; ++j) S += __shfl(q, j, kWave);
    if (lane < k) w[t * k + lane] = (renorm ? q / S : q) * scale;
}

template <typename LT, typename IT, int EPL>
__global__ __launch_bounds__(kRouterWaves* kWave) void router_backward_kernel(
    const typename LT::storage* __restrict__ logits, const IT* __restrict__ idx, const float* __restrict__ gw,
    int64_t T, int E, int k, int scoring, int renorm, float scale, typename LT::storage* __restrict__ dl) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * kRouterWaves + threadIdx.x / kWave;
    if (t >= T) return;
    const typename LT::storage* row = logits + t * (int64_t)E;
    typename LT::storage* drow = dl + t * (int64_t)E;
    const int64_t my_e = lane < k ? index_of<IT>::get(idx[t * k + lane]) : 0;
    if (__any(lane < k && (my_e < 0 || my_e >= E))) {
        for (int e = lane; e < E; e += kWave) drow[e] = fmt<LT>::store(__uint_as_float(0x7fc00000u));
        return;
    }
    float v[EPL], pe[EPL], m, s;
    row_scores<LT, EPL>(row, E, scoring, v, pe, &m, &s);
    const float q = lane < k ? slot_score<LT>(row, my_e, scoring, m, s) : 0.0f;
    const float g = lane < k ? gw[t * k + lane] : 0.0f;
    float S = 0.0f, dot = 0.0f;
    for (int j = 0; j < k; ++j) {
        S += __shfl(q, j, kWave);
        dot += __shfl(g, j, kWave) * __shfl(q, j, kWave);
    }
    const float dq = renorm ? scale * (g / S - dot / (S * S)) : scale * g;
    float dp[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) dp[i] = 0.0f;
    float mdot = 0.0f;  // sum_j q_j dq_j = sum_e p_e dp_e
    for (int j = 0; j < k; ++j) {
        const int ej = __shfl((int)my_e, j, kWave);
        const float dqj = __shfl(dq, j, kWave);
        mdot += __shfl(q, j, kWave) * dqj;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane + kWave * i == ej) dp[i] += dqj;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        if (e < E) {
            const float d = scoring == 0 ? pe[i] * (dp[i] - mdot) : dp[i] * pe[i] * (1.0f - pe[i]);
            drow[e] = fmt<LT>::store(d);
        }
    }
}

template <typename LT, typename IT, bool BACKWARD>
hipError_t launch_typed(const RouterWeightArgs& a, hipStream_t s) {
    using S = typename LT::storage;
    const dim3 grid((unsigned)((a.T + kRouterWaves - 1) / kRouterWaves)), block(kRouterWaves * kWave);
    const S* lg = (const S*)a.logits;
    const IT* ix = (const IT*)a.idx;
    const int epl = (a.E + kWave - 1) / kWave;
#define MOE_RW_CASE(N)                                                                                     \
    if (epl <= N) {                                                                                        \
        if (BACKWARD)                                                                                      \
            router_backward_kernel<LT, IT, N><<<grid, block, 0, s>>>(lg, ix, a.gw, a.T, a.E, a.k, a.scoring, \
                                                                    a.renorm, a.scale, (S*)a.dl);          \
        else                                                                                               \
            router_weights_kernel<LT, IT, N><<<grid, block, 0, s>>>(lg, ix, a.T, a.E, a.k, a.scoring,       \
                                                                   a.renorm, a.scale, a.w);                \
        return hipGetLastError();                                                                          \
    }
    MOE_RW_CASE(1)
    MOE_RW_CASE(2)
    MOE_RW_CASE(4)
    MOE_RW_CASE(8)
    MOE_RW_CASE(16)
    MOE_RW_CASE(32)
    MOE_RW_CASE(64)
#undef MOE_RW_CASE
    return hipErrorInvalidValue;
}

template <typename LT, bool BACKWARD>
hipError_t launch_idx(const RouterWeightArgs& a, hipStream_t s) {
    switch (a.idx_dtype) {
    case MOE_U32: return launch_typed<LT, uint32_t, BACKWARD>(a, s);
    case MOE_I32: return launch_typed<LT, int32_t, BACKWARD>(a, s);
    case MOE_I64: return launch_typed<LT, int64_t, BACKWARD>(a, s);
    default: return hipErrorInvalidValue;
    }
}

template <bool BACKWARD>
hipError_t launch_router(const RouterWeightArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    // the kernels keep one slot per lane
    if (a.k < 1 || a.k > kWave || a.k > a.E || a.E > kWave * 64) return hipErrorInvalidValue;
    if ((a.T + kRouterWaves - 1) / kRouterWaves > 0x7fffffff) return hipErrorInvalidValue;
    switch (a.ldtype) {
    case MOE_F32: return launch_idx<f32_t, BACKWARD>(a, s);
    case MOE_F16: return launch_idx<f16_t, BACKWARD>(a, s);
    case MOE_BF16: return launch_idx<bf16_t, BACKWARD>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_router_weights(const RouterWeightArgs& a, hipStream_t s) { return launch_router<false>(a, s); }
hipError_t launch_router_backward(const RouterWeightArgs& a, hipStream_t s) { return launch_router<true>(a, s); }

}  // namespace moe
