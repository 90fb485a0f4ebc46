// route.hip -- softmax + top-k routing, one wavefront per token.
//
// Follows the ruDNN User Guide, section 4 "Routing contract": the logits row
// is widened to FP32, softmax runs over all E experts, the top_k largest
// probabilities are selected with ties going to the lower expert id, the
// selected weights are optionally renormalised by their FP32 sum and then
// rounded to the logits dtype.  A row with a NaN or +inf, or with only -inf,
// keeps NaN weights; its indices are 0..k-1 (the order that the tie rule
// gives when no probability compares larger than another).
//
// Layout: lane l holds experts l, l+64, ..., so each load of the row is a
// coalesced 64-wide read.  Max and sum are butterfly reductions over the
// wave; top-k is k rounds of a wave arg-max over the 64-bit key
// (probability bits << 32 | ~expert id): probabilities are >= 0, so their
// bit patterns order like their values, and the complemented id makes the
// lower id win among equal probabilities.
#include "moe_internal.h"

namespace moe {
namespace {

template <typename LT, int EPL>
__global__ __launch_bounds__(256) void route_kernel(const typename LT::storage* __restrict__ logits,
                                                    int64_t T, int E, int k, int renorm,
                                                    uint32_t* __restrict__ idx,
                                                    typename LT::storage* __restrict__ w) {
    const int lane = lane_id();
    const int64_t t = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
    if (t >= T) return;
    const typename LT::storage* row = logits + t * (int64_t)E;

    float v[EPL];
    bool nan_or_pinf = false, finite_or_pinf = false;
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        // loaded unconditionally (lanes past E re-read the last logit), so
        // that the lane's loads go out together
        const float x = fmt<LT>::load(row[min(e, E - 1)]);
        v[i] = (e < E) ? x : -INFINITY;
        if (e < E) {
            nan_or_pinf |= (v[i] != v[i]) || (v[i] == INFINITY);
            finite_or_pinf |= (v[i] != -INFINITY);
        }
        m = fmaxf(m, v[i]);
    }
    const bool nan_row = __any(nan_or_pinf) || !__any(finite_or_pinf);

    // selections: lane (j % 64) keeps slot j in register (j / 64)
    uint32_t sel_e[EPL];
    float sel_p[EPL];
    float R = 0.0f;
    if (nan_row) {
#pragma unroll
        for (int c = 0; c < EPL; ++c) {
            sel_e[c] = (uint32_t)(c * kWave + lane);
            sel_p[c] = __uint_as_float(0x7fc00000u);
        }
        R = 1.0f;
    } else {
        m = wave_max(m);
        float q[EPL];
        float s = 0.0f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + kWave * i;
            q[i] = (e < E) ? expf(v[i] - m) : 0.0f;
            s += q[i];
        }
        s = wave_sum(s);
        uint64_t taken = 0;  // bit i: expert lane + 64 i already selected
#pragma unroll
        for (int i = 0; i < EPL; ++i) q[i] = q[i] / s;
#pragma unroll
        for (int c = 0; c < EPL; ++c) { sel_e[c] = 0; sel_p[c] = 0.0f; }
        for (int j = 0; j < k; ++j) {
            uint64_t best = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane + kWave * i;
                const bool ok = (e < E) && !((taken >> i) & 1ull);
                const uint64_t key = ((uint64_t)__float_as_uint(q[i]) << 32) | (uint32_t)(~(uint32_t)e);
                if (ok && key > best) best = key;
            }
            best = wave_max_u64(best);
            const uint32_t eb = ~(uint32_t)best;
            const float pb = __uint_as_float((uint32_t)(best >> 32));
            if ((int)(eb & (kWave - 1)) == lane) taken |= 1ull << (eb / kWave);
            R += pb;  // FP32 sum of the selected probabilities, in slot order
#pragma unroll
            for (int c = 0; c < EPL; ++c) {
                if (j == c * kWave + lane) {
                    sel_e[c] = eb;
                    sel_p[c] = pb;
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < EPL; ++c) {
        const int j = c * kWave + lane;
        if (j < k) {
            float wj = sel_p[c];
            if (renorm) wj = wj / R;
            idx[t * k + j] = sel_e[c];
            w[t * k + j] = fmt<LT>::store(wj);
        }
    }
}

template <typename LT>
hipError_t launch_typed(const RouteArgs& a, hipStream_t s) {
    using S = typename LT::storage;
    const int wpb = 4;
    const dim3 grid((unsigned)((a.T + wpb - 1) / wpb)), block(wpb * kWave);
    const S* lg = (const S*)a.logits;
    S* w = (S*)a.w;
    const int epl = (a.E + kWave - 1) / kWave;
#define MOE_ROUTE_CASE(N)                                                                      \
    if (epl <= N) {                                                                            \
        route_kernel<LT, N><<<grid, block, 0, s>>>(lg, a.T, a.E, a.k, a.renorm, a.idx, w);     \
        return hipGetLastError();                                                              \
    }
    MOE_ROUTE_CASE(1)
    MOE_ROUTE_CASE(2)
    MOE_ROUTE_CASE(4)
    MOE_ROUTE_CASE(8)
    MOE_ROUTE_CASE(16)
    MOE_ROUTE_CASE(32)
    MOE_ROUTE_CASE(64)
#undef MOE_ROUTE_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    switch (a.ldtype) {
    case MOE_F32: return launch_typed<f32_t>(a, s);
    case MOE_F16: return launch_typed<f16_t>(a, s);
    case MOE_BF16: return launch_typed<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
