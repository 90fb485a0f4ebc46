// route_grouped.hip -- group-limited sigmoid routing, one wavefront per token.
//
// Follows the ruDNN user guide, section 10 (group-limited sigmoid MoE
// routing).  Per token:
//   1. s_e = sigmoid(l_e) in FP32; the corrected score c_e = s_e + bias_e
//      steers the selection only;
//   2. the E experts form G contiguous groups of E/G; a group scores its
//      largest corrected score, or the sum of its two largest;
//   3. the best `selected` groups are kept, ties to the lower group id;
//   4. the top_k experts of the kept groups by corrected score, ties to the
//      lower expert id, in slot order of decreasing score;
//   5. the weights are the uncorrected s of the chosen experts, optionally
//      divided by their FP32 sum (slot order), times `scale`, rounded once
//      to the logits dtype.
// A row with a NaN corrected score (a NaN logit or bias) has no order: it
// gets experts 0..k-1 and NaN weights, as the softmax routing does.
//
// Layout: lane l holds experts l, l+64, ...; the row's scores also go to
// LDS so one lane can scan a whole group (lane g scores groups g and
// g+64).  Group and expert choices are rounds of a wave arg-max over the
// 64-bit key (order-preserving bits of the score << 32 | ~id).
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kGroupedWaves = 4;  // tokens per workgroup

// Unsigned image of a non-NaN float that orders like the float (-0 and +0
// are made equal by the caller adding +0).
__device__ __forceinline__ uint32_t ordered_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <typename LT, int EPL>
__global__ __launch_bounds__(kGroupedWaves* kWave) void route_grouped_kernel(
    const typename LT::storage* __restrict__ logits, const float* __restrict__ bias, int64_t T, int E, int k,
    int G, int selected, int top_two, int renorm, float scale, uint32_t* __restrict__ idx,
    typename LT::storage* __restrict__ w) {
    __shared__ float corr_lds[kGroupedWaves][64 * EPL];
    __shared__ float sig_lds[kGroupedWaves][64 * EPL];
    const int lane = lane_id(), wv = threadIdx.x / kWave;
    const int64_t t = (int64_t)blockIdx.x * kGroupedWaves + wv;
    if (t >= T) return;  // no workgroup barrier below: a wave may leave
    float* cs = corr_lds[wv];
    float* ss = sig_lds[wv];
    const typename LT::storage* row = logits + t * (int64_t)E;

    float c[EPL];
    bool nan_seen = false;
    // the lane's logits and biases, loaded unconditionally (lanes past E
    // re-read the last expert's) so that the loads go out together
    float xs[EPL], bs[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int ec = min(lane + kWave * i, E - 1);
        xs[i] = fmt<LT>::load(row[ec]);
        bs[i] = bias ? bias[ec] : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        c[i] = 0.0f;
        if (e < E) {
            const float x = xs[i];
            const float s = 1.0f / (1.0f + expf(-x));
            c[i] = (s + bs[i]) + 0.0f;  // + 0 turns -0 into +0
            nan_seen |= (c[i] != c[i]);
            cs[e] = c[i];
            ss[e] = s;
        }
    }
    if (__any(nan_seen)) {
        if (lane < k) {
            idx[t * k + lane] = (uint32_t)lane;
            w[t * k + lane] = fmt<LT>::store(__uint_as_float(0x7fc00000u));
        }
        return;
    }
    // the scores written above are read by other lanes of this wave: wait
    // for the LDS writes, and keep the compiler from moving reads above them
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_wave_barrier();

    // group scores: lane l owns groups l and l + 64
    const int gsz = E / G;
    uint64_t gkey[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int g = lane + kWave * h;
        gkey[h] = 0;
        if (g < G) {
            float a = -INFINITY, b = -INFINITY;
            for (int e = g * gsz; e < (g + 1) * gsz; ++e) {
                const float v = cs[e];
                if (v > a) {
                    b = a;
                    a = v;
                } else if (v > b) {
                    b = v;
                }
            }
            const float score = (top_two ? a + b : a) + 0.0f;
            gkey[h] = ((uint64_t)ordered_bits(score) << 32) | (uint32_t)(~(uint32_t)g);
        }
    }
    // the `selected` best groups, as a 128-bit mask every lane holds
    uint64_t gmask[2] = {0, 0};
    for (int r = 0; r < selected; ++r) {
        const uint64_t best = wave_max_u64(gkey[0] > gkey[1] ? gkey[0] : gkey[1]);
        const uint32_t gb = ~(uint32_t)best;
        gmask[gb >> 6] |= 1ull << (gb & 63);
        if ((int)(gb & 63) == lane) gkey[gb >> 6] = 0;
    }

    // top_k experts of the kept groups
    uint64_t ekey[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        ekey[i] = 0;
        if (e < E) {
            const int g = e / gsz;
            if ((gmask[g >> 6] >> (g & 63)) & 1ull)
                ekey[i] = ((uint64_t)ordered_bits(c[i]) << 32) | (uint32_t)(~(uint32_t)e);
        }
    }
    uint32_t my_e = 0;
    float my_s = 0.0f, R = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = ekey[i] > best ? ekey[i] : best;
        best = wave_max_u64(best);
        const uint32_t eb = ~(uint32_t)best;
        if ((int)(eb & (kWave - 1)) == lane) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if (i == (int)(eb / kWave)) ekey[i] = 0;
        }
        const float sb = ss[eb];  // the uncorrected score of the pick
        R += sb;                  // FP32 sum in slot order
        if (j == lane) {
            my_e = eb;
            my_s = sb;
        }
    }
    if (lane < k) {
        float wj = my_s;
        if (renorm) wj = wj / R;
        wj = wj * scale;
        idx[t * k + lane] = my_e;
        w[t * k + lane] = fmt<LT>::store(wj);
    }
}

template <typename LT>
hipError_t launch_typed(const GroupRouteArgs& a, hipStream_t s) {
    using S = typename LT::storage;
    const dim3 grid((unsigned)((a.T + kGroupedWaves - 1) / kGroupedWaves)), block(kGroupedWaves * kWave);
    const S* lg = (const S*)a.logits;
    S* w = (S*)a.w;
    const int epl = (a.E + kWave - 1) / kWave;
#define MOE_GROUPED_CASE(N)                                                                              \
    if (epl <= N) {                                                                                      \
        route_grouped_kernel<LT, N><<<grid, block, 0, s>>>(lg, a.bias, a.T, a.E, a.k, a.groups, a.selected, \
                                                           a.top_two, a.renorm, a.scale, a.idx, w);      \
        return hipGetLastError();                                                                        \
    }
    MOE_GROUPED_CASE(1)
    MOE_GROUPED_CASE(2)
    MOE_GROUPED_CASE(4)
    MOE_GROUPED_CASE(8)
    MOE_GROUPED_CASE(16)
#undef MOE_GROUPED_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_route_grouped(const GroupRouteArgs& a, hipStream_t s) {
    if (a.T == 0) return hipSuccess;
    // the host checks these; the kernel's rounds rely on them to always find
    // a group and an expert to pick
    if (a.E < 1 || a.E > 1024 || a.groups < 1 || a.groups > 128 || a.E % a.groups || a.k < 1 || a.k > 64 ||
        a.selected < 1 || a.selected > a.groups || (int64_t)a.k > (int64_t)a.selected * (a.E / a.groups))
        return hipErrorInvalidValue;
    switch (a.ldtype) {
    case MOE_F32: return launch_typed<f32_t>(a, s);
    case MOE_F16: return launch_typed<f16_t>(a, s);
    case MOE_BF16: return launch_typed<bf16_t>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
