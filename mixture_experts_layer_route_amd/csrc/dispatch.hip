// dispatch.hip -- compact, drop-free dispatch of tokens by expert.
//
// Follows the ruDNN User Guide, section 5 "Expert weights and dispatch":
// every selected (token, slot) pair gets its own row (no capacity drop),
// rows are grouped by expert, the order inside an expert comes from atomics
// and is not fixed, and a saved mapping (row_of_slot / token_of_row) lets the
// combine restore token order.
//
// Three kernels:
//   hist    -- per-workgroup LDS histogram; the LDS atomic returns each slot's
//              rank inside its workgroup, and one global atomic per
//              (workgroup, expert) reserves that workgroup's base, so
//              rank_in_expert = base + local rank.
//   scan    -- one workgroup: exclusive prefix sum of the counts, ascending
//              expert id, into offsets[E+1].
//   gather  -- one thread per (token, 16-byte unit): the unit is read once
//              and written to each of the token's k dispatched rows.
// When only the mapping is asked for and the batch has at most
// kSmallDispatchSlots slots, one workgroup does all of it instead (LDS
// histogram, scan, mapping): one launch instead of four, which at decode
// sizes, where each launch is a few microseconds of latency, is most of the
// dispatch's time.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kHistThreads = 256;
constexpr int kHistSlotsPerThread = 8;

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t v) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = v;
}

__global__ __launch_bounds__(kHistThreads) void hist_kernel(const uint32_t* __restrict__ idx, int64_t N,
                                                            int E, uint32_t* __restrict__ counts,
                                                            uint32_t* __restrict__ rank) {
    extern __shared__ uint32_t h[];  // [E]
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kHistThreads * kHistSlotsPerThread;
    uint32_t ex[kHistSlotsPerThread], loc[kHistSlotsPerThread];
#pragma unroll
    for (int i = 0; i < kHistSlotsPerThread; ++i) {
        const int64_t s = base + (int64_t)i * kHistThreads + threadIdx.x;
        ex[i] = (s < N) ? idx[s] : kInvalidRow;
        loc[i] = 0;
        if (ex[i] < (uint32_t)E) loc[i] = atomicAdd(&h[ex[i]], 1u);
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const uint32_t c = h[e];
        if (c) h[e] = atomicAdd(&counts[e], c);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kHistSlotsPerThread; ++i) {
        const int64_t s = base + (int64_t)i * kHistThreads + threadIdx.x;
        if (s < N) rank[s] = (ex[i] < (uint32_t)E) ? h[ex[i]] + loc[i] : kInvalidRow;
    }
}

// exclusive scan of the block's values; 1024 threads (16 waves)
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* total) {
    __shared__ uint32_t wsum[16];
    const int lane = lane_id(), wid = threadIdx.x / kWave;
    const uint32_t inc = wave_inclusive_scan(v);
    if (lane == kWave - 1) wsum[wid] = inc;
    __syncthreads();
    if (wid == 0) {
        const int nw = blockDim.x / kWave;
        uint32_t s = (lane < nw) ? wsum[lane] : 0u;
        s = wave_inclusive_scan(s);
        if (lane < nw) wsum[lane] = s;
    }
    __syncthreads();
    const uint32_t prefix = wid ? wsum[wid - 1] : 0u;
    *total = wsum[blockDim.x / kWave - 1];
    __syncthreads();
    return prefix + inc - v;
}

__global__ __launch_bounds__(1024) void scan_kernel(const uint32_t* __restrict__ counts, int E,
                                                    uint32_t* __restrict__ offsets) {
    const int per = (E + blockDim.x - 1) / blockDim.x;  // contiguous experts per thread
    const int e0 = threadIdx.x * per;
    uint32_t local = 0;
    for (int i = 0; i < per; ++i)
        if (e0 + i < E) local += counts[e0 + i];
    uint32_t total;
    uint32_t run = block_exclusive_scan(local, &total);
    for (int i = 0; i < per; ++i) {
        if (e0 + i < E) {
            offsets[e0 + i] = run;
            run += counts[e0 + i];
        }
    }
    if (threadIdx.x == 0) offsets[E] = total;
}

// V: copy unit (uint4 = 16 bytes when rows allow it, else 4 or 2 bytes).
// grid (tokens, unit chunks): each thread reads one unit of its token once
// and writes it to the token's k dispatched rows; the first chunk's threads
// also record the mapping.
template <typename V>
__global__ __launch_bounds__(256) void gather_kernel(const V* __restrict__ x, int64_t row_units, int k, int E,
                                                     const uint32_t* __restrict__ idx,
                                                     const uint32_t* __restrict__ rank,
                                                     const uint32_t* __restrict__ offsets,
                                                     V* __restrict__ dispatched,
                                                     uint32_t* __restrict__ row_of_slot,
                                                     uint32_t* __restrict__ token_of_row) {
    const int64_t t = blockIdx.x;
    const uint32_t* it = idx + t * k;
    const uint32_t* rt = rank + t * k;
    if (blockIdx.y == 0) {
        for (int j = threadIdx.x; j < k; j += blockDim.x) {
            const uint32_t e = it[j];
            uint32_t row = kInvalidRow;
            if (e < (uint32_t)E) {
                row = offsets[e] + rt[j];
                token_of_row[row] = (uint32_t)t;
            }
            row_of_slot[t * k + j] = row;
        }
    }
    const int64_t u = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
    if (u >= row_units) return;
    const V val = x[t * row_units + u];
    for (int j = 0; j < k; ++j) {
        const uint32_t e = it[j];  // wave-uniform
        if (e < (uint32_t)E) dispatched[(int64_t)(offsets[e] + rt[j]) * row_units + u] = val;
    }
}

// The mapping-only dispatch of a batch of at most kSmallDispatchSlots slots
// in one workgroup of 1024 threads.  Thread t owns slots i * 1024 + t; it
// loads all of their expert ids first (one round of memory latency), then
// takes each slot's rank inside its expert from the LDS atomic that counts it
// (order inside an expert comes from atomics, as in hist_kernel) and keeps
// expert and rank packed in one register: expert in the low kSmallExpertBits
// bits, rank above them (rank < 16384, expert < 4096).  The counts are scanned
// in ascending expert id into offsets[E+1]; then row = offsets[e] + rank.  A
// slot whose index is >= E gets kInvalidRow and no row.  Past 16384 slots
// the one CU's LDS atomics take longer than the four launches of the general
// path (49152 slots: 31 us against 19 us).
constexpr int kSmallDispatchSlots = 16384;
constexpr int kSmallPer = kSmallDispatchSlots / 1024;
constexpr int kSmallExpertBits = 12;
constexpr int kMaxDispatchExperts = 1 << kSmallExpertBits;

__global__ __launch_bounds__(1024) void dispatch_small_kernel(const uint32_t* __restrict__ idx, int N, int k,
                                                              int E, uint32_t* __restrict__ offsets,
                                                              uint32_t* __restrict__ row_of_slot,
                                                              uint32_t* __restrict__ token_of_row) {
    __shared__ uint32_t cnt[kMaxDispatchExperts];
    for (int e = threadIdx.x; e < E; e += blockDim.x) cnt[e] = 0;
    uint32_t st[kSmallPer];
#pragma unroll
    for (int i = 0; i < kSmallPer; ++i) {
        const int sl = i * 1024 + (int)threadIdx.x;
        st[i] = sl < N ? idx[sl] : kInvalidRow;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSmallPer; ++i)
        if (i * 1024 < N)  // uniform
            st[i] = st[i] < (uint32_t)E ? st[i] | (atomicAdd(&cnt[st[i]], 1u) << kSmallExpertBits) : kInvalidRow;
    __syncthreads();
    // exclusive scan, each thread over a contiguous run of experts
    const int per = (E + 1023) / 1024, e0 = (int)threadIdx.x * per;
    uint32_t local = 0;
    for (int j = 0; j < per; ++j)
        if (e0 + j < E) local += cnt[e0 + j];
    uint32_t total;
    uint32_t run = block_exclusive_scan(local, &total);
    for (int j = 0; j < per; ++j) {
        if (e0 + j < E) {
            const uint32_t c = cnt[e0 + j];
            cnt[e0 + j] = run;
            offsets[e0 + j] = run;
            run += c;
        }
    }
    if (threadIdx.x == 0) offsets[E] = total;
    __syncthreads();
    // token of slot i * 1024 + t, stepped by 1024 = qs * k + rs
    const uint32_t qs = 1024u / (uint32_t)k, rs = 1024u % (uint32_t)k;
    uint32_t tok = threadIdx.x / (uint32_t)k, rem = threadIdx.x % (uint32_t)k;
    constexpr uint32_t kExpertMask = (1u << kSmallExpertBits) - 1;
    // the slot offsets are recomputed here rather than kept live from the
    // loads, which would take one register per slot
    int t3 = (int)threadIdx.x;
    asm volatile("" : "+v"(t3));
#pragma unroll
    for (int i = 0; i < kSmallPer; ++i) {
        const int sl = i * 1024 + t3;
        if (sl < N) {
            uint32_t row = kInvalidRow;
            if (st[i] != kInvalidRow) {
                row = cnt[st[i] & kExpertMask] + (st[i] >> kSmallExpertBits);
                token_of_row[row] = tok;
            }
            row_of_slot[sl] = row;
        }
        tok += qs;
        rem += rs;
        if (rem >= (uint32_t)k) {
            rem -= (uint32_t)k;
            ++tok;
        }
    }
}

template <typename V>
hipError_t launch_gather(const DispatchArgs& a, hipStream_t s) {
    const int64_t units = a.dispatched ? a.row_bytes / (int64_t)sizeof(V) : 0;
    const int64_t chunks = (units + 255) / 256;
    if (a.T > 0x7fffffff || chunks > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.T, (unsigned)(chunks > 0 ? chunks : 1)), block(256);
    gather_kernel<V><<<grid, block, 0, s>>>((const V*)a.x, units, a.k, a.E, a.idx, a.rank, a.offsets,
                                            (V*)a.dispatched, a.row_of_slot, a.token_of_row);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
    hipError_t err;
    const int64_t slots = a.T * (int64_t)a.k;
    if (!a.dispatched && slots <= kSmallDispatchSlots && a.E <= kMaxDispatchExperts) {
        dispatch_small_kernel<<<1, 1024, 0, s>>>(a.idx, (int)slots, a.k, a.E, a.offsets, a.row_of_slot,
                                                 a.token_of_row);
        return hipGetLastError();
    }
    fill_u32_kernel<<<(a.E + 255) / 256, 256, 0, s>>>(a.counts, a.E, 0u);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    const int64_t N = a.T * (int64_t)a.k;
    if (N > 0) {
        const int64_t per_block = (int64_t)kHistThreads * kHistSlotsPerThread;
        hist_kernel<<<(unsigned)((N + per_block - 1) / per_block), kHistThreads, a.E * sizeof(uint32_t), s>>>(
            a.idx, N, a.E, a.counts, a.rank);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    scan_kernel<<<1, 1024, 0, s>>>(a.counts, a.E, a.offsets);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if (a.T == 0) return hipSuccess;
    const uintptr_t al = (uintptr_t)a.x | (uintptr_t)a.dispatched;
    if (a.row_bytes % 16 == 0 && al % 16 == 0) return launch_gather<uint4>(a, s);
    if (a.row_bytes % 4 == 0 && al % 4 == 0) return launch_gather<uint32_t>(a, s);
    return launch_gather<uint16_t>(a, s);
}

}  // namespace moe
