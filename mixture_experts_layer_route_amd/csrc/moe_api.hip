// moe_api.hip -- the C ABI of include/moe.h: argument checks, workspace
// layout and kernel enqueueing.  No host sync, no device allocation.
//
// The error cases follow the ruDNN User Guide: section 4 (logits dtype,
// 1 <= top_k <= E, U32 indices, [T,top_k] outputs), section 5 (one float
// dtype and one device for the weights; expert count and extents must agree
// with routing and input) and section 6 (shape, dtype or device mismatches
// are reported as errors rather than computed).
#include <string.h>

#include <mutex>

#include "moe_internal.h"

using namespace moe;

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

int elem_size(int dt) { return dt == MOE_F32 || dt == MOE_U32 ? 4 : 2; }

bool is_float(int dt) { return dt == MOE_F32 || dt == MOE_F16 || dt == MOE_BF16; }

int64_t numel(const moe_tensor* t) {
    int64_t n = 1;
    for (int i = 0; i < t->ndim; ++i) n *= t->dims[i];
    return n;
}

// null / ndim / negative extents / null data of a non-empty tensor
moe_status check_tensor(const moe_tensor* t, int ndim) {
    if (!t) return MOE_ERR_INVALID_ARGUMENT;
    if (t->ndim != ndim) return MOE_ERR_INVALID_ARGUMENT;
    for (int i = 0; i < ndim; ++i)
        if (t->dims[i] < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (numel(t) > 0 && !t->data) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

#define MOE_TRY(expr)                          \
    do {                                       \
        moe_status _st = (expr);               \
        if (_st != MOE_OK) return _st;         \
    } while (0)

moe_status stream_device(hipStream_t s, int* dev) {
    hipError_t e = s ? hipStreamGetDevice(s, dev) : hipGetDevice(dev);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_DEVICE;
    }
    return MOE_OK;
}

moe_status check_device_ptr(const void* p, int dev) {
    if (!p) return MOE_OK;  // empty tensor
    hipPointerAttribute_t attr;
    memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return MOE_ERR_DEVICE;
    }
    if (attr.type != hipMemoryTypeDevice && !attr.isManaged) return MOE_ERR_DEVICE;
    if (attr.device != dev) return MOE_ERR_DEVICE;
    return MOE_OK;
}

moe_status check_devices(hipStream_t s, std::initializer_list<const void*> ptrs) {
    int dev = 0;
    MOE_TRY(stream_device(s, &dev));
    for (const void* p : ptrs) MOE_TRY(check_device_ptr(p, dev));
    return MOE_OK;
}

moe_status launch_status(hipError_t e) {
    if (e == hipSuccess) return MOE_OK;
    (void)hipGetLastError();
    return MOE_ERR_LAUNCH;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------- workspace layouts
struct DispatchWs {
    size_t counts, rank, total;
};
DispatchWs dispatch_ws(int64_t T, int64_t E, int64_t k) {
    DispatchWs w;
    w.counts = 0;
    w.rank = align_up((size_t)E * 4);
    w.total = w.rank + align_up((size_t)(T * k) * 4);
    return w;
}

struct ExpertsWs {
    size_t tiles, h, total;
};
ExpertsWs experts_ws(int64_t N, int64_t I, int64_t E, int dtype) {
    ExpertsWs w;
    w.tiles = 0;
    w.h = align_up(experts_tile_bytes(N, E));
    w.total = w.h + align_up((size_t)N * (size_t)I * elem_size(dtype));
    return w;
}

struct ForwardWs {
    size_t idx, w, offsets, ros, tor, y, dws, ews, total;
};
ForwardWs forward_ws(int64_t T, int64_t H, int64_t I, int64_t E, int64_t k, int dtype) {
    ForwardWs f;
    const int64_t N = T * k;
    const size_t es = elem_size(dtype);
    size_t o = 0;
    f.idx = o;     o += align_up((size_t)N * 4);
    f.w = o;       o += align_up((size_t)N * 4);
    f.offsets = o; o += align_up((size_t)(E + 1) * 4);
    f.ros = o;     o += align_up((size_t)N * 4);
    f.tor = o;     o += align_up((size_t)N * 4);
    f.y = o;       o += align_up((size_t)N * H * es);
    f.dws = o;     o += dispatch_ws(T, E, k).total;
    f.ews = o;     o += experts_ws(N, I, E, dtype).total;
    f.total = o;
    return f;
}

// ---------------------------------------------------------------- checks per call
moe_status check_route(const moe_tensor* logits, moe_routing_options opt, const moe_tensor* indices,
                       const moe_tensor* weights) {
    MOE_TRY(check_tensor(logits, 2));
    MOE_TRY(check_tensor(indices, 2));
    MOE_TRY(check_tensor(weights, 2));
    if (!is_float(logits->dtype)) return MOE_ERR_DTYPE;
    if (indices->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (weights->dtype != logits->dtype) return MOE_ERR_DTYPE;
    const int64_t T = logits->dims[0], E = logits->dims[1];
    if (E < 1) return MOE_ERR_SHAPE;
    if (opt.top_k < 1 || opt.top_k > E) return MOE_ERR_TOP_K;
    if (opt.renormalize != 0 && opt.renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (indices->dims[0] != T || indices->dims[1] != opt.top_k) return MOE_ERR_SHAPE;
    if (weights->dims[0] != T || weights->dims[1] != opt.top_k) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (T * opt.top_k >= (int64_t)0xFFFFFFFF) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_group_options(moe_group_routing_options o, int64_t E) {
    if (o.groups < 1 || o.groups > 128 || o.selected_groups < 1 || o.selected_groups > o.groups)
        return MOE_ERR_INVALID_ARGUMENT;
    if ((o.group_top_two != 0 && o.group_top_two != 1) || (o.renormalize != 0 && o.renormalize != 1))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!(o.scale > 0.0f) || o.scale == INFINITY) return MOE_ERR_INVALID_ARGUMENT;
    if (E % o.groups) return MOE_ERR_INVALID_ARGUMENT;
    if (o.group_top_two && E / o.groups < 2) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

moe_status check_route_grouped(const moe_tensor* logits, const moe_tensor* bias, moe_group_routing_options opt,
                               const moe_tensor* indices, const moe_tensor* weights) {
    MOE_TRY(check_tensor(logits, 2));
    if (bias) MOE_TRY(check_tensor(bias, 1));
    MOE_TRY(check_tensor(indices, 2));
    MOE_TRY(check_tensor(weights, 2));
    const int64_t T = logits->dims[0], E = logits->dims[1];
    if (E >= 1) MOE_TRY(check_group_options(opt, E));
    if (!is_float(logits->dtype)) return MOE_ERR_DTYPE;
    if (bias && bias->dtype != MOE_F32) return MOE_ERR_DTYPE;
    if (indices->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (weights->dtype != logits->dtype) return MOE_ERR_DTYPE;
    if (E < 1) return MOE_ERR_SHAPE;
    if (bias && bias->dims[0] != E) return MOE_ERR_SHAPE;
    if (opt.top_k < 1 || opt.top_k > 64 || (int64_t)opt.top_k > (int64_t)opt.selected_groups * (E / opt.groups))
        return MOE_ERR_TOP_K;
    if (indices->dims[0] != T || indices->dims[1] != opt.top_k) return MOE_ERR_SHAPE;
    if (weights->dims[0] != T || weights->dims[1] != opt.top_k) return MOE_ERR_SHAPE;
    if (E > 1024) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_dispatch(const moe_tensor* input, const moe_tensor* indices, int64_t E,
                          const moe_tensor* dispatched, const moe_tensor* offsets,
                          const moe_tensor* ros, const moe_tensor* tor) {
    MOE_TRY(check_tensor(input, 2));
    MOE_TRY(check_tensor(indices, 2));
    if (dispatched) MOE_TRY(check_tensor(dispatched, 2));
    MOE_TRY(check_tensor(offsets, 1));
    MOE_TRY(check_tensor(ros, 1));
    MOE_TRY(check_tensor(tor, 1));
    if (E < 0) return MOE_ERR_INVALID_ARGUMENT;
    if (!is_float(input->dtype)) return MOE_ERR_DTYPE;
    if (indices->dtype != MOE_U32 || offsets->dtype != MOE_U32 || ros->dtype != MOE_U32 ||
        tor->dtype != MOE_U32)
        return MOE_ERR_DTYPE;
    if (dispatched && dispatched->dtype != input->dtype) return MOE_ERR_DTYPE;
    const int64_t T = input->dims[0], H = input->dims[1], k = indices->dims[1];
    if (E < 1) return MOE_ERR_SHAPE;
    if (k < 1 || k > E) return MOE_ERR_TOP_K;
    if (indices->dims[0] != T) return MOE_ERR_SHAPE;
    if (dispatched && (dispatched->dims[0] != T * k || dispatched->dims[1] != H)) return MOE_ERR_SHAPE;
    if (offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    if (ros->dims[0] != T * k || tor->dims[0] != T * k) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (T * k >= (int64_t)0xFFFFFFFF) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_weights(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down) {
    MOE_TRY(check_tensor(gate, 3));
    MOE_TRY(check_tensor(up, 3));
    MOE_TRY(check_tensor(down, 3));
    if (!is_float(gate->dtype)) return MOE_ERR_DTYPE;
    if (up->dtype != gate->dtype || down->dtype != gate->dtype) return MOE_ERR_DTYPE;
    const int64_t E = gate->dims[0], I = gate->dims[1], H = gate->dims[2];
    if (up->dims[0] != E || up->dims[1] != I || up->dims[2] != H) return MOE_ERR_SHAPE;
    if (down->dims[0] != E || down->dims[1] != H || down->dims[2] != I) return MOE_ERR_SHAPE;
    if (E < 1 || H < 1 || I < 1) return MOE_ERR_SHAPE;
    return MOE_OK;
}

moe_status check_gemm_limits(int64_t E, int64_t H, int64_t I, int64_t N,
                             const std::initializer_list<const void*>& ptrs) {
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (H % MOE_DIM_MULTIPLE || I % MOE_DIM_MULTIPLE) return MOE_ERR_UNSUPPORTED;
    if (H > (1 << 30) / 4 || I > (1 << 30) / 4) return MOE_ERR_UNSUPPORTED;
    if (N >= (int64_t)0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
    for (const void* p : ptrs)
        if (!aligned16(p)) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

moe_status check_experts(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                         const moe_tensor* dispatched, const moe_tensor* offsets, const moe_tensor* out) {
    MOE_TRY(check_weights(gate, up, down));
    MOE_TRY(check_tensor(dispatched, 2));
    MOE_TRY(check_tensor(offsets, 1));
    MOE_TRY(check_tensor(out, 2));
    if (dispatched->dtype != gate->dtype || out->dtype != gate->dtype) return MOE_ERR_DTYPE;
    if (offsets->dtype != MOE_U32) return MOE_ERR_DTYPE;
    const int64_t E = gate->dims[0], H = gate->dims[2], N = dispatched->dims[0];
    if (dispatched->dims[1] != H) return MOE_ERR_SHAPE;
    if (offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    if (out->dims[0] != N || out->dims[1] != H) return MOE_ERR_SHAPE;
    return check_gemm_limits(E, H, gate->dims[1], N, {gate->data, up->data, down->data, dispatched->data, out->data});
}

moe_status check_combine(const moe_tensor* y, const moe_tensor* ros, const moe_tensor* w,
                         const moe_tensor* out) {
    MOE_TRY(check_tensor(y, 2));
    MOE_TRY(check_tensor(ros, 1));
    MOE_TRY(check_tensor(w, 2));
    MOE_TRY(check_tensor(out, 2));
    if (!is_float(y->dtype) || !is_float(w->dtype)) return MOE_ERR_DTYPE;
    if (ros->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (out->dtype != y->dtype) return MOE_ERR_DTYPE;
    const int64_t T = w->dims[0], k = w->dims[1], H = y->dims[1];
    if (k < 1) return MOE_ERR_TOP_K;
    if (ros->dims[0] != T * k) return MOE_ERR_SHAPE;
    if (out->dims[0] != T || out->dims[1] != H) return MOE_ERR_SHAPE;
    return MOE_OK;
}

// ---------------------------------------------------------------- enqueue helpers
moe_status enqueue_route(const moe_tensor* logits, moe_routing_options opt, uint32_t* idx, void* w,
                         hipStream_t s) {
    RouteArgs a;
    a.logits = logits->data;
    a.ldtype = logits->dtype;
    a.T = logits->dims[0];
    a.E = (int)logits->dims[1];
    a.k = opt.top_k;
    a.renorm = opt.renormalize;
    a.idx = idx;
    a.w = w;
    return launch_status(launch_route(a, s));
}

moe_status enqueue_route_grouped(const moe_tensor* logits, const moe_tensor* bias, moe_group_routing_options o,
                                 uint32_t* idx, void* w, hipStream_t s) {
    GroupRouteArgs a;
    a.logits = logits->data;
    a.ldtype = logits->dtype;
    a.bias = bias ? (const float*)bias->data : nullptr;
    a.T = logits->dims[0];
    a.E = (int)logits->dims[1];
    a.k = o.top_k;
    a.groups = o.groups;
    a.selected = o.selected_groups;
    a.top_two = o.group_top_two;
    a.renorm = o.renormalize;
    a.scale = o.scale;
    a.idx = idx;
    a.w = w;
    return launch_status(launch_route_grouped(a, s));
}

moe_status enqueue_dispatch(const void* x, int dtype, int64_t T, int64_t H, const uint32_t* idx, int k,
                            int64_t E, void* dispatched, uint32_t* offsets, uint32_t* ros, uint32_t* tor,
                            void* ws, hipStream_t s) {
    const DispatchWs l = dispatch_ws(T, E, k);
    DispatchArgs a;
    a.x = x;
    a.T = T;
    a.row_bytes = H * elem_size(dtype);
    a.k = k;
    a.E = (int)E;
    a.idx = idx;
    a.counts = (uint32_t*)((char*)ws + l.counts);
    a.rank = (uint32_t*)((char*)ws + l.rank);
    a.offsets = offsets;
    a.dispatched = dispatched;
    a.row_of_slot = ros;
    a.token_of_row = tor;
    return launch_status(launch_dispatch(a, s));
}

// x_rows: null when x holds the N dispatched rows; else token_of_row, and x
// holds the x_nrows token rows the products read through it.
moe_status enqueue_experts(int dtype, int64_t E, int64_t H, int64_t I, const void* gate, const void* up,
                           const void* down, const void* x, const uint32_t* x_rows, int64_t x_nrows, int64_t N,
                           const uint32_t* offsets, void* y, void* h, void* ws, hipStream_t s, ExpertsPart part,
                           float* gu = nullptr) {
    const ExpertsWs l = experts_ws(N, I, E, dtype);
    ExpertsArgs a;
    a.dtype = dtype;
    a.gate = gate;
    a.up = up;
    a.down = down;
    a.x = x;
    a.x_rows = x_rows;
    a.x_nrows = x_nrows;
    a.offsets = offsets;
    a.y = y;
    a.h = h ? h : (char*)ws + l.h;
    a.gu = gu;
    a.tiles = (char*)ws + l.tiles;
    a.N = N;
    a.H = H;
    a.I = I;
    a.E = (int)E;
    return launch_status(launch_experts(a, s, part));
}

moe_status enqueue_combine(const void* y, int dtype, int64_t N, const uint32_t* ros, const void* w,
                           int wdtype, int64_t T, int k, int64_t H, void* out, hipStream_t s) {
    CombineArgs a;
    a.y = y;
    a.dtype = dtype;
    a.N = N;
    a.row_of_slot = ros;
    a.w = w;
    a.wdtype = wdtype;
    a.T = T;
    a.k = k;
    a.H = H;
    a.out = out;
    return launch_status(launch_combine(a, s));
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status st) {
    switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT: null pointer, bad ndim or negative extent";
    case MOE_ERR_DTYPE: return "MOE_ERR_DTYPE: dtype not allowed by the routing/expert contract";
    case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE: extents disagree";
    case MOE_ERR_TOP_K: return "MOE_ERR_TOP_K: top_k must satisfy 1 <= top_k <= E";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE: buffer is not device memory of the stream's device";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE: workspace missing or too small";
    case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH: HIP launch error";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside this implementation's limits";
    default: return "unknown moe_status";
    }
}

moe_status moe_route(const moe_tensor* logits, moe_routing_options options, moe_tensor* indices,
                     moe_tensor* weights, void* stream) {
    MOE_TRY(check_route(logits, options, indices, weights));
    if (logits->dims[0] == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {logits->data, indices->data, weights->data}));
    return enqueue_route(logits, options, (uint32_t*)indices->data, weights->data, s);
}

moe_status moe_route_sigmoid_grouped(const moe_tensor* logits, const moe_tensor* bias,
                                     moe_group_routing_options options, moe_tensor* indices, moe_tensor* weights,
                                     void* stream) {
    MOE_TRY(check_route_grouped(logits, bias, options, indices, weights));
    if (logits->dims[0] == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {logits->data, bias ? bias->data : logits->data, indices->data, weights->data}));
    return enqueue_route_grouped(logits, bias, options, (uint32_t*)indices->data, weights->data, s);
}

size_t moe_dispatch_workspace_bytes(int64_t T, int64_t E, int32_t top_k) {
    if (T < 0 || E < 1 || top_k < 1) return 0;
    return dispatch_ws(T, E, top_k).total;
}

moe_status moe_dispatch(const moe_tensor* input, const moe_tensor* indices, int64_t num_experts,
                        moe_tensor* dispatched, moe_tensor* expert_offsets, moe_tensor* row_of_slot,
                        moe_tensor* token_of_row, void* workspace, size_t workspace_bytes, void* stream) {
    MOE_TRY(check_dispatch(input, indices, num_experts, dispatched, expert_offsets, row_of_slot, token_of_row));
    const int64_t T = input->dims[0], H = input->dims[1], k = indices->dims[1];
    if (!workspace || workspace_bytes < dispatch_ws(T, num_experts, k).total) return MOE_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    void* disp = dispatched ? dispatched->data : nullptr;
    MOE_TRY(check_devices(s, {input->data, indices->data, disp ? disp : input->data, expert_offsets->data,
                              row_of_slot->data, token_of_row->data, workspace}));
    return enqueue_dispatch(input->data, input->dtype, T, H, (const uint32_t*)indices->data, (int)k,
                            num_experts, disp, (uint32_t*)expert_offsets->data,
                            (uint32_t*)row_of_slot->data, (uint32_t*)token_of_row->data, workspace, s);
}

size_t moe_experts_workspace_bytes(int64_t N, int64_t H, int64_t I, int64_t E, int32_t dtype) {
    (void)H;
    if (N < 0 || I < 1 || E < 1 || !is_float(dtype)) return 0;
    return experts_ws(N, I, E, dtype).total;
}

moe_status moe_experts_forward(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                               const moe_tensor* dispatched, const moe_tensor* expert_offsets,
                               moe_tensor* expert_out, void* workspace, size_t workspace_bytes,
                               void* stream) {
    MOE_TRY(check_experts(gate, up, down, dispatched, expert_offsets, expert_out));
    const int64_t N = dispatched->dims[0], E = gate->dims[0], I = gate->dims[1];
    if (!workspace || workspace_bytes < experts_ws(N, I, E, gate->dtype).total) return MOE_ERR_WORKSPACE;
    if (N == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {gate->data, up->data, down->data, dispatched->data, expert_offsets->data,
                              expert_out->data, workspace}));
    return enqueue_experts(gate->dtype, E, gate->dims[2], I, gate->data, up->data, down->data, dispatched->data,
                           nullptr, 0, N, (const uint32_t*)expert_offsets->data, expert_out->data, nullptr, workspace, s,
                           kBoth);
}

moe_status moe_experts_gate_up(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* dispatched,
                               const moe_tensor* expert_offsets, moe_tensor* h, void* workspace,
                               size_t workspace_bytes, void* stream) {
    MOE_TRY(check_tensor(gate, 3));
    MOE_TRY(check_tensor(up, 3));
    MOE_TRY(check_tensor(dispatched, 2));
    MOE_TRY(check_tensor(expert_offsets, 1));
    MOE_TRY(check_tensor(h, 2));
    if (!is_float(gate->dtype)) return MOE_ERR_DTYPE;
    if (up->dtype != gate->dtype || dispatched->dtype != gate->dtype || h->dtype != gate->dtype)
        return MOE_ERR_DTYPE;
    if (expert_offsets->dtype != MOE_U32) return MOE_ERR_DTYPE;
    const int64_t E = gate->dims[0], I = gate->dims[1], H = gate->dims[2], N = dispatched->dims[0];
    if (up->dims[0] != E || up->dims[1] != I || up->dims[2] != H) return MOE_ERR_SHAPE;
    if (E < 1 || H < 1 || I < 1) return MOE_ERR_SHAPE;
    if (dispatched->dims[1] != H || expert_offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    if (h->dims[0] != N || h->dims[1] != I) return MOE_ERR_SHAPE;
    MOE_TRY(check_gemm_limits(E, H, I, N, {gate->data, up->data, dispatched->data, h->data}));
    if (!workspace || workspace_bytes < align_up(experts_tile_bytes(N, E))) return MOE_ERR_WORKSPACE;
    if (N == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {gate->data, up->data, dispatched->data, expert_offsets->data, h->data, workspace}));
    return enqueue_experts(gate->dtype, E, H, I, gate->data, up->data, nullptr, dispatched->data, nullptr, 0, N,
                           (const uint32_t*)expert_offsets->data, nullptr, h->data, workspace, s, kGateUp);
}

moe_status moe_experts_gate_up_gathered(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* input,
                                       const moe_tensor* token_of_row, const moe_tensor* expert_offsets,
                                       moe_tensor* h, void* workspace, size_t workspace_bytes, void* stream) {
    MOE_TRY(check_tensor(gate, 3));
    MOE_TRY(check_tensor(up, 3));
    MOE_TRY(check_tensor(input, 2));
    MOE_TRY(check_tensor(token_of_row, 1));
    MOE_TRY(check_tensor(expert_offsets, 1));
    MOE_TRY(check_tensor(h, 2));
    if (!is_float(gate->dtype)) return MOE_ERR_DTYPE;
    if (up->dtype != gate->dtype || input->dtype != gate->dtype || h->dtype != gate->dtype)
        return MOE_ERR_DTYPE;
    if (token_of_row->dtype != MOE_U32 || expert_offsets->dtype != MOE_U32) return MOE_ERR_DTYPE;
    const int64_t E = gate->dims[0], I = gate->dims[1], H = gate->dims[2];
    const int64_t T = input->dims[0], N = token_of_row->dims[0];
    if (up->dims[0] != E || up->dims[1] != I || up->dims[2] != H) return MOE_ERR_SHAPE;
    if (E < 1 || H < 1 || I < 1) return MOE_ERR_SHAPE;
    if (input->dims[1] != H || expert_offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    if (h->dims[0] != N || h->dims[1] != I) return MOE_ERR_SHAPE;
    if (N > 0 && T < 1) return MOE_ERR_SHAPE;
    MOE_TRY(check_gemm_limits(E, H, I, N, {gate->data, up->data, input->data, h->data}));
    if (!workspace || workspace_bytes < align_up(experts_tile_bytes(N, E))) return MOE_ERR_WORKSPACE;
    if (N == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {gate->data, up->data, input->data, token_of_row->data, expert_offsets->data,
                              h->data, workspace}));
    return enqueue_experts(gate->dtype, E, H, I, gate->data, up->data, nullptr, input->data,
                           (const uint32_t*)token_of_row->data, T, N, (const uint32_t*)expert_offsets->data,
                           nullptr, h->data, workspace, s, kGateUp);
}

moe_status moe_experts_down(const moe_tensor* down, const moe_tensor* h, const moe_tensor* expert_offsets,
                            moe_tensor* expert_out, void* workspace, size_t workspace_bytes, void* stream) {
    MOE_TRY(check_tensor(down, 3));
    MOE_TRY(check_tensor(h, 2));
    MOE_TRY(check_tensor(expert_offsets, 1));
    MOE_TRY(check_tensor(expert_out, 2));
    if (!is_float(down->dtype)) return MOE_ERR_DTYPE;
    if (h->dtype != down->dtype || expert_out->dtype != down->dtype) return MOE_ERR_DTYPE;
    if (expert_offsets->dtype != MOE_U32) return MOE_ERR_DTYPE;
    const int64_t E = down->dims[0], H = down->dims[1], I = down->dims[2], N = h->dims[0];
    if (E < 1 || H < 1 || I < 1) return MOE_ERR_SHAPE;
    if (h->dims[1] != I || expert_offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    if (expert_out->dims[0] != N || expert_out->dims[1] != H) return MOE_ERR_SHAPE;
    MOE_TRY(check_gemm_limits(E, H, I, N, {down->data, h->data, expert_out->data}));
    if (!workspace || workspace_bytes < align_up(experts_tile_bytes(N, E))) return MOE_ERR_WORKSPACE;
    if (N == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {down->data, h->data, expert_offsets->data, expert_out->data, workspace}));
    return enqueue_experts(down->dtype, E, H, I, nullptr, nullptr, down->data, nullptr, nullptr, 0, N,
                           (const uint32_t*)expert_offsets->data, expert_out->data, h->data, workspace, s,
                           kDown);
}

moe_status moe_combine(const moe_tensor* expert_out, const moe_tensor* row_of_slot, const moe_tensor* weights,
                       moe_tensor* output, void* stream) {
    MOE_TRY(check_combine(expert_out, row_of_slot, weights, output));
    const int64_t T = weights->dims[0], k = weights->dims[1], H = expert_out->dims[1];
    if (T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {expert_out->data, row_of_slot->data, weights->data, output->data}));
    return enqueue_combine(expert_out->data, expert_out->dtype, expert_out->dims[0],
                           (const uint32_t*)row_of_slot->data, weights->data, weights->dtype, T, (int)k, H,
                           output->data, s);
}

size_t moe_forward_workspace_bytes(int64_t T, int64_t H, int64_t I, int64_t E, int32_t top_k, int32_t dtype) {
    if (T < 0 || H < 1 || I < 1 || E < 1 || top_k < 1 || !is_float(dtype)) return 0;
    return forward_ws(T, H, I, E, top_k, dtype).total;
}

}  // extern "C"

namespace {
// The chain after the routing options were checked: shapes, limits and
// workspace, then route (through `route`, which writes indices and weights
// into the workspace), mapping-only dispatch, experts reading the tokens in
// place, combine.
template <typename RouteFn>
moe_status forward_chain(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                         const moe_tensor* input, const moe_tensor* logits, const moe_tensor* bias, int64_t k,
                         moe_tensor* output, void* workspace, size_t workspace_bytes, void* stream,
                         RouteFn route, bool check_workspace_device = true) {
    const int64_t E = gate->dims[0], I = gate->dims[1], H = gate->dims[2];
    const int64_t T = input->dims[0];
    if (input->dims[1] != H) return MOE_ERR_SHAPE;
    if (logits->dims[0] != T || logits->dims[1] != E) return MOE_ERR_SHAPE;
    if (output->dims[0] != T || output->dims[1] != H) return MOE_ERR_SHAPE;
    const int64_t N = T * k;
    if (N >= (int64_t)0x7FFFFFFF) return MOE_ERR_UNSUPPORTED;
    MOE_TRY(check_gemm_limits(E, H, I, N, {gate->data, up->data, down->data, input->data, output->data}));
    const ForwardWs l = forward_ws(T, H, I, E, k, gate->dtype);
    if (!workspace || workspace_bytes < l.total) return MOE_ERR_WORKSPACE;
    if (T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {gate->data, up->data, down->data, input->data, logits->data,
                              bias ? bias->data : logits->data, output->data,
                              check_workspace_device ? workspace : nullptr}));
    char* ws = (char*)workspace;
    uint32_t* idx = (uint32_t*)(ws + l.idx);
    void* w = ws + l.w;
    uint32_t* offsets = (uint32_t*)(ws + l.offsets);
    uint32_t* ros = (uint32_t*)(ws + l.ros);
    uint32_t* tor = (uint32_t*)(ws + l.tor);
    void* y = ws + l.y;
    MOE_TRY(route(idx, w, s));
    MOE_TRY(enqueue_dispatch(input->data, input->dtype, T, H, idx, (int)k, E, nullptr, offsets, ros, tor,
                             ws + l.dws, s));
    // the gate/up products read the token rows through token_of_row, so the
    // dispatch writes only the mapping and no dispatched copy of the rows
    MOE_TRY(enqueue_experts(gate->dtype, E, H, I, gate->data, up->data, down->data, input->data, tor, T, N,
                            offsets, y, nullptr, ws + l.ews, s, kBoth));
    return enqueue_combine(y, input->dtype, N, ros, w, logits->dtype, T, (int)k, H, output->data, s);
}

moe_status check_forward_tensors(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                 const moe_tensor* input, const moe_tensor* logits, const moe_tensor* output) {
    MOE_TRY(check_weights(gate, up, down));
    MOE_TRY(check_tensor(input, 2));
    MOE_TRY(check_tensor(logits, 2));
    MOE_TRY(check_tensor(output, 2));
    if (!is_float(logits->dtype)) return MOE_ERR_DTYPE;
    if (input->dtype != gate->dtype || output->dtype != gate->dtype) return MOE_ERR_DTYPE;
    return MOE_OK;
}
}  // namespace

extern "C" {

moe_status moe_forward(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                       const moe_tensor* input, const moe_tensor* logits, moe_routing_options options,
                       moe_tensor* output, void* workspace, size_t workspace_bytes, void* stream) {
    MOE_TRY(check_forward_tensors(gate, up, down, input, logits, output));
    const int64_t E = gate->dims[0];
    if (logits->dims[1] == E && (options.top_k < 1 || options.top_k > E)) return MOE_ERR_TOP_K;
    if (options.renormalize != 0 && options.renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    return forward_chain(gate, up, down, input, logits, nullptr, options.top_k, output, workspace, workspace_bytes,
                         stream, [&](uint32_t* idx, void* w, hipStream_t s) {
                             return enqueue_route(logits, options, idx, w, s);
                         });
}

moe_status moe_forward_sigmoid_grouped(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                       const moe_tensor* input, const moe_tensor* logits, const moe_tensor* bias,
                                       moe_group_routing_options options, moe_tensor* output,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    MOE_TRY(check_forward_tensors(gate, up, down, input, logits, output));
    if (bias) MOE_TRY(check_tensor(bias, 1));
    const int64_t E = gate->dims[0];
    MOE_TRY(check_group_options(options, E));
    if (bias && bias->dtype != MOE_F32) return MOE_ERR_DTYPE;
    if (bias && bias->dims[0] != E) return MOE_ERR_SHAPE;
    if (options.top_k < 1 || options.top_k > 64 ||
        (int64_t)options.top_k > (int64_t)options.selected_groups * (E / options.groups))
        return MOE_ERR_TOP_K;
    if (E > 1024) return MOE_ERR_UNSUPPORTED;
    return forward_chain(gate, up, down, input, logits, bias, options.top_k, output, workspace, workspace_bytes,
                         stream, [&](uint32_t* idx, void* w, hipStream_t s) {
                             return enqueue_route_grouped(logits, bias, options, idx, w, s);
                         });
}

}  // extern "C"

// ---------------------------------------------------------------- forward without allocation
// moe_forward for callers that cannot allocate: the forward's workspace is a
// static device array of kNoAllocScratchBytes, of which every device the
// library runs on holds its own copy until the process ends.  Host code never
// passes the array's name to a kernel (on the host it only stands in for the
// symbol): the device address comes from hipGetSymbolAddress, taken once per
// device with that device current, and is kept per device.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 256;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices];

// The device address of device dev's scratch array (set up on the first call
// on that device).
moe_status scratch_of_device(int dev, void** ptr) {
    if (dev < 0 || dev >= kMaxScratchDevices) return MOE_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_ERR_DEVICE;
        }
        if (cur != dev && hipSetDevice(dev) != hipSuccess) {
            (void)hipGetLastError();
            return MOE_ERR_DEVICE;
        }
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return MOE_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}
}  // namespace

extern "C" moe_status moe_forward_no_alloc(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                           const moe_tensor* input, const moe_tensor* logits,
                                           moe_routing_options options, moe_tensor* output, void* stream) {
    MOE_TRY(check_forward_tensors(gate, up, down, input, logits, output));
    const int64_t E = gate->dims[0];
    if (logits->dims[1] == E && (options.top_k < 1 || options.top_k > E)) return MOE_ERR_TOP_K;
    if (options.renormalize != 0 && options.renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    // the stream's device, and that device's array (set up on the first call
    // there); then the checks and launches of moe_forward, with the array as
    // the workspace: a batch whose forward workspace exceeds it gets
    // MOE_ERR_WORKSPACE
    int dev = 0;
    MOE_TRY(stream_device((hipStream_t)stream, &dev));
    void* ws = nullptr;
    MOE_TRY(scratch_of_device(dev, &ws));
    return forward_chain(gate, up, down, input, logits, nullptr, options.top_k, output, ws, kNoAllocScratchBytes,
                         stream, [&](uint32_t* idx, void* w, hipStream_t s) {
                             return enqueue_route(logits, options, idx, w, s);
                         }, false);
}

// ---------------------------------------------------------------- first-order training
namespace {

bool is_index(int dt) { return dt == MOE_U32 || dt == MOE_I32 || dt == MOE_I64; }

moe_status check_router_options(moe_router_weight_options o) {
    if (o.scoring != MOE_SCORING_SOFTMAX && o.scoring != MOE_SCORING_SIGMOID) return MOE_ERR_INVALID_ARGUMENT;
    if (o.renormalize != 0 && o.renormalize != 1) return MOE_ERR_INVALID_ARGUMENT;
    if (!(o.scale > 0.0f) || o.scale == INFINITY) return MOE_ERR_INVALID_ARGUMENT;
    return MOE_OK;
}

// logits [T,E], indices [T,k], a [T,k] F32 tensor (weights or their gradient)
moe_status check_router_train(const moe_tensor* logits, const moe_tensor* indices, const moe_tensor* tk,
                              moe_router_weight_options o) {
    MOE_TRY(check_tensor(logits, 2));
    MOE_TRY(check_tensor(indices, 2));
    MOE_TRY(check_tensor(tk, 2));
    MOE_TRY(check_router_options(o));
    if (!is_float(logits->dtype)) return MOE_ERR_DTYPE;
    if (!is_index(indices->dtype)) return MOE_ERR_DTYPE;
    if (tk->dtype != MOE_F32) return MOE_ERR_DTYPE;
    const int64_t T = logits->dims[0], E = logits->dims[1], k = indices->dims[1];
    if (E < 1) return MOE_ERR_SHAPE;
    if (indices->dims[0] != T) return MOE_ERR_SHAPE;
    if (k < 1 || k > E || k > 64) return MOE_ERR_TOP_K;
    if (tk->dims[0] != T || tk->dims[1] != k) return MOE_ERR_SHAPE;
    if (E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

RouterWeightArgs router_args(const moe_tensor* logits, const moe_tensor* indices, moe_router_weight_options o) {
    RouterWeightArgs a = {};
    a.logits = logits->data;
    a.ldtype = logits->dtype;
    a.idx = indices->data;
    a.idx_dtype = indices->dtype;
    a.T = logits->dims[0];
    a.E = (int)logits->dims[1];
    a.k = (int)indices->dims[1];
    a.scoring = o.scoring;
    a.renorm = o.renormalize;
    a.scale = o.scale;
    return a;
}

// rows [R,H] with an optional token_of_row [N]: the product rows; *N gets N
moe_status check_product_rows(const moe_tensor* rows, const moe_tensor* tor, int dtype, int64_t H, int64_t* N) {
    MOE_TRY(check_tensor(rows, 2));
    if (tor) MOE_TRY(check_tensor(tor, 1));
    if (rows->dtype != dtype) return MOE_ERR_DTYPE;
    if (tor && tor->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (rows->dims[1] != H) return MOE_ERR_SHAPE;
    *N = tor ? tor->dims[0] : rows->dims[0];
    if (tor && *N > 0 && rows->dims[0] < 1) return MOE_ERR_SHAPE;
    return MOE_OK;
}

moe_status check_2d(const moe_tensor* t, int dtype, int64_t d0, int64_t d1) {
    MOE_TRY(check_tensor(t, 2));
    if (t->dtype != dtype) return MOE_ERR_DTYPE;
    if (t->dims[0] != d0 || t->dims[1] != d1) return MOE_ERR_SHAPE;
    return MOE_OK;
}

moe_status check_3d(const moe_tensor* t, int dtype, int64_t d0, int64_t d1, int64_t d2) {
    MOE_TRY(check_tensor(t, 3));
    if (t->dtype != dtype) return MOE_ERR_DTYPE;
    if (t->dims[0] != d0 || t->dims[1] != d1 || t->dims[2] != d2) return MOE_ERR_SHAPE;
    return MOE_OK;
}

struct BackwardWs {
    size_t tiles, dgu, xg, total;
};
BackwardWs backward_ws(int64_t N, int64_t H, int64_t I, int64_t E, int dtype) {
    BackwardWs w;
    w.tiles = 0;
    w.dgu = align_up(experts_backward_tile_bytes(N, E));
    w.xg = w.dgu + align_up((size_t)N * 2 * (size_t)I * elem_size(dtype));
    w.total = w.xg + align_up((size_t)N * (size_t)H * elem_size(dtype));
    return w;
}

}  // namespace

extern "C" {

moe_status moe_router_weights(const moe_tensor* logits, const moe_tensor* indices,
                              moe_router_weight_options options, moe_tensor* weights, void* stream) {
    MOE_TRY(check_router_train(logits, indices, weights, options));
    if (logits->dims[0] == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {logits->data, indices->data, weights->data}));
    RouterWeightArgs a = router_args(logits, indices, options);
    a.w = (float*)weights->data;
    return launch_status(launch_router_weights(a, s));
}

moe_status moe_router_backward(const moe_tensor* logits, const moe_tensor* indices,
                               const moe_tensor* grad_weights, moe_router_weight_options options,
                               moe_tensor* grad_logits, void* stream) {
    MOE_TRY(check_router_train(logits, indices, grad_weights, options));
    MOE_TRY(check_2d(grad_logits, logits->dtype, logits->dims[0], logits->dims[1]));
    if (logits->dims[0] == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {logits->data, indices->data, grad_weights->data, grad_logits->data}));
    RouterWeightArgs a = router_args(logits, indices, options);
    a.gw = (const float*)grad_weights->data;
    a.dl = grad_logits->data;
    return launch_status(launch_router_backward(a, s));
}

moe_status moe_combine_backward(const moe_tensor* expert_out, const moe_tensor* row_of_slot,
                                const moe_tensor* weights, const moe_tensor* grad_output,
                                moe_tensor* grad_expert_out, moe_tensor* grad_weights, void* stream) {
    MOE_TRY(check_tensor(expert_out, 2));
    MOE_TRY(check_tensor(row_of_slot, 1));
    MOE_TRY(check_tensor(weights, 2));
    MOE_TRY(check_tensor(grad_output, 2));
    MOE_TRY(check_tensor(grad_expert_out, 2));
    MOE_TRY(check_tensor(grad_weights, 2));
    if (!is_float(expert_out->dtype) || !is_float(weights->dtype)) return MOE_ERR_DTYPE;
    if (row_of_slot->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (grad_output->dtype != expert_out->dtype || grad_expert_out->dtype != expert_out->dtype)
        return MOE_ERR_DTYPE;
    if (grad_weights->dtype != MOE_F32) return MOE_ERR_DTYPE;
    const int64_t N = expert_out->dims[0], H = expert_out->dims[1];
    const int64_t T = weights->dims[0], k = weights->dims[1];
    if (k < 1) return MOE_ERR_TOP_K;
    if (row_of_slot->dims[0] != T * k) return MOE_ERR_SHAPE;
    if (grad_output->dims[0] != T || grad_output->dims[1] != H) return MOE_ERR_SHAPE;
    if (grad_expert_out->dims[0] != N || grad_expert_out->dims[1] != H) return MOE_ERR_SHAPE;
    if (grad_weights->dims[0] != T || grad_weights->dims[1] != k) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {expert_out->data, row_of_slot->data, weights->data, grad_output->data,
                              grad_expert_out->data, grad_weights->data}));
    CombineBackwardArgs a;
    a.y = expert_out->data;
    a.dtype = expert_out->dtype;
    a.N = N;
    a.row_of_slot = (const uint32_t*)row_of_slot->data;
    a.w = weights->data;
    a.wdtype = weights->dtype;
    a.g = grad_output->data;
    a.T = T;
    a.k = (int)k;
    a.H = H;
    a.dy = grad_expert_out->data;
    a.dw = (float*)grad_weights->data;
    return launch_status(launch_combine_backward(a, s));
}

moe_status moe_experts_forward_training(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                        const moe_tensor* rows, const moe_tensor* token_of_row,
                                        const moe_tensor* expert_offsets, moe_tensor* expert_out,
                                        moe_tensor* preact, moe_tensor* h, void* workspace,
                                        size_t workspace_bytes, void* stream) {
    MOE_TRY(check_weights(gate, up, down));
    const int dt = gate->dtype;
    const int64_t E = gate->dims[0], I = gate->dims[1], H = gate->dims[2];
    int64_t N = 0;
    MOE_TRY(check_product_rows(rows, token_of_row, dt, H, &N));
    MOE_TRY(check_tensor(expert_offsets, 1));
    if (expert_offsets->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (expert_offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    MOE_TRY(check_2d(expert_out, dt, N, H));
    MOE_TRY(check_2d(preact, MOE_F32, N, 2 * I));
    MOE_TRY(check_2d(h, dt, N, I));
    MOE_TRY(check_gemm_limits(E, H, I, N, {gate->data, up->data, down->data, rows->data, expert_out->data,
                                           preact->data, h->data}));
    if (!workspace || workspace_bytes < experts_ws(N, I, E, dt).total) return MOE_ERR_WORKSPACE;
    if (N == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t* tor = token_of_row ? (const uint32_t*)token_of_row->data : nullptr;
    MOE_TRY(check_devices(s, {gate->data, up->data, down->data, rows->data, tor ? (const void*)tor : rows->data,
                              expert_offsets->data, expert_out->data, preact->data, h->data, workspace}));
    return enqueue_experts(dt, E, H, I, gate->data, up->data, down->data, rows->data, tor, rows->dims[0], N,
                           (const uint32_t*)expert_offsets->data, expert_out->data, h->data, workspace, s, kBoth,
                           (float*)preact->data);
}

size_t moe_experts_backward_workspace_bytes(int64_t N, int64_t H, int64_t I, int64_t E, int32_t dtype) {
    if (N < 0 || H < 1 || I < 1 || E < 1 || !is_float(dtype)) return 0;
    return backward_ws(N, H, I, E, dtype).total;
}

moe_status moe_experts_backward(const moe_tensor* gate, const moe_tensor* up, const moe_tensor* down,
                                const moe_tensor* rows, const moe_tensor* token_of_row,
                                const moe_tensor* expert_offsets, const moe_tensor* preact, const moe_tensor* h,
                                const moe_tensor* grad_expert_out, moe_tensor* grad_rows, moe_tensor* grad_gate,
                                moe_tensor* grad_up, moe_tensor* grad_down, void* workspace,
                                size_t workspace_bytes, void* stream) {
    MOE_TRY(check_weights(gate, up, down));
    const int dt = gate->dtype;
    const int64_t E = gate->dims[0], I = gate->dims[1], H = gate->dims[2];
    int64_t N = 0;
    MOE_TRY(check_product_rows(rows, token_of_row, dt, H, &N));
    MOE_TRY(check_tensor(expert_offsets, 1));
    if (expert_offsets->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (expert_offsets->dims[0] != E + 1) return MOE_ERR_SHAPE;
    MOE_TRY(check_2d(preact, MOE_F32, N, 2 * I));
    MOE_TRY(check_2d(h, dt, N, I));
    MOE_TRY(check_2d(grad_expert_out, dt, N, H));
    MOE_TRY(check_2d(grad_rows, dt, N, H));
    MOE_TRY(check_3d(grad_gate, MOE_F32, E, I, H));
    MOE_TRY(check_3d(grad_up, MOE_F32, E, I, H));
    MOE_TRY(check_3d(grad_down, MOE_F32, E, H, I));
    MOE_TRY(check_gemm_limits(E, H, I, N, {gate->data, up->data, down->data, rows->data, preact->data, h->data,
                                           grad_expert_out->data, grad_rows->data, grad_gate->data, grad_up->data,
                                           grad_down->data}));
    const BackwardWs l = backward_ws(N, H, I, E, dt);
    if (!workspace || workspace_bytes < l.total) return MOE_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const uint32_t* tor = token_of_row ? (const uint32_t*)token_of_row->data : nullptr;
    MOE_TRY(check_devices(s, {gate->data, up->data, down->data, rows->data, tor ? (const void*)tor : rows->data,
                              expert_offsets->data, preact->data, h->data, grad_expert_out->data, grad_rows->data,
                              grad_gate->data, grad_up->data, grad_down->data, workspace}));
    ExpertsBackwardArgs a;
    a.dtype = dt;
    a.gate = gate->data;
    a.up = up->data;
    a.down = down->data;
    a.x = rows->data;
    a.x_rows = tor;
    a.x_nrows = rows->dims[0];
    a.offsets = (const uint32_t*)expert_offsets->data;
    a.gu = (const float*)preact->data;
    a.h = h->data;
    a.dy = grad_expert_out->data;
    a.dx = grad_rows->data;
    a.dgate = (float*)grad_gate->data;
    a.dup = (float*)grad_up->data;
    a.ddown = (float*)grad_down->data;
    a.dgu = (char*)workspace + l.dgu;
    a.xg = (char*)workspace + l.xg;
    a.tiles = (char*)workspace + l.tiles;
    a.N = N;
    a.H = H;
    a.I = I;
    a.E = (int)E;
    // N == 0 still runs: every expert's weight gradients are written as zeros
    return launch_status(launch_experts_backward(a, s));
}

moe_status moe_dispatch_backward(const moe_tensor* grad_rows, const moe_tensor* row_of_slot, int32_t top_k,
                                 moe_tensor* grad_input, void* stream) {
    MOE_TRY(check_tensor(grad_rows, 2));
    MOE_TRY(check_tensor(row_of_slot, 1));
    MOE_TRY(check_tensor(grad_input, 2));
    if (!is_float(grad_rows->dtype)) return MOE_ERR_DTYPE;
    if (row_of_slot->dtype != MOE_U32) return MOE_ERR_DTYPE;
    if (grad_input->dtype != grad_rows->dtype) return MOE_ERR_DTYPE;
    if (top_k < 1) return MOE_ERR_TOP_K;
    const int64_t N = grad_rows->dims[0], H = grad_rows->dims[1], T = grad_input->dims[0];
    if (grad_input->dims[1] != H) return MOE_ERR_SHAPE;
    if (row_of_slot->dims[0] != T * top_k) return MOE_ERR_SHAPE;
    if (T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    MOE_TRY(check_devices(s, {grad_rows->data, row_of_slot->data, grad_input->data}));
    DispatchBackwardArgs a;
    a.drows = grad_rows->data;
    a.dtype = grad_rows->dtype;
    a.N = N;
    a.row_of_slot = (const uint32_t*)row_of_slot->data;
    a.T = T;
    a.k = top_k;
    a.H = H;
    a.dx = grad_input->data;
    return launch_status(launch_dispatch_backward(a, s));
}

}  // extern "C"
