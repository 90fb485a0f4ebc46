"""Host-side tests of the C ABI: the library loads, exports what include/moe.h
declares, sizes workspaces, and rejects bad arguments before touching a device.

Every call here fails validation (or the device check) on the host, so no
kernel is launched; these run without a GPU.
"""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_route_amd as moe
from mixture_experts_layer_route_amd import _lib
from mixture_experts_layer_route_amd._lib import MoeRoutingOptions, raw_tensor

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
F32, F16, BF16, U32 = _lib.MOE_F32, _lib.MOE_F16, _lib.MOE_BF16, _lib.MOE_U32
OK, INVALID, DTYPE, SHAPE, TOPK, DEVICE, WORKSPACE, LAUNCH, UNSUPPORTED = range(9)
FAKE = 0x10000  # never dereferenced: validation rejects the call first


@pytest.fixture(scope="module")
def L():
    return _lib.load()


def header_functions():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w\*\s]+?\b(moe_\w+)\s*\(", src, re.M)))


def test_library_exports_every_declared_function(L):
    declared = header_functions()
    assert set(declared) == set(_lib.EXPORTS), declared
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in _lib.STATUS.items():
        assert L.moe_status_string(code).decode().startswith(name)


def test_header_limits_match_binding():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert f"#define MOE_MAX_EXPERTS {_lib.MAX_EXPERTS}" in src
    assert f"#define MOE_DIM_MULTIPLE {_lib.DIM_MULTIPLE}" in src


def test_workspace_sizes(L):
    assert L.moe_dispatch_workspace_bytes(100, 8, 2) >= 100 * 2 * 4 + 8 * 4
    assert L.moe_dispatch_workspace_bytes(-1, 8, 2) == 0
    assert L.moe_experts_workspace_bytes(256, 128, 64, 8, BF16) >= 256 * 64 * 2
    assert L.moe_experts_workspace_bytes(256, 128, 64, 8, U32) == 0
    small = L.moe_forward_workspace_bytes(64, 128, 256, 8, 2, F32)
    big = L.moe_forward_workspace_bytes(8192, 2048, 1408, 64, 6, BF16)
    assert 0 < small < big
    # expert outputs and the activation must fit; the fused forward reads
    # token rows in place, so no dispatched copy is needed
    N = 8192 * 6
    assert big >= N * 2048 * 2 + N * 1408 * 2
    assert big < N * 2048 * 2 * 2 + N * 1408 * 2
    assert L.moe_forward_workspace_bytes(64, 128, 256, 8, 0, F32) == 0


def _route(L, logits, k, idx, w, renorm=1):
    return L.moe_route(ctypes.byref(logits), MoeRoutingOptions(k, renorm), ctypes.byref(idx),
                       ctypes.byref(w), None)


def test_route_validation(L):
    T, E, k = 16, 8, 2
    lg = raw_tensor(FAKE, F32, (T, E))
    idx = raw_tensor(FAKE, U32, (T, k))
    w = raw_tensor(FAKE, F32, (T, k))
    assert _route(L, raw_tensor(None, F32, (T, E)), k, idx, w) == INVALID
    assert _route(L, raw_tensor(FAKE, F32, (T, E, 1)), k, idx, w) == INVALID
    assert _route(L, raw_tensor(FAKE, F32, (-1, E)), k, idx, w) == INVALID
    assert _route(L, raw_tensor(FAKE, U32, (T, E)), k, idx, w) == DTYPE       # quantised/int logits
    assert _route(L, lg, k, raw_tensor(FAKE, F32, (T, k)), w) == DTYPE        # indices must be U32
    assert _route(L, lg, k, idx, raw_tensor(FAKE, BF16, (T, k))) == DTYPE     # weights in logits dtype
    assert _route(L, lg, 0, raw_tensor(FAKE, U32, (T, 0)), raw_tensor(FAKE, F32, (T, 0))) == TOPK
    assert _route(L, lg, E + 1, raw_tensor(FAKE, U32, (T, E + 1)), raw_tensor(FAKE, F32, (T, E + 1))) == TOPK
    assert _route(L, lg, k, raw_tensor(FAKE, U32, (T + 1, k)), w) == SHAPE
    assert _route(L, lg, k, idx, raw_tensor(FAKE, F32, (T, k + 1))) == SHAPE
    assert _route(L, lg, k, idx, w, renorm=2) == INVALID
    big = raw_tensor(FAKE, F32, (T, _lib.MAX_EXPERTS + 1))
    assert _route(L, big, k, idx, w) == UNSUPPORTED
    # T = 0 is a valid no-op
    assert _route(L, raw_tensor(None, F32, (0, E)), k, raw_tensor(None, U32, (0, k)),
                  raw_tensor(None, F32, (0, k))) == OK


def test_route_device_check_without_device(L):
    """A well-formed call whose buffers are not device memory of the stream's
    device is refused with MOE_ERR_DEVICE, never launched."""
    T, E, k = 16, 8, 2
    st = _route(L, raw_tensor(FAKE, F32, (T, E)), k, raw_tensor(FAKE, U32, (T, k)), raw_tensor(FAKE, F32, (T, k)))
    assert st == DEVICE


def _dispatch(L, x, idx, E, rows, off, ros, tor, ws=FAKE, wsb=1 << 30):
    return L.moe_dispatch(ctypes.byref(x), ctypes.byref(idx), E, ctypes.byref(rows), ctypes.byref(off),
                          ctypes.byref(ros), ctypes.byref(tor), ctypes.c_void_p(ws), wsb, None)


def test_dispatch_validation(L):
    T, H, E, k = 10, 16, 4, 2
    x = raw_tensor(FAKE, BF16, (T, H))
    idx = raw_tensor(FAKE, U32, (T, k))
    rows = raw_tensor(FAKE, BF16, (T * k, H))
    off = raw_tensor(FAKE, U32, (E + 1,))
    ros = raw_tensor(FAKE, U32, (T * k,))
    tor = raw_tensor(FAKE, U32, (T * k,))
    assert _dispatch(L, x, idx, E, raw_tensor(FAKE, F16, (T * k, H)), off, ros, tor) == DTYPE
    assert _dispatch(L, x, raw_tensor(FAKE, F32, (T, k)), E, rows, off, ros, tor) == DTYPE
    assert _dispatch(L, x, idx, E, raw_tensor(FAKE, BF16, (T * k, H + 1)), off, ros, tor) == SHAPE
    assert _dispatch(L, x, idx, E, rows, raw_tensor(FAKE, U32, (E,)), ros, tor) == SHAPE
    assert _dispatch(L, x, idx, E, rows, off, raw_tensor(FAKE, U32, (T,)), tor) == SHAPE
    assert _dispatch(L, x, raw_tensor(FAKE, U32, (T, 5)), E, raw_tensor(FAKE, BF16, (T * 5, H)), off,
                     raw_tensor(FAKE, U32, (T * 5,)), raw_tensor(FAKE, U32, (T * 5,))) == TOPK
    assert _dispatch(L, x, idx, E, rows, off, ros, tor, ws=0) == WORKSPACE
    assert _dispatch(L, x, idx, E, rows, off, ros, tor, wsb=8) == WORKSPACE
    assert _dispatch(L, x, idx, -1, rows, off, ros, tor) == INVALID


def test_dispatch_mapping_only_validation(L):
    """A NULL dispatched tensor asks for the mapping only; the other
    arguments are still checked, and a well-formed call reaches the device
    check."""
    T, H, E, k = 10, 16, 4, 2
    x = raw_tensor(FAKE, BF16, (T, H))
    idx = raw_tensor(FAKE, U32, (T, k))
    off = raw_tensor(FAKE, U32, (E + 1,))
    ros = raw_tensor(FAKE, U32, (T * k,))
    tor = raw_tensor(FAKE, U32, (T * k,))

    def d(idx=idx, off=off, ros=ros):
        return L.moe_dispatch(ctypes.byref(x), ctypes.byref(idx), E, None, ctypes.byref(off), ctypes.byref(ros),
                              ctypes.byref(tor), ctypes.c_void_p(FAKE), 1 << 30, None)

    assert d(idx=raw_tensor(FAKE, F32, (T, k))) == DTYPE
    assert d(off=raw_tensor(FAKE, U32, (E,))) == SHAPE
    assert d(ros=raw_tensor(FAKE, U32, (T,))) == SHAPE
    assert d() == DEVICE


def test_gate_up_gathered_validation(L):
    E, I, H, T, N = 4, 32, 16, 10, 20
    g = raw_tensor(FAKE, BF16, (E, I, H))
    u = raw_tensor(FAKE, BF16, (E, I, H))
    x = raw_tensor(FAKE, BF16, (T, H))
    tor = raw_tensor(FAKE, U32, (N,))
    off = raw_tensor(FAKE, U32, (E + 1,))
    h = raw_tensor(FAKE, BF16, (N, I))

    def f(u=u, x=x, tor=tor, off=off, h=h, wsb=1 << 30):
        return L.moe_experts_gate_up_gathered(ctypes.byref(g), ctypes.byref(u), ctypes.byref(x), ctypes.byref(tor),
                                              ctypes.byref(off), ctypes.byref(h), ctypes.c_void_p(FAKE), wsb, None)

    assert f(x=raw_tensor(FAKE, F16, (T, H))) == DTYPE
    assert f(tor=raw_tensor(FAKE, F32, (N,))) == DTYPE
    assert f(x=raw_tensor(FAKE, BF16, (T, H + 8))) == SHAPE
    assert f(h=raw_tensor(FAKE, BF16, (N + 1, I))) == SHAPE     # h has a row per token_of_row entry
    assert f(off=raw_tensor(FAKE, U32, (E,))) == SHAPE
    assert f(x=raw_tensor(FAKE, BF16, (0, H))) == SHAPE         # rows to gather but no tokens
    assert f(x=raw_tensor(FAKE + 2, BF16, (T, H))) == UNSUPPORTED
    assert f(wsb=16) == WORKSPACE
    assert f() == DEVICE


def _experts(L, g, u, d, rows, off, out, ws=FAKE, wsb=1 << 30):
    return L.moe_experts_forward(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ctypes.byref(rows),
                                 ctypes.byref(off), ctypes.byref(out), ctypes.c_void_p(ws), wsb, None)


def test_experts_validation(L):
    E, I, H, N = 4, 32, 16, 20
    g = raw_tensor(FAKE, BF16, (E, I, H))
    u = raw_tensor(FAKE, BF16, (E, I, H))
    d = raw_tensor(FAKE, BF16, (E, H, I))
    rows = raw_tensor(FAKE, BF16, (N, H))
    off = raw_tensor(FAKE, U32, (E + 1,))
    out = raw_tensor(FAKE, BF16, (N, H))
    assert _experts(L, g, raw_tensor(FAKE, F16, (E, I, H)), d, rows, off, out) == DTYPE   # one weight dtype
    assert _experts(L, g, u, d, raw_tensor(FAKE, F32, (N, H)), off, out) == DTYPE         # input = weight dtype
    assert _experts(L, g, u, raw_tensor(FAKE, BF16, (E, I, H)), rows, off, out) == SHAPE  # down is [E,H,I]
    assert _experts(L, g, raw_tensor(FAKE, BF16, (E + 1, I, H)), d, rows, off, out) == SHAPE
    assert _experts(L, g, u, d, raw_tensor(FAKE, BF16, (N, H + 8)), off, out) == SHAPE
    assert _experts(L, g, u, d, rows, raw_tensor(FAKE, U32, (E + 2,)), out) == SHAPE
    assert _experts(L, g, u, d, rows, off, raw_tensor(FAKE, BF16, (N + 1, H))) == SHAPE
    odd = (E, 12, H)
    assert _experts(L, raw_tensor(FAKE, BF16, odd), raw_tensor(FAKE, BF16, odd),
                    raw_tensor(FAKE, BF16, (E, H, 12)), rows, off, out) == UNSUPPORTED
    assert _experts(L, g, u, d, raw_tensor(FAKE + 2, BF16, (N, H)), off, out) == UNSUPPORTED  # unaligned
    assert _experts(L, g, u, d, rows, off, out, wsb=16) == WORKSPACE


def test_combine_validation(L):
    T, k, H, N = 8, 2, 16, 16
    y = raw_tensor(FAKE, F32, (N, H))
    ros = raw_tensor(FAKE, U32, (T * k,))
    w = raw_tensor(FAKE, F32, (T, k))
    out = raw_tensor(FAKE, F32, (T, H))
    c = lambda *a: L.moe_combine(*[ctypes.byref(t) for t in a], None)
    assert c(y, ros, w, raw_tensor(FAKE, BF16, (T, H))) == DTYPE
    assert c(y, raw_tensor(FAKE, F32, (T * k,)), w, out) == DTYPE
    assert c(y, raw_tensor(FAKE, U32, (T * k + 1,)), w, out) == SHAPE
    assert c(y, ros, w, raw_tensor(FAKE, F32, (T, H + 1))) == SHAPE
    assert c(y, ros, w, out) == DEVICE


def test_forward_validation(L):
    E, I, H, T, k = 8, 64, 32, 16, 2
    g = raw_tensor(FAKE, BF16, (E, I, H))
    u = raw_tensor(FAKE, BF16, (E, I, H))
    d = raw_tensor(FAKE, BF16, (E, H, I))
    x = raw_tensor(FAKE, BF16, (T, H))
    lg = raw_tensor(FAKE, F32, (T, E))   # logits dtype is independent of the input dtype
    out = raw_tensor(FAKE, BF16, (T, H))
    ws = L.moe_forward_workspace_bytes(T, H, I, E, k, BF16)

    def f(x=x, lg=lg, out=out, k=k, renorm=1, wsb=ws, g=g):
        return L.moe_forward(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ctypes.byref(x),
                             ctypes.byref(lg), MoeRoutingOptions(k, renorm), ctypes.byref(out),
                             ctypes.c_void_p(FAKE), wsb, None)

    assert f(lg=raw_tensor(FAKE, U32, (T, E))) == DTYPE
    assert f(x=raw_tensor(FAKE, F16, (T, H))) == DTYPE
    assert f(lg=raw_tensor(FAKE, F32, (T, E + 1))) == SHAPE
    assert f(lg=raw_tensor(FAKE, F32, (T + 1, E))) == SHAPE
    assert f(x=raw_tensor(FAKE, BF16, (T, H + 8))) == SHAPE
    assert f(k=0) == TOPK and f(k=E + 1) == TOPK
    assert f(wsb=ws - 1) == WORKSPACE
    assert f(g=raw_tensor(FAKE, F32, (E, I, H))) == DTYPE
    assert f() == DEVICE  # well-formed: only the device check is left


def test_python_layer_rejects_non_contiguous():
    import torch
    x = torch.zeros(4, 6)[:, ::2]
    with pytest.raises(moe.MoeError):
        moe.api._desc(x)


def test_route_sigmoid_grouped_validation(L):
    from mixture_experts_layer_route_amd._lib import MoeGroupRoutingOptions
    T, E = 16, 64
    lg = raw_tensor(FAKE, BF16, (T, E))
    bias = raw_tensor(FAKE, F32, (E,))

    def r(k=8, G=8, m=4, two=1, renorm=1, scale=2.5, lg=lg, bias=bias, idx=None, w=None):
        idx = idx or raw_tensor(FAKE, U32, (T, k))
        w = w or raw_tensor(FAKE, BF16, (T, k))
        o = MoeGroupRoutingOptions(k, G, m, two, renorm, scale)
        return L.moe_route_sigmoid_grouped(ctypes.byref(lg), ctypes.byref(bias) if bias is not None else None, o,
                                           ctypes.byref(idx), ctypes.byref(w), None)

    assert r(G=0) == INVALID and r(G=129) == INVALID and r(G=6) == INVALID   # 6 does not divide 64
    assert r(m=0) == INVALID and r(m=9) == INVALID
    assert r(two=2) == INVALID and r(renorm=2) == INVALID
    assert r(G=64, m=8, two=1) == INVALID                                    # one expert per group
    assert r(scale=0.0) == INVALID and r(scale=float("inf")) == INVALID and r(scale=float("nan")) == INVALID
    assert r(bias=raw_tensor(FAKE, F16, (E,))) == DTYPE
    assert r(lg=raw_tensor(FAKE, U32, (T, E))) == DTYPE
    assert r(w=raw_tensor(FAKE, F32, (T, 8))) == DTYPE                      # weights follow the logits dtype
    assert r(bias=raw_tensor(FAKE, F32, (E + 1,))) == SHAPE
    assert r(k=0) == TOPK and r(k=65) == TOPK
    assert r(k=33, m=4) == TOPK                                              # only 4 x 8 experts are kept
    assert r(idx=raw_tensor(FAKE, U32, (T, 7))) == SHAPE
    assert r(lg=raw_tensor(FAKE, BF16, (T, 2048)), bias=None) == UNSUPPORTED
    assert r() == DEVICE and r(bias=None) == DEVICE


def test_forward_sigmoid_grouped_validation(L):
    from mixture_experts_layer_route_amd._lib import MoeGroupRoutingOptions
    E, I, H, T, k = 16, 64, 32, 8, 2
    g = raw_tensor(FAKE, BF16, (E, I, H))
    u = raw_tensor(FAKE, BF16, (E, I, H))
    d = raw_tensor(FAKE, BF16, (E, H, I))
    x = raw_tensor(FAKE, BF16, (T, H))
    lg = raw_tensor(FAKE, F32, (T, E))
    out = raw_tensor(FAKE, BF16, (T, H))
    ws = L.moe_forward_workspace_bytes(T, H, I, E, k, BF16)

    def f(k=k, G=4, m=2, bias=None, lg=lg, wsb=ws):
        o = MoeGroupRoutingOptions(k, G, m, 1, 1, 1.0)
        return L.moe_forward_sigmoid_grouped(ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ctypes.byref(x),
                                             ctypes.byref(lg), ctypes.byref(bias) if bias is not None else None, o,
                                             ctypes.byref(out), ctypes.c_void_p(FAKE), wsb, None)

    assert f(G=3) == INVALID
    assert f(k=9, m=2) == TOPK
    assert f(bias=raw_tensor(FAKE, F32, (E - 1,))) == SHAPE
    assert f(bias=raw_tensor(FAKE, BF16, (E,))) == DTYPE
    assert f(lg=raw_tensor(FAKE, F32, (T, E + 4))) == SHAPE
    assert f(wsb=ws - 1) == WORKSPACE
    assert f() == DEVICE and f(bias=raw_tensor(FAKE, F32, (E,))) == DEVICE


# ---------------------------------------------------------------- first-order training
I32, I64 = _lib.MOE_I32, _lib.MOE_I64


def _rw(L, lg, idx, w, scoring=0, renorm=1, scale=1.0):
    return L.moe_router_weights(ctypes.byref(lg), ctypes.byref(idx), _lib.MoeRouterWeightOptions(scoring, renorm, scale),
                                ctypes.byref(w), None)


def _rb(L, lg, idx, gw, dl, scoring=0, renorm=1, scale=1.0):
    return L.moe_router_backward(ctypes.byref(lg), ctypes.byref(idx), ctypes.byref(gw),
                                 _lib.MoeRouterWeightOptions(scoring, renorm, scale), ctypes.byref(dl), None)


def test_router_training_validation(L):
    T, E, k = 16, 8, 2
    lg = raw_tensor(FAKE, BF16, (T, E))
    idx = raw_tensor(FAKE, I64, (T, k))
    w = raw_tensor(FAKE, F32, (T, k))
    dl = raw_tensor(FAKE, BF16, (T, E))
    assert _rw(L, lg, raw_tensor(FAKE, F32, (T, k)), w) == DTYPE                 # float indices
    assert _rw(L, raw_tensor(FAKE, U32, (T, E)), idx, w) == DTYPE                # integer logits
    assert _rw(L, lg, idx, raw_tensor(FAKE, BF16, (T, k))) == DTYPE              # weights are F32
    assert _rw(L, lg, idx, w, scoring=2) == INVALID
    assert _rw(L, lg, idx, w, renorm=2) == INVALID
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert _rw(L, lg, idx, w, scale=bad) == INVALID
    assert _rw(L, lg, raw_tensor(FAKE, U32, (T + 1, k)), w) == SHAPE
    assert _rw(L, lg, idx, raw_tensor(FAKE, F32, (T, k + 1))) == SHAPE
    assert _rw(L, lg, raw_tensor(FAKE, I32, (T, E + 1)), raw_tensor(FAKE, F32, (T, E + 1))) == TOPK
    big = raw_tensor(FAKE, F32, (T, 128))
    assert _rw(L, big, raw_tensor(FAKE, U32, (T, 65)), raw_tensor(FAKE, F32, (T, 65))) == TOPK  # k <= 64
    assert _rw(L, raw_tensor(FAKE, F32, (T, 5000)), idx, w) == UNSUPPORTED
    for dt in (U32, I32, I64):
        assert _rw(L, lg, raw_tensor(FAKE, dt, (T, k)), w) == DEVICE             # valid up to the device check
    assert _rb(L, lg, idx, w, dl) == DEVICE
    assert _rb(L, lg, idx, w, raw_tensor(FAKE, F32, (T, E))) == DTYPE            # gradient in the logits dtype
    assert _rb(L, lg, idx, w, raw_tensor(FAKE, BF16, (T, E + 1))) == SHAPE
    assert _rb(L, lg, idx, raw_tensor(FAKE, BF16, (T, k)), dl) == DTYPE          # grad_weights are F32


def test_combine_and_dispatch_backward_validation(L):
    T, k, H, N = 8, 2, 64, 16
    y = raw_tensor(FAKE, BF16, (N, H))
    ros = raw_tensor(FAKE, U32, (T * k,))
    w = raw_tensor(FAKE, F32, (T, k))
    g = raw_tensor(FAKE, BF16, (T, H))
    dy = raw_tensor(FAKE, BF16, (N, H))
    dw = raw_tensor(FAKE, F32, (T, k))

    def cb(*a):
        return L.moe_combine_backward(*[ctypes.byref(x) for x in a], None)

    assert cb(y, ros, w, g, dy, dw) == DEVICE
    assert cb(y, ros, w, raw_tensor(FAKE, F32, (T, H)), dy, dw) == DTYPE
    assert cb(y, ros, w, g, dy, raw_tensor(FAKE, BF16, (T, k))) == DTYPE
    assert cb(y, raw_tensor(FAKE, U32, (T * k + 1,)), w, g, dy, dw) == SHAPE
    assert cb(y, ros, w, g, raw_tensor(FAKE, BF16, (N + 1, H)), dw) == SHAPE
    assert cb(y, ros, w, raw_tensor(FAKE, BF16, (T, H + 8)), dy, dw) == SHAPE

    def db(rows, r, kk, dx):
        return L.moe_dispatch_backward(ctypes.byref(rows), ctypes.byref(r), kk, ctypes.byref(dx), None)

    dx = raw_tensor(FAKE, BF16, (T, H))
    assert db(dy, ros, k, dx) == DEVICE
    assert db(dy, ros, 0, dx) == TOPK
    assert db(dy, ros, k + 1, dx) == SHAPE
    assert db(dy, ros, k, raw_tensor(FAKE, F16, (T, H))) == DTYPE
    assert db(dy, ros, k, raw_tensor(FAKE, BF16, (T, H + 8))) == SHAPE
    assert db(dy, raw_tensor(None, U32, (0,)), k, raw_tensor(None, BF16, (0, H))) == OK  # T = 0


def test_experts_training_validation(L):
    E, I, H, N, T = 4, 64, 128, 32, 16
    gate = raw_tensor(FAKE, BF16, (E, I, H))
    up = raw_tensor(FAKE, BF16, (E, I, H))
    down = raw_tensor(FAKE, BF16, (E, H, I))
    rows = raw_tensor(FAKE, BF16, (T, H))
    tor = raw_tensor(FAKE, U32, (N,))
    off = raw_tensor(FAKE, U32, (E + 1,))
    out = raw_tensor(FAKE, BF16, (N, H))
    pre = raw_tensor(FAKE, F32, (N, 2 * I))
    h = raw_tensor(FAKE, BF16, (N, I))
    ws_n = L.moe_experts_workspace_bytes(N, H, I, E, BF16)

    def fwd(rows_, tor_, out_, pre_, h_, ws=ws_n):
        return L.moe_experts_forward_training(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down),
                                              ctypes.byref(rows_), ctypes.byref(tor_) if tor_ is not None else None,
                                              ctypes.byref(off), ctypes.byref(out_), ctypes.byref(pre_),
                                              ctypes.byref(h_), FAKE, ws, None)

    assert fwd(rows, tor, out, pre, h) == DEVICE
    assert fwd(rows, None, out, pre, h) == SHAPE                       # rows are then the N dispatched rows
    assert fwd(raw_tensor(FAKE, BF16, (N, H)), None, out, pre, h) == DEVICE
    assert fwd(rows, tor, out, raw_tensor(FAKE, BF16, (N, 2 * I)), h) == DTYPE   # preact is F32
    assert fwd(rows, tor, out, raw_tensor(FAKE, F32, (N, I)), h) == SHAPE
    assert fwd(rows, tor, out, pre, raw_tensor(FAKE, F32, (N, I))) == DTYPE
    assert fwd(rows, tor, out, pre, h, ws=ws_n - 1) == WORKSPACE
    assert fwd(rows, tor, out, pre, raw_tensor(FAKE + 8, BF16, (N, I))) == UNSUPPORTED  # misaligned

    ws_b = L.moe_experts_backward_workspace_bytes(N, H, I, E, BF16)
    assert ws_b >= N * 2 * I * 2
    assert L.moe_experts_backward_workspace_bytes(N, H, I, E, U32) == 0
    dy = raw_tensor(FAKE, BF16, (N, H))
    dx = raw_tensor(FAKE, BF16, (N, H))
    dg = raw_tensor(FAKE, F32, (E, I, H))
    du = raw_tensor(FAKE, F32, (E, I, H))
    dd = raw_tensor(FAKE, F32, (E, H, I))

    def bwd(dg_=dg, du_=du, dd_=dd, dy_=dy, ws=ws_b):
        return L.moe_experts_backward(ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), ctypes.byref(rows),
                                      ctypes.byref(tor), ctypes.byref(off), ctypes.byref(pre), ctypes.byref(h),
                                      ctypes.byref(dy_), ctypes.byref(dx), ctypes.byref(dg_), ctypes.byref(du_),
                                      ctypes.byref(dd_), FAKE, ws, None)

    assert bwd() == DEVICE
    assert bwd(dg_=raw_tensor(FAKE, BF16, (E, I, H))) == DTYPE          # weight gradients are F32
    assert bwd(dd_=raw_tensor(FAKE, F32, (E, I, H))) == SHAPE           # ddown is [E,H,I]
    assert bwd(dy_=raw_tensor(FAKE, BF16, (N + 1, H))) == SHAPE
    assert bwd(ws=ws_b - 1) == WORKSPACE
