"""Plain CPU oracle of the local MoE forward chain (ctypes wrapper of moe_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product
package never does.  It shares no code with the HIP library.

The chain follows the ruDNN User Guide (ruDNN 0.1.5 on docs.rs), sections 3-6:
FP32 softmax over all experts, top-k with ties to the lower expert id,
optional renormalisation, cast of the weights to the logits dtype, a
drop-free dispatch grouped by expert, SwiGLU experts
``down_e(silu(gate_e x) * up_e x)`` and a weighted combine in token order.
Expert and combine sums are taken in binary64 (tiny-llm deep dive 5, the
RMSNorm block's reason for wide accumulators).

The first-order training functions follow the RUDA ruDNN library guide,
section 12: router weights of a fixed selection and their logits gradient,
the combine, expert and dispatch backward passes.

Arrays are numpy: F32 data as ``float32``; F16 and BF16 data as their raw
``uint16`` bit patterns; indices and mappings as ``uint32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

DT = {"f32": 0, "f16": 1, "bf16": 2}
INVALID_ROW = 0xFFFFFFFF


def build(force: bool = True) -> str:
    """Compile moe_oracle.c with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-std=c11", "-O2", "-fPIC", "-shared", "-pthread",
               "-ffp-contract=off", "-fno-fast-math", "-D_GNU_SOURCE",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_double
        L.oracle_round_f32.restype = dp
        L.oracle_round_f16.restype = dp
        L.oracle_round_bf16.restype = dp
        for f in (L.oracle_round_f32, L.oracle_round_f16, L.oracle_round_bf16):
            f.argtypes = [dp]
        L.oracle_silu.restype = dp
        L.oracle_silu.argtypes = [dp]
        L.oracle_widen.argtypes = [vp, i32, i64, vp]
        L.oracle_narrow.argtypes = [vp, i32, i64, vp]
        L.oracle_softmax.argtypes = [vp, i32, i64, i64, vp]
        L.oracle_route.restype = i32
        L.oracle_route.argtypes = [vp, i32, i64, i64, i32, i32, vp, vp, vp, i32]
        L.oracle_route_sigmoid_grouped.restype = i32
        L.oracle_route_sigmoid_grouped.argtypes = [vp, i32, vp, i64, i64, i32, i32, i32, i32, i32,
                                                   ctypes.c_float, vp, vp, vp, vp, i32]
        L.oracle_dispatch.restype = i32
        L.oracle_dispatch.argtypes = [vp, i64, i32, i64, vp, i64, i32, vp, vp, vp, vp]
        L.oracle_experts.restype = i32
        L.oracle_experts.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, vp, vp, i32]
        L.oracle_combine.restype = i32
        L.oracle_combine.argtypes = [vp, i32, vp, vp, i32, i64, i32, i64, vp, i32]
        f32 = ctypes.c_float
        L.oracle_router_weights.restype = i32
        L.oracle_router_weights.argtypes = [vp, i32, vp, i64, i64, i32, i32, i32, f32, vp, i32]
        L.oracle_router_backward.restype = i32
        L.oracle_router_backward.argtypes = [vp, i32, vp, vp, i64, i64, i32, i32, i32, f32, vp, i32]
        L.oracle_combine_backward.restype = i32
        L.oracle_combine_backward.argtypes = [vp, i32, vp, vp, i32, vp, i64, i32, i64, i64, vp, vp, i32]
        L.oracle_dispatch_backward.restype = i32
        L.oracle_dispatch_backward.argtypes = [vp, i32, vp, i64, i32, i64, i64, vp, i32]
        L.oracle_experts_train_forward.restype = i32
        L.oracle_experts_train_forward.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, vp, vp, vp, vp, i32]
        L.oracle_experts_backward.restype = i32
        L.oracle_experts_backward.argtypes = [vp, vp, vp, i32, vp, vp, i64, i64, i64, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, i32]
        _lib = L
    return _lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


def _ptr(a: np.ndarray) -> int:
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


def storage_dtype(dt: str):
    return np.float32 if dt == "f32" else np.uint16


def _check(a: np.ndarray, dt: str, name: str) -> np.ndarray:
    want = storage_dtype(dt)
    if a.dtype != want:
        raise TypeError(f"{name}: expected {np.dtype(want)} storage for {dt}, got {a.dtype}")
    return np.ascontiguousarray(a)


# ---------------------------------------------------------------- formats
def round_scalar(x: float, dt: str) -> float:
    return {"f32": lib().oracle_round_f32, "f16": lib().oracle_round_f16,
            "bf16": lib().oracle_round_bf16}[dt](float(x))


def widen(bits: np.ndarray, dt: str) -> np.ndarray:
    """Values of a stored array, as float64 (exact)."""
    a = _check(bits, dt, "bits")
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_widen(_ptr(a), DT[dt], a.size, _ptr(out))
    return out


def narrow(vals: np.ndarray, dt: str) -> np.ndarray:
    """Round float64 values once (nearest, ties to even) to dtype ``dt``."""
    v = np.ascontiguousarray(vals, dtype=np.float64)
    out = np.empty(v.shape, dtype=storage_dtype(dt))
    lib().oracle_narrow(_ptr(v), DT[dt], v.size, _ptr(out))
    return out


def silu(z: float) -> float:
    return lib().oracle_silu(float(z))


# ---------------------------------------------------------------- routing
def softmax(logits: np.ndarray, dt: str) -> np.ndarray:
    lg = _check(logits, dt, "logits")
    T, E = lg.shape
    p = np.empty((T, E), dtype=np.float32)
    lib().oracle_softmax(_ptr(lg), DT[dt], T, E, _ptr(p))
    return p


def route(logits: np.ndarray, dt: str, top_k: int, renormalize: bool, nthreads: int | None = None):
    """Returns (indices u32 [T,k], weights [T,k] in the logits dtype, FP32 weights before the cast)."""
    lg = _check(logits, dt, "logits")
    T, E = lg.shape
    idx = np.empty((T, top_k), dtype=np.uint32)
    w = np.empty((T, top_k), dtype=storage_dtype(dt))
    w32 = np.empty((T, top_k), dtype=np.float32)
    rc = lib().oracle_route(_ptr(lg), DT[dt], T, E, int(top_k), int(bool(renormalize)),
                            _ptr(idx), _ptr(w), _ptr(w32), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_route: bad arguments")
    return idx, w, w32


def route_sigmoid_grouped(logits: np.ndarray, dt: str, bias: np.ndarray | None, top_k: int, groups: int,
                          selected_groups: int, group_top_two: bool, renormalize: bool, scale: float,
                          nthreads: int | None = None):
    """Group-limited sigmoid routing (ruDNN user guide, section 10).

    Returns (indices u32 [T,k], weights [T,k] in the logits dtype, FP32
    weights before the cast, corrected scores sigmoid(l) + bias [T,E] FP32)."""
    lg = _check(logits, dt, "logits")
    T, E = lg.shape
    b = None if bias is None else np.ascontiguousarray(bias, dtype=np.float32)
    if b is not None and b.shape != (E,):
        raise ValueError("bias must be [E] float32")
    idx = np.empty((T, top_k), dtype=np.uint32)
    w = np.empty((T, top_k), dtype=storage_dtype(dt))
    w32 = np.empty((T, top_k), dtype=np.float32)
    corr = np.empty((T, E), dtype=np.float32)
    rc = lib().oracle_route_sigmoid_grouped(_ptr(lg), DT[dt], _ptr(b) if b is not None else None, T, E,
                                            int(top_k), int(groups), int(selected_groups),
                                            int(bool(group_top_two)), int(bool(renormalize)), float(scale),
                                            _ptr(idx), _ptr(w), _ptr(w32), _ptr(corr),
                                            nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_route_sigmoid_grouped: options outside the section's limits")
    return idx, w, w32, corr


# ---------------------------------------------------------------- dispatch
def dispatch(indices: np.ndarray, E: int, x: np.ndarray, dt: str):
    """Returns (offsets [E+1], row_of_slot [T*k], token_of_row [n_valid], rows [n_valid,H])."""
    idx = np.ascontiguousarray(indices, dtype=np.uint32)
    xs = _check(x, dt, "x")
    T, k = idx.shape
    H = xs.shape[1]
    n_valid = int(np.count_nonzero(idx < E))
    offsets = np.empty(E + 1, dtype=np.uint32)
    ros = np.empty(T * k, dtype=np.uint32)
    tor = np.empty(max(n_valid, 1), dtype=np.uint32)
    rows = np.empty((max(n_valid, 1), H), dtype=storage_dtype(dt))
    rc = lib().oracle_dispatch(_ptr(idx), T, k, E, _ptr(xs), H, DT[dt],
                               _ptr(offsets), _ptr(ros), _ptr(tor), _ptr(rows))
    if rc != 0:
        raise ValueError("oracle_dispatch: bad arguments")
    return offsets, ros, tor[:n_valid], rows[:n_valid]


# ---------------------------------------------------------------- experts
def _expert_ptrs(w, E: int, dt: str, keep: list):
    """w: full array [E, a, b] or dict {expert: [a, b]} -> array of E pointers."""
    arr = (ctypes.c_void_p * E)()
    if isinstance(w, dict):
        for e, m in w.items():
            m = _check(m, dt, "weight")
            keep.append(m)
            arr[int(e)] = _ptr(m)
    else:
        w = _check(w, dt, "weight")
        keep.append(w)
        step = w.shape[1] * w.shape[2] * w.itemsize
        for e in range(E):
            arr[e] = w.ctypes.data + e * step
    return arr


def experts(gate, up, down, dt: str, rows: np.ndarray, offsets: np.ndarray, E: int, H: int, I: int,
            with_h: bool = False, nthreads: int | None = None):
    """SwiGLU experts on grouped rows: y_r = down_e (silu(gate_e x_r) * up_e x_r)."""
    keep: list = []
    g = _expert_ptrs(gate, E, dt, keep)
    u = _expert_ptrs(up, E, dt, keep)
    d = _expert_ptrs(down, E, dt, keep)
    r = _check(rows, dt, "rows") if rows.size else np.empty((1, H), dtype=storage_dtype(dt))
    off = np.ascontiguousarray(offsets, dtype=np.uint32)
    n = int(off[E])
    out = np.empty((max(n, 1), H), dtype=storage_dtype(dt))
    h = np.empty((max(n, 1), I), dtype=storage_dtype(dt)) if with_h else None
    rc = lib().oracle_experts(ctypes.cast(g, ctypes.c_void_p), ctypes.cast(u, ctypes.c_void_p),
                              ctypes.cast(d, ctypes.c_void_p), DT[dt], _ptr(r), _ptr(off),
                              E, H, I, _ptr(out), _ptr(h) if with_h else None,
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_experts: a row's expert has no weights")
    if with_h:
        return out[:n], h[:n]
    return out[:n]


# ---------------------------------------------------------------- combine
def combine(Y: np.ndarray, dt: str, row_of_slot: np.ndarray, weights: np.ndarray, wdt: str,
            T: int, k: int, H: int, nthreads: int | None = None) -> np.ndarray:
    Ys = _check(Y, dt, "Y") if Y.size else np.empty((1, H), dtype=storage_dtype(dt))
    ros = np.ascontiguousarray(row_of_slot, dtype=np.uint32)
    w = _check(weights, wdt, "weights")
    out = np.empty((T, H), dtype=storage_dtype(dt))
    rc = lib().oracle_combine(_ptr(Ys), DT[dt], _ptr(ros), _ptr(w), DT[wdt], T, k, H, _ptr(out),
                              nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_combine: bad arguments")
    return out


# ---------------------------------------------------------------- whole chain
def forward(x: np.ndarray, logits: np.ndarray, gate, up, down, dt: str, ldt: str, top_k: int,
            renormalize: bool, nthreads: int | None = None) -> dict:
    """The whole local chain; returns every intermediate in a dict."""
    T, H = x.shape
    E = logits.shape[1]
    if isinstance(gate, dict):
        I = next(iter(gate.values())).shape[0]
    else:
        I = gate.shape[1]
    idx, w, w32 = route(logits, ldt, top_k, renormalize, nthreads)
    offsets, ros, tor, rows = dispatch(idx, E, x, dt)
    Y, h = experts(gate, up, down, dt, rows, offsets, E, H, I, with_h=True, nthreads=nthreads)
    out = combine(Y, dt, ros, w, ldt, T, top_k, H, nthreads)
    return {"indices": idx, "weights": w, "weights_f32": w32, "offsets": offsets,
            "row_of_slot": ros, "token_of_row": tor, "dispatched": rows, "h": h, "Y": Y,
            "output": out}


# ---------------------------------------------------------------- training
SCORING = {"softmax": 0, "sigmoid": 1}


def _indices_i64(indices: np.ndarray) -> np.ndarray:
    """U32, I32 or I64 indices as int64 values (a U32 index keeps its value)."""
    a = np.asarray(indices)
    if a.dtype not in (np.uint32, np.int32, np.int64):
        raise TypeError(f"indices must be u32, i32 or i64, got {a.dtype}")
    return np.ascontiguousarray(a.astype(np.int64))


def router_weights(logits: np.ndarray, dt: str, indices: np.ndarray, scoring: str, renormalize: bool,
                   scale: float, nthreads: int | None = None) -> np.ndarray:
    """FP32 [T,k] weights of a fixed selection (RUDA ruDNN guide, section 12)."""
    lg = _check(logits, dt, "logits")
    T, E = lg.shape
    idx = _indices_i64(indices)
    k = idx.shape[1]
    w = np.empty((T, k), dtype=np.float32)
    rc = lib().oracle_router_weights(_ptr(lg), DT[dt], _ptr(idx), T, E, k, SCORING[scoring],
                                     int(bool(renormalize)), float(scale), _ptr(w), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_router_weights: bad arguments")
    return w


def router_backward(logits: np.ndarray, dt: str, indices: np.ndarray, grad_weights: np.ndarray, scoring: str,
                    renormalize: bool, scale: float, nthreads: int | None = None) -> np.ndarray:
    """[T,E] logits gradient in the logits dtype for FP32 weight gradients [T,k]."""
    lg = _check(logits, dt, "logits")
    T, E = lg.shape
    idx = _indices_i64(indices)
    k = idx.shape[1]
    gw = np.ascontiguousarray(grad_weights, dtype=np.float32)
    if gw.shape != (T, k):
        raise ValueError("grad_weights must be [T,k]")
    dl = np.empty((T, E), dtype=storage_dtype(dt))
    rc = lib().oracle_router_backward(_ptr(lg), DT[dt], _ptr(idx), _ptr(gw), T, E, k, SCORING[scoring],
                                      int(bool(renormalize)), float(scale), _ptr(dl), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_router_backward: bad arguments")
    return dl


def combine_backward(Y: np.ndarray, dt: str, row_of_slot: np.ndarray, weights: np.ndarray, wdt: str,
                     grad_output: np.ndarray, T: int, k: int, H: int, nthreads: int | None = None):
    """Returns (dY [N,H] in the expert dtype, dweights [T,k] FP32)."""
    N = Y.shape[0]
    Ys = _check(Y, dt, "Y") if Y.size else np.empty((1, H), dtype=storage_dtype(dt))
    ros = np.ascontiguousarray(row_of_slot, dtype=np.uint32)
    w = _check(weights, wdt, "weights")
    g = _check(grad_output, dt, "grad_output")
    dY = np.empty((max(N, 1), H), dtype=storage_dtype(dt))
    dw = np.empty((T, k), dtype=np.float32)
    rc = lib().oracle_combine_backward(_ptr(Ys), DT[dt], _ptr(ros), _ptr(w), DT[wdt], _ptr(g), T, k, H, N,
                                       _ptr(dY), _ptr(dw), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_combine_backward: bad arguments")
    return dY[:N], dw


def dispatch_backward(dinput: np.ndarray, dt: str, row_of_slot: np.ndarray, T: int, k: int, H: int,
                      nthreads: int | None = None) -> np.ndarray:
    """dx [T,H]: each token's dispatched-row gradients summed, weights not applied."""
    N = dinput.shape[0]
    d = _check(dinput, dt, "dinput") if dinput.size else np.empty((1, H), dtype=storage_dtype(dt))
    ros = np.ascontiguousarray(row_of_slot, dtype=np.uint32)
    dx = np.empty((T, H), dtype=storage_dtype(dt))
    rc = lib().oracle_dispatch_backward(_ptr(d), DT[dt], _ptr(ros), T, k, H, N, _ptr(dx),
                                        nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_dispatch_backward: bad arguments")
    return dx


def experts_train_forward(gate, up, down, dt: str, rows: np.ndarray, offsets: np.ndarray, E: int, H: int, I: int,
                          nthreads: int | None = None) -> dict:
    """The experts' forward plus what their backward needs: the FP32
    pre-activations g = gate x, u = up x and the stored activation h."""
    keep: list = []
    gp = _expert_ptrs(gate, E, dt, keep)
    up_ = _expert_ptrs(up, E, dt, keep)
    dp = _expert_ptrs(down, E, dt, keep)
    r = _check(rows, dt, "rows") if rows.size else np.empty((1, H), dtype=storage_dtype(dt))
    off = np.ascontiguousarray(offsets, dtype=np.uint32)
    n = int(off[E])
    m = max(n, 1)
    out = np.empty((m, H), dtype=storage_dtype(dt))
    h = np.empty((m, I), dtype=storage_dtype(dt))
    g = np.empty((m, I), dtype=np.float32)
    u = np.empty((m, I), dtype=np.float32)
    rc = lib().oracle_experts_train_forward(ctypes.cast(gp, ctypes.c_void_p), ctypes.cast(up_, ctypes.c_void_p),
                                            ctypes.cast(dp, ctypes.c_void_p), DT[dt], _ptr(r), _ptr(off),
                                            E, H, I, _ptr(out), _ptr(h), _ptr(g), _ptr(u),
                                            nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_experts_train_forward: a row's expert has no weights")
    return {"output": out[:n], "h": h[:n], "g": g[:n], "u": u[:n]}


def experts_backward(gate, up, down, dt: str, rows: np.ndarray, offsets: np.ndarray, E: int, H: int, I: int,
                     g: np.ndarray, u: np.ndarray, h: np.ndarray, dY: np.ndarray, nthreads: int | None = None,
                     with_dgu: bool = False):
    """Returns (dinput [N,H] in the expert dtype, dgate [E,I,H], dup [E,I,H], ddown [E,H,I] FP32), and with
    ``with_dgu`` also the rounded intermediates dg | du [N,2I] as float64."""
    keep: list = []
    gp = _expert_ptrs(gate, E, dt, keep)
    up_ = _expert_ptrs(up, E, dt, keep)
    dp = _expert_ptrs(down, E, dt, keep)
    off = np.ascontiguousarray(offsets, dtype=np.uint32)
    n = int(off[E])
    m = max(n, 1)

    def pad(a, cols, storage):
        a = np.ascontiguousarray(a, dtype=storage) if storage == np.float32 else _check(a, dt, "array")
        return a if a.size else np.zeros((1, cols), dtype=storage)

    r = pad(rows, H, storage_dtype(dt))
    g_ = pad(g, I, np.float32)
    u_ = pad(u, I, np.float32)
    h_ = pad(h, I, storage_dtype(dt))
    dy = pad(dY, H, storage_dtype(dt))
    dx = np.empty((m, H), dtype=storage_dtype(dt))
    dgate = np.empty((E, I, H), dtype=np.float32)
    dup = np.empty((E, I, H), dtype=np.float32)
    ddown = np.empty((E, H, I), dtype=np.float32)
    dgu = np.empty((m, 2 * I), dtype=np.float64) if with_dgu else None
    rc = lib().oracle_experts_backward(ctypes.cast(gp, ctypes.c_void_p), ctypes.cast(up_, ctypes.c_void_p),
                                       ctypes.cast(dp, ctypes.c_void_p), DT[dt], _ptr(r), _ptr(off), E, H, I,
                                       _ptr(g_), _ptr(u_), _ptr(h_), _ptr(dy), _ptr(dx), _ptr(dgate), _ptr(dup),
                                       _ptr(ddown), _ptr(dgu) if with_dgu else None, nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle_experts_backward: a row's expert has no weights")
    if with_dgu:
        return dx[:n], dgate, dup, ddown, dgu[:n]
    return dx[:n], dgate, dup, ddown


def train_step(x: np.ndarray, logits: np.ndarray, gate, up, down, dt: str, ldt: str, top_k: int,
               renormalize: bool, grad_output: np.ndarray, nthreads: int | None = None,
               indices: np.ndarray | None = None, scoring: str = "softmax", scale: float = 1.0) -> dict:
    """Forward of the chain with training caches, then the section's four
    backward steps in order: combine, experts, dispatch, router.  The
    selection is the softmax route's unless ``indices`` [T,k] (U32) is given."""
    T, H = x.shape
    E = logits.shape[1]
    I = gate.shape[1]
    if indices is None:
        idx, _, _ = route(logits, ldt, top_k, renormalize, nthreads)
    else:
        idx = np.ascontiguousarray(indices, dtype=np.uint32)
    w32 = router_weights(logits, ldt, idx, scoring, renormalize, scale, nthreads)
    offsets, ros, tor, rows = dispatch(idx, E, x, dt)
    fw = experts_train_forward(gate, up, down, dt, rows, offsets, E, H, I, nthreads)
    out = combine(fw["output"], dt, ros, w32, "f32", T, top_k, H, nthreads)
    dY, dw = combine_backward(fw["output"], dt, ros, w32, "f32", grad_output, T, top_k, H, nthreads)
    drows, dgate, dup, ddown, dgu = experts_backward(gate, up, down, dt, rows, offsets, E, H, I, fw["g"],
                                                     fw["u"], fw["h"], dY, nthreads, with_dgu=True)
    dx = dispatch_backward(drows, dt, ros, T, top_k, H, nthreads)
    dl = router_backward(logits, ldt, idx, dw, scoring, renormalize, scale, nthreads)
    return {"indices": idx, "weights_f32": w32, "offsets": offsets, "row_of_slot": ros, "dispatched": rows,
            "Y": fw["output"], "h": fw["h"], "g": fw["g"], "u": fw["u"], "output": out, "dY": dY,
            "dweights": dw, "drows": drows, "dgu": dgu, "dgate": dgate, "dup": dup, "ddown": ddown, "dx": dx,
            "dlogits": dl}
