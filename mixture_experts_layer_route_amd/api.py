"""Python face of libmoe.so, shaped like the ruDNN MoE API.

The objects mirror the ruDNN User Guide (ruDNN 0.1.5 on docs.rs), section 6
"Call MoE": ``route(logits, options)`` gives a ``RoutingPlan`` with
``expert_indices()``, ``weights()`` and ``dispatch(input)``; dispatching gives
``DispatchedTokens`` whose ``combine(expert_output)`` restores token order;
``SwiGluExperts(gate, up, down)`` holds the weights and runs ``forward`` (the
whole chain from precomputed logits) or ``forward_dispatched``.  Errors come
back as ``MoeError`` (the guide's section 3 error convention).

First-order training follows the RUDA ruDNN library guide, section 12:
``RoutingPlan.into_training(logits, options)`` keeps the selection and
recomputes FP32 weights (``selected_router_weights``);
``SwiGluExperts.forward_dispatched_training`` returns the output and an
``ExpertsCache``; the backward then runs ``DispatchedTokens.combine_backward``,
``ExpertsCache.backward``, ``DispatchedTokens.dispatch_backward`` and
``RouterTrainingPlan.backward``, in that order.

This module only allocates torch tensors and passes pointers and extents
to the C ABI: every step of the chain runs in the HIP kernels.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import MoeError, MoeGroupRoutingOptions, MoeRouterWeightOptions, MoeRoutingOptions, MoeTensor

_DTYPES = {
    torch.float32: _lib.MOE_F32,
    torch.float16: _lib.MOE_F16,
    torch.bfloat16: _lib.MOE_BF16,
    torch.uint32: _lib.MOE_U32,
    torch.int32: _lib.MOE_I32,
    torch.int64: _lib.MOE_I64,
}


def _dtype_code(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise MoeError(2, f"unsupported tensor dtype {t.dtype}") from None


def _desc(t: torch.Tensor) -> MoeTensor:
    if not t.is_contiguous():
        raise MoeError(1, "tensors must be contiguous (dense row-major)")
    if t.dim() < 1 or t.dim() > 3:
        raise MoeError(1, f"tensors must have 1 to 3 dims, got {t.dim()}")
    d = MoeTensor()
    d.data = t.data_ptr() if t.numel() else None
    d.dtype = _dtype_code(t)
    d.ndim = t.dim()
    for i, s in enumerate(t.shape):
        d.dims[i] = int(s)
    return d


def _stream(device: torch.device) -> ctypes.c_void_p:
    # a tensor that is not on a GPU still gets the current stream; the
    # library's device check then refuses its pointer with MOE_ERR_DEVICE
    if device.type != "cuda":
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _ref(d: MoeTensor):
    return ctypes.byref(d)


@dataclass(frozen=True)
class RoutingOptions:
    """top_k with 1 <= top_k <= E; renormalize the selected weights or not."""
    top_k: int
    renormalize: bool = True

    def _c(self) -> MoeRoutingOptions:
        return MoeRoutingOptions(int(self.top_k), int(bool(self.renormalize)))


@dataclass(frozen=True)
class GroupRoutingOptions:
    """Group-limited sigmoid routing (section 10): top_k in 1..64; `groups`
    contiguous groups of E/groups experts (1..128); the `selected_groups` best
    groups, scored by their largest corrected score or, with group_top_two,
    the sum of their two largest; renormalize; a finite positive scale."""
    top_k: int
    groups: int
    selected_groups: int
    group_top_two: bool = True
    renormalize: bool = True
    scale: float = 1.0

    def _c(self) -> MoeGroupRoutingOptions:
        return MoeGroupRoutingOptions(int(self.top_k), int(self.groups), int(self.selected_groups),
                                      int(bool(self.group_top_two)), int(bool(self.renormalize)), float(self.scale))


@dataclass(frozen=True)
class RouterWeightOptions:
    """Weights of a fixed selection (section 12): scoring "softmax" (FP32
    softmax over all experts) or "sigmoid"; renormalize over the selection;
    a finite positive scale applied last."""
    scoring: str = "softmax"
    renormalize: bool = True
    scale: float = 1.0

    def _c(self) -> MoeRouterWeightOptions:
        codes = {"softmax": _lib.MOE_SCORING_SOFTMAX, "sigmoid": _lib.MOE_SCORING_SIGMOID}
        if self.scoring not in codes:
            raise MoeError(1, f"scoring must be 'softmax' or 'sigmoid', got {self.scoring!r}")
        return MoeRouterWeightOptions(codes[self.scoring], int(bool(self.renormalize)), float(self.scale))


def _workspace(nbytes: int, device) -> torch.Tensor:
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


class RoutingPlan:
    """Selected experts [T,k] (U32) and weights [T,k] (logits dtype)."""

    def __init__(self, indices: torch.Tensor, weights: torch.Tensor, num_experts: int):
        self._indices = indices
        self._weights = weights
        self.num_experts = int(num_experts)

    def expert_indices(self) -> torch.Tensor:
        return self._indices

    def weights(self) -> torch.Tensor:
        return self._weights

    @property
    def top_k(self) -> int:
        return int(self._indices.shape[1])

    def dispatch(self, input: torch.Tensor, copy_rows: bool = True) -> "DispatchedTokens":
        return dispatch(input, self._indices, self.num_experts, self._weights, copy_rows)

    def into_training(self, logits: torch.Tensor, options: RouterWeightOptions) -> "RouterTrainingPlan":
        """Keep this selection and recompute its weights in FP32 (selected_router_weights)."""
        return RouterTrainingPlan(logits, self._indices, options)


class RouterTrainingPlan:
    """A fixed selection with FP32 weights recomputed from the logits; the
    logits and indices are kept for the backward and must not change."""

    def __init__(self, logits: torch.Tensor, indices: torch.Tensor, options: RouterWeightOptions):
        self.logits, self.indices, self.options = logits, indices, options
        self._weights = router_weights(logits, indices, options)

    def weights(self) -> torch.Tensor:
        return self._weights

    def routing(self) -> RoutingPlan:
        """The plan to dispatch and combine with (FP32 weights)."""
        if self.indices.dtype != torch.uint32:
            raise MoeError(2, "dispatch takes U32 indices")
        return RoutingPlan(self.indices, self._weights, int(self.logits.shape[1]))

    def backward(self, grad_weights: torch.Tensor) -> torch.Tensor:
        """d loss / d logits (selected_router_backward)."""
        return router_backward(self.logits, self.indices, grad_weights, self.options)


def router_weights(logits: torch.Tensor, indices: torch.Tensor, options: RouterWeightOptions) -> torch.Tensor:
    """FP32 [T,k] weights of the experts in `indices` (moe_router_weights)."""
    L = _lib.load()
    T, k = indices.shape
    w = torch.empty((T, k), dtype=torch.float32, device=logits.device)
    dl, di, dw = _desc(logits), _desc(indices), _desc(w)
    _lib.check(L.moe_router_weights(_ref(dl), _ref(di), options._c(), _ref(dw), _stream(logits.device)),
               "moe_router_weights")
    return w


def router_backward(logits: torch.Tensor, indices: torch.Tensor, grad_weights: torch.Tensor,
                    options: RouterWeightOptions) -> torch.Tensor:
    """[T,E] logits gradient in the logits dtype (moe_router_backward)."""
    L = _lib.load()
    dlog = torch.empty_like(logits)
    d = [_desc(x) for x in (logits, indices, grad_weights, dlog)]
    _lib.check(L.moe_router_backward(_ref(d[0]), _ref(d[1]), _ref(d[2]), options._c(), _ref(d[3]),
                                     _stream(logits.device)), "moe_router_backward")
    return dlog


def route(logits: torch.Tensor, options: RoutingOptions) -> RoutingPlan:
    """FP32 softmax + top-k routing of [T,E] logits (moe_route)."""
    L = _lib.load()
    T, E = logits.shape
    k = int(options.top_k)
    idx = torch.empty((T, max(k, 0)), dtype=torch.uint32, device=logits.device)
    w = torch.empty((T, max(k, 0)), dtype=logits.dtype, device=logits.device)
    dl, di, dw = _desc(logits), _desc(idx), _desc(w)
    _lib.check(L.moe_route(_ref(dl), options._c(), _ref(di), _ref(dw), _stream(logits.device)), "moe_route")
    return RoutingPlan(idx, w, E)


def route_sigmoid_grouped(logits: torch.Tensor, bias: torch.Tensor | None,
                          options: GroupRoutingOptions) -> RoutingPlan:
    """Group-limited sigmoid routing of [T,E] logits with an optional FP32
    correction bias [E] that steers the choice only (moe_route_sigmoid_grouped)."""
    L = _lib.load()
    T, E = logits.shape
    k = int(options.top_k)
    idx = torch.empty((T, max(k, 0)), dtype=torch.uint32, device=logits.device)
    w = torch.empty((T, max(k, 0)), dtype=logits.dtype, device=logits.device)
    dl, di, dw = _desc(logits), _desc(idx), _desc(w)
    db = _desc(bias) if bias is not None else None
    _lib.check(L.moe_route_sigmoid_grouped(_ref(dl), _ref(db) if db is not None else None, options._c(),
                                           _ref(di), _ref(dw), _stream(logits.device)),
               "moe_route_sigmoid_grouped")
    return RoutingPlan(idx, w, E)


class DispatchedTokens:
    """Rows grouped by expert plus the saved mapping back to tokens."""

    def __init__(self, rows, expert_offsets, row_of_slot, token_of_row, weights, num_tokens, top_k):
        self.rows = rows                      # [T*k, H], or None when no rows were copied
        self.expert_offsets = expert_offsets  # [E+1] U32
        self.row_of_slot = row_of_slot        # [T*k] U32
        self.token_of_row = token_of_row      # [T*k] U32
        self.routing_weights = weights        # [T,k] or None
        self.num_tokens = int(num_tokens)
        self.top_k = int(top_k)

    def combine(self, expert_output: torch.Tensor, weights: torch.Tensor | None = None) -> torch.Tensor:
        w = self.routing_weights if weights is None else weights
        if w is None:
            raise MoeError(1, "combine needs routing weights")
        return combine(expert_output, self.row_of_slot, w)

    def combine_backward(self, expert_output: torch.Tensor, grad_output: torch.Tensor,
                         weights: torch.Tensor | None = None):
        """Step 1 of the backward: (dexpert [N,H], FP32 dweights [T,k]) (moe_combine_backward)."""
        w = self.routing_weights if weights is None else weights
        if w is None:
            raise MoeError(1, "combine_backward needs routing weights")
        return combine_backward(expert_output, self.row_of_slot, w, grad_output)

    def dispatch_backward(self, grad_rows: torch.Tensor) -> torch.Tensor:
        """Step 3: each token's row gradients summed, weights not applied (moe_dispatch_backward)."""
        return dispatch_backward(grad_rows, self.row_of_slot, self.top_k, self.num_tokens)


def dispatch(input: torch.Tensor, indices: torch.Tensor, num_experts: int,
             weights: torch.Tensor | None = None, copy_rows: bool = True) -> DispatchedTokens:
    """Compact, drop-free dispatch of [T,H] tokens by expert (moe_dispatch).

    With copy_rows=False only the offsets and the mapping are written (for
    SwiGluExperts.gate_up_gathered, which reads the tokens in place)."""
    L = _lib.load()
    T, H = input.shape
    k = int(indices.shape[1])
    dev = input.device
    rows = torch.empty((T * k, H), dtype=input.dtype, device=dev) if copy_rows else None
    offsets = torch.empty((num_experts + 1,), dtype=torch.uint32, device=dev)
    ros = torch.empty((T * k,), dtype=torch.uint32, device=dev)
    tor = torch.empty((T * k,), dtype=torch.uint32, device=dev)
    ws = _workspace(L.moe_dispatch_workspace_bytes(T, num_experts, k), dev)
    d = [_desc(x) if x is not None else None for x in (input, indices, rows, offsets, ros, tor)]
    st = L.moe_dispatch(_ref(d[0]), _ref(d[1]), int(num_experts), _ref(d[2]) if d[2] is not None else None,
                        _ref(d[3]), _ref(d[4]), _ref(d[5]), ctypes.c_void_p(ws.data_ptr()), ws.numel(),
                        _stream(dev))
    _lib.check(st, "moe_dispatch")
    return DispatchedTokens(rows, offsets, ros, tor, weights, T, k)


def combine(expert_output: torch.Tensor, row_of_slot: torch.Tensor, weights: torch.Tensor) -> torch.Tensor:
    """Weighted combine back into token order (moe_combine)."""
    L = _lib.load()
    T = weights.shape[0]
    out = torch.empty((T, expert_output.shape[1]), dtype=expert_output.dtype, device=expert_output.device)
    d = [_desc(x) for x in (expert_output, row_of_slot, weights, out)]
    _lib.check(L.moe_combine(_ref(d[0]), _ref(d[1]), _ref(d[2]), _ref(d[3]), _stream(out.device)),
               "moe_combine")
    return out


def combine_backward(expert_output: torch.Tensor, row_of_slot: torch.Tensor, weights: torch.Tensor,
                     grad_output: torch.Tensor):
    """(grad_expert_out [N,H], grad_weights [T,k] FP32) (moe_combine_backward)."""
    L = _lib.load()
    T, k = weights.shape
    dy = torch.empty_like(expert_output)
    dw = torch.empty((T, k), dtype=torch.float32, device=expert_output.device)
    d = [_desc(x) for x in (expert_output, row_of_slot, weights, grad_output, dy, dw)]
    _lib.check(L.moe_combine_backward(*[_ref(x) for x in d], _stream(expert_output.device)),
               "moe_combine_backward")
    return dy, dw


def dispatch_backward(grad_rows: torch.Tensor, row_of_slot: torch.Tensor, top_k: int, num_tokens: int) -> torch.Tensor:
    """[T,H] token gradients (moe_dispatch_backward)."""
    L = _lib.load()
    dx = torch.empty((num_tokens, grad_rows.shape[1]), dtype=grad_rows.dtype, device=grad_rows.device)
    d = [_desc(x) for x in (grad_rows, row_of_slot, dx)]
    _lib.check(L.moe_dispatch_backward(_ref(d[0]), _ref(d[1]), int(top_k), _ref(d[2]), _stream(dx.device)),
               "moe_dispatch_backward")
    return dx


class ExpertsCache:
    """What the experts backward needs: the product rows (dispatched, or the
    tokens with token_of_row), the offsets, the FP32 pre-activations g | u
    [N,2I] and the activation h [N,I]."""

    def __init__(self, experts, rows, token_of_row, expert_offsets, preact, h):
        self.experts = experts
        self.rows, self.token_of_row, self.expert_offsets = rows, token_of_row, expert_offsets
        self.preact, self.h = preact, h

    def backward(self, grad_expert_out: torch.Tensor, workspace: torch.Tensor | None = None):
        """Step 2: (grad_rows [N,H], grad_gate, grad_up [E,I,H], grad_down [E,H,I] FP32) (moe_experts_backward)."""
        ex = self.experts
        L = _lib.load()
        N = self.h.shape[0]
        dev = self.h.device
        dx = torch.empty((N, ex.hidden), dtype=self.h.dtype, device=dev)
        dg = torch.empty((ex.num_experts, ex.intermediate, ex.hidden), dtype=torch.float32, device=dev)
        du = torch.empty_like(dg)
        dd = torch.empty((ex.num_experts, ex.hidden, ex.intermediate), dtype=torch.float32, device=dev)
        need = L.moe_experts_backward_workspace_bytes(N, ex.hidden, ex.intermediate, ex.num_experts,
                                                      _dtype_code(self.h))
        if workspace is None or workspace.numel() < need:
            workspace = _workspace(need, dev)
        tor = _desc(self.token_of_row) if self.token_of_row is not None else None
        d = [_desc(x) for x in (self.rows, self.expert_offsets, self.preact, self.h, grad_expert_out, dx, dg, du, dd)]
        g, u, w = ex._dw
        st = L.moe_experts_backward(_ref(g), _ref(u), _ref(w), _ref(d[0]), _ref(tor) if tor is not None else None,
                                    *[_ref(x) for x in d[1:]], ctypes.c_void_p(workspace.data_ptr()),
                                    workspace.numel(), _stream(dev))
        _lib.check(st, "moe_experts_backward")
        return dx, dg, du, dd


class SwiGluExperts:
    """Bias-free SwiGLU expert weights: gate, up [E,I,H]; down [E,H,I]."""

    def __init__(self, gate: torch.Tensor, up: torch.Tensor, down: torch.Tensor):
        if gate.dim() != 3 or up.shape != gate.shape or down.dim() != 3:
            raise MoeError(3, "gate/up must be [E,I,H] and down [E,H,I]")
        E, I, H = gate.shape
        if tuple(down.shape) != (E, H, I):
            raise MoeError(3, "down must be [E,H,I]")
        if up.dtype != gate.dtype or down.dtype != gate.dtype:
            raise MoeError(2, "gate, up and down must share one float dtype")
        if up.device != gate.device or down.device != gate.device:
            raise MoeError(5, "gate, up and down must share one device")
        self.gate, self.up, self.down = gate, up, down
        self.num_experts, self.intermediate, self.hidden = E, I, H
        self._dw = [_desc(w) for w in (gate, up, down)]

    def forward(self, input: torch.Tensor, logits: torch.Tensor, options: RoutingOptions,
                workspace: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
        """The whole local chain from precomputed logits (moe_forward)."""
        L = _lib.load()
        T, H = input.shape
        if out is None:
            out = torch.empty((T, H), dtype=input.dtype, device=input.device)
        need = L.moe_forward_workspace_bytes(T, self.hidden, self.intermediate, self.num_experts,
                                             int(options.top_k), _dtype_code(input))
        if workspace is None or workspace.numel() < need:
            workspace = _workspace(need, input.device)
        dx, dl, do = _desc(input), _desc(logits), _desc(out)
        g, u, d = self._dw
        st = L.moe_forward(_ref(g), _ref(u), _ref(d), _ref(dx), _ref(dl), options._c(), _ref(do),
                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel(), _stream(input.device))
        _lib.check(st, "moe_forward")
        return out

    def forward_no_alloc(self, input: torch.Tensor, logits: torch.Tensor, options: RoutingOptions,
                         out: torch.Tensor) -> torch.Tensor:
        """moe_forward without a workspace (moe_forward_no_alloc): the library
        runs on its static per-device scratch array; the caller provides out."""
        L = _lib.load()
        dx, dl, do = _desc(input), _desc(logits), _desc(out)
        g, u, d = self._dw
        st = L.moe_forward_no_alloc(_ref(g), _ref(u), _ref(d), _ref(dx), _ref(dl), options._c(), _ref(do),
                                    _stream(input.device))
        _lib.check(st, "moe_forward_no_alloc")
        return out

    def forward_sigmoid_grouped(self, input: torch.Tensor, logits: torch.Tensor, bias: torch.Tensor | None,
                                options: GroupRoutingOptions, workspace: torch.Tensor | None = None,
                                out: torch.Tensor | None = None) -> torch.Tensor:
        """The whole local chain with group-limited sigmoid routing (moe_forward_sigmoid_grouped)."""
        L = _lib.load()
        T, H = input.shape
        if out is None:
            out = torch.empty((T, H), dtype=input.dtype, device=input.device)
        need = L.moe_forward_workspace_bytes(T, self.hidden, self.intermediate, self.num_experts,
                                             int(options.top_k), _dtype_code(input))
        if workspace is None or workspace.numel() < need:
            workspace = _workspace(need, input.device)
        dx, dl, do = _desc(input), _desc(logits), _desc(out)
        db = _desc(bias) if bias is not None else None
        g, u, d = self._dw
        st = L.moe_forward_sigmoid_grouped(_ref(g), _ref(u), _ref(d), _ref(dx), _ref(dl),
                                           _ref(db) if db is not None else None, options._c(), _ref(do),
                                           ctypes.c_void_p(workspace.data_ptr()), workspace.numel(),
                                           _stream(input.device))
        _lib.check(st, "moe_forward_sigmoid_grouped")
        return out

    def forward_workspace_bytes(self, T: int, top_k: int, dtype: torch.dtype) -> int:
        return int(_lib.load().moe_forward_workspace_bytes(T, self.hidden, self.intermediate,
                                                          self.num_experts, int(top_k), _DTYPES[dtype]))

    def forward_dispatched(self, dispatched: DispatchedTokens | torch.Tensor,
                           expert_offsets: torch.Tensor | None = None) -> torch.Tensor:
        """SwiGLU experts on rows grouped by expert (moe_experts_forward)."""
        L = _lib.load()
        if isinstance(dispatched, DispatchedTokens):
            rows, offsets = dispatched.rows, dispatched.expert_offsets
        else:
            rows, offsets = dispatched, expert_offsets
        N = rows.shape[0]
        out = torch.empty((N, self.hidden), dtype=rows.dtype, device=rows.device)
        ws = _workspace(L.moe_experts_workspace_bytes(N, self.hidden, self.intermediate, self.num_experts,
                                                      _dtype_code(rows)), rows.device)
        dr, do_, dy = _desc(rows), _desc(offsets), _desc(out)
        g, u, d = self._dw
        st = L.moe_experts_forward(_ref(g), _ref(u), _ref(d), _ref(dr), _ref(do_), _ref(dy),
                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(rows.device))
        _lib.check(st, "moe_experts_forward")
        return out

    def forward_dispatched_training(self, dispatched: DispatchedTokens, input: torch.Tensor | None = None,
                                    workspace: torch.Tensor | None = None):
        """The experts forward plus its cache (moe_experts_forward_training):
        on the dispatched copy, or -- with `input` -- on the token rows read
        in place through token_of_row.  Returns (output [N,H], ExpertsCache)."""
        L = _lib.load()
        if input is None:
            if dispatched.rows is None:
                raise MoeError(1, "no dispatched rows: pass the token rows as `input`")
            rows, tor = dispatched.rows, None
        else:
            rows, tor = input, dispatched.token_of_row
        offsets = dispatched.expert_offsets
        N = tor.shape[0] if tor is not None else rows.shape[0]
        dev = rows.device
        out = torch.empty((N, self.hidden), dtype=rows.dtype, device=dev)
        preact = torch.empty((N, 2 * self.intermediate), dtype=torch.float32, device=dev)
        h = torch.empty((N, self.intermediate), dtype=rows.dtype, device=dev)
        need = L.moe_experts_workspace_bytes(N, self.hidden, self.intermediate, self.num_experts, _dtype_code(rows))
        if workspace is None or workspace.numel() < need:
            workspace = _workspace(need, dev)
        dt = _desc(tor) if tor is not None else None
        d = [_desc(x) for x in (rows, offsets, out, preact, h)]
        g, u, w = self._dw
        st = L.moe_experts_forward_training(_ref(g), _ref(u), _ref(w), _ref(d[0]), _ref(dt) if dt is not None else None,
                                            *[_ref(x) for x in d[1:]], ctypes.c_void_p(workspace.data_ptr()),
                                            workspace.numel(), _stream(dev))
        _lib.check(st, "moe_experts_forward_training")
        return out, ExpertsCache(self, rows, tor, offsets, preact, h)

    def gate_up(self, rows: torch.Tensor, expert_offsets: torch.Tensor,
                workspace: torch.Tensor | None = None) -> torch.Tensor:
        """First half of the experts: h = silu(gate_e x) * up_e x (moe_experts_gate_up)."""
        L = _lib.load()
        N = rows.shape[0]
        h = torch.empty((N, self.intermediate), dtype=rows.dtype, device=rows.device)
        ws = workspace if workspace is not None else _workspace(
            L.moe_experts_workspace_bytes(N, self.hidden, self.intermediate, self.num_experts, _dtype_code(rows)),
            rows.device)
        dr, do_, dh = _desc(rows), _desc(expert_offsets), _desc(h)
        g, u, _ = self._dw
        st = L.moe_experts_gate_up(_ref(g), _ref(u), _ref(dr), _ref(do_), _ref(dh),
                                   ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(rows.device))
        _lib.check(st, "moe_experts_gate_up")
        return h

    def gate_up_gathered(self, input: torch.Tensor, token_of_row: torch.Tensor, expert_offsets: torch.Tensor,
                         workspace: torch.Tensor | None = None) -> torch.Tensor:
        """gate_up reading token rows in place through token_of_row (moe_experts_gate_up_gathered)."""
        L = _lib.load()
        N = token_of_row.shape[0]
        h = torch.empty((N, self.intermediate), dtype=input.dtype, device=input.device)
        ws = workspace if workspace is not None else _workspace(
            L.moe_experts_workspace_bytes(N, self.hidden, self.intermediate, self.num_experts, _dtype_code(input)),
            input.device)
        dx, dt, do_, dh = _desc(input), _desc(token_of_row), _desc(expert_offsets), _desc(h)
        g, u, _ = self._dw
        st = L.moe_experts_gate_up_gathered(_ref(g), _ref(u), _ref(dx), _ref(dt), _ref(do_), _ref(dh),
                                            ctypes.c_void_p(ws.data_ptr()), ws.numel(), _stream(input.device))
        _lib.check(st, "moe_experts_gate_up_gathered")
        return h

    def down_proj(self, h: torch.Tensor, expert_offsets: torch.Tensor,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
        """Second half of the experts: y = down_e h (moe_experts_down)."""
        L = _lib.load()
        N = h.shape[0]
        out = torch.empty((N, self.hidden), dtype=h.dtype, device=h.device)
        ws = workspace if workspace is not None else _workspace(
            L.moe_experts_workspace_bytes(N, self.hidden, self.intermediate, self.num_experts, _dtype_code(h)),
            h.device)
        dh, do_, dy = _desc(h), _desc(expert_offsets), _desc(out)
        _, _, d = self._dw
        st = L.moe_experts_down(_ref(d), _ref(dh), _ref(do_), _ref(dy), ctypes.c_void_p(ws.data_ptr()),
                                ws.numel(), _stream(h.device))
        _lib.check(st, "moe_experts_down")
        return out
