"""Pins of the oracle's first-order training functions (RUDA ruDNN library
guide, section 12) against torch's float64 autograd -- a library
differentiator that shares nothing with the oracle's hand-written chain
rule -- plus central finite differences and the section's special cases
(gathered duplicates, NaN rows for invalid indices, no re-weighting in the
dispatch backward).
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def f64(a):
    return torch.from_numpy(np.asarray(a, np.float64))


def rand_idx(rng, T, E, k, distinct=True):
    if distinct:
        return np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.uint32)
    return rng.integers(0, E, size=(T, k)).astype(np.uint32)


def torch_router(lg, idx, scoring, renorm, scale):
    """w(l) of a fixed selection, written with torch ops on float64 leaves."""
    lt = f64(lg).requires_grad_(True)
    s = torch.softmax(lt, dim=1) if scoring == "softmax" else torch.sigmoid(lt)
    q = torch.gather(s, 1, torch.from_numpy(idx.astype(np.int64)))
    w = q / q.sum(dim=1, keepdim=True) if renorm else q
    return lt, w * scale


@pytest.mark.parametrize("scoring", ["softmax", "sigmoid"])
@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("distinct", [True, False])
def test_router_weights_and_backward_match_autograd(scoring, renorm, distinct):
    rng = np.random.default_rng(1)
    T, E, k, scale = 200, 24, 5, 1.75
    lg = (rng.standard_normal((T, E)) * 2).astype(np.float32)
    idx = rand_idx(rng, T, E, k, distinct)
    gw = rng.standard_normal((T, k)).astype(np.float32)
    w = oracle.router_weights(lg, "f32", idx, scoring, renorm, scale)
    dl = oracle.router_backward(lg, "f32", idx, gw, scoring, renorm, scale)
    lt, wt = torch_router(lg, idx, scoring, renorm, scale)
    (wt * f64(gw)).sum().backward()
    assert np.allclose(w, wt.detach().numpy(), rtol=4e-7 * (k + 4), atol=1e-30)
    ref = lt.grad.numpy()
    assert np.max(np.abs(dl - ref) / (1e-7 + np.abs(ref).max(axis=1, keepdims=True))) < 1e-5
    # the selection is fixed: experts outside it get no gradient under sigmoid scoring
    if scoring == "sigmoid":
        mask = np.ones((T, E), bool)
        np.put_along_axis(mask, idx.astype(np.int64), False, axis=1)
        assert np.all(dl[mask] == 0.0)


def test_router_backward_finite_differences():
    """Central differences of sum(gw * w(l)) on a few logits of tiny rows."""
    rng = np.random.default_rng(2)
    T, E, k = 6, 7, 3
    lg = rng.standard_normal((T, E)).astype(np.float64)
    idx = rand_idx(rng, T, E, k)
    gw = rng.standard_normal((T, k)).astype(np.float32)
    for scoring in ("softmax", "sigmoid"):
        dl = oracle.router_backward(lg.astype(np.float32), "f32", idx, gw, scoring, True, 2.0)
        eps = 1e-2
        for t, e in [(0, 0), (1, 3), (2, int(idx[2, 0])), (5, 6)]:
            def loss(v):
                a = lg.copy()
                a[t, e] = v
                w = oracle.router_weights(a.astype(np.float32), "f32", idx, scoring, True, 2.0)
                return float(np.sum(gw.astype(np.float64) * w))
            fd = (loss(lg[t, e] + eps) - loss(lg[t, e] - eps)) / (2 * eps)
            # eps^2 truncation and binary32 rounding of the weights bound the error
            assert abs(fd - dl[t, e]) < 2e-3 * (1 + abs(fd)), (scoring, t, e, fd, dl[t, e])


def test_router_invalid_index_rows_are_nan():
    rng = np.random.default_rng(3)
    T, E, k = 5, 8, 2
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx = rand_idx(rng, T, E, k).astype(np.int64)
    idx[1, 0] = E         # past the end
    idx[3, 1] = -1        # negative (an I32/I64 index)
    gw = np.ones((T, k), np.float32)
    for scoring in ("softmax", "sigmoid"):
        w = oracle.router_weights(lg, "f32", idx, scoring, True, 1.0)
        dl = oracle.router_backward(lg, "f32", idx, gw, scoring, True, 1.0)
        for t in range(T):
            bad = t in (1, 3)
            assert np.all(np.isnan(w[t])) == bad and np.all(np.isfinite(w[t])) != bad
            assert np.all(np.isnan(dl[t])) == bad and np.all(np.isfinite(dl[t])) != bad
    # a U32 index of 2^32 - 1 is out of range too, not -1
    u = rand_idx(rng, T, E, k)
    u[0, 0] = 0xFFFFFFFF
    assert np.all(np.isnan(oracle.router_weights(lg, "f32", u, "softmax", False, 1.0)[0]))


def test_router_renormalised_weights_sum_to_scale_and_dtypes():
    rng = np.random.default_rng(4)
    T, E, k = 64, 64, 6
    lg32 = rng.standard_normal((T, E)).astype(np.float32)
    idx = rand_idx(rng, T, E, k)
    gw = rng.standard_normal((T, k)).astype(np.float32)
    for dt in ("bf16", "f16"):
        bits = oracle.narrow(lg32, dt)
        wide = oracle.widen(bits, dt).astype(np.float32)
        w = oracle.router_weights(bits, dt, idx, "softmax", True, 2.5)
        assert np.array_equal(w, oracle.router_weights(wide, "f32", idx, "softmax", True, 2.5))
        assert np.allclose(w.sum(axis=1), 2.5, rtol=0, atol=1e-5)
        dl = oracle.router_backward(bits, dt, idx, gw, "softmax", True, 2.5)
        d32 = oracle.router_backward(wide, "f32", idx, gw, "softmax", True, 2.5)
        assert np.array_equal(dl, oracle.narrow(d32.astype(np.float64), dt)) or \
            np.max(np.abs(oracle.widen(dl, dt) - d32)) <= np.max(np.abs(d32)) * 2.0 ** -7
    # renormalised softmax weights do not change under a shift of the row
    w0 = oracle.router_weights(lg32, "f32", idx, "softmax", True, 1.0)
    w1 = oracle.router_weights(lg32 + np.float32(3.0), "f32", idx, "softmax", True, 1.0)
    assert np.allclose(w0, w1, rtol=1e-6)
    # and the logits gradient of a softmax row sums to zero
    d = oracle.router_backward(lg32, "f32", idx, gw, "softmax", False, 1.0)
    assert np.allclose(d.sum(axis=1), 0.0, atol=1e-6)


@pytest.mark.parametrize("scale", [0.0, -1.0, float("inf"), float("nan")])
def test_router_scale_must_be_finite_and_positive(scale):
    lg = np.zeros((2, 4), np.float32)
    idx = np.array([[0, 1], [2, 3]], np.uint32)
    with pytest.raises(ValueError):
        oracle.router_weights(lg, "f32", idx, "softmax", True, scale)
    with pytest.raises(ValueError):
        oracle.router_backward(lg, "f32", idx, np.zeros((2, 2), np.float32), "softmax", True, scale)


def test_router_topk_limits():
    lg = np.zeros((2, 70), np.float32)
    with pytest.raises(ValueError):
        oracle.router_weights(lg, "f32", np.zeros((2, 65), np.uint32), "softmax", True, 1.0)
    with pytest.raises(ValueError):
        oracle.router_weights(lg[:, :3], "f32", np.zeros((2, 4), np.uint32), "softmax", True, 1.0)


def combine_autograd(Y, ros, w, g, T, k):
    Yt = f64(Y).requires_grad_(True)
    wt = f64(w).requires_grad_(True)
    rows = torch.from_numpy(ros.astype(np.int64)).view(T, k)
    out = (Yt[rows] * wt.unsqueeze(2)).sum(dim=1)
    (out * f64(g)).sum().backward()
    return Yt.grad.numpy(), wt.grad.numpy()


def test_combine_backward_matches_autograd():
    rng = np.random.default_rng(5)
    T, E, k, H = 50, 6, 3, 40
    idx = rand_idx(rng, T, E, k)
    x = rng.standard_normal((T, H)).astype(np.float32)
    offsets, ros, tor, rows = oracle.dispatch(idx, E, x, "f32")
    Y = rng.standard_normal((rows.shape[0], H)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    g = rng.standard_normal((T, H)).astype(np.float32)
    dY, dw = oracle.combine_backward(Y, "f32", ros, w, "f32", g, T, k, H)
    rY, rw = combine_autograd(Y, ros, w, g, T, k)
    assert np.allclose(dY, rY, rtol=1e-7, atol=0)
    assert np.allclose(dw, rw, rtol=1e-6, atol=1e-6)


def test_combine_backward_bf16_and_invalid_slot():
    rng = np.random.default_rng(6)
    T, E, k, H = 20, 4, 2, 16
    idx = rand_idx(rng, T, E, k)
    idx[7, 1] = E  # invalid: the forward gives token 7 a NaN row
    x = oracle.narrow(rng.standard_normal((T, H)), "bf16")
    offsets, ros, tor, rows = oracle.dispatch(idx, E, x, "bf16")
    Y = oracle.narrow(rng.standard_normal((rows.shape[0], H)), "bf16")
    w = rng.random((T, k)).astype(np.float32)
    g = oracle.narrow(rng.standard_normal((T, H)), "bf16")
    dY, dw = oracle.combine_backward(Y, "bf16", ros, w, "f32", g, T, k, H)
    valid = ros != oracle.INVALID_ROW
    rY, rw = combine_autograd(oracle.widen(Y, "bf16"), np.where(valid, ros, 0), np.where(valid.reshape(T, k), w, 0),
                              oracle.widen(g, "bf16"), T, k)
    # every dispatched row is some slot's: the bf16 product is rounded once
    assert np.array_equal(dY, oracle.narrow(rY, "bf16"))
    assert np.all(np.isnan(dw[7])) and np.all(np.isfinite(np.delete(dw, 7, axis=0)))
    assert np.allclose(np.delete(dw, 7, axis=0), np.delete(rw, 7, axis=0), rtol=1e-6, atol=1e-6)


def test_dispatch_backward_sums_rows_without_weights():
    rng = np.random.default_rng(7)
    T, E, k, H = 40, 5, 3, 24
    idx = rand_idx(rng, T, E, k)
    x = rng.standard_normal((T, H)).astype(np.float32)
    offsets, ros, tor, rows = oracle.dispatch(idx, E, x, "f32")
    d = rng.standard_normal(rows.shape).astype(np.float32)
    dx = oracle.dispatch_backward(d, "f32", ros, T, k, H)
    xt = f64(x).requires_grad_(True)
    r = xt[torch.from_numpy(tor.astype(np.int64))]   # the dispatch as a gather
    (r * f64(d)).sum().backward()
    assert np.allclose(dx, xt.grad.numpy(), rtol=1e-7, atol=1e-7)
    idx[3, 2] = 99
    offsets, ros, tor, rows = oracle.dispatch(idx, E, x, "f32")
    dx = oracle.dispatch_backward(np.zeros(rows.shape, np.float32), "f32", ros, T, k, H)
    assert np.all(np.isnan(dx[3])) and np.all(dx[np.arange(T) != 3] == 0)


def experts_autograd(gate, up, down, rows, offsets, dY):
    """Per expert: y = down (silu(gate x) * (up x)); float64 autograd of sum(y * dY)."""
    E = gate.shape[0]
    G, U, D = (f64(a).requires_grad_(True) for a in (gate, up, down))
    X = f64(rows).requires_grad_(True)
    outs = []
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        xe = X[a:b]
        g = xe @ G[e].T
        u = xe @ U[e].T
        outs.append((torch.nn.functional.silu(g) * u) @ D[e].T)
    y = torch.cat(outs)
    (y * f64(dY)).sum().backward()
    return y.detach().numpy(), X.grad.numpy(), G.grad.numpy(), U.grad.numpy(), D.grad.numpy()


def expert_case(rng, T, E, k, H, I, dt, skip_expert=None):
    idx = rand_idx(rng, T, E, k)
    if skip_expert is not None:
        idx[idx == skip_expert] = (skip_expert + 1) % E
        idx = np.sort(idx, axis=1)
        for t in range(T):  # keep the row's experts distinct
            s = sorted(set(idx[t].tolist()) | set(range(E)) - {skip_expert})
            idx[t] = np.array(s[:k], np.uint32)
    x = oracle.narrow(rng.standard_normal((T, H)), dt)
    offsets, ros, tor, rows = oracle.dispatch(idx, E, x, dt)
    gate = oracle.narrow(rng.standard_normal((E, I, H)) / np.sqrt(H), dt)
    up = oracle.narrow(rng.standard_normal((E, I, H)) / np.sqrt(H), dt)
    down = oracle.narrow(rng.standard_normal((E, H, I)) / np.sqrt(I), dt)
    dY = oracle.narrow(rng.standard_normal((rows.shape[0], H)), dt)
    return gate, up, down, rows, offsets, dY


def test_experts_train_forward_caches():
    rng = np.random.default_rng(8)
    E, H, I = 4, 32, 48
    gate, up, down, rows, offsets, _ = expert_case(rng, 30, E, 2, H, I, "f32")
    fw = oracle.experts_train_forward(gate, up, down, "f32", rows, offsets, E, H, I)
    y, h = oracle.experts(gate, up, down, "f32", rows, offsets, E, H, I, with_h=True)
    assert np.array_equal(fw["output"], y) and np.array_equal(fw["h"], h)
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        g = rows[a:b].astype(np.float64) @ gate[e].astype(np.float64).T
        u = rows[a:b].astype(np.float64) @ up[e].astype(np.float64).T
        assert np.allclose(fw["g"][a:b], g, rtol=1e-6, atol=1e-6)
        assert np.allclose(fw["u"][a:b], u, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("skip", [None, 2])
def test_experts_backward_matches_autograd_f32(skip):
    """F32 weights: the only roundings are binary32 ones, so every gradient
    agrees with float64 autograd to a few binary32 ulps of its row scale.
    With ``skip`` one expert owns no row: its weight gradients are zero."""
    rng = np.random.default_rng(9)
    E, H, I = 5, 40, 56
    gate, up, down, rows, offsets, dY = expert_case(rng, 36, E, 2, H, I, "f32", skip)
    fw = oracle.experts_train_forward(gate, up, down, "f32", rows, offsets, E, H, I)
    dx, dg, du, dd = oracle.experts_backward(gate, up, down, "f32", rows, offsets, E, H, I,
                                             fw["g"], fw["u"], fw["h"], dY)
    y, rx, rg, ru, rd = experts_autograd(gate, up, down, rows, offsets, dY)
    assert np.allclose(fw["output"], y, rtol=1e-5, atol=1e-5)
    for got, ref in ((dx, rx), (dg, rg), (du, ru), (dd, rd)):
        assert np.max(np.abs(got - ref)) <= 1e-5 * (1 + np.max(np.abs(ref)))
    if skip is not None:
        assert np.all(dg[skip] == 0) and np.all(du[skip] == 0) and np.all(dd[skip] == 0)


def test_experts_backward_bf16_within_rounding():
    """BF16: h, dg and du are rounded to bf16 once each; the gradients stay
    within bf16's relative step of float64 autograd on the same values."""
    rng = np.random.default_rng(10)
    E, H, I = 3, 64, 64
    gate, up, down, rows, offsets, dY = expert_case(rng, 40, E, 2, H, I, "bf16")
    fw = oracle.experts_train_forward(gate, up, down, "bf16", rows, offsets, E, H, I)
    dx, dg, du, dd = oracle.experts_backward(gate, up, down, "bf16", rows, offsets, E, H, I,
                                             fw["g"], fw["u"], fw["h"], dY)
    w = lambda a: oracle.widen(a, "bf16")
    _, rx, rg, ru, rd = experts_autograd(w(gate), w(up), w(down), w(rows), offsets, w(dY))
    for got, ref in ((w(dx), rx), (dg, rg), (du, ru), (dd, rd)):
        err = np.abs(got - ref)
        assert np.max(err) <= 2e-2 * (1 + np.max(np.abs(ref)))
        assert np.median(err) <= 2.0 ** -8 * np.median(np.abs(ref)) + 1e-6


def test_silu_derivative_special_values():
    """silu'(0) = 1/2: with g = 0 (a zero gate), du = 0 and dg = dh * u / 2."""
    E, H, I = 1, 4, 3
    gate = np.zeros((E, I, H), np.float32)
    rng = np.random.default_rng(11)
    up = rng.standard_normal((E, I, H)).astype(np.float32)
    down = rng.standard_normal((E, H, I)).astype(np.float32)
    rows = rng.standard_normal((2, H)).astype(np.float32)
    offsets = np.array([0, 2], np.uint32)
    dY = rng.standard_normal((2, H)).astype(np.float32)
    fw = oracle.experts_train_forward(gate, up, down, "f32", rows, offsets, E, H, I)
    assert np.all(fw["h"] == 0) and np.all(fw["output"] == 0)
    dx, dg, du, dd = oracle.experts_backward(gate, up, down, "f32", rows, offsets, E, H, I,
                                             fw["g"], fw["u"], fw["h"], dY)
    assert np.all(du == 0) and np.all(dd == 0)
    dh = dY.astype(np.float64) @ down[0].astype(np.float64)           # [2, I]
    dgr = (dh * fw["u"].astype(np.float64) / 2).T @ rows.astype(np.float64)
    assert np.allclose(dg[0], dgr, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("renorm", [True, False])
def test_train_step_matches_autograd_of_the_dense_chain(renorm):
    """The section's four steps, composed, against autograd of the dense
    per-token form out_t = sum_j w_j(l_t) FFN_{e_j}(x_t) with the selection
    fixed: dx, dlogits, dgate, dup, ddown."""
    rng = np.random.default_rng(12)
    T, E, k, H, I = 24, 6, 2, 16, 20
    x = rng.standard_normal((T, H)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    gate = (rng.standard_normal((E, I, H)) / 4).astype(np.float32)
    up = (rng.standard_normal((E, I, H)) / 4).astype(np.float32)
    down = (rng.standard_normal((E, H, I)) / 4).astype(np.float32)
    gout = rng.standard_normal((T, H)).astype(np.float32)
    r = oracle.train_step(x, lg, gate, up, down, "f32", "f32", k, renorm, gout)
    idx = torch.from_numpy(r["indices"].astype(np.int64))
    X, L, G, U, D = (f64(a).requires_grad_(True) for a in (x, lg, gate, up, down))
    p = torch.softmax(L, dim=1)
    q = torch.gather(p, 1, idx)
    w = q / q.sum(dim=1, keepdim=True) if renorm else q
    out = torch.zeros(T, H, dtype=torch.float64)
    for j in range(k):
        e = idx[:, j]
        g = torch.einsum("th,tih->ti", X, G[e])
        u = torch.einsum("th,tih->ti", X, U[e])
        y = torch.einsum("ti,thi->th", torch.nn.functional.silu(g) * u, D[e])
        out = out + w[:, j:j + 1] * y
    (out * f64(gout)).sum().backward()
    assert np.allclose(r["output"], out.detach().numpy(), rtol=1e-5, atol=1e-5)
    for got, ref in ((r["dx"], X.grad), (r["dlogits"], L.grad), (r["dgate"], G.grad), (r["dup"], U.grad),
                     (r["ddown"], D.grad)):
        ref = ref.numpy()
        assert np.max(np.abs(got - ref)) <= 1e-5 * (1 + np.max(np.abs(ref)))
