"""First-order training on the HIP path vs the CPU oracle (RUDA ruDNN library
guide, section 12), through the C ABI on a gfx950 GPU.

Each backward step is checked on its own against the oracle fed the same
inputs, then the whole step (route, FP32 router weights, mapping-only
dispatch, experts forward with its cache, combine, and the four backward
steps) against the oracle's composition.  Small cases span several 128-row
tiles, ragged tails, an expert without rows and every dtype; the prefill
workload runs at full size with sampled checks.

Tolerances: values computed in FP32 from F32 data (router weights, the
pre-activation cache, F32 chains) use 1e-4 * (1 + |ref|); results whose
inputs are BF16/F16 use 2e-2 * (1 + |ref|).  The FP32 weight gradients are
sums over an expert's rows of products whose 16-bit factor (dg, du or h) both
sides round separately; they must stay within 2e-2 * (1 + |ref|) plus one
rounding step of that factor times the sum of |terms|, with at most 0.1% of
elements beyond the plain 2e-2 * (1 + |ref|).
"""
import sys
import zlib

import numpy as np
import pytest
import torch

import mixture_experts_layer_route_amd as moe
import moe_synth as S
import oracle
from parity import TOL, assert_close, assert_close_sum, host_bits, values

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NTHREADS = min(16, oracle.default_threads())


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    moe.load()
    yield
    torch.cuda.synchronize()


def u32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint32).view(np.int32)).view(torch.uint32).to(DEV)


def f32_close(got, ref, what):
    assert_close(np.asarray(got, np.float64), np.asarray(ref, np.float64), "f32", what)


def wgrad_l1(offsets, dgu, rows, dY, h, dt, E, I):
    """Sums of |terms| of the weight gradients, per element: |dg|^T |x|,
    |du|^T |x| (per expert, [E,I,H]) and |dy|^T |h| ([E,H,I])."""
    x, y, hh = (np.abs(oracle.widen(a, dt)) for a in (rows, dY, h))
    H = x.shape[1]
    lg, lu, ld = np.zeros((E, I, H)), np.zeros((E, I, H)), np.zeros((E, H, I))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b > a:
            lg[e] = np.abs(dgu[a:b, :I]).T @ x[a:b]
            lu[e] = np.abs(dgu[a:b, I:]).T @ x[a:b]
            ld[e] = y[a:b].T @ hh[a:b]
    return lg, lu, ld


def check_wgrads(got, ref, l1, dt, tag):
    for gt, rf, m, what in zip(got, ref, l1, ("grad_gate", "grad_up", "grad_down")):
        assert_close_sum(gt.cpu().double().numpy(), rf, m, dt, f"{what} {tag}")


# ------------------------------------------------------------------ router weights
ROUTER_CASES = [
    dict(name="softmax_f32", T=300, E=16, k=4, dt="f32", scoring="softmax", renorm=True, scale=1.0, idx="u32"),
    dict(name="sigmoid_bf16", T=257, E=64, k=6, dt="bf16", scoring="sigmoid", renorm=False, scale=2.5, idx="i32"),
    dict(name="softmax_dups_f16", T=200, E=256, k=8, dt="f16", scoring="softmax", renorm=True, scale=1.0,
         idx="i64", dups=True),
    dict(name="sigmoid_renorm_f32", T=128, E=48, k=8, dt="f32", scoring="sigmoid", renorm=True, scale=0.5,
         idx="u32", dups=True),
    dict(name="edge_invalid_f32", T=400, E=16, k=4, dt="f32", scoring="softmax", renorm=True, scale=1.0,
         idx="i64", edge=True, invalid=True),
    dict(name="edge_sigmoid_invalid_bf16", T=300, E=32, k=3, dt="bf16", scoring="sigmoid", renorm=True,
         scale=1.0, idx="i32", edge=True, invalid=True),
    dict(name="wide_bf16", T=40, E=4096, k=64, dt="bf16", scoring="softmax", renorm=True, scale=1.0, idx="u32"),
    dict(name="k_equals_e_f32", T=50, E=5, k=5, dt="f32", scoring="softmax", renorm=False, scale=3.0, idx="u32"),
]


def router_inputs(c):
    rng = np.random.default_rng(zlib.crc32(c["name"].encode()))
    T, E, k = c["T"], c["E"], c["k"]
    cfg = S.small_config(c["name"], T=T, H=8, I=8, E=E, top_k=k, dtype="f32", logits_dtype=c["dt"], seed=77,
                         edge_rows=c.get("edge", False))
    _, lg = S.make_tokens(cfg)
    if c.get("dups"):
        idx = rng.integers(0, E, size=(T, k)).astype(np.int64)
    else:
        idx = np.argsort(rng.random((T, E)), axis=1)[:, :k].astype(np.int64)
    if c.get("invalid"):
        rows = rng.choice(T, size=T // 20, replace=False)
        idx[rows, rng.integers(0, k, size=rows.size)] = E if c["idx"] == "u32" else -1
        idx[rows[: rows.size // 2], 0] = E + 7
    gw = rng.standard_normal((T, k)).astype(np.float32)
    tidx = {"u32": lambda a: u32(a.astype(np.uint32)), "i32": lambda a: torch.from_numpy(a.astype(np.int32)).to(DEV),
            "i64": lambda a: torch.from_numpy(a).to(DEV)}[c["idx"]](idx)
    return lg, idx, gw, tidx


@pytest.mark.parametrize("c", ROUTER_CASES, ids=lambda c: c["name"])
def test_router_weights_and_backward_parity(c):
    log(f"router training {c['name']}")
    lg, idx, gw, tidx = router_inputs(c)
    opt = moe.RouterWeightOptions(c["scoring"], c["renorm"], c["scale"])
    glg = lg.to(DEV)
    w = moe.router_weights(glg, tidx, opt)
    dl = moe.router_backward(glg, tidx, torch.from_numpy(gw).to(DEV), opt)
    torch.cuda.synchronize()
    lb = host_bits(lg)
    ow = oracle.router_weights(lb, c["dt"], idx, c["scoring"], c["renorm"], c["scale"], NTHREADS)
    odl = oracle.router_backward(lb, c["dt"], idx, gw, c["scoring"], c["renorm"], c["scale"], NTHREADS)
    f32_close(w.cpu().numpy(), ow, f"router weights {c['name']}")
    assert_close(values(dl, c["dt"]), oracle.widen(odl, c["dt"]), c["dt"], f"logits gradient {c['name']}")
    if c.get("invalid"):
        bad = ~((idx >= 0) & (idx < c["E"])).all(axis=1)
        assert bad.any() and torch.isnan(w.cpu()[torch.from_numpy(bad)]).all()


# ------------------------------------------------------------------ combine / dispatch backward
BWD_CASES = [
    S.small_config("cb_tiny_f32", T=64, H=128, I=8, E=8, top_k=2, dtype="f32", seed=301),
    S.small_config("cb_ragged_bf16", T=301, H=200, I=8, E=5, top_k=3, dtype="bf16", seed=302),
    S.small_config("cb_odd_h_f16", T=77, H=36, I=8, E=3, top_k=2, dtype="f16", logits_dtype="f32", seed=303),
    S.small_config("cb_wide_bf16", T=129, H=7168, I=8, E=16, top_k=8, dtype="bf16", seed=304),
    # more slots than one batch of row loads (8) in the dispatch backward
    S.small_config("cb_many_slots_bf16", T=50, H=64, I=8, E=24, top_k=11, dtype="bf16", seed=305),
]


@pytest.mark.parametrize("cfg", BWD_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("wdt", ["f32", "logits"])
def test_combine_and_dispatch_backward_parity(cfg, wdt):
    log(f"combine/dispatch backward {cfg.name} weights {wdt}")
    rng = np.random.default_rng(cfg.seed)
    x, lg = S.make_tokens(cfg)
    idx, w, w32 = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    idx[5, 1] = cfg.E  # one token with an invalid slot: NaN weight gradients and a NaN dx row
    offsets, ros, tor, rows = oracle.dispatch(idx, cfg.E, host_bits(x), cfg.dtype)
    N = rows.shape[0]
    Y = S.to_bits(torch.randn((N, cfg.H), generator=torch.Generator().manual_seed(cfg.seed)).to(S.TORCH_DT[cfg.dtype]))
    g = host_bits(S.make_grad_output(cfg))
    wb, wname = (w32, "f32") if wdt == "f32" else (w, cfg.logits_dtype)
    gdy, gdw = moe.combine_backward(S.from_bits(Y, cfg.dtype, DEV), u32(ros), S.from_bits(wb, wname, DEV),
                                    S.from_bits(g, cfg.dtype, DEV))
    drows = S.to_bits(torch.from_numpy(rng.standard_normal((N, cfg.H)).astype(np.float32)).to(S.TORCH_DT[cfg.dtype]))
    gdx = moe.dispatch_backward(S.from_bits(drows, cfg.dtype, DEV), u32(ros), cfg.top_k, cfg.T)
    torch.cuda.synchronize()
    ody, odw = oracle.combine_backward(Y, cfg.dtype, ros, wb, wname, g, cfg.T, cfg.top_k, cfg.H, NTHREADS)
    odx = oracle.dispatch_backward(drows, cfg.dtype, ros, cfg.T, cfg.top_k, cfg.H, NTHREADS)
    assert_close(values(gdy, cfg.dtype), oracle.widen(ody, cfg.dtype), cfg.dtype, "grad_expert_out")
    f32_close(gdw.cpu().numpy(), odw, "grad_weights")
    assert_close(values(gdx, cfg.dtype), oracle.widen(odx, cfg.dtype), cfg.dtype, "grad_input")
    assert torch.isnan(gdw[5]).all() and torch.isnan(gdx[5].float()).all()


# ------------------------------------------------------------------ experts forward with cache + backward
EXPERT_CASES = [
    S.small_config("ex_tiny_f32", T=64, H=128, I=256, E=8, top_k=2, dtype="f32", seed=401),
    S.small_config("ex_ragged_bf16", T=301, H=200, I=136, E=5, top_k=2, dtype="bf16", seed=402),
    S.small_config("ex_ragged_f16", T=77, H=264, I=72, E=3, top_k=3, dtype="f16", logits_dtype="f32", seed=403),
    S.small_config("ex_many_experts_bf16", T=96, H=64, I=96, E=40, top_k=4, dtype="bf16", seed=404),
    S.small_config("ex_pipe64_bf16", T=600, H=192, I=128, E=6, top_k=2, dtype="bf16", seed=405),
    S.small_config("ex_long_k_bf16", T=1500, H=128, I=64, E=2, top_k=1, dtype="bf16", seed=406),
    S.small_config("ex_f32_odd", T=90, H=48, I=40, E=3, top_k=2, dtype="f32", seed=407),
    # more weight-gradient tiles (16 experts x 8 x 8 of 128 x 256) than the
    # GPU runs at once
    S.small_config("ex_many_tiles_bf16", T=1100, H=2048, I=512, E=16, top_k=2, dtype="bf16", seed=409),
    # experts of at most 64 rows: stream tiles of the 64-K kernel, which also
    # save the FP32 pre-activations
    S.small_config("ex_stream_bf16", T=40, H=128, I=192, E=16, top_k=4, dtype="bf16", seed=410),
]


def compare_experts_training(cfg, x_bits, idx, W, gathered: bool):
    """Runs the GPU forward-with-cache and backward on the GPU dispatch of idx,
    and the oracle on the same per-expert rows; compares every output."""
    E, H, I = cfg.E, cfg.H, cfg.I
    gx = S.from_bits(x_bits, cfg.dtype, DEV)
    gidx = u32(idx)
    d = moe.dispatch(gx, gidx, E, copy_rows=not gathered)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    y, cache = ex.forward_dispatched_training(d, input=gx if gathered else None)
    n = int(host_bits(d.expert_offsets)[E])
    rng = np.random.default_rng(cfg.seed + 5)
    dY = S.to_bits(torch.from_numpy(rng.standard_normal((d.token_of_row.shape[0], H)).astype(np.float32))
                   .to(S.TORCH_DT[cfg.dtype]))
    gdx, gdg, gdu, gdd = cache.backward(S.from_bits(dY, cfg.dtype, DEV))
    torch.cuda.synchronize()
    tor = host_bits(d.token_of_row)[:n]
    offsets = host_bits(d.expert_offsets)
    rows = x_bits[tor]
    Wb = [host_bits(w) for w in W]
    fw = oracle.experts_train_forward(*Wb, cfg.dtype, rows, offsets, E, H, I, NTHREADS)
    odx, odg, odu, odd, odgu = oracle.experts_backward(*Wb, cfg.dtype, rows, offsets, E, H, I, fw["g"], fw["u"],
                                                       fw["h"], dY[:n], NTHREADS, with_dgu=True)
    tag = f"{cfg.name} {'gathered' if gathered else 'copied'}"
    dt = cfg.dtype
    assert_close(values(y[:n], dt), oracle.widen(fw["output"], dt), dt, f"output {tag}")
    pre = cache.preact[:n].cpu().numpy()
    f32_close(pre[:, :I], fw["g"], f"saved g {tag}")
    f32_close(pre[:, I:], fw["u"], f"saved u {tag}")
    assert_close(values(cache.h[:n], dt), oracle.widen(fw["h"], dt), dt, f"saved h {tag}")
    assert_close(values(gdx[:n], dt), oracle.widen(odx, dt), dt, f"grad_rows {tag}")
    check_wgrads((gdg, gdu, gdd), (odg, odu, odd), wgrad_l1(offsets, odgu, rows, dY[:n], fw["h"], dt, E, I), dt, tag)
    # the cache's forward is the plain forward, bit for bit
    if not gathered:
        y_plain = ex.forward_dispatched(d)
        torch.cuda.synchronize()
        bits = torch.int32 if y.dtype == torch.float32 else torch.int16
        assert torch.equal(y[:n].view(bits), y_plain[:n].view(bits))
    return gdd


@pytest.mark.parametrize("cfg", EXPERT_CASES, ids=lambda c: c.name)
@pytest.mark.parametrize("gathered", [False, True], ids=["copied", "gathered"])
def test_experts_training_parity(cfg, gathered):
    log(f"experts training {cfg.name} gathered={gathered}")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    idx, _, _ = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    compare_experts_training(cfg, host_bits(x), idx, W, gathered)


def test_expert_without_rows_gets_zero_gradients():
    cfg = S.small_config("ex_idle_bf16", T=200, H=64, I=128, E=6, top_k=2, dtype="bf16", seed=408)
    log("experts training with idle experts")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    idx, _, _ = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    idx[idx == 2] = 3           # experts 2 and 5 own no rows
    idx[idx == 5] = 0
    dup = idx[:, 0] == idx[:, 1]
    idx[dup, 1] = np.where(idx[dup, 0] == 1, 4, 1)
    gdd = compare_experts_training(cfg, host_bits(x), idx, W, gathered=True)
    assert float(gdd[2].abs().max()) == 0.0 and float(gdd[5].abs().max()) == 0.0


# ------------------------------------------------------------------ the whole training step
def gpu_train_step(cfg, x, lg, W, gout, opt: "moe.RouterWeightOptions", grouped=None):
    gx, glg = x.to(DEV), lg.to(DEV)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    if grouped is None:
        plan = moe.route(glg, moe.RoutingOptions(cfg.top_k, cfg.renormalize))
    else:
        plan = moe.route_sigmoid_grouped(glg, None, grouped)
    tp = plan.into_training(glg, opt)
    d = tp.routing().dispatch(gx, copy_rows=False)
    y, cache = ex.forward_dispatched_training(d, input=gx)
    out = d.combine(y)
    dy, dw = d.combine_backward(y, gout.to(DEV))
    drows, dgate, dup, ddown = cache.backward(dy)
    dx = d.dispatch_backward(drows)
    dlg = tp.backward(dw)
    torch.cuda.synchronize()
    return dict(indices=host_bits(plan.expert_indices()), output=out, dx=dx, dlogits=dlg, dgate=dgate, dup=dup,
                ddown=ddown, dweights=dw)


STEP_CASES = [
    (S.small_config("step_f32", T=64, H=128, I=256, E=8, top_k=2, dtype="f32", seed=501), "softmax"),
    (S.small_config("step_bf16", T=400, H=192, I=136, E=6, top_k=3, dtype="bf16", seed=502), "softmax"),
    (S.small_config("step_f16_f32logits", T=150, H=64, I=96, E=5, top_k=2, dtype="f16", logits_dtype="f32",
                    renormalize=False, seed=503), "softmax"),
]


@pytest.mark.parametrize("cfg,scoring", STEP_CASES, ids=lambda c: getattr(c, "name", str(c)))
def test_training_step_parity(cfg, scoring):
    log(f"training step {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    gout = S.make_grad_output(cfg)
    opt = moe.RouterWeightOptions(scoring, cfg.renormalize, 1.0)
    g = gpu_train_step(cfg, x, lg, W, gout, opt)
    r = oracle.train_step(host_bits(x), host_bits(lg), *[host_bits(w) for w in W], cfg.dtype, cfg.logits_dtype,
                          cfg.top_k, cfg.renormalize, host_bits(gout), NTHREADS, indices=g["indices"],
                          scoring=scoring)
    dt = cfg.dtype
    assert_close(values(g["output"], dt), oracle.widen(r["output"], dt), dt, "step output")
    assert_close(values(g["dx"], dt), oracle.widen(r["dx"], dt), dt, "step dx")
    if dt == "f32":
        f32_close(g["dweights"].cpu().numpy(), r["dweights"], "step dweights")
    else:
        assert_close(g["dweights"].cpu().double().numpy(), r["dweights"], dt, "step dweights")
    assert_close(values(g["dlogits"], cfg.logits_dtype), oracle.widen(r["dlogits"], cfg.logits_dtype),
                 cfg.logits_dtype if dt == "f32" else dt, "step dlogits")
    l1 = wgrad_l1(r["offsets"], r["dgu"], r["dispatched"], r["dY"], r["h"], dt, cfg.E, cfg.I)
    check_wgrads((g["dgate"], g["dup"], g["ddown"]), (r["dgate"], r["dup"], r["ddown"]), l1, dt, "step")


def test_training_step_with_group_limited_sigmoid_routing():
    cfg = S.small_config("step_grouped_bf16", T=300, H=128, I=64, E=32, top_k=4, dtype="bf16", seed=504)
    log("training step, group-limited sigmoid routing")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    gout = S.make_grad_output(cfg)
    gopt = moe.GroupRoutingOptions(top_k=4, groups=8, selected_groups=2, group_top_two=True, renormalize=True,
                                   scale=2.5)
    opt = moe.RouterWeightOptions("sigmoid", True, 2.5)
    g = gpu_train_step(cfg, x, lg, W, gout, opt, grouped=gopt)
    r = oracle.train_step(host_bits(x), host_bits(lg), *[host_bits(w) for w in W], "bf16", "bf16", 4, True,
                          host_bits(gout), NTHREADS, indices=g["indices"], scoring="sigmoid", scale=2.5)
    for k, dt in (("output", "bf16"), ("dx", "bf16"), ("dlogits", "bf16")):
        assert_close(values(g[k], dt), oracle.widen(r[k], dt), dt, f"grouped step {k}")
    l1 = wgrad_l1(r["offsets"], r["dgu"], r["dispatched"], r["dY"], r["h"], "bf16", cfg.E, cfg.I)
    check_wgrads((g["dgate"], g["dup"], g["ddown"]), (r["dgate"], r["dup"], r["ddown"]), l1, "bf16", "grouped step")


# ------------------------------------------------------------------ full size, sampled
def run_step_on_device(cfg):
    """The benchmark's training step on device-drawn inputs; returns every result."""
    x, lg = S.make_tokens(cfg, device=DEV)
    W = S.make_weights(cfg, device=DEV)
    gout = S.make_grad_output(cfg, device=DEV)
    opt = moe.RouterWeightOptions("softmax", cfg.renormalize, 1.0)
    ex = moe.SwiGluExperts(*W)
    plan = moe.route(lg, moe.RoutingOptions(cfg.top_k, cfg.renormalize))
    tp = plan.into_training(lg, opt)
    d = tp.routing().dispatch(x, copy_rows=False)
    y, cache = ex.forward_dispatched_training(d, input=x)
    dy, dw = d.combine_backward(y, gout)
    drows, dgate, dup, ddown = cache.backward(dy)
    dx = d.dispatch_backward(drows)
    dlg = tp.backward(dw)
    torch.cuda.synchronize()
    return dict(x=x, lg=lg, W=W, gout=gout, plan=plan, d=d, dy=dy, drows=drows, dgate=dgate, dup=dup,
                ddown=ddown, dx=dx, dlg=dlg)


def check_tokens(cfg, r, tokens):
    """dx and dlogits of some tokens, each token's k rows through the oracle
    with the full expert weights (dx sums the token's k row gradients, and
    dlogits needs the combine backward's weight gradients of all k slots)."""
    H, I, k = cfg.H, cfg.I, cfg.top_k
    W = r["W"]
    idx = host_bits(r["plan"].expert_indices())
    ros = host_bits(r["d"].row_of_slot)
    xb, lb, gb = host_bits(r["x"]), host_bits(r["lg"]), host_bits(r["gout"])
    ldt = cfg.logits_dtype
    for t in tokens:
        rows_t = ros[t * k:(t + 1) * k]
        w32 = oracle.router_weights(lb[t:t + 1], ldt, idx[t:t + 1], "softmax", cfg.renormalize, 1.0)
        gdx_t = np.zeros(H)
        dw_t = np.zeros((1, k), np.float32)
        for j in range(k):
            e = int(idx[t, j])
            We = [host_bits(w[e:e + 1]) for w in W]
            off1 = np.array([0, 1], np.uint32)
            fw = oracle.experts_train_forward(*We, cfg.dtype, xb[t:t + 1], off1, 1, H, I)
            ody, odw = oracle.combine_backward(fw["output"], cfg.dtype, np.array([0], np.uint32), w32[:, j:j + 1],
                                               "f32", gb[t:t + 1], 1, 1, H)
            odx, _, _, _ = oracle.experts_backward(*We, cfg.dtype, xb[t:t + 1], off1, 1, H, I, fw["g"], fw["u"],
                                                   fw["h"], ody)
            gdx_t += oracle.widen(odx, cfg.dtype)[0]
            dw_t[0, j] = odw[0, 0]
            assert_close(values(r["drows"][int(rows_t[j])], cfg.dtype), oracle.widen(odx, cfg.dtype)[0], cfg.dtype,
                         f"{cfg.name} grad_rows token {t} slot {j}")
        odl = oracle.router_backward(lb[t:t + 1], ldt, idx[t:t + 1], dw_t, "softmax", cfg.renormalize, 1.0)
        assert_close(values(r["dx"][t], cfg.dtype), oracle.widen(oracle.narrow(gdx_t, cfg.dtype), cfg.dtype),
                     cfg.dtype, f"{cfg.name} dx token {t}")
        assert_close(values(r["dlg"][t], ldt), oracle.widen(odl, ldt)[0], cfg.dtype, f"{cfg.name} dlogits token {t}")


def check_rows_of_every_tile(cfg, r, tile_rows=128):
    """The combine backward's dY and the experts backward's grad_rows on the
    first and last row of every tile_rows-row tile of every expert (the row
    products' tiles are 128 rows, the forward's 256), each row through the
    oracle with its expert's full weights.  A row's results depend on that
    row alone, so these rows are exact references at any batch size."""
    E, H, I, k = cfg.E, cfg.H, cfg.I, cfg.top_k
    W = r["W"]
    idx = host_bits(r["plan"].expert_indices())
    offsets = host_bits(r["d"].expert_offsets).astype(np.int64)
    tor = host_bits(r["d"].token_of_row).astype(np.int64)
    ros = host_bits(r["d"].row_of_slot).astype(np.int64).reshape(cfg.T, k)
    xb, lb, gb = host_bits(r["x"]), host_bits(r["lg"]), host_bits(r["gout"])
    n_checked = 0
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if b == a:
            continue
        starts = list(range(a, b, tile_rows))
        rows = np.array(sorted(set(starts) | {min(s + tile_rows, b) - 1 for s in starts}), np.int64)
        toks = tor[rows]
        slot = np.argmax(ros[toks] == rows[:, None], axis=1)
        assert np.all(ros[toks, slot] == rows)
        w32 = oracle.router_weights(lb[toks], cfg.logits_dtype, idx[toks], "softmax", cfg.renormalize, 1.0)
        wsel = np.ascontiguousarray(w32[np.arange(rows.size), slot][:, None])
        We = [host_bits(w[e:e + 1]) for w in W]
        n = rows.size
        off1 = np.array([0, n], np.uint32)
        fw = oracle.experts_train_forward(*We, cfg.dtype, xb[toks], off1, 1, H, I, NTHREADS)
        ody, _ = oracle.combine_backward(fw["output"], cfg.dtype, np.arange(n, dtype=np.uint32), wsel, "f32",
                                         gb[toks], n, 1, H)
        odx, _, _, _ = oracle.experts_backward(*We, cfg.dtype, xb[toks], off1, 1, H, I, fw["g"], fw["u"], fw["h"],
                                               ody, NTHREADS)
        ti = torch.as_tensor(rows, device=DEV)
        tag = f"{cfg.name} expert {e} ({b - a} rows, {n} rows checked)"
        assert_close(values(r["dy"][ti], cfg.dtype), oracle.widen(ody, cfg.dtype), cfg.dtype, f"dY {tag}")
        assert_close(values(r["drows"][ti], cfg.dtype), oracle.widen(odx, cfg.dtype), cfg.dtype, f"grad_rows {tag}")
        n_checked += n
    log(f"  dY and grad_rows checked on {n_checked} rows (first and last of every {tile_rows}-row tile)")


def check_expert_columns(cfg, r, experts, cols_of):
    """dgate, dup and ddown of the given experts on columns cols_of(e) of the
    intermediate dimension: column i of these gradients depends only on
    column i of g, u, h and dh, so the oracle on the expert's weights sliced
    to those columns gives them exactly (rows [i, :] of dgate and dup,
    column [:, i] of ddown)."""
    H = cfg.H
    W = r["W"]
    offsets = host_bits(r["d"].expert_offsets)
    tor = host_bits(r["d"].token_of_row)
    xb = host_bits(r["x"])
    for e in experts:
        a, b = int(offsets[e]), int(offsets[e + 1])
        cols = np.asarray(cols_of(e), np.int64)
        gate_s = host_bits(W[0][e, cols])[None]
        up_s = host_bits(W[1][e, cols])[None]
        down_s = np.ascontiguousarray(host_bits(W[2][e][:, cols]))[None]
        rows_e = xb[tor[a:b]]
        off1 = np.array([0, b - a], np.uint32)
        dy_e = host_bits(r["dy"][a:b])
        fw = oracle.experts_train_forward(gate_s, up_s, down_s, cfg.dtype, rows_e, off1, 1, H, len(cols), NTHREADS)
        _, odg, odu, odd, odgu = oracle.experts_backward(gate_s, up_s, down_s, cfg.dtype, rows_e, off1, 1, H,
                                                         len(cols), fw["g"], fw["u"], fw["h"], dy_e, NTHREADS,
                                                         with_dgu=True)
        lg, lu, ld = wgrad_l1(off1, odgu, rows_e, dy_e, fw["h"], cfg.dtype, 1, len(cols))
        tag = f"{cfg.name} expert {e} ({b - a} rows)"
        assert_close_sum(r["dgate"][e, cols].cpu().double().numpy(), odg[0], lg[0], cfg.dtype, f"dgate {tag}")
        assert_close_sum(r["dup"][e, cols].cpu().double().numpy(), odu[0], lu[0], cfg.dtype, f"dup {tag}")
        assert_close_sum(r["ddown"][e][:, cols].cpu().double().numpy(), odd[0], ld[0], cfg.dtype, f"ddown {tag}")


def one_column_per_block(I, rng, block=128):
    """A random column in every block of 128 intermediate columns (the
    weight-gradient tiles' extent along I), plus one more anywhere."""
    cols = {int(rng.integers(s, min(s + block, I))) for s in range(0, I, block)}
    cols.add(int(rng.integers(0, I)))
    return sorted(cols)


def test_training_step_full_size_sampled():
    """Prefill BF16 (T=8192, H=2048, I=1408, E=64, top_k=6) through the same
    calls the benchmark times: dY and grad_rows on the first and last row of
    every row tile of every expert, the weight gradients of every expert on
    a column in every 128-column block, and dx and dlogits of 16 tokens."""
    cfg = S.CONFIGS["prefill_bf16"]
    log("training full size: prefill_bf16")
    r = run_step_on_device(cfg)
    log("  device step done; checking")
    rng = np.random.default_rng(9)
    check_rows_of_every_tile(cfg, r)
    check_expert_columns(cfg, r, range(cfg.E), lambda e: one_column_per_block(cfg.I, rng))
    log(f"  weight gradients checked on all {cfg.E} experts")
    check_tokens(cfg, r, rng.choice(cfg.T, size=16, replace=False))


def test_training_step_skewed_routing_sampled():
    """Zipf(1.1)-skewed routing over 256 experts (the skewed workload's
    routing at H=1024, I=512): the hottest expert owns thousands of rows, so
    the weight-gradient products run long K loops and the row products many
    tiles of one expert, while cold experts own a few rows or none.  dY and
    grad_rows on the first and last row of every row tile, the weight
    gradients of every expert with rows on a column per 128-column block,
    zero gradients for experts without rows, and dx and dlogits of 4 tokens."""
    cfg = S.small_config("skewed_train_bf16", T=8192, H=1024, I=512, E=256, top_k=8, dtype="bf16", zipf_s=1.1,
                         seed=1104)
    log("training skewed routing: T=8192 H=1024 I=512 E=256 k=8")
    r = run_step_on_device(cfg)
    off = host_bits(r["d"].expert_offsets).astype(np.int64)
    counts = np.diff(off)
    log(f"  rows per expert: max {counts.max()}, median {int(np.median(counts))}, empty {int((counts == 0).sum())}")
    assert counts[0] > 2000
    rng = np.random.default_rng(10)
    check_rows_of_every_tile(cfg, r)
    check_expert_columns(cfg, r, np.nonzero(counts > 0)[0], lambda e: one_column_per_block(cfg.I, rng))
    check_tokens(cfg, r, rng.choice(cfg.T, size=4, replace=False))
    empty = np.nonzero(counts == 0)[0]
    for e in empty[:3]:
        assert float(r["dgate"][e].abs().max()) == 0.0 and float(r["ddown"][e].abs().max()) == 0.0


def test_training_all_tokens_to_one_expert():
    """Every token picks expert 3 first: one expert owns a third of the rows
    (a K loop of 2048 rows in its weight gradients) and the others share the
    rest."""
    cfg = S.small_config("one_hot_train_bf16", T=2048, H=256, I=192, E=8, top_k=3, dtype="bf16", seed=1105)
    log("training with one dominant expert")
    x, lg = S.make_tokens(cfg)
    lg[:, 3] = 30.0
    W = S.make_weights(cfg)
    gout = S.make_grad_output(cfg)
    opt = moe.RouterWeightOptions("softmax", True, 1.0)
    g = gpu_train_step(cfg, x, lg, W, gout, opt)
    assert (g["indices"][:, 0] == 3).all()
    r = oracle.train_step(host_bits(x), host_bits(lg), *[host_bits(w) for w in W], "bf16", "bf16", 3, True,
                          host_bits(gout), NTHREADS, indices=g["indices"])
    for k, dt in (("output", "bf16"), ("dx", "bf16"), ("dlogits", "bf16")):
        assert_close(values(g[k], dt), oracle.widen(r[k], dt), dt, f"one-hot step {k}")
    l1 = wgrad_l1(r["offsets"], r["dgu"], r["dispatched"], r["dY"], r["h"], "bf16", cfg.E, cfg.I)
    check_wgrads((g["dgate"], g["dup"], g["ddown"]), (r["dgate"], r["dup"], r["ddown"]), l1, "bf16", "one-hot step")


def test_training_empty_batch_and_single_token():
    """T = 0: no rows, every weight gradient is written as zeros; T = 1."""
    E, H, I = 4, 64, 64
    cfg = S.small_config("t1_bf16", T=1, H=H, I=I, E=E, top_k=2, dtype="bf16", seed=1106)
    W = [w.to(DEV) for w in S.make_weights(cfg)]
    ex = moe.SwiGluExperts(*W)
    x0 = torch.empty((0, H), dtype=torch.bfloat16, device=DEV)
    d0 = moe.dispatch(x0, torch.empty((0, 2), dtype=torch.uint32, device=DEV), E, copy_rows=False)
    y0, cache0 = ex.forward_dispatched_training(d0, input=x0)
    grads = cache0.backward(torch.empty((0, H), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()
    assert y0.shape == (0, H) and grads[0].shape == (0, H)
    for gw in grads[1:]:
        assert float(gw.abs().max()) == 0.0
    x, lg = S.make_tokens(cfg)
    gout = S.make_grad_output(cfg)
    g = gpu_train_step(cfg, x, lg, [w.cpu() for w in W], gout, moe.RouterWeightOptions("softmax", True, 1.0))
    r = oracle.train_step(host_bits(x), host_bits(lg), *[host_bits(w) for w in W], "bf16", "bf16", 2, True,
                          host_bits(gout), NTHREADS, indices=g["indices"])
    for k in ("output", "dx", "dlogits"):
        assert_close(values(g[k], "bf16"), oracle.widen(r[k], "bf16"), "bf16", f"single token {k}")
    l1 = wgrad_l1(r["offsets"], r["dgu"], r["dispatched"], r["dY"], r["h"], "bf16", E, I)
    check_wgrads((g["dgate"], g["dup"], g["ddown"]), (r["dgate"], r["dup"], r["ddown"]), l1, "bf16", "single token")
