"""moe_forward_no_alloc against moe_forward, through the C ABI, on a gfx950 GPU.

The entry point runs moe_forward's kernels on the library's static per-device
scratch array instead of a caller's workspace, so its output must equal
moe_forward's bit for bit; it is also compared with the CPU oracle.  Two
calls run back to back, the second on a smaller batch, so the second reads
an array the first left full of its own values.
"""
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_route_amd as moe
import moe_synth as S
import oracle
from parity import assert_close, compare_routing, host_bits, values

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
NTHREADS = min(16, oracle.default_threads())
SCRATCH_BYTES = 64 << 20


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def check_against_oracle(cfg, x, lg, W, out):
    res = oracle.forward(host_bits(x), host_bits(lg), *[host_bits(w) for w in W], cfg.dtype, cfg.logits_dtype,
                         cfg.top_k, cfg.renormalize, NTHREADS)
    plan = moe.route(lg.to(DEV), moe.RoutingOptions(cfg.top_k, cfg.renormalize))
    torch.cuda.synchronize()
    _, near = compare_routing(host_bits(plan.expert_indices()), plan.weights().cpu(), host_bits(lg),
                              cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    assert near.mean() < 0.01
    assert_close(values(out, cfg.dtype), oracle.widen(res["output"], cfg.dtype), cfg.dtype,
                 f"no-alloc forward {cfg.name}", rows_mask=~near)


@pytest.mark.parametrize("first,second", [
    # 16-bit: the 64-K pipelined kernel (many rows per expert), then a batch
    # small enough for the 16-row tile
    (S.small_config("na_pipe_bf16", T=700, H=256, I=192, E=16, top_k=4, dtype="bf16", seed=91),
     S.small_config("na_small_bf16", T=37, H=256, I=192, E=16, top_k=4, dtype="bf16", seed=92)),
    # F32 through the register-staged kernel
    (S.small_config("na_f32", T=300, H=128, I=96, E=8, top_k=2, dtype="f32", seed=93),
     S.small_config("na_f32_small", T=21, H=128, I=96, E=8, top_k=2, dtype="f32", seed=94)),
], ids=lambda c: c.name)
def test_no_alloc_equals_forward_twice(first, second):
    W = S.make_weights(first)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    for cfg in (first, second):
        log(f"no-alloc {cfg.name}")
        assert (cfg.H, cfg.I, cfg.E) == (first.H, first.I, first.E)
        x, lg = S.make_tokens(cfg)
        gx, glg = x.to(DEV), lg.to(DEV)
        opts = moe.RoutingOptions(cfg.top_k, cfg.renormalize)
        ref = ex.forward(gx, glg, opts)
        got = ex.forward_no_alloc(gx, glg, opts, out=torch.full_like(gx, float("nan")))
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"{cfg.name}: no-alloc output differs from moe_forward"
        check_against_oracle(cfg, x, lg, W, got)


def test_no_alloc_decode_workload():
    """The decode workload at full size (T=32, H=4096, I=1536, E=128, top_k=8),
    then its first 5 tokens, against moe_forward bit for bit."""
    cfg = S.CONFIGS["decode_bf16"]
    log("no-alloc decode: generating inputs on the GPU")
    x, lg = S.make_tokens(cfg, device=DEV)
    W = S.make_weights(cfg, device=DEV)
    ex = moe.SwiGluExperts(*W)
    opts = moe.RoutingOptions(cfg.top_k, cfg.renormalize)
    for T in (cfg.T, 5):
        ref = ex.forward(x[:T], lg[:T], opts)
        got = ex.forward_no_alloc(x[:T], lg[:T], opts, out=torch.empty_like(x[:T]))
        torch.cuda.synchronize()
        assert torch.equal(bits(got), bits(ref)), f"decode T={T}: no-alloc output differs from moe_forward"


def test_no_alloc_rejects_batches_beyond_the_array():
    """A forward workspace above 64 MiB is refused before anything runs; the
    output keeps its contents."""
    cfg = S.small_config("na_big", T=200000, H=64, I=64, E=4, top_k=4, dtype="bf16", seed=95)
    L = moe.load()
    assert L.moe_forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, 2) > SCRATCH_BYTES
    W = [w.to(DEV) for w in S.make_weights(cfg)]
    ex = moe.SwiGluExperts(*W)
    x = torch.zeros(cfg.T, cfg.H, dtype=torch.bfloat16, device=DEV)
    lg = torch.zeros(cfg.T, cfg.E, dtype=torch.bfloat16, device=DEV)
    out = torch.full_like(x, 3.0)
    with pytest.raises(moe.MoeError) as e:
        ex.forward_no_alloc(x, lg, moe.RoutingOptions(cfg.top_k, True), out=out)
    assert e.value.name == "MOE_ERR_WORKSPACE"
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
    # the largest batch of these extents that fits still runs
    T = 1
    while L.moe_forward_workspace_bytes(2 * T, cfg.H, cfg.I, cfg.E, cfg.top_k, 2) <= SCRATCH_BYTES:
        T *= 2
    got = ex.forward_no_alloc(x[:T], lg[:T], moe.RoutingOptions(cfg.top_k, True), out=out[:T])
    ref = ex.forward(x[:T], lg[:T], moe.RoutingOptions(cfg.top_k, True))
    torch.cuda.synchronize()
    assert torch.equal(bits(got), bits(ref))
