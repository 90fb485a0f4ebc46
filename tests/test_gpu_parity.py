"""HIP path vs the CPU oracle, through the C ABI, on a gfx950 GPU.

Small cases run every stage against the oracle element by element; they span
several GEMM tiles and a ragged tail.  The full-size workloads run the fused
forward exactly as the benchmark launches it and compare routing and
dispatch in full and the output on sampled tokens.
"""
import os
import sys

import numpy as np
import pytest
import torch

import mixture_experts_layer_route_amd as moe
import moe_synth as S
import oracle
from parity import (TOL, assert_close, compare_dispatch, compare_grouped_routing, compare_routing, host_bits,
                    values)

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


def upload(cfg, x, lg, weights):
    return (x.to(DEV), lg.to(DEV), [w.to(DEV) for w in weights])


def small_cases():
    return [
        S.CONFIGS["tiny_f32"],
        S.small_config("ragged_bf16", T=301, H=200, I=136, E=5, top_k=2, dtype="bf16", seed=11),
        S.small_config("ragged_f16", T=77, H=264, I=72, E=3, top_k=3, dtype="f16", logits_dtype="f32", seed=12),
        S.small_config("many_experts_bf16", T=96, H=64, I=96, E=40, top_k=4, dtype="bf16", seed=13),
        S.small_config("wide_rows_bf16", T=700, H=128, I=128, E=4, top_k=2, dtype="bf16", seed=14),
        S.small_config("one_expert_f32", T=50, H=64, I=64, E=1, top_k=1, dtype="f32", seed=15),
        S.small_config("k_equals_e_f32", T=40, H=32, I=48, E=6, top_k=6, renormalize=False, seed=16),
        # large-tile pipelined kernel (16-bit, H and I multiples of 32): ragged
        # token tiles, one and two K stages, f16
        S.small_config("pipe_f16", T=500, H=96, I=160, E=3, top_k=2, dtype="f16", seed=17),
        S.small_config("pipe_short_k_bf16", T=600, H=64, I=32, E=4, top_k=2, dtype="bf16", seed=18),
        S.small_config("pipe_many_tiles_bf16", T=1100, H=256, I=320, E=5, top_k=3, dtype="bf16", seed=19),
        # 64-wide K stages (H and I multiples of 64): a single K step each way,
        # and several steps with ragged tiles in f16
        S.small_config("pipe64_one_step_bf16", T=600, H=64, I=64, E=3, top_k=2, dtype="bf16", seed=20),
        S.small_config("pipe64_f16", T=900, H=192, I=128, E=6, top_k=2, dtype="f16", seed=27),
        # few rows per expert (the 16-row tile) with a partial last K slice on
        # both products: K = 72 and 40 values of f16
        S.small_config("small_tile_k_tail_f16", T=40, H=72, I=40, E=8, top_k=2, dtype="f16", seed=28),
    ]


def deep_cases():
    """The 64-K kernel's steady state and long tile groups, element by
    element: H and I multiples of 64 with 6-8 K steps each way (both rings
    wrap several times, the two-steps-ahead weight loads land in reused
    slots), and experts owning 9-12 token tiles of 256 rows, so the tile
    list splits them into two groups of 5-6."""
    return [
        S.small_config("pipe64_deep_bf16", T=5000, H=512, I=448, E=2, top_k=1, dtype="bf16", seed=81),
        S.small_config("pipe64_deep_f16", T=4500, H=448, I=384, E=3, top_k=2, dtype="f16", seed=82),
    ]


def stream_cases():
    """The 64-K kernel's per-expert tile choice: experts of at most 64 rows run
    as stream tiles (64 token slots against 256 weight rows), the others on
    256-row tiles, in the same launch.  All-stream batches (decode-sized), f16,
    and a Zipf-skewed batch mixing both (1024 tokens, top-8 of 256 experts)."""
    return [
        S.small_config("stream_decode_bf16", T=32, H=256, I=192, E=16, top_k=4, dtype="bf16", seed=83),
        S.small_config("stream_f16", T=60, H=128, I=128, E=8, top_k=2, dtype="f16", logits_dtype="f32", seed=84),
        S.small_config("stream_mixed_zipf_bf16", T=1024, H=512, I=256, E=256, top_k=8, dtype="bf16", zipf_s=1.1,
                       seed=85),
    ]


def decode_cases():
    """The decode stream kernel (experts of a few rows): H and I not
    multiples of 256, so the last K step of each product holds 3 and 1 of
    its 4 quarters; a Zipf-hot expert that owns most of the 64 tokens, i.e.
    several 16-row token tiles of one expert; 1024 experts for 16 tokens;
    and K = 64, a single quarter per step."""
    return [
        S.small_config("decode_partial_k_bf16", T=50, H=448, I=320, E=64, top_k=4, dtype="bf16", seed=87),
        S.small_config("decode_hot_f16", T=64, H=256, I=192, E=32, top_k=2, dtype="f16", zipf_s=2.0, seed=88),
        # 1024 experts for 16 tokens: most units belong to experts of one row
        S.small_config("decode_many_experts_bf16", T=16, H=128, I=64, E=1024, top_k=8, dtype="bf16", seed=90),
        # K = 64 on both products: every step holds a single quarter
        S.small_config("decode_k64_bf16", T=24, H=64, I=64, E=16, top_k=4, dtype="bf16", seed=91),
    ]


# ------------------------------------------------------------------ routing
@pytest.mark.parametrize("cfg", [
    S.CONFIGS["tiny_f32"],
    S.CONFIGS["edge_f32"],
    S.small_config("edge_norenorm", T=1024, H=8, I=8, E=16, top_k=4, renormalize=False, edge_rows=True,
                   seed=1001),
    S.small_config("route_bf16", T=513, H=8, I=8, E=64, top_k=6, dtype="bf16", seed=21),
    S.small_config("route_f16", T=300, H=8, I=8, E=128, top_k=8, dtype="f16", seed=22),
    S.small_config("route_bigE", T=64, H=8, I=8, E=1000, top_k=10, dtype="f32", seed=23),
    S.small_config("route_maxE", T=8, H=8, I=8, E=4096, top_k=70, dtype="bf16", seed=24),
    S.small_config("route_k_eq_e", T=100, H=8, I=8, E=7, top_k=7, dtype="f32", seed=25),
    S.small_config("route_ties_bf16", T=400, H=8, I=8, E=256, top_k=8, dtype="bf16", edge_rows=True, seed=26),
], ids=lambda c: c.name)
def test_route_parity(cfg):
    log(f"route parity {cfg.name}")
    _, lg = S.make_tokens(cfg)
    plan = moe.route(lg.to(DEV), moe.RoutingOptions(cfg.top_k, cfg.renormalize))
    torch.cuda.synchronize()
    gi = host_bits(plan.expert_indices())
    compare_routing(gi, plan.weights().cpu(), host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize,
                    NTHREADS)


def test_route_exact_ties_pick_lower_id():
    lg = torch.tensor([[0.5, 2.0, 2.0, 2.0, -1.0, 2.0]] * 3, dtype=torch.float32)
    plan = moe.route(lg.to(DEV), moe.RoutingOptions(3, True))
    assert host_bits(plan.expert_indices()).tolist() == [[1, 2, 3]] * 3


def test_route_nan_rows_keep_nan():
    E, k = 6, 3
    rows = []
    for pos in range(E):
        r = [0.0] * E; r[pos] = float("nan"); rows.append(r)
        r = [0.0] * E; r[pos] = float("inf"); rows.append(r)
    rows.append([float("-inf")] * E)
    for dt in ("f32", "bf16", "f16"):
        lg = torch.tensor(rows).to(S.TORCH_DT[dt])
        plan = moe.route(lg.to(DEV), moe.RoutingOptions(k, True))
        assert (host_bits(plan.expert_indices()) == np.arange(k)[None, :]).all()
        assert torch.isnan(plan.weights().float().cpu()).all()


# ------------------------------------------------------------------ dispatch
@pytest.mark.parametrize("cfg", small_cases() + [S.CONFIGS["edge_f32"]], ids=lambda c: c.name)
def test_dispatch_parity(cfg):
    log(f"dispatch parity {cfg.name}")
    x, lg = S.make_tokens(cfg)
    idx, _, _ = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    xb = host_bits(x)
    o = oracle.dispatch(idx, cfg.E, xb, cfg.dtype)
    gidx = torch.from_numpy(idx.view(np.int32)).view(torch.uint32).to(DEV)
    d = moe.dispatch(x.to(DEV), gidx, cfg.E)
    torch.cuda.synchronize()
    gpu = {"rows": host_bits(d.rows), "offsets": host_bits(d.expert_offsets),
           "row_of_slot": host_bits(d.row_of_slot), "token_of_row": host_bits(d.token_of_row)}
    compare_dispatch(gpu, *o, xb, idx, cfg.E)


def test_dispatch_all_tokens_to_one_expert():
    cfg = S.small_config("hot", T=3000, H=64, I=64, E=32, top_k=2, dtype="bf16", seed=31)
    x, _ = S.make_tokens(cfg)
    idx = np.zeros((cfg.T, 2), np.uint32)
    idx[:, 1] = 7
    xb = host_bits(x)
    o = oracle.dispatch(idx, cfg.E, xb, "bf16")
    d = moe.dispatch(x.to(DEV), torch.from_numpy(idx.view(np.int32)).view(torch.uint32).to(DEV), cfg.E)
    torch.cuda.synchronize()
    gpu = {"rows": host_bits(d.rows), "offsets": host_bits(d.expert_offsets),
           "row_of_slot": host_bits(d.row_of_slot), "token_of_row": host_bits(d.token_of_row)}
    compare_dispatch(gpu, *o, xb, idx, cfg.E)


def test_invalid_indices_give_nan_rows_without_oob():
    """An expert id >= E is skipped by dispatch and turns the token's output row
    NaN at combine (the training section's convention for bad indices)."""
    T, H, E, k = 33, 64, 4, 2
    x = torch.randn(T, H).to(torch.bfloat16)
    idx = np.tile(np.array([[0, 1]], np.uint32), (T, 1))
    idx[3, 1] = 4
    idx[10, 0] = 0xFFFFFFFF
    d = moe.dispatch(x.to(DEV), torch.from_numpy(idx.view(np.int32)).view(torch.uint32).to(DEV), E,
                     weights=torch.full((T, k), 0.5, dtype=torch.bfloat16, device=DEV))
    out = d.combine(d.rows).float().cpu()
    torch.cuda.synchronize()
    assert int(host_bits(d.expert_offsets)[E]) == T * k - 2
    ros = host_bits(d.row_of_slot)
    assert ros[3 * k + 1] == 0xFFFFFFFF and ros[10 * k] == 0xFFFFFFFF
    nan_rows = torch.isnan(out).all(dim=1)
    assert nan_rows[3] and nan_rows[10] and int(nan_rows.sum()) == 2


@pytest.mark.parametrize("T,k,E,skew", [
    (8192, 6, 64, 0.0),      # 49152 slots, the prefill routing's shape
    (16384, 4, 128, 1.5),    # 65536 slots, skewed
    (4096, 4, 128, 1.5),     # 16384 slots, the most one workgroup maps; skewed
    (4097, 4, 128, 0.0),     # one token more: the multi-kernel path
    (2001, 7, 4096, 0.0),    # ragged, the most experts one workgroup counts
    (3000, 2, 4096, 1.2),    # the same, skewed
    (16000, 1, 3, 0.0),      # k = 1, few experts
    (10, 1500, 2048, 0.0),   # k > 1024
], ids=lambda v: str(v))
def test_mapping_only_dispatch_at_batch_sizes(T, k, E, skew):
    """The mapping-only dispatch across the sizes its one-workgroup kernel
    takes (at most 16384 slots and 4096 experts) and past them, with invalid
    ids sprinkled in: offsets bit-exact, mapping valid and equal per expert to
    the oracle's."""
    log(f"mapping-only dispatch T={T} k={k} E={E}")
    rng = np.random.default_rng(T + k + E)
    if skew:
        p = 1.0 / np.arange(1, E + 1) ** skew
        idx = rng.choice(E, size=(T, k), p=p / p.sum()).astype(np.uint32)
    else:
        idx = rng.integers(0, E, size=(T, k), dtype=np.uint32)
    bad = rng.random((T, k)) < 0.001
    idx[bad] = np.where(rng.random(int(bad.sum())) < 0.5, E, 0xFFFFFFFF).astype(np.uint32)
    x = torch.from_numpy(rng.integers(-2**15, 2**15, size=(T, 8), dtype=np.int16)).view(torch.bfloat16)
    xb = host_bits(x)
    o = oracle.dispatch(idx, E, xb, "bf16")
    m = moe.dispatch(x.to(DEV), torch.from_numpy(idx.view(np.int32)).view(torch.uint32).to(DEV), E,
                     copy_rows=False)
    torch.cuda.synchronize()
    tor = host_bits(m.token_of_row)
    gpu = {"rows": xb[np.minimum(tor, T - 1)], "offsets": host_bits(m.expert_offsets),
           "row_of_slot": host_bits(m.row_of_slot), "token_of_row": tor}
    compare_dispatch(gpu, *o, xb, idx, E)


# ------------------------------------------------------------------ experts
@pytest.mark.parametrize("cfg", small_cases() + deep_cases() + stream_cases() + decode_cases() +
                         [S.CONFIGS["edge_f32"]], ids=lambda c: c.name)
def test_experts_parity(cfg):
    log(f"experts parity {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    Wb = [host_bits(w) for w in W]
    idx, _, _ = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    offsets, ros, tor, rows = oracle.dispatch(idx, cfg.E, host_bits(x), cfg.dtype)
    Y, h = oracle.experts(*Wb, cfg.dtype, rows, offsets, cfg.E, cfg.H, cfg.I, with_h=True, nthreads=NTHREADS)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    g_rows = S.from_bits(rows, cfg.dtype, DEV)
    g_off = torch.from_numpy(offsets.view(np.int32)).view(torch.uint32).to(DEV)
    gy = ex.forward_dispatched(g_rows, g_off)
    torch.cuda.synchronize()
    assert_close(values(gy, cfg.dtype), oracle.widen(Y, cfg.dtype), cfg.dtype, f"expert outputs {cfg.name}")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_experts_tile_choice_at_its_boundaries(dt):
    """Experts of 1, 63 and 64 rows (one stream tile), 65, 200 and 256 (one
    256-row tile), 257, 300 and 576 (256-row tiles and a stream tile of the
    last 1, 44 and 64 rows), 577 (three 256-row tiles, the last of 65 rows)
    and an empty one, in one launch, against the oracle."""
    counts = [64, 65, 1, 0, 200, 257, 63, 256, 300, 1, 576, 577]
    E, H, I = len(counts), 128, 192
    cfg = S.small_config(f"boundary_{dt}", T=sum(counts), H=H, I=I, E=E, top_k=1, dtype=dt, seed=86)
    x, _ = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    rows = host_bits(x)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    Y = oracle.experts(*[host_bits(w) for w in W], dt, rows, offsets, E, H, I, nthreads=NTHREADS)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    g_off = torch.from_numpy(offsets.view(np.int32)).view(torch.uint32).to(DEV)
    gy = ex.forward_dispatched(x.to(DEV), g_off)
    torch.cuda.synchronize()
    assert_close(values(gy, dt), oracle.widen(Y, dt), dt, f"expert outputs, tile boundaries ({dt})")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_leftover_rows_with_deep_k_and_several_weight_tiles(dt):
    """Experts whose last token tile holds 1, 10, 33 and 64 rows after full
    256-row tiles (a stream tile in the gate/up product, a 256-row tile in
    the down product), whole experts of 64 and 65 rows, an empty expert and
    one of exactly three tiles, with K of 8 (gate/up) and 7 (down) 64-wide
    steps and 4 and 2 weight tiles: the persistent launch moves between
    prefetched 256-row tiles and stream tiles in both products."""
    counts = [3 * 256 + 10, 2 * 256 + 64, 256 + 1, 64, 4 * 256 + 33, 65, 0, 3 * 256]
    E, H, I = len(counts), 512, 448
    cfg = S.small_config(f"leftover_{dt}", T=sum(counts), H=H, I=I, E=E, top_k=1, dtype=dt, seed=90)
    x, _ = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    rows = host_bits(x)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    Y = oracle.experts(*[host_bits(w) for w in W], dt, rows, offsets, E, H, I, nthreads=NTHREADS)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    g_off = torch.from_numpy(offsets.view(np.int32)).view(torch.uint32).to(DEV)
    gy = ex.forward_dispatched(x.to(DEV), g_off)
    torch.cuda.synchronize()
    assert_close(values(gy, dt), oracle.widen(Y, dt), dt, f"expert outputs, leftover rows ({dt})")


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_decode_kernel_token_tiles_at_their_boundaries(dt):
    """Experts of 15, 16 (one 16-row token tile), 17, 33 and 48 rows (two to
    three tiles), 1, 2 and none, among 40 experts (132 rows, at most 4 per
    expert on average, so the decode stream kernel runs), against the
    oracle."""
    counts = [15, 16, 17, 0, 1, 33, 48, 2] + [0] * 32
    E, H, I = len(counts), 128, 192
    cfg = S.small_config(f"decode_boundary_{dt}", T=sum(counts), H=H, I=I, E=E, top_k=1, dtype=dt, seed=89)
    x, _ = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    rows = host_bits(x)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.uint32)
    Y = oracle.experts(*[host_bits(w) for w in W], dt, rows, offsets, E, H, I, nthreads=NTHREADS)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    g_off = torch.from_numpy(offsets.view(np.int32)).view(torch.uint32).to(DEV)
    gy = ex.forward_dispatched(x.to(DEV), g_off)
    torch.cuda.synchronize()
    assert_close(values(gy, dt), oracle.widen(Y, dt), dt, f"expert outputs, decode token tiles ({dt})")


@pytest.mark.parametrize("cfg", [
    S.small_config("gather_pipe_bf16", T=700, H=128, I=96, E=5, top_k=2, dtype="bf16", seed=51),
    S.small_config("gather_small_f16", T=24, H=64, I=64, E=32, top_k=3, dtype="f16", seed=52),
    S.small_config("gather_f32", T=90, H=48, I=40, E=3, top_k=2, dtype="f32", seed=53),
    S.small_config("gather_edge_bf16", T=1024, H=64, I=64, E=16, top_k=4, dtype="bf16", edge_rows=True, seed=54),
], ids=lambda c: c.name)
def test_mapping_only_dispatch_and_gathered_gate_up(cfg):
    """moe_dispatch with no dispatched buffer writes the same offsets and a
    valid mapping; gate/up reading the tokens in place through token_of_row
    gives the bits of gate/up on the copied rows, and matches the oracle."""
    log(f"gathered gate/up {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    idx, _, _ = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    xb = host_bits(x)
    o = oracle.dispatch(idx, cfg.E, xb, cfg.dtype)
    gx = x.to(DEV)
    gidx = torch.from_numpy(idx.view(np.int32)).view(torch.uint32).to(DEV)
    m = moe.dispatch(gx, gidx, cfg.E, copy_rows=False)
    torch.cuda.synchronize()
    assert m.rows is None
    tor = host_bits(m.token_of_row)
    gpu = {"rows": xb[np.minimum(tor, cfg.T - 1)], "offsets": host_bits(m.expert_offsets),
           "row_of_slot": host_bits(m.row_of_slot), "token_of_row": tor}
    compare_dispatch(gpu, *o, xb, idx, cfg.E)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    d = moe.dispatch(gx, gidx, cfg.E)
    h_copy = ex.gate_up(d.rows, d.expert_offsets)
    h_in_place = ex.gate_up_gathered(gx, d.token_of_row, d.expert_offsets)
    torch.cuda.synchronize()
    n = int(host_bits(d.expert_offsets)[cfg.E])
    bits = torch.int32 if h_copy.dtype == torch.float32 else torch.int16
    assert torch.equal(h_copy[:n].view(bits), h_in_place[:n].view(bits))
    # the oracle's activation for the same per-expert rows (row order inside
    # an expert is the device's; map each row to its token)
    Wb = [host_bits(w) for w in W]
    _, h_ref = oracle.experts(*Wb, cfg.dtype, xb[host_bits(d.token_of_row)[:n]], host_bits(d.expert_offsets),
                              cfg.E, cfg.H, cfg.I, with_h=True, nthreads=NTHREADS)
    assert_close(values(h_in_place[:n], cfg.dtype), oracle.widen(h_ref[:n], cfg.dtype), cfg.dtype,
                 f"gathered activation {cfg.name}")


# ------------------------------------------------------------------ combine
@pytest.mark.parametrize("cfg", small_cases(), ids=lambda c: c.name)
def test_combine_parity(cfg):
    log(f"combine parity {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = [host_bits(w) for w in S.make_weights(cfg)]
    res = oracle.forward(host_bits(x), host_bits(lg), *W, cfg.dtype, cfg.logits_dtype, cfg.top_k,
                         cfg.renormalize, NTHREADS)
    gy = S.from_bits(res["Y"], cfg.dtype, DEV)
    gros = torch.from_numpy(res["row_of_slot"].view(np.int32)).view(torch.uint32).to(DEV)
    gw = S.from_bits(res["weights"], cfg.logits_dtype, DEV)
    out = moe.combine(gy, gros, gw)
    torch.cuda.synchronize()
    assert_close(values(out, cfg.dtype), oracle.widen(res["output"], cfg.dtype), cfg.dtype, "combine")


# ------------------------------------------------------------------ whole chain
def run_forward_case(cfg, repeat_check=True):
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    res = oracle.forward(host_bits(x), host_bits(lg), *[host_bits(w) for w in W], cfg.dtype, cfg.logits_dtype,
                         cfg.top_k, cfg.renormalize, NTHREADS)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    opts = moe.RoutingOptions(cfg.top_k, cfg.renormalize)
    gx, glg = x.to(DEV), lg.to(DEV)
    out = ex.forward(gx, glg, opts)
    plan = moe.route(glg, opts)
    torch.cuda.synchronize()
    _, near = compare_routing(host_bits(plan.expert_indices()), plan.weights().cpu(), host_bits(lg),
                              cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    assert near.mean() < 0.01, f"too many near-tie tokens: {near.sum()}"
    assert_close(values(out, cfg.dtype), oracle.widen(res["output"], cfg.dtype), cfg.dtype,
                 f"forward {cfg.name}", rows_mask=~near)
    if repeat_check:
        out2 = ex.forward(gx, glg, opts)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8) if out.dtype != torch.float32 else out.view(torch.int32),
                           out2.view(torch.uint8) if out.dtype != torch.float32 else out2.view(torch.int32)), \
            "forward must be bitwise reproducible"
    return out


@pytest.mark.parametrize("cfg", small_cases() + deep_cases() + stream_cases() + decode_cases() + [
    S.CONFIGS["edge_f32"],
    S.small_config("edge_norenorm", T=1024, H=256, I=512, E=16, top_k=4, renormalize=False, edge_rows=True,
                   seed=1001),
], ids=lambda c: c.name)
def test_forward_parity(cfg):
    log(f"forward parity {cfg.name}")
    run_forward_case(cfg)


@pytest.mark.parametrize("cfg", [
    # pipelined large-tile kernel, 16-row small-tile kernel, f32 kernel: the
    # fused forward reads token rows through token_of_row, the split path
    # reads the dispatched copy; both must give the same bits
    S.small_config("split", T=257, H=128, I=192, E=9, top_k=3, dtype="bf16", seed=41),
    S.small_config("split_small", T=20, H=96, I=64, E=16, top_k=2, dtype="f16", seed=43),
    S.small_config("split_f32", T=130, H=40, I=24, E=4, top_k=2, dtype="f32", seed=44),
    S.small_config("split_edge", T=300, H=64, I=96, E=16, top_k=4, dtype="bf16", edge_rows=True, seed=45),
    S.small_config("split_stream_mixed", T=1024, H=512, I=256, E=256, top_k=8, dtype="bf16", zipf_s=1.1, seed=46),
    S.small_config("split_decode", T=40, H=448, I=320, E=64, top_k=4, dtype="bf16", seed=47),
], ids=lambda c: c.name)
def test_split_stages_equal_fused_forward(cfg):
    log(f"split == fused {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = [w.to(DEV) for w in S.make_weights(cfg)]
    ex = moe.SwiGluExperts(*W)
    opts = moe.RoutingOptions(cfg.top_k, True)
    gx, glg = x.to(DEV), lg.to(DEV)
    fused = ex.forward(gx, glg, opts)
    plan = moe.route(glg, opts)
    disp = plan.dispatch(gx)
    y = ex.forward_dispatched(disp)
    split = disp.combine(y)
    torch.cuda.synchronize()
    bits = torch.int32 if fused.dtype == torch.float32 else torch.int16
    assert torch.equal(fused.view(bits), split.view(bits))


@pytest.mark.parametrize("cfg", [
    # the 64-K kernel's persistent launch (its claim words cleared by the
    # tile-list kernel of each call), and the decode stream kernel
    S.small_config("graph_pipe64", T=2048, H=512, I=384, E=16, top_k=2, dtype="bf16", seed=61),
    S.small_config("graph_decode", T=24, H=256, I=192, E=32, top_k=4, dtype="bf16", seed=62),
], ids=lambda c: c.name)
def test_fused_forward_replays_in_a_hip_graph(cfg):
    """The fused forward captured in a HIP graph: no memset, copy or
    allocation of its own inside, so every replay must give the eager bits.
    Replays are separated by eager forwards on other inputs, which leave the
    workspace (tile list, claim words) in another state each time."""
    log(f"graph replay {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = [w.to(DEV) for w in S.make_weights(cfg)]
    ex = moe.SwiGluExperts(*W)
    opts = moe.RoutingOptions(cfg.top_k, True)
    gx, glg = x.to(DEV), lg.to(DEV)
    need = moe.load().moe_forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.top_k, 2)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty_like(gx)
    eager = ex.forward(gx, glg, opts, workspace=ws).clone()
    other_x, other_lg = torch.randn_like(gx), torch.randn_like(glg)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ex.forward(gx, glg, opts, workspace=ws, out=out)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ex.forward(gx, glg, opts, workspace=ws, out=out)
    bits = torch.int16
    for rep in range(3):
        out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(bits), eager.view(bits)), f"replay {rep}"
        ex.forward(other_x, other_lg, opts, workspace=ws)
        torch.cuda.synchronize()


def test_forward_empty_batch():
    cfg = S.small_config("empty", T=0, H=64, I=64, E=4, top_k=2, dtype="bf16")
    W = [w.to(DEV) for w in S.make_weights(cfg)]
    ex = moe.SwiGluExperts(*W)
    out = ex.forward(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV),
                     torch.empty(0, 4, dtype=torch.bfloat16, device=DEV), moe.RoutingOptions(2, True))
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_forward_single_token():
    run_forward_case(S.small_config("single", T=1, H=64, I=128, E=8, top_k=2, dtype="bf16", seed=42))


def test_errors_surface_as_moeerror():
    W = [w.to(DEV) for w in S.make_weights(S.small_config("err", T=4, H=64, I=64, E=4, top_k=2, dtype="bf16"))]
    ex = moe.SwiGluExperts(*W)
    x = torch.zeros(4, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(moe.MoeError) as e:
        ex.forward(x, torch.zeros(4, 5, dtype=torch.bfloat16, device=DEV), moe.RoutingOptions(2, True))
    assert e.value.name == "MOE_ERR_SHAPE"
    with pytest.raises(moe.MoeError) as e:
        ex.forward(x, torch.zeros(4, 4, dtype=torch.bfloat16, device=DEV), moe.RoutingOptions(5, True))
    assert e.value.name == "MOE_ERR_TOP_K"
    with pytest.raises(moe.MoeError) as e:
        ex.forward(x.cpu(), torch.zeros(4, 4, dtype=torch.bfloat16, device=DEV), moe.RoutingOptions(2, True))
    assert e.value.name == "MOE_ERR_DEVICE"


# ------------------------------------------------------------------ full-size workloads
def tile_covering_tokens(offsets, tor, BM=256):
    """One token at the first and one at the last row of every BM-row token
    tile of every expert (the tiles the expert products walk), so every live
    (expert, token tile) pair of the forward has checked rows."""
    pick = set()
    for e in range(len(offsets) - 1):
        for r0 in range(int(offsets[e]), int(offsets[e + 1]), BM):
            r1 = min(r0 + BM, int(offsets[e + 1]))
            pick.add(int(tor[r0]))
            pick.add(int(tor[r1 - 1]))
    return np.array(sorted(pick), dtype=np.int64)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["prefill_bf16", "decode_bf16", "skewed_bf16"])
def test_full_size(name):
    """The benchmark's workloads at full size, on the kernels and launch
    configuration the benchmark times.  The fused forward is run, then the
    same chain as split calls (route, mapping-only dispatch, gate/up through
    token_of_row, down, combine), whose mapping the test keeps: the two must
    agree bit for bit, so the split run's tiles are the fused run's.  Routing
    and dispatch are compared in full; the output is compared against the
    oracle on every token for prefill and decode, and for the skewed workload
    on the tokens at the first and last row of every token tile of every
    expert."""
    cfg = S.CONFIGS[name]
    log(f"full-size {name}: generating inputs on the GPU")
    x, lg = S.make_tokens(cfg, device=DEV)
    W = S.make_weights(cfg, device=DEV)
    ex = moe.SwiGluExperts(*W)
    opts = moe.RoutingOptions(cfg.top_k, cfg.renormalize)
    out = ex.forward(x, lg, opts)
    plan = moe.route(lg, opts)
    m = plan.dispatch(x, copy_rows=False)
    h = ex.gate_up_gathered(x, m.token_of_row, m.expert_offsets)
    split = m.combine(ex.down_proj(h, m.expert_offsets))
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), split.view(torch.int16)), "fused and split forwards differ"
    del h, split
    log(f"full-size {name}: routing parity over all {cfg.T} tokens")
    lgb = host_bits(lg)
    (o_idx, _), near = compare_routing(host_bits(plan.expert_indices()), plan.weights().cpu(), lgb,
                                       cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    assert near.mean() < 0.01
    log(f"full-size {name}: dispatch invariants over all rows")
    xb = host_bits(x)
    d = plan.dispatch(x)
    torch.cuda.synchronize()
    gidx = host_bits(plan.expert_indices())
    o = oracle.dispatch(gidx, cfg.E, xb, cfg.dtype)
    gpu = {"rows": host_bits(d.rows), "offsets": host_bits(d.expert_offsets),
           "row_of_slot": host_bits(d.row_of_slot), "token_of_row": host_bits(d.token_of_row)}
    compare_dispatch(gpu, *o, xb, gidx, cfg.E)
    del d, gpu, o
    if name == "skewed_bf16":
        sample = tile_covering_tokens(host_bits(m.expert_offsets), host_bits(m.token_of_row))
    else:
        sample = np.arange(cfg.T)
    sample = sample[~near[sample]]
    experts = sorted(set(o_idx[sample].reshape(-1).tolist()))
    log(f"full-size {name}: oracle on {len(sample)} of {cfg.T} tokens, {len(experts)} experts, "
        f"{NTHREADS} threads")
    g = {e: host_bits(W[0][e]) for e in experts}
    u = {e: host_bits(W[1][e]) for e in experts}
    dn = {e: host_bits(W[2][e]) for e in experts}
    res = oracle.forward(xb[sample], lgb[sample], g, u, dn, cfg.dtype, cfg.logits_dtype, cfg.top_k,
                         cfg.renormalize, NTHREADS)
    assert_close(values(out, cfg.dtype)[sample], oracle.widen(res["output"], cfg.dtype), cfg.dtype,
                 f"forward {name} ({len(sample)} tokens)")
    log(f"full-size {name}: {len(sample)} tokens match")
    # properties at every token: finite output, bitwise reproducible
    assert torch.isfinite(out.float()).all()
    out2 = ex.forward(x, lg, opts)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))


def test_token_buffer_over_4gib_sampled():
    """A token buffer of 4.4 GB: the 64-K kernel addresses token rows with
    32-bit offsets, so the host must send this size to the 64-bit kernel.  A
    wrapped offset would read a lower row of the same buffer (wrong values,
    no access outside it), which the sampled tokens past 2^32 bytes catch."""
    cfg = S.small_config("tokens_over_4gib_bf16", T=270000, H=8192, I=64, E=4, top_k=1, dtype="bf16", seed=61)
    assert cfg.T * cfg.H * 2 > 1 << 32
    log(f"{cfg.name}: generating {cfg.T * cfg.H * 2 / 1e9:.1f} GB of tokens on the GPU")
    x, lg = S.make_tokens(cfg, device=DEV)
    W = S.make_weights(cfg, device=DEV)
    ex = moe.SwiGluExperts(*W)
    opts = moe.RoutingOptions(cfg.top_k, cfg.renormalize)
    out = ex.forward(x, lg, opts)
    torch.cuda.synchronize()
    # tokens whose rows start past 2^32 bytes, and a few below
    first_high = (1 << 32) // (cfg.H * 2)
    rng = np.random.default_rng(cfg.seed)
    sample = np.sort(np.concatenate([rng.choice(np.arange(first_high, cfg.T), 12, replace=False),
                                     rng.choice(first_high, 4, replace=False)]))
    st = torch.from_numpy(sample).to(DEV)
    log(f"{cfg.name}: oracle on {len(sample)} sampled tokens")
    g = {e: host_bits(W[0][e]) for e in range(cfg.E)}
    u = {e: host_bits(W[1][e]) for e in range(cfg.E)}
    dn = {e: host_bits(W[2][e]) for e in range(cfg.E)}
    res = oracle.forward(host_bits(x[st]), host_bits(lg[st]), g, u, dn, cfg.dtype, cfg.logits_dtype, cfg.top_k,
                         cfg.renormalize, NTHREADS)
    assert_close(values(out[st], cfg.dtype), oracle.widen(res["output"], cfg.dtype), cfg.dtype,
                 f"forward {cfg.name} (sampled tokens)")


@pytest.mark.parametrize("cfg", [
    S.small_config("halves_bf16", T=300, H=128, I=192, E=6, top_k=2, dtype="bf16", seed=51),
    S.small_config("halves_small_f16", T=20, H=64, I=96, E=16, top_k=4, dtype="f16", seed=52),
], ids=lambda c: c.name)
def test_gate_up_and_down_halves_equal_experts_forward(cfg):
    """moe_experts_gate_up followed by moe_experts_down runs the same kernels
    as moe_experts_forward: the results are bitwise equal, and h matches the
    oracle's stored activation."""
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    Wb = [host_bits(w) for w in W]
    idx, _, _ = oracle.route(host_bits(lg), cfg.logits_dtype, cfg.top_k, cfg.renormalize, NTHREADS)
    offsets, _, _, rows = oracle.dispatch(idx, cfg.E, host_bits(x), cfg.dtype)
    _, h_ref = oracle.experts(*Wb, cfg.dtype, rows, offsets, cfg.E, cfg.H, cfg.I, with_h=True, nthreads=NTHREADS)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    g_rows = S.from_bits(rows, cfg.dtype, DEV)
    g_off = torch.from_numpy(offsets.view(np.int32)).view(torch.uint32).to(DEV)
    whole = ex.forward_dispatched(g_rows, g_off)
    h = ex.gate_up(g_rows, g_off)
    y = ex.down_proj(h, g_off)
    torch.cuda.synchronize()
    assert torch.equal(whole.view(torch.int16), y.view(torch.int16))
    assert_close(values(h, cfg.dtype), oracle.widen(h_ref, cfg.dtype), cfg.dtype, "activation h")


# ------------------------------------------------------------------ group-limited sigmoid routing
def grouped_case(name, T, E, dtype, k, G, m, top_two, renorm, scale, seed, bias="normal", ties=False,
                 nan_rows=False):
    return dict(name=name, T=T, E=E, dtype=dtype, k=k, G=G, m=m, top_two=top_two, renorm=renorm, scale=scale,
                seed=seed, bias=bias, ties=ties, nan_rows=nan_rows)


GROUPED_CASES = [
    # the skewed workload's routing shape: 256 experts in 8 groups, the best 4
    # by their top two corrected scores, top-8, renormalised, scaled 2.5
    grouped_case("ds_bf16", 2048, 256, "bf16", 8, 8, 4, True, True, 2.5, 61),
    grouped_case("ds_f32", 1024, 256, "f32", 8, 8, 4, True, True, 2.5, 62),
    grouped_case("ds_f16_nobias", 1024, 256, "f16", 8, 8, 4, True, False, 1.0, 63, bias=None),
    grouped_case("one_group_f32", 512, 64, "f32", 6, 1, 1, False, True, 1.0, 64),
    grouped_case("max_shape_bf16", 256, 1024, "bf16", 64, 128, 32, True, True, 2.0, 65),
    grouped_case("small_groups_f32", 700, 96, "f32", 5, 32, 3, False, False, 0.5, 66),
    grouped_case("ties_f32", 2000, 16, "f32", 4, 4, 2, True, True, 1.0, 67, ties=True),
    grouped_case("ties_max_bf16", 2000, 32, "bf16", 3, 8, 2, False, True, 1.0, 68, ties=True),
    grouped_case("nan_rows_bf16", 600, 64, "bf16", 4, 8, 2, True, True, 1.0, 69, nan_rows=True),
    grouped_case("odd_E_f32", 300, 40, "f32", 7, 5, 3, True, True, 1.5, 70),
]


def make_grouped_inputs(c):
    g = torch.Generator().manual_seed(c["seed"])
    if c["ties"]:
        lg = torch.randint(-1, 2, (c["T"], c["E"]), generator=g).float()
        bias = torch.tensor([0.0, 0.25, -0.25])[torch.randint(0, 3, (c["E"],), generator=g)]
    else:
        lg = torch.randn(c["T"], c["E"], generator=g)
        bias = torch.randn(c["E"], generator=g) * 0.3
    if c["nan_rows"]:
        rows = torch.randperm(c["T"], generator=g)[: c["T"] // 10]
        lg[rows[: len(rows) // 2], 3] = float("nan")
        lg[rows[len(rows) // 2:], :] = float("inf")  # sigmoid 1 everywhere: ties, lower ids
    lg = lg.to(S.TORCH_DT[c["dtype"]])
    return lg, (None if c["bias"] is None else bias.float().contiguous())


@pytest.mark.parametrize("c", GROUPED_CASES, ids=lambda c: c["name"])
def test_route_sigmoid_grouped_parity(c):
    log(f"grouped routing {c['name']}")
    lg, bias = make_grouped_inputs(c)
    opts = moe.GroupRoutingOptions(c["k"], c["G"], c["m"], c["top_two"], c["renorm"], c["scale"])
    plan = moe.route_sigmoid_grouped(lg.to(DEV), None if bias is None else bias.to(DEV), opts)
    torch.cuda.synchronize()
    compare_grouped_routing(host_bits(plan.expert_indices()), plan.weights().cpu(), host_bits(lg), c["dtype"],
                            None if bias is None else bias.numpy(), c["k"], c["G"], c["m"], c["top_two"],
                            c["renorm"], c["scale"], NTHREADS)


@pytest.mark.parametrize("cfg", [
    S.small_config("grouped_fwd_bf16", T=700, H=128, I=192, E=32, top_k=4, dtype="bf16", seed=71),
    S.small_config("grouped_fwd_f32", T=200, H=64, I=96, E=16, top_k=3, dtype="f32", seed=72),
], ids=lambda c: c.name)
def test_forward_sigmoid_grouped_parity(cfg):
    """The chain with group-limited sigmoid routing against the oracle's
    routing, dispatch, experts and combine, and bitwise against the split
    calls fed by the same routing."""
    log(f"grouped forward {cfg.name}")
    x, lg = S.make_tokens(cfg)
    W = S.make_weights(cfg)
    bias = (torch.randn(cfg.E, generator=torch.Generator().manual_seed(cfg.seed)) * 0.3).float()
    G, m = 4, 2
    opts = moe.GroupRoutingOptions(cfg.top_k, G, m, True, True, 2.5)
    ex = moe.SwiGluExperts(*[w.to(DEV) for w in W])
    gx, glg, gb = x.to(DEV), lg.to(DEV), bias.to(DEV)
    out = ex.forward_sigmoid_grouped(gx, glg, gb, opts)
    plan = moe.route_sigmoid_grouped(glg, gb, opts)
    d = plan.dispatch(gx)
    split = d.combine(ex.forward_dispatched(d))
    torch.cuda.synchronize()
    bits = torch.int32 if out.dtype == torch.float32 else torch.int16
    assert torch.equal(out.view(bits), split.view(bits))
    (o_idx, o_w), near = compare_grouped_routing(host_bits(plan.expert_indices()), plan.weights().cpu(),
                                                 host_bits(lg), cfg.logits_dtype, bias.numpy(), cfg.top_k, G, m,
                                                 True, True, 2.5, NTHREADS)
    Wb = [host_bits(w) for w in W]
    xb = host_bits(x)
    offsets, ros, _, rows = oracle.dispatch(o_idx, cfg.E, xb, cfg.dtype)
    Y = oracle.experts(*Wb, cfg.dtype, rows, offsets, cfg.E, cfg.H, cfg.I, nthreads=NTHREADS)
    ref = oracle.combine(Y, cfg.dtype, ros, o_w, cfg.logits_dtype, cfg.T, cfg.top_k, cfg.H, NTHREADS)
    assert_close(values(out, cfg.dtype), oracle.widen(ref, cfg.dtype), cfg.dtype, f"grouped forward {cfg.name}",
                 rows_mask=~near)
