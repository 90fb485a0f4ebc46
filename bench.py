#!/usr/bin/env python3
"""Benchmark of the local MoE forward chain (route -> dispatch -> SwiGLU
experts -> combine) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload prefill_bf16]

A step is one fused moe_forward over the whole batch (all stages), with the
inputs and weights already resident in HBM.  Prints one JSON line:
  value        whole-job tokens/s of the timed fused forwards;
  event_ms_per_step  their per-step device times (mean, median), and the
               median of K more forwards each run after a 512 MiB scratch
               read that flushes the last-level cache (cold_median);
  roofline     the dominant kernel (the gate/up grouped GEMM), its
               algorithmic FLOPs (or bytes, at decode) per launch over its
               average launch time, measured with HIP events recorded on the
               stream it runs on, against the MI355X dense peak;
  stages_ms    per-stage times of the split calls (same kernels), and the
               algorithmic HBM GB/s of routing, dispatch (mapping only, and
               the split API's copying dispatch) and combine;
  cpu_baseline the CPU oracle timed on a bounded sample of the same workload;
  secondary    the decode and skewed workloads, same measurement;
  grouped_routing  the skewed workload's forward with group-limited sigmoid
               routing, and that routing kernel's HBM roofline;
  training     one first-order training step on the prefill workload (route,
               FP32 router weights, dispatch, experts forward with its cache,
               combine, then the combine, experts, dispatch and router
               backward), its stage times, the experts backward's MFMA
               roofline and the oracle's step on a bounded token sample.
The pages publish no throughput for this chain, so vs_baseline is null.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import re
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE forward tokens/s + TFLOP/s (% bf16 MFMA peak) / HBM GB/s at decode"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")
_CSRC = os.path.join(ROOT, "mixture_experts_layer_route_amd", "csrc")
# every source compiled into the expert GEMM kernels
GEMM_SRCS = [os.path.join(_CSRC, f) for f in ("experts.hip", "mfma.h", "tiles.h", "moe_internal.h")]


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # the first ~30 forward steps after the GPU starts working run up to 10%
    # slower while its clock settles (a kernel trace of 30 fused, 30 split and
    # 30 fused forwards: gate/up 606, 554 and 550 us on average), so the
    # untimed warmup covers that transient
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="prefill_bf16",
                    choices=["prefill_bf16", "decode_bf16", "skewed_bf16"])
    ap.add_argument("--secondary", default="decode_bf16,skewed_bf16",
                    help="comma-separated extra workloads to measure ('' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    ap.add_argument("--grouped", default="skewed_bf16",
                    help="workload for the forward with group-limited sigmoid routing ('' to skip)")
    ap.add_argument("--training", default="prefill_bf16",
                    help="workload of the training-step measurement ('' to skip)")
    ap.add_argument("--only-training", action="store_true",
                    help="measure only the training step (for profiler runs)")
    ap.add_argument("--only-forward", action="store_true",
                    help="time only the fused forward (for profiler runs)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after measuring, copy this many MiB device-to-device once: a kernel of known "
                         "traffic for scaling HBM byte counters (FETCH_SIZE / WRITE_SIZE)")
    return ap.parse_args()


def kernel_hash() -> str:
    """sha256 prefix of the GEMM kernels' sources (the kernel file and the
    headers compiled into it) with comments and blank space removed, so an
    edit of a comment does not retire the counters."""
    parts = []
    for path in GEMM_SRCS:
        with open(path) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        parts.append(" ".join(src.split()))
    return hashlib.sha256("\n".join(parts).encode()).hexdigest()[:16]


def traffic_for(workload: str):
    """HBM bytes per launch of the dominant kernel from the committed PMC
    counter summary, or None when absent or taken on an older kernel."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else w.get("bytes_per_launch")


STAGE_WARMUP = 40


def measure(name: str, steps: int, warmup: int, only_forward: bool = False) -> dict:
    import torch

    import mixture_experts_layer_route_amd as moe
    import moe_synth as S

    cfg = S.CONFIGS[name]
    dev = "cuda:0"
    x, lg = S.make_tokens(cfg, device=dev)
    W = S.make_weights(cfg, device=dev)
    ex = moe.SwiGluExperts(*W)
    opts = moe.RoutingOptions(cfg.top_k, cfg.renormalize)
    ws = torch.empty(ex.forward_workspace_bytes(cfg.T, cfg.top_k, x.dtype), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    res = {"workload": name, "cfg": cfg}
    # The split-stage loop (at least 40 untimed iterations, then K timed) is
    # only enqueued here, and the fused forwards follow it with no idle gap:
    # the GPU's power control answers any idle gap of 10 ms or more with ~30
    # forwards that run up to 30% slower before settling (prefill, per-step
    # events: 0.89, 0.92, 1.01, 1.09, 1.11, ... back to 0.89 ms by the 30th),
    # which a warmup of a few steps would otherwise leave in the timed region.
    stage = None
    if not only_forward:
        stage = stage_loop(moe, ex, x, lg, opts, cfg, steps, max(warmup, STAGE_WARMUP))

    # The timed region: W untimed fused forwards, then exactly K, bracketed
    # by synchronisations; an event before each step gives per-step device
    # times (their median sits next to the wall-clock mean).
    for _ in range(warmup):
        ex.forward(x, lg, opts, ws, out)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i].record()
        ex.forward(x, lg, opts, ws, out)
    evs[steps].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    ms_step = wall * 1e3 / steps
    res.update({"ms_per_step": ms_step, "event_ms_mean": sum(per) / steps,
                "event_ms_median": (per[(steps - 1) // 2] + per[steps // 2]) / 2,
                "tokens_per_s": cfg.T * steps / wall})
    res["tflops"] = cfg.flops() / (ms_step * 1e-3) / 1e12
    if stage is not None:
        res["event_ms_cold_median"] = cold_forwards(ex, x, lg, opts, ws, out, steps)
        res.update(stage_results(stage, x, steps, warmup))
    return res


COLD_SCRATCH_MIB = 512


def cold_forwards(ex, x, lg, opts, ws, out, steps: int) -> float:
    """Median device time of K fused forwards, each after a 512 MiB scratch
    read that evicts the 256 MB last-level cache, so no input of the forward
    is cached when it starts (timed after the K steps of record, back to
    back, with events around each forward only).  The scratch is written once
    beforehand: flushing with writes would leave the forward ~256 MB of dirty
    lines to write back, which added ~50 us to the decode forward."""
    import torch

    scratch = torch.ones(COLD_SCRATCH_MIB << 17, dtype=torch.int32, device=x.device)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        scratch.sum()
        a.record()
        ex.forward(x, lg, opts, ws, out)
        b.record()
    torch.cuda.synchronize()
    per = sorted(a.elapsed_time(b) for a, b in evs)
    del scratch
    return (per[(steps - 1) // 2] + per[steps // 2]) / 2


def stage_loop(moe, ex, x, lg, opts, cfg, steps: int, warmup: int) -> dict:
    """Enqueues the per-stage timing loop: the split calls run the kernels of
    the fused forward (mapping-only dispatch, gate/up reading the tokens in
    place), back to back like the forward steps, with events on the stream
    every call is launched on (torch's current stream).  Nothing here waits
    for the GPU; stage_results reads the events."""
    import torch

    ews = torch.empty(moe.load().moe_experts_workspace_bytes(cfg.N, cfg.H, cfg.I, cfg.E, 2 if cfg.dtype == "bf16"
                                                              else (1 if cfg.dtype == "f16" else 0)),
                      dtype=torch.uint8, device=x.device)
    plan = None
    marks = []
    for it in range(warmup + steps):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
        evs[0].record()
        plan = moe.route(lg, opts)
        evs[1].record()
        disp = plan.dispatch(x, copy_rows=False)
        evs[2].record()
        h = ex.gate_up_gathered(x, disp.token_of_row, disp.expert_offsets, ews)
        evs[3].record()
        y = ex.down_proj(h, disp.expert_offsets, ews)
        evs[4].record()
        disp.combine(y)
        evs[5].record()
        if it >= warmup:
            marks.append(evs)
    return {"marks": marks, "plan": plan}


def stage_results(stage: dict, x, steps: int, warmup: int) -> dict:
    """Per-stage times from the loop stage_loop enqueued (the GPU has
    finished it), then the split API's copying dispatch alone, timed after
    everything else."""
    import torch

    names = ["route", "dispatch", "experts_gate_up", "experts_down", "combine"]
    acc = {n: 0.0 for n in names}
    for evs in stage["marks"]:
        for i, n in enumerate(names):
            acc[n] += evs[i].elapsed_time(evs[i + 1])
    res = {"stages_ms": {n: acc[n] / steps for n in names}}
    plan = stage["plan"]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(warmup):
        plan.dispatch(x)
    e0.record()
    for _ in range(steps):
        plan.dispatch(x)
    e1.record()
    torch.cuda.synchronize()
    res["dispatch_copy_ms"] = e0.elapsed_time(e1) / steps
    idx = plan.expert_indices().view(torch.int32).long()
    res["active_experts"] = int(torch.unique(idx).numel())
    return res


def event_ms(res: dict) -> dict:
    """Per-step device times of the fused forward: the mean and median of the
    timed steps, and the median with the last-level cache flushed first."""
    d = {"mean": round(res["event_ms_mean"], 4), "median": round(res["event_ms_median"], 4)}
    if "event_ms_cold_median" in res:
        d["cold_median"] = round(res["event_ms_cold_median"], 4)
    return d


def roofline(res: dict) -> dict:
    cfg = res["cfg"]
    t = res["stages_ms"]["experts_gate_up"] * 1e-3
    es = 2 if cfg.dtype in ("bf16", "f16") else 4
    if res["workload"] == "decode_bf16":
        # weight streaming: each active expert's gate and up rows are read
        # once; plus the token rows read (in place, once per token) and the
        # activation written
        nbytes = res["active_experts"] * 2 * cfg.I * cfg.H * es + cfg.T * cfg.H * es + cfg.N * cfg.I * es
        ach = nbytes / t / 1e9
        r = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": round(ach / PEAK_HBM_GBS, 4)}
    else:
        flops = 4.0 * cfg.N * cfg.H * cfg.I  # gate and up products
        ach = flops / t / 1e12
        r = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
             "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
    r["kernel"] = ("decode_stream_kernel (gate/up, fused SiLU*mul)"
                   if res["workload"] == "decode_bf16" else "grouped_gemm_pipe64_kernel (gate/up, fused SiLU*mul)")
    r["avg_launch_ms"] = round(res["stages_ms"]["experts_gate_up"], 4)
    r["traffic"] = traffic_for(res["workload"])
    return r


def hbm_bytes_forward(res: dict) -> float:
    """Algorithmic HBM bytes of one forward: active experts' weights once,
    tokens/logits/output once, the routing and mapping arrays once, the
    expert outputs written and read once, the activation written and read
    once (the token rows are read in place, no dispatched copy)."""
    cfg = res["cfg"]
    es = 2 if cfg.dtype in ("bf16", "f16") else 4
    w = res["active_experts"] * 3 * cfg.H * cfg.I * es
    io = cfg.T * cfg.H * es * 2 + cfg.T * cfg.E * es + cfg.N * (4 + es)
    inter = 2 * cfg.N * cfg.H * es + 2 * cfg.N * cfg.I * es
    return w + io + inter


def oracle_threads() -> int:
    """Every core this process may run on."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(name: str, target_s: float) -> dict:
    """The oracle's whole forward on the first n tokens of workload `name`
    (n sized for about target_s seconds), on every core this process may run
    on; then its per-stage times on every workload (cpu_stages)."""
    import torch

    import moe_synth as S
    import oracle

    cfg = S.CONFIGS[name]
    threads = oracle_threads()
    x, lg = S.make_tokens(cfg, device="cuda:0")
    xb, lgb = S.to_bits(x), S.to_bits(lg)
    cache = {}

    def run(n):
        idx, _, _ = oracle.route(lgb[:n], cfg.logits_dtype, cfg.top_k, cfg.renormalize, threads)
        g, u, d = expert_bits(cfg, sorted(set(idx.reshape(-1).tolist())), cache)
        t0 = time.perf_counter()
        oracle.forward(xb[:n], lgb[:n], g, u, d, cfg.dtype, cfg.logits_dtype, cfg.top_k, cfg.renormalize, threads)
        return time.perf_counter() - t0

    probe = 16
    dt = run(probe)
    n = int(max(probe, min(cfg.T, probe * target_s / max(dt, 1e-3))))
    dt = run(n)
    cache.clear()
    torch.cuda.empty_cache()
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens of {name}, whole forward (route, dispatch, experts, "
                      f"combine), {dt:.1f} s on {threads} threads",
            "stages": cpu_stages(threads)}


def expert_bits(cfg, experts, cache):
    """Host bits of the gate, up and down matrices of `experts`, each drawn on
    the GPU from its own stream (the values make_weights draws)."""
    import moe_synth as S

    for e in experts:
        if e not in cache:
            cache[e] = tuple(S.to_bits(w) for w in S.make_expert(cfg, e, device="cuda:0"))
    return ({e: cache[e][0] for e in experts}, {e: cache[e][1] for e in experts},
            {e: cache[e][2] for e in experts})


# tokens of each workload the per-stage oracle timing covers: the small
# workloads whole, the large ones on their first tokens (seconds each)
CPU_STAGE_TOKENS = {"tiny_f32": 64, "edge_f32": 1024, "prefill_bf16": 1024, "decode_bf16": 32,
                    "skewed_bf16": 64}


def cpu_stages(threads: int) -> dict:
    """Wall seconds of each oracle stage (route, dispatch, experts, combine)
    on every workload, on the first CPU_STAGE_TOKENS tokens of each."""
    import moe_synth as S
    import oracle

    out = {}
    for name, n in CPU_STAGE_TOKENS.items():
        cfg = S.CONFIGS[name]
        x, lg = S.make_tokens(cfg, device="cuda:0")
        n = min(n, cfg.T)
        xb, lgb = S.to_bits(x[:n]), S.to_bits(lg[:n])
        t = {}
        t0 = time.perf_counter()
        idx, w, _ = oracle.route(lgb, cfg.logits_dtype, cfg.top_k, cfg.renormalize, threads)
        t["route"] = time.perf_counter() - t0
        t0 = time.perf_counter()
        offsets, ros, _, rows = oracle.dispatch(idx, cfg.E, xb, cfg.dtype)
        t["dispatch"] = time.perf_counter() - t0
        experts = sorted(e for e in set(idx.reshape(-1).tolist()) if e < cfg.E)
        g, u, d = expert_bits(cfg, experts, {})
        t0 = time.perf_counter()
        Y = oracle.experts(g, u, d, cfg.dtype, rows, offsets, cfg.E, cfg.H, cfg.I, nthreads=threads)
        t["experts"] = time.perf_counter() - t0
        del g, u, d
        t0 = time.perf_counter()
        oracle.combine(Y, cfg.dtype, ros, w, cfg.logits_dtype, n, cfg.top_k, cfg.H, threads)
        t["combine"] = time.perf_counter() - t0
        total = sum(t.values())
        out[name] = {"tokens": n, "of": cfg.T, "active_experts": len(experts),
                     "seconds": {k: round(v, 4) for k, v in t.items()}, "total_s": round(total, 4),
                     "tokens_per_s": round(n / total, 2)}
    return out


def measure_grouped(name: str, steps: int, warmup: int) -> dict:
    """The forward with group-limited sigmoid routing on workload `name`
    (8 groups, the best 4 by their top-two corrected scores, renormalised,
    scale 2.5, a small seeded FP32 correction bias), and the routing kernel
    alone, both timed back to back with HIP events."""
    import torch

    import mixture_experts_layer_route_amd as moe
    import moe_synth as S

    cfg = S.CONFIGS[name]
    dev = "cuda:0"
    x, lg = S.make_tokens(cfg, device=dev)
    W = S.make_weights(cfg, device=dev)
    ex = moe.SwiGluExperts(*W)
    bias = (torch.randn(cfg.E, generator=torch.Generator().manual_seed(cfg.seed)) * 0.1).float().to(dev)
    opts = moe.GroupRoutingOptions(cfg.top_k, 8, 4, True, True, 2.5)
    ws = torch.empty(ex.forward_workspace_bytes(cfg.T, cfg.top_k, x.dtype), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    for _ in range(warmup):
        ex.forward_sigmoid_grouped(x, lg, bias, opts, ws, out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        ex.forward_sigmoid_grouped(x, lg, bias, opts, ws, out)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    reps = max(steps, 20)
    for _ in range(warmup):
        moe.route_sigmoid_grouped(lg, bias, opts)
    ev[0].record()
    for _ in range(reps):
        plan = moe.route_sigmoid_grouped(lg, bias, opts)
    ev[1].record()
    torch.cuda.synchronize()
    route_ms = ev[0].elapsed_time(ev[1]) / reps
    ls = 2 if cfg.logits_dtype in ("bf16", "f16") else 4
    nbytes = cfg.T * cfg.E * ls + cfg.E * 4 + cfg.T * cfg.top_k * (4 + ls)
    ach = nbytes / (route_ms * 1e-3) / 1e9
    idx = plan.expert_indices().view(torch.int32).long()
    return {"workload": name, "routing": "group-limited sigmoid: 8 groups, best 4 by top-two, renormalised, scale 2.5",
            "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
            "tflops": round(cfg.flops() / (ms * 1e-3) / 1e12, 2),
            "active_experts": int(torch.unique(idx).numel()),
            "route_roofline": {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                               "frac": round(ach / PEAK_HBM_GBS, 4), "kernel": "route_grouped_kernel",
                               "avg_launch_ms": round(route_ms, 4), "bytes_per_launch": nbytes}}


def training_step(moe, ex, x, lg, gout, cfg, opt, marks=None):
    """One first-order training step through the public calls; with `marks`
    (a list) HIP events are recorded between the stages on the current stream."""
    import torch

    def mark():
        if marks is not None:
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            marks.append(e)

    mark()
    plan = moe.route(lg, moe.RoutingOptions(cfg.top_k, cfg.renormalize))
    tp = plan.into_training(lg, opt)
    mark()
    d = tp.routing().dispatch(x, copy_rows=False)
    mark()
    y, cache = ex.forward_dispatched_training(d, input=x)
    mark()
    d.combine(y)
    mark()
    dy, dw = d.combine_backward(y, gout)
    mark()
    grads = cache.backward(dy)
    mark()
    d.dispatch_backward(grads[0])
    mark()
    tp.backward(dw)
    mark()
    return plan


TRAIN_STAGES = ["route_and_weights", "dispatch", "experts_forward_training", "combine", "combine_backward",
                "experts_backward", "dispatch_backward", "router_backward"]


def measure_training(name: str, steps: int, warmup: int, cpu_seconds: float | None) -> dict:
    """Whole training steps back to back (wall time, one sync), then the
    same steps with HIP events between the stages (on the stream they are
    launched on), then the oracle's step on the first tokens of the batch."""
    import torch

    import mixture_experts_layer_route_amd as moe
    import moe_synth as S

    cfg = S.CONFIGS[name]
    dev = "cuda:0"
    x, lg = S.make_tokens(cfg, device=dev)
    W = S.make_weights(cfg, device=dev)
    gout = S.make_grad_output(cfg, device=dev)
    ex = moe.SwiGluExperts(*W)
    opt = moe.RouterWeightOptions("softmax", cfg.renormalize, 1.0)
    for _ in range(warmup):
        training_step(moe, ex, x, lg, gout, cfg, opt)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        plan = training_step(moe, ex, x, lg, gout, cfg, opt)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    all_marks = []
    for _ in range(steps):
        m = []
        training_step(moe, ex, x, lg, gout, cfg, opt, m)
        all_marks.append(m)
    torch.cuda.synchronize()
    st = {n: sum(m[i].elapsed_time(m[i + 1]) for m in all_marks) / steps for i, n in enumerate(TRAIN_STAGES)}
    # algorithmic FLOPs: forward 6 N H I (gate, up, down), backward 12 N H I
    # (dh, dx over K = 2I, dgate + dup, ddown)
    nhi = float(cfg.N) * cfg.H * cfg.I
    t_bwd = st["experts_backward"] * 1e-3
    ach = 12.0 * nhi / t_bwd / 1e12
    idx = plan.expert_indices().view(torch.int32).long()
    out = {"workload": f"{name}: {cfg.description}", "ms_per_step": round(ms, 4),
           "tokens_per_s": round(cfg.T / (ms * 1e-3), 1), "tflops": round(18.0 * nhi / (ms * 1e-3) / 1e12, 2),
           "active_experts": int(torch.unique(idx).numel()),
           "stages_ms": {k: round(v, 4) for k, v in st.items()},
           "roofline": {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                        "kernel": "train_pipe2_kernel x4 (experts backward: dh, dx, dgate+dup, ddown)",
                        "avg_launch_ms": round(st["experts_backward"], 4), "flops_per_launch": 12.0 * nhi,
                        "traffic": None}}
    del W, ex
    torch.cuda.empty_cache()
    if cpu_seconds:
        out["cpu_baseline"] = cpu_training_baseline(cfg, cpu_seconds)
    return out


def cpu_training_baseline(cfg, target_s: float) -> dict:
    """The oracle's training step (forward with caches and the four
    backward steps) on the first n tokens of the same batch."""
    import moe_synth as S
    import oracle

    threads = oracle_threads()
    x, lg = S.make_tokens(cfg, device="cuda:0")
    gout = S.make_grad_output(cfg, device="cuda:0")
    Wb = [S.to_bits(w) for w in S.make_weights(cfg, device="cuda:0")]
    xb, lgb, gb = S.to_bits(x), S.to_bits(lg), S.to_bits(gout)

    def run(n):
        t0 = time.perf_counter()
        oracle.train_step(xb[:n], lgb[:n], *Wb, cfg.dtype, cfg.logits_dtype, cfg.top_k, cfg.renormalize, gb[:n],
                          threads)
        return time.perf_counter() - t0

    probe = 8
    dt = run(probe)
    n = int(max(probe, min(cfg.T, probe * target_s / max(dt, 1e-3))))
    dt = run(n)
    return {"value": round(n / dt, 2), "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens, whole training step, {dt:.1f} s"}


def stage_gbs(res: dict) -> dict:
    """Algorithmic HBM GB/s of the memory-bound stages: routing reads the
    logits and writes indices and weights; the mapping-only dispatch reads
    the indices and writes the offsets and both mappings; the copying
    dispatch also reads the tokens and writes their k copies; combine reads
    the expert rows, the mapping and the weights and writes the output."""
    cfg = res["cfg"]
    es = 2 if cfg.dtype in ("bf16", "f16") else 4
    ls = 2 if cfg.logits_dtype in ("bf16", "f16") else 4
    T, N, E, H = cfg.T, cfg.N, cfg.E, cfg.H
    st = res["stages_ms"]
    nbytes = {
        "route": T * E * ls + N * (4 + ls),
        "dispatch": N * 4 + 2 * N * 4 + (E + 1) * 4,
        "dispatch_copy": N * 4 + T * H * es + N * H * es + 2 * N * 4 + (E + 1) * 4,
        "combine": N * H * es + N * (4 + ls) + T * H * es,
    }
    ms = {"route": st["route"], "dispatch": st["dispatch"], "dispatch_copy": res["dispatch_copy_ms"],
          "combine": st["combine"]}
    return {k: round(nbytes[k] / (ms[k] * 1e-3) / 1e9, 1) for k in nbytes}


def summary(res: dict) -> dict:
    cfg = res["cfg"]
    d = {"workload": res["workload"], "tokens_per_s": round(res["tokens_per_s"], 1),
         "ms_per_step": round(res["ms_per_step"], 4),
         "event_ms_per_step": event_ms(res),
         "tflops": round(res["tflops"], 2),
         "pct_bf16_peak": round(100 * res["tflops"] / PEAK_BF16_TFLOPS, 2)}
    if "stages_ms" in res:
        d["stages_ms"] = {k: round(v, 4) for k, v in res["stages_ms"].items()}
        d["active_experts"] = res["active_experts"]
        d["hbm_gbs_forward"] = round(hbm_bytes_forward(res) / (res["ms_per_step"] * 1e-3) / 1e9, 1)
        d["dispatch_copy_ms"] = round(res["dispatch_copy_ms"], 4)
        d["stage_hbm_gbs"] = stage_gbs(res)
        d["roofline"] = roofline(res)
    d["config"] = {"T": cfg.T, "H": cfg.H, "I": cfg.I, "E": cfg.E, "top_k": cfg.top_k,
                   "renormalize": cfg.renormalize, "dtype": cfg.dtype}
    return d


def progress(msg: str) -> None:
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the MoE chain here runs on a single device "
              "(no multi-GPU path is built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch

    import mixture_experts_layer_route_amd as moe

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    moe.load()
    if args.only_training:
        print(json.dumps({"training": measure_training(args.training or args.workload, args.steps, args.warmup,
                                                       None)}), flush=True)
        return
    progress(f"measuring {args.workload}")
    res = measure(args.workload, args.steps, args.warmup, args.only_forward)
    head = summary(res)
    cfg = res["cfg"]
    line = {
        "metric": METRIC,
        "value": round(res["tokens_per_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 4),
        "event_ms_per_step": event_ms(res),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; weights ~N(0,1/sqrt(fan_in)), no checkpoint)",
        "config": {"workload": f"{args.workload}: {cfg.description}", "T": cfg.T, "H": cfg.H, "I": cfg.I,
                   "E": cfg.E, "top_k": cfg.top_k, "renormalize": cfg.renormalize, "parallelism": "single GPU"},
        "tflops": head["tflops"],
        "pct_bf16_peak": head["pct_bf16_peak"],
    }
    if "roofline" in head:
        line["roofline"] = head["roofline"]
        line["stages_ms"] = head["stages_ms"]
        line["hbm_gbs_forward"] = head["hbm_gbs_forward"]
        line["dispatch_copy_ms"] = head["dispatch_copy_ms"]
        line["stage_hbm_gbs"] = head["stage_hbm_gbs"]
        line["active_experts"] = head["active_experts"]
    if not args.only_forward:
        sec = [s for s in args.secondary.split(",") if s and s != args.workload]
        line["secondary"] = {}
        for s in sec:
            torch.cuda.empty_cache()
            progress(f"measuring {s}")
            r = measure(s, args.steps, args.warmup)
            line["secondary"][s] = summary(r)
            del r
        torch.cuda.empty_cache()
        if args.grouped:
            progress("measuring the forward with group-limited sigmoid routing")
            line["grouped_routing"] = measure_grouped(args.grouped, args.steps, args.warmup)
            torch.cuda.empty_cache()
        if args.training:
            progress("measuring the training step")
            line["training"] = measure_training(args.training, args.steps, args.warmup,
                                                None if args.no_cpu_baseline else args.cpu_seconds)
            torch.cuda.empty_cache()
        if not args.no_cpu_baseline:
            progress("timing the CPU oracle")
            line["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_seconds)
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        line["calibration_copy_bytes"] = n
        del src, dst
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
