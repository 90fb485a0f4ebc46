"""Seeded synthetic inputs for the MoE forward chain.

This module serves both the HIP path and the CPU oracle and holds none of
the method's arithmetic: it only draws numbers, scales them, rounds them to
the storage dtype and moves bytes between torch and numpy.

Recipe (the same for every consumer):
  * each tensor -- and, for expert weights, each expert -- draws from its own
    torch generator, seeded by ``stream_seed(seed, tensor_id, expert)``, so a
    single expert can be regenerated without drawing the rest;
  * values are float32 standard normals, scaled, then rounded once to the
    storage dtype (round to nearest even, torch's ``.to``);
  * x ~ N(0, 1); logits ~ N(0, 1); gate and up have std 1/sqrt(H) (fan-in H);
    down has std 1/sqrt(I) (fan-in I);
  * the routing edge workload rounds its logits to integers (half to even)
    clamped to [-3, 3] and plants, in a seeded random set of rows, one NaN
    (5% of rows), one +inf (5%) or a row of -inf (2%);
  * the training step's output gradient is N(0, 1) [T,H] in the input dtype;
  * the skewed workload adds to every logit column e the bias
    2 * ln(w_(e+1)) with Zipf weights w_r = r^-1.1 / sum_j j^-1.1 (expert e
    has Zipf rank e + 1), so a few low-id experts are hot.

Values depend on the device that draws them (torch's CPU and GPU generators
differ); a test draws once and hands the same bytes to both sides.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

# tensor ids of the per-tensor streams
_X, _LOGITS, _GATE, _UP, _DOWN, _EDGE, _GRAD_OUT = 1, 2, 3, 4, 5, 6, 7


@dataclass(frozen=True)
class MoeConfig:
    name: str
    T: int
    H: int
    I: int
    E: int
    top_k: int
    renormalize: bool
    dtype: str        # input and weight dtype
    logits_dtype: str
    seed: int
    edge_rows: bool = False
    zipf_s: float | None = None
    description: str = field(default="", compare=False)

    @property
    def N(self) -> int:
        return self.T * self.top_k

    def flops(self) -> float:
        """6 * N * H * I: the two gate/up products and the down product."""
        return 6.0 * self.N * self.H * self.I


CONFIGS = {
    "tiny_f32": MoeConfig("tiny_f32", 64, 128, 256, 8, 2, True, "f32", "f32", 1000,
                          description="Tiny F32 MoE, T=64 H=128 I=256 E=8 top_k=2"),
    "edge_f32": MoeConfig("edge_f32", 1024, 256, 512, 16, 4, True, "f32", "f32", 1001, edge_rows=True,
                          description="Routing edge cases F32, T=1024 H=256 I=512 E=16 top_k=4"),
    "prefill_bf16": MoeConfig("prefill_bf16", 8192, 2048, 1408, 64, 6, True, "bf16", "bf16", 1002,
                              description="Prefill BF16, T=8192 H=2048 I=1408 E=64 top_k=6"),
    "decode_bf16": MoeConfig("decode_bf16", 32, 4096, 1536, 128, 8, True, "bf16", "bf16", 1003,
                             description="Decode BF16, T=32 H=4096 I=1536 E=128 top_k=8"),
    "skewed_bf16": MoeConfig("skewed_bf16", 8192, 7168, 2048, 256, 8, True, "bf16", "bf16", 1004,
                             zipf_s=1.1,
                             description="Skewed BF16, T=8192 H=7168 I=2048 E=256 top_k=8, Zipf(1.1) bias"),
}


def stream_seed(seed: int, tensor_id: int, expert: int = 0) -> int:
    """Deterministic 63-bit seed of one stream (numpy SeedSequence hash)."""
    st = np.random.SeedSequence([int(seed), int(tensor_id), int(expert)]).generate_state(2, dtype=np.uint32)
    return int((int(st[0]) << 31) ^ int(st[1])) & ((1 << 63) - 1)


def _gen(device, seed: int, tensor_id: int, expert: int = 0) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, tensor_id, expert))
    return g


def _normal(shape, device, seed, tensor_id, expert=0) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(device, seed, tensor_id, expert), device=device,
                       dtype=torch.float32)


def zipf_bias(E: int, s: float) -> torch.Tensor:
    """2 * ln(w_r), w_r = r^-s / sum_j j^-s, with rank r = e + 1 (float64)."""
    r = torch.arange(1, E + 1, dtype=torch.float64)
    w = r.pow(-s)
    w = w / w.sum()
    return 2.0 * torch.log(w)


def make_tokens(cfg: MoeConfig, device="cpu", seed: int | None = None, T: int | None = None):
    """x [T,H] (cfg.dtype) and logits [T,E] (cfg.logits_dtype) on ``device``."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    x = _normal((T, cfg.H), device, seed, _X).to(TORCH_DT[cfg.dtype])
    lg = _normal((T, cfg.E), device, seed, _LOGITS)
    if cfg.zipf_s is not None:
        lg = lg + zipf_bias(cfg.E, cfg.zipf_s).to(device=device, dtype=torch.float32)[None, :]
    if cfg.edge_rows:
        lg = torch.clamp(torch.round(lg), -3.0, 3.0)
        g = _gen("cpu", seed, _EDGE)
        perm = torch.randperm(T, generator=g)
        n_nan, n_inf, n_ninf = int(0.05 * T), int(0.05 * T), int(0.02 * T)
        cols = torch.randint(0, cfg.E, (n_nan + n_inf,), generator=g)
        rows_nan = perm[:n_nan]
        rows_inf = perm[n_nan:n_nan + n_inf]
        rows_ninf = perm[n_nan + n_inf:n_nan + n_inf + n_ninf]
        lg = lg.cpu()
        lg[rows_nan, cols[:n_nan]] = float("nan")
        lg[rows_inf, cols[n_nan:]] = float("inf")
        lg[rows_ninf, :] = float("-inf")
        lg = lg.to(device)
    return x, lg.to(TORCH_DT[cfg.logits_dtype])


def make_expert(cfg: MoeConfig, e: int, device="cpu", seed: int | None = None):
    """gate_e [I,H], up_e [I,H], down_e [H,I] of one expert, in cfg.dtype."""
    seed = cfg.seed if seed is None else seed
    dt = TORCH_DT[cfg.dtype]
    sg = 1.0 / math.sqrt(cfg.H)
    sd = 1.0 / math.sqrt(cfg.I)
    gate = (_normal((cfg.I, cfg.H), device, seed, _GATE, e) * sg).to(dt)
    up = (_normal((cfg.I, cfg.H), device, seed, _UP, e) * sg).to(dt)
    down = (_normal((cfg.H, cfg.I), device, seed, _DOWN, e) * sd).to(dt)
    return gate, up, down


def make_weights(cfg: MoeConfig, device="cpu", seed: int | None = None):
    """gate [E,I,H], up [E,I,H], down [E,H,I], filled expert by expert."""
    dt = TORCH_DT[cfg.dtype]
    gate = torch.empty((cfg.E, cfg.I, cfg.H), dtype=dt, device=device)
    up = torch.empty((cfg.E, cfg.I, cfg.H), dtype=dt, device=device)
    down = torch.empty((cfg.E, cfg.H, cfg.I), dtype=dt, device=device)
    for e in range(cfg.E):
        g, u, d = make_expert(cfg, e, device, seed)
        gate[e].copy_(g)
        up[e].copy_(u)
        down[e].copy_(d)
    return gate, up, down


def make_grad_output(cfg: MoeConfig, device="cpu", seed: int | None = None, T: int | None = None):
    """d loss / d output [T,H] of one training step, N(0, 1) in cfg.dtype."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    return _normal((T, cfg.H), device, seed, _GRAD_OUT).to(TORCH_DT[cfg.dtype])


def to_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's bytes: float32 stays float32, 16-bit
    floats become their uint16 bit patterns, uint32 stays uint32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.float16, torch.bfloat16):
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.uint32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.int32:
        return t.numpy().view(np.uint32)
    raise TypeError(f"to_bits: unsupported dtype {t.dtype}")


def from_bits(a: np.ndarray, dt: str, device="cpu") -> torch.Tensor:
    """Inverse of to_bits for a float dtype name."""
    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16))
    return t.view(TORCH_DT[dt]).to(device)


def small_config(name: str, T: int, H: int, I: int, E: int, top_k: int, renormalize: bool = True,
                 dtype: str = "f32", logits_dtype: str | None = None, seed: int = 7,
                 edge_rows: bool = False, zipf_s: float | None = None) -> MoeConfig:
    return MoeConfig(name, T, H, I, E, top_k, renormalize, dtype, logits_dtype or dtype, seed,
                     edge_rows=edge_rows, zipf_s=zipf_s)
