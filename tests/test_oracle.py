"""Pins of the CPU oracle against facts the pages and the mathematics fix.

No pin re-types the oracle's own formula: each compares against a library
routine, a closed form, brute force on tiny inputs, an invariant, or values
a page prints.  Citations name the page and section the fact comes from.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import moe_synth as S

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def ulp32(x):
    return np.spacing(np.abs(np.float32(x))).astype(np.float64)


def fp32_softmax_bound(ref, logits):
    """A-priori bound of an FP32 max-shifted softmax over E experts: the shift
    d = l - max rounds once (relative error 2^-24, which exp turns into an
    absolute |d| 2^-24 in the exponent), each exp and the quotient round once,
    and a sequential E-term sum adds at most E-1 roundings, so to first order
    |p - p_exact| <= (E + 3 + |d|) 2^-24 p_exact."""
    l = np.asarray(logits, dtype=np.float64)
    d = np.abs(l - l.max(axis=-1, keepdims=True))
    E = l.shape[-1]
    return (E + 3 + d) * 2.0 ** -24 * np.abs(ref) + 1e-45


# ------------------------------------------------------------------ formats
def test_round_f32_matches_hardware_cast(oracle_lib):
    rng = np.random.default_rng(1)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-160, 130, 20000))
    v = np.concatenate([v, [0.0, -0.0, 3.4028235677973366e38, 3.4028235e38 * 1.0000001,
                            1.401298464324817e-45 * 0.5, 1.401298464324817e-45 * 0.5000001]])
    with np.errstate(over="ignore"):
        ref = v.astype(np.float32)
    got = oracle_lib.narrow(v, "f32")
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_round_f16_matches_numpy(oracle_lib):
    rng = np.random.default_rng(2)
    v = rng.standard_normal(20000) * np.exp2(rng.integers(-30, 16, 20000))
    # exact ties, the overflow boundary, subnormal ties
    ties = (np.arange(1, 2000) + 0.5) * 2.0 ** -10
    v = np.concatenate([v, ties, -ties, [65504.0, 65519.99, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26,
                                         2.0 ** -25 * 1.0000001, np.inf, -np.inf]])
    ref = v.astype(np.float16)
    got = oracle_lib.narrow(v, "f16")
    assert np.array_equal(got, ref.view(np.uint16))


def test_round_bf16_matches_torch(oracle_lib):
    rng = np.random.default_rng(3)
    v32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-130, 126, 20000))).astype(np.float32)
    # halfway cases between bf16 neighbours, both parities
    base = np.arange(0x3F80, 0x3F80 + 512, dtype=np.uint32) << 16
    half = (base | 0x8000).view(np.float32)
    v32 = np.concatenate([v32, half, -half, np.float32([3.3895314e38, 3.39e38, np.inf, 1e-40])])
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle_lib.narrow(v32.astype(np.float64), "bf16")
    assert np.array_equal(got, ref)


def test_nan_survives_every_cast(oracle_lib):
    for dt in ("f32", "f16", "bf16"):
        back = oracle_lib.widen(oracle_lib.narrow(np.array([np.nan, -np.nan]), dt), dt)
        assert np.isnan(back).all()


def test_widen_every_16bit_pattern(oracle_lib):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f16 = oracle_lib.widen(bits, "f16")
    ref16 = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(f16), np.isnan(ref16))
    ok = ~np.isnan(ref16)
    assert np.array_equal(f16[ok], ref16[ok])
    bf = oracle_lib.widen(bits, "bf16")
    refb = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    assert np.array_equal(np.isnan(bf), np.isnan(refb))
    ok = ~np.isnan(refb)
    assert np.array_equal(bf[ok], refb[ok])


# ------------------------------------------------------------------ softmax
# ruDNN User Guide section 4: FP32 softmax over all experts; tiny-llm ops.rs
# softmax block: the max-shifted form is mathematically the plain softmax.
def test_softmax_single_expert_is_one(oracle_lib):
    lg = np.float32([[0.3], [-7.0], [1e30]])
    assert np.array_equal(oracle_lib.softmax(lg, "f32"), np.ones((3, 1), np.float32))


@pytest.mark.parametrize("E", [2, 3, 7, 64, 256])
def test_softmax_equal_logits_is_uniform(oracle_lib, E):
    lg = np.full((2, E), 1.25, np.float32)
    p = oracle_lib.softmax(lg, "f32")
    assert np.array_equal(p, np.full((2, E), np.float32(1.0) / np.float32(E)))


def test_softmax_two_experts_closed_form(oracle_lib):
    rng = np.random.default_rng(4)
    lg = rng.standard_normal((500, 2)).astype(np.float32) * 4
    p = oracle_lib.softmax(lg, "f32").astype(np.float64)
    l = lg.astype(np.float64)
    p0 = 1.0 / (1.0 + np.exp(l[:, 1] - l[:, 0]))
    p1 = 1.0 / (1.0 + np.exp(l[:, 0] - l[:, 1]))
    bound = fp32_softmax_bound(np.stack([p0, p1], 1), lg)
    assert np.all(np.abs(p[:, 0] - p0) <= bound[:, 0])
    assert np.all(np.abs(p[:, 1] - p1) <= bound[:, 1])


@pytest.mark.parametrize("E", [3, 8, 64, 256])
def test_softmax_vs_torch_float64(oracle_lib, E):
    rng = np.random.default_rng(5 + E)
    lg = (rng.standard_normal((200, E)) * 3).astype(np.float32)
    ref = torch.softmax(torch.from_numpy(lg).double(), dim=-1).numpy()
    p = oracle_lib.softmax(lg, "f32").astype(np.float64)
    assert np.all(np.abs(p - ref) <= fp32_softmax_bound(ref, lg))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_softmax_low_precision_logits_widen_exactly(oracle_lib, dt):
    """F16/BF16 logits are widened exactly, then FP32 softmax (section 4)."""
    rng = np.random.default_rng(6)
    lg = torch.from_numpy(rng.standard_normal((64, 16)).astype(np.float32)).to(S.TORCH_DT[dt])
    ref = torch.softmax(lg.double(), dim=-1).numpy()
    p = oracle_lib.softmax(S.to_bits(lg), dt).astype(np.float64)
    assert np.all(np.abs(p - ref) <= fp32_softmax_bound(ref, lg.double().numpy()))


# ------------------------------------------------------------------ top-k and ties
# ruDNN User Guide section 4: top-k after softmax, ties favour the lower id.
@pytest.mark.parametrize("E", [1, 2, 3, 4, 5])
def test_topk_brute_force_all_small_rows(oracle_lib, E):
    rows = np.array(list(itertools.product([-1.0, 0.0, 1.0], repeat=E)), dtype=np.float32)
    p = oracle_lib.softmax(rows, "f32")
    for k in range(1, E + 1):
        idx, _, w32 = oracle_lib.route(rows, "f32", k, False, nthreads=1)
        for r in range(len(rows)):
            by_p = sorted(range(E), key=lambda e: (-float(p[r, e]), e))[:k]
            by_logit = sorted(range(E), key=lambda e: (-float(rows[r, e]), e))[:k]
            assert list(idx[r]) == by_p
            assert list(idx[r]) == by_logit
            assert np.array_equal(w32[r], p[r, by_p])


def test_topk_exact_ties_take_lower_id(oracle_lib):
    lg = np.float32([[0.5, 2.0, 2.0, 2.0, -1.0, 2.0]])
    idx, _, _ = oracle_lib.route(lg, "f32", 3, True)
    assert list(idx[0]) == [1, 2, 3]


# ------------------------------------------------------------------ NaN rows
# ruDNN User Guide section 4: NaN, +inf or all -inf rows keep NaN weights and
# are not turned into a uniform distribution.
def _nan_rows(E):
    rows = []
    for pos in range(E):
        r = np.zeros(E, np.float32); r[pos] = np.nan; rows.append(r)
        r = np.zeros(E, np.float32); r[pos] = np.inf; rows.append(r)
        r = np.linspace(-1, 1, E).astype(np.float32); r[pos] = np.nan; r[(pos + 1) % E] = np.inf
        rows.append(r)
        r = np.full(E, -np.inf, np.float32); r[pos] = np.nan; rows.append(r)
    rows.append(np.full(E, -np.inf, np.float32))
    r = np.full(E, np.inf, np.float32); rows.append(r)
    return np.stack(rows)


@pytest.mark.parametrize("renorm", [False, True])
@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
def test_nan_rows(oracle_lib, renorm, dt):
    E, k = 6, 3
    rows32 = _nan_rows(E)
    rows = rows32 if dt == "f32" else S.to_bits(torch.from_numpy(rows32).to(S.TORCH_DT[dt]))
    idx, w, w32 = oracle_lib.route(rows, dt, k, renorm)
    assert np.isnan(w32).all()
    assert np.isnan(oracle_lib.widen(w, dt)).all()
    assert (idx == np.arange(k, dtype=np.uint32)[None, :]).all()
    # all-or-none: every probability of such a row is NaN
    assert np.isnan(oracle_lib.softmax(rows, dt)).all()


def test_partial_neg_inf_row_is_finite(oracle_lib):
    lg = np.float32([[-np.inf, 0.0, -np.inf, 1.0, -np.inf]])
    p = oracle_lib.softmax(lg, "f32")
    assert np.isfinite(p).all()
    assert p[0, 0] == 0 and p[0, 2] == 0 and p[0, 4] == 0
    idx, _, w32 = oracle_lib.route(lg, "f32", 4, False)
    assert list(idx[0]) == [3, 1, 0, 2]  # zero probabilities go by lower id
    assert w32[0, 2] == 0 and w32[0, 3] == 0


# ------------------------------------------------------------------ renormalisation and cast
def test_renormalised_weights_sum_to_one(oracle_lib):
    rng = np.random.default_rng(7)
    for E, k in [(8, 2), (64, 6), (128, 8), (256, 8), (16, 16)]:
        lg = rng.standard_normal((300, E)).astype(np.float32)
        _, _, w32 = oracle_lib.route(lg, "f32", k, True)
        s = w32.astype(np.float64).sum(axis=1)
        assert np.all(np.abs(s - 1.0) <= k * 2.0 ** -23)


def test_k1_renormalised_weight_is_exactly_one(oracle_lib):
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((100, 16)).astype(np.float32)
    _, w, w32 = oracle_lib.route(lg, "f32", 1, True)
    assert np.all(w32 == 1.0) and np.all(w == 1.0)


def test_k_equals_e_renormalised_matches_probabilities(oracle_lib):
    rng = np.random.default_rng(9)
    lg = rng.standard_normal((100, 12)).astype(np.float32)
    p = oracle_lib.softmax(lg, "f32").astype(np.float64)
    idx, _, w32 = oracle_lib.route(lg, "f32", 12, True)
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    assert np.all(np.abs(w32 - sel) <= 4 * ulp32(sel))


def test_without_renorm_weights_are_the_probabilities(oracle_lib):
    rng = np.random.default_rng(10)
    lg = rng.standard_normal((100, 32)).astype(np.float32)
    p = oracle_lib.softmax(lg, "f32")
    idx, _, w32 = oracle_lib.route(lg, "f32", 5, False)
    assert np.array_equal(w32, np.take_along_axis(p, idx.astype(np.int64), axis=1))


@pytest.mark.parametrize("dt", ["f16", "bf16"])
def test_weights_cast_to_logits_dtype(oracle_lib, dt):
    """Section 4: after (optional) renormalisation the weights take the logits dtype."""
    rng = np.random.default_rng(11)
    lg = S.to_bits(torch.from_numpy(rng.standard_normal((200, 16)).astype(np.float32)).to(S.TORCH_DT[dt]))
    for renorm in (False, True):
        _, w, w32 = oracle_lib.route(lg, dt, 4, renorm)
        ref = torch.from_numpy(w32).to(S.TORCH_DT[dt])
        assert np.array_equal(w, S.to_bits(ref))


# ------------------------------------------------------------------ dispatch
def _gather_fixture():
    with open(os.path.join(GOLDEN, "gather_example.json")) as f:
        return json.load(f)


def test_gather_semantics_of_dispatch_and_combine(oracle_lib):
    """The page's printed torch.gather example, reproduced by the oracle's
    dispatch (rows copied from token x[token_of_row]) and combine (a weight-1
    slot reads Y[row_of_slot])."""
    g = _gather_fixture()
    x = np.array(g["x"], dtype=np.float32)
    index = np.array(g["index"])
    expected = np.array(g["expected"], dtype=np.float32)
    # combine: treat x as 12 one-wide rows; output (i, j) owns one slot with weight 1
    Y = x.reshape(12, 1).copy()
    ros = (4 * np.arange(3)[:, None] + index).reshape(-1).astype(np.uint32)
    w = np.ones((6, 1), np.float32)
    out = oracle_lib.combine(Y, "f32", ros, w, "f32", 6, 1, 1)
    assert np.array_equal(out.reshape(3, 2), expected)
    # dispatch: tokens are the 12 scalars; slot (i,j) routes token 4i+index[i,j]
    # to expert 0 with k=1 -> dispatched rows hold exactly the gathered values
    tok_idx = np.zeros((12, 1), np.uint32)
    offsets, ros2, tor, rows = oracle_lib.dispatch(tok_idx, 1, x.reshape(12, 1), "f32")
    picked = rows[ros2[(4 * np.arange(3)[:, None] + index).reshape(-1)], 0]
    assert np.array_equal(picked.reshape(3, 2), expected)


def test_dispatch_invariants(oracle_lib):
    rng = np.random.default_rng(12)
    T, E, k, H = 300, 11, 3, 5
    lg = rng.standard_normal((T, E)).astype(np.float32)
    idx, _, _ = oracle_lib.route(lg, "f32", k, True)
    x = rng.standard_normal((T, H)).astype(np.float32)
    offsets, ros, tor, rows = oracle_lib.dispatch(idx, E, x, "f32")
    counts = np.bincount(idx.reshape(-1), minlength=E)
    assert offsets[0] == 0 and offsets[E] == T * k
    assert np.array_equal(np.diff(offsets.astype(np.int64)), counts)
    assert sorted(ros.tolist()) == list(range(T * k))  # every slot exactly once
    for e in range(E):
        toks = set(tor[offsets[e]:offsets[e + 1]].tolist())
        assert toks == {t for t in range(T) if e in idx[t]}
    assert np.array_equal(rows, x[tor])  # bit copies
    # row_of_slot points at a row owned by the slot's expert and token
    for s in range(T * k):
        r = ros[s]
        assert tor[r] == s // k
        assert offsets[idx.reshape(-1)[s]] <= r < offsets[idx.reshape(-1)[s] + 1]


def test_dispatch_invalid_index_is_skipped_and_combine_gives_nan(oracle_lib):
    """A slot naming an expert >= E is not copied; its token's output row is
    NaN (the training section's convention for bad indices)."""
    T, E, k, H = 4, 3, 2, 3
    idx = np.array([[0, 1], [2, 7], [1, 0], [3, 2]], np.uint32)
    x = np.arange(T * H, dtype=np.float32).reshape(T, H)
    offsets, ros, tor, rows = oracle_lib.dispatch(idx, E, x, "f32")
    assert offsets[E] == 6
    assert ros[3] == oracle_lib.INVALID_ROW and ros[6] == oracle_lib.INVALID_ROW
    Y = rows.copy()
    w = np.full((T, k), 0.5, np.float32)
    out = oracle_lib.combine(Y, "f32", ros, w, "f32", T, k, H)
    assert np.isnan(out[1]).all() and np.isnan(out[3]).all()
    assert np.array_equal(out[0], 0.5 * x[0] + 0.5 * x[0])


# ------------------------------------------------------------------ experts
def test_silu_special_values(oracle_lib):
    """tiny-llm ops.rs SiLU block: silu(z) = z * sigmoid(z)."""
    assert oracle_lib.silu(0.0) == 0.0
    assert oracle_lib.silu(60.0) == 60.0
    v = oracle_lib.silu(-800.0)
    assert v == 0.0 and math.copysign(1.0, v) < 0
    for z in np.linspace(-20, 20, 81):
        ref = float(torch.nn.functional.silu(torch.tensor(z, dtype=torch.float64)))
        assert abs(oracle_lib.silu(z) - ref) <= 4e-16 * max(1.0, abs(ref))


def _textbook_swiglu(x, gate, up, down):
    """tiny-llm ops.rs SiLU block: FFN(x) = W_down(SiLU(W_gate x) * W_up x)."""
    x = torch.as_tensor(x, dtype=torch.float64)
    g = x @ torch.as_tensor(gate, dtype=torch.float64).T
    u = x @ torch.as_tensor(up, dtype=torch.float64).T
    return ((torch.nn.functional.silu(g) * u) @ torch.as_tensor(down, dtype=torch.float64).T).numpy()


@pytest.mark.parametrize("dt,tol", [("f32", 2e-6), ("bf16", 3e-2), ("f16", 4e-3)])
def test_single_expert_reduces_to_swiglu_ffn(oracle_lib, dt, tol):
    cfg = S.small_config("one", T=24, H=48, I=40, E=1, top_k=1, dtype=dt)
    x, lg = S.make_tokens(cfg)
    gate, up, down = S.make_weights(cfg)
    res = oracle_lib.forward(S.to_bits(x), S.to_bits(lg), S.to_bits(gate), S.to_bits(up),
                             S.to_bits(down), dt, dt, 1, True)
    got = oracle_lib.widen(res["output"], dt)
    ref = _textbook_swiglu(x.double(), gate[0].double(), up[0].double(), down[0].double())
    assert np.all(np.abs(got - ref) <= tol * (1 + np.abs(ref)))
    assert np.all(oracle_lib.widen(res["weights"], dt) == 1.0)


def test_expert_weight_layout_is_not_transposed(oracle_lib):
    """gate [E,I,H] multiplies x over H (section 5): with H != I a transposed
    operand would not even line up; check one hand-made case exactly."""
    H, I = 2, 3
    x = np.float32([[1.0, 2.0]])
    gate = np.float32([[[1, 0], [0, 1], [1, 1]]])   # g = [1, 2, 3]
    up = np.float32([[[1, 0], [1, 0], [1, 0]]])     # u = [1, 1, 1]
    down = np.float32([[[1, 0, 0], [0, 0, 1]]])     # y = [h0, h2]
    offsets = np.uint32([0, 1])
    y = oracle_lib.experts(gate, up, down, "f32", x, offsets, 1, H, I)
    s = lambda z: z / (1 + math.exp(-z))
    assert np.allclose(y[0], [s(1.0), s(3.0)], rtol=1e-7, atol=0)


# ------------------------------------------------------------------ whole chain
def _dense_mixture(x, lg, gate, up, down):
    """top_k = E without renormalisation is the softmax-weighted sum over all
    experts; computed the per-token way of the torch_general_ops page's
    einsum MoE (gather each token's expert weights, contract, weight-sum)."""
    x = torch.as_tensor(x, dtype=torch.float64)
    p = torch.softmax(torch.as_tensor(lg, dtype=torch.float64), dim=-1)
    T, E = p.shape
    ids = torch.arange(E).expand(T, E)
    g = torch.as_tensor(gate, dtype=torch.float64)[ids]       # [T, E, I, H]
    u = torch.as_tensor(up, dtype=torch.float64)[ids]
    d = torch.as_tensor(down, dtype=torch.float64)[ids]       # [T, E, H, I]
    a = torch.nn.functional.silu(torch.einsum("th,taih->tai", x, g)) * torch.einsum("th,taih->tai", x, u)
    y = torch.einsum("tai,tahi->tah", a, d)
    return torch.einsum("tah,ta->th", y, p).numpy()


def test_top_k_equal_e_is_dense_softmax_mixture(oracle_lib):
    cfg = S.small_config("dense", T=16, H=24, I=20, E=5, top_k=5, renormalize=False)
    x, lg = S.make_tokens(cfg)
    gate, up, down = S.make_weights(cfg)
    res = oracle_lib.forward(S.to_bits(x), S.to_bits(lg), S.to_bits(gate), S.to_bits(up),
                             S.to_bits(down), "f32", "f32", 5, False)
    ref = _dense_mixture(x, lg, gate, up, down)
    assert np.all(np.abs(res["output"] - ref) <= 1e-5 * (1 + np.abs(ref)))


def test_token_permutation_permutes_outputs(oracle_lib):
    cfg = S.small_config("perm", T=40, H=16, I=24, E=6, top_k=2, dtype="bf16")
    x, lg = S.make_tokens(cfg)
    W = [S.to_bits(w) for w in S.make_weights(cfg)]
    a = oracle_lib.forward(S.to_bits(x), S.to_bits(lg), *W, "bf16", "bf16", 2, True)["output"]
    perm = torch.randperm(40, generator=torch.Generator().manual_seed(3))
    b = oracle_lib.forward(S.to_bits(x[perm]), S.to_bits(lg[perm]), *W, "bf16", "bf16", 2, True)["output"]
    assert np.array_equal(a[perm.numpy()], b)


def test_expert_relabelling_leaves_output_unchanged(oracle_lib):
    cfg = S.small_config("relabel", T=40, H=16, I=24, E=6, top_k=3)
    x, lg = S.make_tokens(cfg)
    gate, up, down = S.make_weights(cfg)
    ra = oracle_lib.forward(S.to_bits(x), S.to_bits(lg), S.to_bits(gate), S.to_bits(up), S.to_bits(down),
                            "f32", "f32", 3, True)
    sigma = torch.tensor([4, 0, 5, 2, 1, 3])
    rb = oracle_lib.forward(S.to_bits(x), S.to_bits(lg[:, sigma]), S.to_bits(gate[sigma]),
                            S.to_bits(up[sigma]), S.to_bits(down[sigma]), "f32", "f32", 3, True)
    # the same experts are chosen, under their new names
    assert np.array_equal(sigma.numpy()[rb["indices"]], ra["indices"])
    # only the order of the softmax sum changed, so outputs agree to rounding
    a, b = ra["output"].astype(np.float64), rb["output"].astype(np.float64)
    assert np.all(np.abs(a - b) <= 1e-6 * (1 + np.abs(a)))


def test_row_order_inside_an_expert_does_not_matter(oracle_lib):
    """Section 5 leaves the order inside an expert unspecified; any order must
    give the same output once the mapping restores token order."""
    cfg = S.small_config("order", T=50, H=16, I=24, E=4, top_k=2, dtype="bf16")
    x, lg = S.make_tokens(cfg)
    W = [S.to_bits(w) for w in S.make_weights(cfg)]
    res = oracle_lib.forward(S.to_bits(x), S.to_bits(lg), *W, "bf16", "bf16", 2, True)
    off, ros, tor, rows = res["offsets"], res["row_of_slot"], res["token_of_row"], res["dispatched"]
    rng = np.random.default_rng(13)
    newpos = np.arange(len(tor))
    for e in range(4):
        seg = np.arange(off[e], off[e + 1])
        newpos[seg] = rng.permutation(seg)
    rows2 = np.empty_like(rows)
    rows2[newpos] = rows
    ros2 = newpos[ros].astype(np.uint32)
    Y2 = oracle_lib.experts(*W, "bf16", rows2, off, 4, 16, 24)
    out2 = oracle_lib.combine(Y2, "bf16", ros2, res["weights"], "bf16", 50, 2, 16)
    assert np.array_equal(out2, res["output"])


def test_no_token_is_dropped(oracle_lib):
    """Section 5: no capacity drop, even when every token picks one expert."""
    T, E, k, H = 257, 8, 2, 4
    lg = np.zeros((T, E), np.float32)
    lg[:, 3] = 5.0
    lg[:, 6] = 4.0
    idx, _, _ = oracle_lib.route(lg, "f32", k, True)
    x = np.random.default_rng(14).standard_normal((T, H)).astype(np.float32)
    off, ros, tor, rows = oracle_lib.dispatch(idx, E, x, "f32")
    assert off[4] - off[3] == T and off[7] - off[6] == T and off[E] == T * k


@pytest.mark.parametrize("ldt", ["bf16", "f16", "f32"])
def test_combine_uses_the_cast_weights(oracle_lib, ldt):
    """Section 6 (Call MoE): the combine sums the expert rows with the routing
    weights, and section 4 makes those weights the logits dtype.  Two experts
    whose outputs are exactly +256 and -256 (a SiLU input of 128 saturates to
    128 in every dtype, times a down weight of +-2) make the output of a token
    256 (w0 - w1) rounded once: with the cast weights this is one value, with
    the FP32 weights before the cast another, and the oracle must give the
    first on every token.  For F32 logits the two coincide."""
    T, H, I, E = 256, 8, 1, 2
    x = np.zeros((T, H), np.float32)
    x[:, 0] = 1.0
    gate = np.zeros((E, I, H), np.float32)
    gate[:, 0, 0] = 128.0
    up = np.zeros((E, I, H), np.float32)
    up[:, 0, 0] = 1.0
    down = np.zeros((E, H, I), np.float32)
    down[0, :, 0] = 2.0
    down[1, :, 0] = -2.0
    to = lambda a, dt: S.to_bits(torch.from_numpy(a).to(S.TORCH_DT[dt]))
    a = np.linspace(-0.1, 0.1, T).astype(np.float32)  # w0 - w1 near 0: a fine output grid
    lg = np.stack([a, np.zeros(T, np.float32)], axis=1)
    res = oracle_lib.forward(to(x, "bf16"), to(lg, ldt), to(gate, "bf16"), to(up, "bf16"), to(down, "bf16"),
                             "bf16", ldt, 2, True)
    Y = oracle_lib.widen(res["Y"], "bf16")
    y_of_expert = np.where(np.arange(T * 2) < res["offsets"][1], 256.0, -256.0)
    assert np.array_equal(Y, np.repeat(y_of_expert[:, None], H, axis=1))
    # the stored weights are the FP32 weights rounded to the logits dtype
    w32 = res["weights_f32"].reshape(T, 2).astype(np.float64)
    wc = torch.from_numpy(res["weights_f32"]).to(S.TORCH_DT[ldt]).double().numpy().reshape(T, 2)
    rnd = lambda v: torch.from_numpy(v).to(torch.bfloat16).double().numpy()
    sign = np.where(res["indices"].reshape(T, 2) == 0, 256.0, -256.0)  # slot j's expert output
    want = rnd((sign * wc).sum(axis=1))       # two exact terms: exact in double, rounded once
    other = rnd((sign * w32).sum(axis=1))
    got = oracle_lib.widen(res["output"], "bf16")
    assert np.array_equal(got, np.repeat(want[:, None], H, axis=1))
    differ = int((want != other).sum())
    if ldt == "f32":
        assert differ == 0
    else:
        assert differ > T // 8, f"the case must tell the two readings apart ({differ} tokens differ)"


# ------------------------------------------------------------------ generator sanity
def test_edge_workload_has_the_planted_rows():
    cfg = S.CONFIGS["edge_f32"]
    _, lg = S.make_tokens(cfg)
    l = lg.numpy()
    nan_rows = np.isnan(l).any(1)
    inf_rows = np.isposinf(l).any(1)
    ninf_rows = np.isneginf(l).all(1)
    assert nan_rows.sum() == 51 and inf_rows.sum() == 51 and ninf_rows.sum() == 20
    fin = ~(nan_rows | inf_rows | ninf_rows)
    assert set(np.unique(l[fin]).tolist()) <= {-3.0, -2.0, -1.0, 0.0, 1.0, 2.0, 3.0}
