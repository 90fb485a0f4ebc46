"""Comparison rules between the HIP path and the CPU oracle.

Agreement is defined as follows (the rules of the build's parity contract):
  * indices match bit-exactly, except where the oracle's FP32 probabilities
    of the two experts in question differ by less than 1e-6 (a near tie, where
    ulp-level differences in exp and summation order may flip the order);
    exact ties -- bit-identical logits -- are not exempt;
  * NaN rows: identical NaN masks, indices 0..k-1;
  * dispatch: the per-expert set of token ids (the order inside an expert
    follows atomics and is not fixed), every row a bit copy of its token;
  * values: |got - ref| <= tol * (1 + |ref|), tol = 1e-4 for F32 and 2e-2
    for F16/BF16, NaN positions identical.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_synth as S
import oracle

TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
# One rounding step relative to the value: the two sides round an
# intermediate (h, dg, du) once each, from slightly different unrounded
# values, so their copies differ by at most this factor of the value.
ROUND_STEP = {"f32": 2.0 ** -23, "f16": 2.0 ** -10, "bf16": 2.0 ** -7}
NEAR_TIE = 1e-6


def host_bits(t: torch.Tensor) -> np.ndarray:
    return S.to_bits(t)


def values(a, dt: str) -> np.ndarray:
    """float64 values of a torch tensor or of oracle bits."""
    if isinstance(a, torch.Tensor):
        return a.detach().cpu().double().numpy()
    return oracle.widen(np.ascontiguousarray(a), dt)


def assert_close(got, ref, dt: str, what: str, rows_mask=None):
    g, r = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    if rows_mask is not None:
        g, r = g[rows_mask], r[rows_mask]
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ ({int((gn != rn).sum())} elements)"
    ok = ~rn
    err = np.abs(g[ok] - r[ok])
    lim = TOL[dt] * (1.0 + np.abs(r[ok]))
    if err.size:
        worst = int(np.argmax(err - lim))
        assert np.all(err <= lim), (f"{what}: max excess {float((err - lim)[worst]):.3g} "
                                    f"(got {g[ok][worst]!r}, ref {r[ok][worst]!r}, tol {TOL[dt]})")


def compare_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, logits_bits: np.ndarray, ldt: str,
                    top_k: int, renorm: bool, nthreads: int | None = None):
    """Checks GPU routing against the oracle; returns (oracle result, near-tie token mask)."""
    o_idx, o_w, _ = oracle.route(logits_bits, ldt, top_k, renorm, nthreads)
    p = oracle.softmax(logits_bits, ldt).astype(np.float64)
    lg = oracle.widen(logits_bits, ldt)
    T, E = p.shape
    k = top_k
    gi = gpu_idx.astype(np.int64)
    oi = o_idx.astype(np.int64)
    assert gi.shape == (T, k)
    nan_rows = np.isnan(p).any(axis=1)
    # the all-or-none property of the oracle's NaN rows
    assert np.array_equal(nan_rows, np.isnan(p).all(axis=1))
    gw, ow = values(gpu_w, ldt), oracle.widen(o_w, ldt)
    # NaN rows
    if nan_rows.any():
        assert (gi[nan_rows] == np.arange(k)[None, :]).all(), "NaN rows must select experts 0..k-1"
        assert np.isnan(gw[nan_rows]).all(), "NaN rows must keep NaN weights"
    fin = ~nan_rows
    assert not np.isnan(gw[fin]).any(), "finite rows must have finite weights"
    assert ((gi >= 0) & (gi < E)).all()
    srt = np.sort(gi, axis=1)
    assert (np.diff(srt, axis=1) > 0).all(), "indices of a token must be distinct"
    mism = (gi != oi) & fin[:, None]
    near = np.zeros(T, bool)
    if mism.any():
        t_ids, j_ids = np.nonzero(mism)
        pa = p[t_ids, oi[t_ids, j_ids]]
        pb = p[t_ids, gi[t_ids, j_ids]]
        la = lg[t_ids, oi[t_ids, j_ids]]
        lb = lg[t_ids, gi[t_ids, j_ids]]
        gap = np.abs(pa - pb)
        bad = (gap >= NEAR_TIE) | (la == lb)
        assert not bad.any(), (
            f"index mismatch outside the near-tie rule at token {t_ids[bad][0]} slot {j_ids[bad][0]}: "
            f"oracle {oi[t_ids[bad][0]]} gpu {gi[t_ids[bad][0]]} gap {gap[bad][0]:.3g}")
        near[t_ids] = True
    assert_close(gw, ow, ldt, "routing weights")
    return (o_idx, o_w), near


def compare_dispatch(gpu: dict, o_offsets, o_ros, o_tor, o_rows, x_bits: np.ndarray, idx: np.ndarray, E: int):
    """gpu: dict of host numpy arrays rows/offsets/row_of_slot/token_of_row."""
    T, k = idx.shape
    offs = gpu["offsets"].astype(np.int64)
    assert np.array_equal(offs, o_offsets.astype(np.int64)), "expert offsets differ"
    n = int(offs[E])
    ros = gpu["row_of_slot"].astype(np.int64)
    tor = gpu["token_of_row"][:n].astype(np.int64)
    flat = idx.reshape(-1).astype(np.int64)
    valid = flat < E
    assert np.array_equal(ros[~valid], np.full((~valid).sum(), 0xFFFFFFFF)), "invalid slots must be unmapped"
    assert np.array_equal(np.sort(ros[valid]), np.arange(n)), "every row must belong to exactly one slot"
    slot_tok = np.nonzero(valid)[0] // k
    assert np.array_equal(tor[ros[valid]], slot_tok), "token_of_row must invert row_of_slot"
    exp_of_row = np.searchsorted(offs, np.arange(n), side="right") - 1
    assert np.array_equal(exp_of_row[ros[valid]], flat[valid]), "a slot's row must lie in its expert's range"
    otor = o_tor.astype(np.int64)
    for e in range(E):
        a, b = offs[e], offs[e + 1]
        assert np.array_equal(np.sort(tor[a:b]), np.sort(otor[a:b])), f"token set of expert {e} differs"
    rows = gpu["rows"][:n]
    assert np.array_equal(rows, x_bits[tor]), "dispatched rows must be bit copies of their tokens"


def compare_grouped_routing(gpu_idx: np.ndarray, gpu_w: np.ndarray, logits_bits: np.ndarray, ldt: str,
                            bias: np.ndarray | None, top_k: int, groups: int, selected: int, top_two: bool,
                            renorm: bool, scale: float, nthreads: int | None = None):
    """Group-limited sigmoid routing against the oracle, with the near-tie
    rule applied to the corrected scores: a slot may differ where the two
    experts' corrected scores are within 1e-6 (unless logit and bias are
    both identical, an exact tie), and a whole row may differ where the
    oracle's group scores at the selection boundary are within 1e-6.
    Returns (oracle result, near-tie token mask)."""
    o_idx, o_w, _, corr = oracle.route_sigmoid_grouped(logits_bits, ldt, bias, top_k, groups, selected, top_two,
                                                       renorm, scale, nthreads)
    lg = oracle.widen(logits_bits, ldt)
    T, E = corr.shape
    k, G, gsz = top_k, groups, E // groups
    b = np.zeros(E, np.float32) if bias is None else bias.astype(np.float32)
    gi, oi = gpu_idx.astype(np.int64), o_idx.astype(np.int64)
    assert gi.shape == (T, k)
    nan_rows = np.isnan(corr).any(axis=1)
    gw, ow = values(gpu_w, ldt), oracle.widen(o_w, ldt)
    if nan_rows.any():
        assert (gi[nan_rows] == np.arange(k)[None, :]).all(), "NaN rows must select experts 0..k-1"
        assert np.isnan(gw[nan_rows]).all(), "NaN rows must keep NaN weights"
    fin = ~nan_rows
    assert not np.isnan(gw[fin]).any(), "finite rows must have finite weights"
    assert ((gi >= 0) & (gi < E)).all()
    assert (np.diff(np.sort(gi, axis=1), axis=1) > 0).all(), "indices of a token must be distinct"
    # the oracle's group scores, to find rows whose group choice is a near tie
    cf = np.where(np.isnan(corr), -np.inf, corr).astype(np.float64)
    top = -np.sort(-cf.reshape(T, G, gsz), axis=2)
    gsc = top[:, :, 0] + (top[:, :, 1] if top_two else 0.0)
    gs_sorted = -np.sort(-gsc, axis=1)
    near_group = np.zeros(T, bool)
    if selected < G:
        # an exact tie (gap 0) comes from identical inputs and must resolve
        # to the lower group id on both sides, so it is not exempt
        ggap = gs_sorted[:, selected - 1] - gs_sorted[:, selected]
        near_group = (ggap > 0) & (ggap < NEAR_TIE)
    near = near_group & fin
    mism = (gi != oi) & fin[:, None] & ~near_group[:, None]
    if mism.any():
        t_ids, j_ids = np.nonzero(mism)
        a, bb = oi[t_ids, j_ids], gi[t_ids, j_ids]
        gap = np.abs(cf[t_ids, a] - cf[t_ids, bb])
        exact = (lg[t_ids, a] == lg[t_ids, bb]) & (b[a] == b[bb])
        bad = (gap >= NEAR_TIE) | exact
        assert not bad.any(), (
            f"index mismatch outside the near-tie rule at token {t_ids[bad][0]} slot {j_ids[bad][0]}: "
            f"oracle {a[bad][0]} gpu {bb[bad][0]} gap {gap[bad][0]:.3g}")
        near[t_ids] = True
    same = fin & ~near
    assert_close(gw[same], ow[same], ldt, "grouped routing weights")
    assert near.mean() < 0.01, f"too many near-tie tokens: {int(near.sum())}"
    return (o_idx, o_w), near


def assert_close_sum(got, ref, l1, dt: str, what: str, max_outliers: float = 1e-3):
    """For results that are K-sums of products with one separately rounded
    16-bit factor (the weight gradients): every element within
    TOL (1 + |ref|) + ROUND_STEP * l1, l1 = the sum of |terms|, which bounds
    what the two sides' independent roundings of that factor can do; and
    at most a fraction `max_outliers` of elements beyond TOL (1 + |ref|),
    since a rounding that lands on the other side of a boundary is rare."""
    g, r, m = (np.asarray(a, np.float64) for a in (got, ref, l1))
    assert g.shape == r.shape == m.shape, (what, g.shape, r.shape, m.shape)
    gn, rn = np.isnan(g), np.isnan(r)
    assert np.array_equal(gn, rn), f"{what}: NaN positions differ"
    ok = ~rn
    err = np.abs(g[ok] - r[ok])
    strict = TOL[dt] * (1.0 + np.abs(r[ok]))
    bound = strict + ROUND_STEP[dt] * m[ok]
    if err.size:
        worst = int(np.argmax(err - bound))
        assert np.all(err <= bound), (f"{what}: max excess {float((err - bound)[worst]):.3g} over the rounding "
                                      f"bound (got {g[ok][worst]!r}, ref {r[ok][worst]!r})")
        frac = float(np.mean(err > strict))
        assert frac <= max_outliers, f"{what}: {frac:.2%} of elements beyond {TOL[dt]} * (1 + |ref|)"
