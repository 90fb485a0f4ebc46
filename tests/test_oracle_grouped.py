"""Pins of the oracle's group-limited sigmoid routing (ruDNN user guide,
section 10) against things other than itself: a brute force that ranks by
stable sorts instead of repeated arg-max, the softmax routing it reduces to,
torch's sigmoid, and invariants of the definition.
"""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def sig32(x: np.ndarray) -> np.ndarray:
    """torch's float64 sigmoid rounded to binary32: a library routine, not the oracle's."""
    return torch.sigmoid(torch.from_numpy(np.asarray(x, np.float64))).to(torch.float32).numpy()


def brute_force(lg, bias, k, G, m, top_two):
    """Selection by definition, with stable sorts: groups by (-score, id),
    experts of the chosen groups by (-corrected score, id)."""
    T, E = lg.shape
    gsz = E // G
    s = sig32(lg)
    c = (s + (np.zeros(E, np.float32) if bias is None else bias)).astype(np.float32)
    out = np.empty((T, k), np.uint32)
    for t in range(T):
        gs = np.empty(G, np.float32)
        for g in range(G):
            v = np.sort(c[t, g * gsz:(g + 1) * gsz])[::-1]
            gs[g] = np.float32(v[0] + v[1]) if top_two else v[0]
        order = sorted(range(G), key=lambda g: (-float(gs[g]), g))
        chosen = set(order[:m])
        allowed = [e for e in range(E) if e // gsz in chosen]
        ranked = sorted(allowed, key=lambda e: (-float(c[t, e]), e))
        out[t] = ranked[:k]
    return out, s, c


def configs_small():
    for E in (4, 6, 8):
        for G in [g for g in range(1, E + 1) if E % g == 0]:
            for m in range(1, G + 1):
                for top_two in (False, True):
                    if top_two and E // G < 2:
                        continue
                    for k in sorted({1, 2, 3, m * (E // G)}):
                        if k <= m * (E // G):
                            yield E, G, m, k, top_two


def test_selection_matches_brute_force_with_ties():
    """Logits and bias from tiny sets force exact ties in scores and group
    scores; every option combination on E <= 8 must pick what the sorted
    brute force picks, ties going to the lower id."""
    rng = np.random.default_rng(7)
    for E, G, m, k, top_two in configs_small():
        lg = rng.integers(-1, 2, size=(60, E)).astype(np.float32)
        bias = rng.choice(np.array([0.0, 0.25, -0.25], np.float32), size=E)
        for b in (None, bias):
            idx, _, _, corr = oracle.route_sigmoid_grouped(lg, "f32", b, k, G, m, top_two, True, 1.0)
            ref, _, c = brute_force(lg, b, k, G, m, top_two)
            assert np.array_equal(corr, c), (E, G, m, k, top_two)
            assert np.array_equal(idx, ref), (E, G, m, k, top_two, b is None)


def test_one_group_without_bias_reduces_to_softmax_routing():
    """sigmoid and softmax are both increasing in the logit, so with one group
    (or every group selected) and no bias the chosen experts and their order
    are the softmax route's, on rows without near ties."""
    rng = np.random.default_rng(3)
    lg = rng.standard_normal((400, 64)).astype(np.float32)
    for G, m in ((1, 1), (8, 8)):
        idx, _, _, corr = oracle.route_sigmoid_grouped(lg, "f32", None, 6, G, m, False, True, 1.0)
        ref, _, _ = oracle.route(lg, "f32", 6, True)
        srt = np.sort(corr, axis=1)[:, ::-1]
        clear = np.all(np.abs(np.diff(srt[:, :7], axis=1)) > 1e-6, axis=1)
        assert clear.mean() > 0.9
        assert np.array_equal(idx[clear], ref[clear])


def test_weights_are_uncorrected_sigmoid_scores():
    """Without renormalisation a weight is sigmoid(logit) * scale, whatever the
    bias; with it the weights are proportional to those scores and sum to
    scale."""
    rng = np.random.default_rng(5)
    T, E, k, G, m, scale = 300, 256, 8, 8, 4, 2.5
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.5).astype(np.float32)
    idx, _, w32, _ = oracle.route_sigmoid_grouped(lg, "f32", bias, k, G, m, True, False, scale)
    s = sig32(lg)
    sel = np.take_along_axis(s, idx.astype(np.int64), axis=1)
    assert np.array_equal(w32, (sel * np.float32(scale)).astype(np.float32))
    idx2, _, w2, _ = oracle.route_sigmoid_grouped(lg, "f32", bias, k, G, m, True, True, scale)
    assert np.array_equal(idx2, idx)
    assert np.allclose(w2.sum(axis=1), scale, rtol=0, atol=16 * k * 2.0 ** -24 * scale)
    assert np.allclose(w2 / w2[:, :1], sel / sel[:, :1], rtol=4e-7 * k)


def test_deepseek_style_invariants():
    """E=256 in 8 groups, the best 4 by the sum of their top two corrected
    scores, top-8 inside them, renormalised and scaled by 2.5 (the skewed
    workload's shape): chosen experts lie in the 4 best groups, beat every
    other candidate of those groups, and come in decreasing order."""
    rng = np.random.default_rng(11)
    T, E, k, G, m = 500, 256, 8, 8, 4
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = (rng.standard_normal(E) * 0.3).astype(np.float32)
    idx, _, w32, corr = oracle.route_sigmoid_grouped(lg, "f32", bias, k, G, m, True, True, 2.5)
    gsz = E // G
    top2 = np.sort(corr.reshape(T, G, gsz), axis=2)[:, :, ::-1]
    gscore = (top2[:, :, 0] + top2[:, :, 1]).astype(np.float32)
    for t in range(T):
        groups = set(int(e) // gsz for e in idx[t])
        assert len(groups) <= m
        chosen_min = min(gscore[t, g] for g in groups)
        assert sum(1 for g in range(G) if gscore[t, g] > chosen_min) < m
        c_sel = corr[t, idx[t]]
        assert np.all(np.diff(c_sel) <= 0)
        best_groups = np.argsort(-gscore[t], kind="stable")[:m]
        cand = np.concatenate([np.arange(g * gsz, (g + 1) * gsz) for g in best_groups])
        rest = np.setdiff1d(cand, idx[t])
        assert corr[t, rest].max() <= c_sel.min()
    assert np.all(w32 > 0)


def test_bias_steers_selection_only():
    rng = np.random.default_rng(13)
    T, E = 50, 32
    lg = rng.standard_normal((T, E)).astype(np.float32)
    bias = np.zeros(E, np.float32)
    bias[[20, 21, 22]] = 10.0  # group 2 of 4 (experts 16..23) dominates
    idx, _, w32, _ = oracle.route_sigmoid_grouped(lg, "f32", bias, 3, 4, 1, False, False, 1.0)
    assert np.array_equal(np.sort(idx, axis=1), np.tile([20, 21, 22], (T, 1)))
    s = sig32(lg)
    assert np.array_equal(w32, np.take_along_axis(s, idx.astype(np.int64), axis=1))


def test_nan_and_infinite_rows():
    E = 16
    lg = np.zeros((4, E), np.float32)
    lg[0, 5] = np.nan
    lg[1, 3] = np.inf       # sigmoid 1: a finite, clear winner
    lg[2, :] = -np.inf      # every score 0: ties, lower ids first
    lg[3, 7] = -np.inf
    idx, _, w32, _ = oracle.route_sigmoid_grouped(lg, "f32", None, 2, 4, 2, False, False, 1.0)
    assert list(idx[0]) == [0, 1] and np.all(np.isnan(w32[0]))
    assert idx[1, 0] == 3 and w32[1, 0] == 1.0
    assert list(idx[2]) == [0, 1] and np.all(w32[2] == 0.0)
    assert np.all(np.isfinite(w32[1:]))
    bias = np.zeros(E, np.float32)
    bias[9] = np.nan        # a NaN correction makes every row a NaN row
    idx, _, w32, _ = oracle.route_sigmoid_grouped(lg[1:], "f32", bias, 2, 4, 2, False, False, 1.0)
    assert np.all(idx == np.array([0, 1], np.uint32)) and np.all(np.isnan(w32))


def test_dtypes_round_the_weights_once():
    rng = np.random.default_rng(17)
    lg32 = rng.standard_normal((64, 128)).astype(np.float32)
    for dt in ("bf16", "f16"):
        bits = oracle.narrow(lg32, dt)
        idx, w, w32, _ = oracle.route_sigmoid_grouped(bits, dt, None, 8, 8, 4, True, True, 2.5)
        wide = oracle.widen(w, dt)
        assert np.array_equal(wide, oracle.widen(oracle.narrow(w32, dt), dt))
        lg_w = oracle.widen(bits, dt).astype(np.float32)  # exact: bf16 and f16 values are binary32 values
        idx32, _, _, _ = oracle.route_sigmoid_grouped(lg_w, "f32", None, 8, 8, 4, True, True, 2.5)
        assert np.array_equal(idx, idx32)


@pytest.mark.parametrize("args", [
    dict(E=1025, k=1, G=1, m=1),
    dict(E=129 * 2, k=1, G=129, m=1),
    dict(E=30, k=1, G=4, m=1),            # E not divisible by G
    dict(E=32, k=1, G=4, m=5),            # more selected groups than groups
    dict(E=32, k=1, G=4, m=0),
    dict(E=256, k=65, G=1, m=1),          # top_k > 64
    dict(E=32, k=9, G=4, m=1),            # top_k beyond the chosen groups' experts
    dict(E=8, k=1, G=8, m=1, top_two=True),  # one expert per group cannot give two
    dict(E=8, k=1, G=2, m=1, scale=0.0),
    dict(E=8, k=1, G=2, m=1, scale=float("inf")),
    dict(E=8, k=1, G=2, m=1, scale=float("nan")),
])
def test_limits(args):
    a = dict(top_two=False, scale=1.0) | args
    lg = np.zeros((2, a["E"]), np.float32)
    with pytest.raises(ValueError):
        oracle.route_sigmoid_grouped(lg, "f32", None, a["k"], a["G"], a["m"], a["top_two"], True, a["scale"])
