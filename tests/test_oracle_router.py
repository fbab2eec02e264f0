"""Pins of the oracle's router (gate order G, canonical sigmoid, top-k, weights)
against things other than the oracle itself: hand-derived values of the fixed
summation order, exact arithmetic within the fp32 error bound, the fp64
sigmoid, subset enumeration, closed forms and scipy's softmax/expit."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import expit, softmax

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _vec(spec, h):
    v = np.zeros(h, dtype=np.float32)
    if spec == "ones":
        v[:] = 1.0
    else:
        for i, val in spec.items():
            v[int(i)] = np.float32(val)
    return v


def test_gate_order_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "gate_order_cases.json")))["cases"]
    for c in cases:
        h = c["h"]
        x = _vec(c["x"], h)[None, :]
        w = _vec(c["w"], h)
        # a second expert row holding the reversed vector makes the (t, e)
        # indexing observable
        W = np.stack([w, w[::-1].copy()])
        b = None if c["bias"] is None else np.array([c["bias"], 0.0], dtype=np.float32)
        got = oracle.gate_logits(x, W, b)
        assert got.shape == (1, 2)
        assert got[0, 0] == np.float32(c["expected"]), (c["name"], got[0, 0])


def _exact_dot(x, w):
    return sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, w))


@pytest.mark.parametrize("h", [64, 128, 200, 4096])
def test_gate_within_fp32_error_bound(h):
    """|l - exact| <= (ceil(h/64) + 6) u sum|x_i w_i| (chain length plus tree
    depth, u = 2^-24), checked with exact rational arithmetic."""
    rng = np.random.default_rng(h)
    T, E = 3, 5
    x = rng.standard_normal((T, h)).astype(np.float32)
    w = (rng.standard_normal((E, h)) / np.sqrt(h)).astype(np.float32)
    l = oracle.gate_logits(x, w)
    u = 2.0 ** -24
    n = -(-h // 64) + 6
    for t in range(T):
        for e in range(E):
            ex = _exact_dot(x[t], w[e])
            s = float(sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(x[t], w[e])))
            err = abs(Fraction(float(l[t, e])) - ex)
            assert float(err) <= 1.01 * n * u * s, (t, e)


@pytest.mark.parametrize("h", [128, 640])
def test_gate_within_error_bound_with_subnormal_products(h):
    """Tokens near fp32's smallest normal against small gate weights, so the
    products and most partial sums are subnormal: there the error of a
    rounding is absolute (at most half the subnormal spacing, 2^-150), so
    |l - exact| <= (ceil(h/64) + 6) u sum|x_i w_i| + (h + 63) 2^-150 (one
    rounding per fma and per tree addition), checked with exact rational
    arithmetic; subnormal results are kept, not flushed."""
    rng = np.random.default_rng(h + 1)
    T, E = 4, 5
    x = (rng.standard_normal((T, h)) * 2.0 ** -118).astype(np.float32)
    x[1] *= 2.0 ** 40                      # a token of ordinary magnitude among them
    x[2] *= 2.0 ** -8                      # logits themselves subnormal
    w = (rng.standard_normal((E, h)) * 2.0 ** -9).astype(np.float32)
    l = oracle.gate_logits(x, w)
    u = 2.0 ** -24
    n = -(-h // 64) + 6
    tiny = 0
    for t in range(T):
        for e in range(E):
            ex = _exact_dot(x[t], w[e])
            prods = [abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(x[t], w[e])]
            tiny += sum(p < Fraction(2) ** -126 for p in prods)
            s = float(sum(prods))
            err = abs(Fraction(float(l[t, e])) - ex)
            assert err <= Fraction(1.01 * n * u * s) + (h + 63) * Fraction(2) ** -150, (t, e)
    assert tiny > (T - 1) * E * h // 2, "most products of the small tokens lie below the normal range"
    assert np.all(l[2] != 0) and np.all(np.abs(l[2]) < 2.0 ** -126), "subnormal logits are kept"


def test_gate_small_integers_exact_and_indexing():
    """Small integer inputs make every step exact: l = x @ w^T exactly."""
    rng = np.random.default_rng(7)
    x = rng.integers(-8, 9, size=(6, 320)).astype(np.float32)
    w = rng.integers(-8, 9, size=(4, 320)).astype(np.float32)
    b = np.array([1, -2, 0, 3], dtype=np.float32)
    got = oracle.gate_logits(x, w, b)
    ref = x.astype(np.int64) @ w.astype(np.int64).T + b.astype(np.int64)
    assert np.array_equal(got, ref.astype(np.float32))


def test_sigmoid_c_exhaustive():
    """Every fp32 input in [-80, 90]: within 0.5 ulp (+ fp64 noise) of the fp64
    sigmoid and non-decreasing."""
    max_ulp, n_dec, n = oracle.sigmoid_c_sweep(-80.0, 90.0)
    assert n > 2_000_000_000
    assert n_dec == 0
    assert max_ulp <= 0.5 + 1e-6


def test_sigmoid_c_special_values():
    s = oracle.sigmoid_c(np.array([0.0, 80.0, 1000.0, -80.0, -1000.0, np.inf, -np.inf],
                                  dtype=np.float32))
    assert s[0] == np.float32(0.5)
    assert s[1] == 1.0 and s[2] == 1.0 and s[5] == 1.0
    assert s[3] == s[4] == s[6] == np.float32(expit(-80.0))
    assert oracle.exp_c(0.0) == 1.0
    x = np.linspace(-30, 30, 1001)
    got = np.array([oracle.exp_c(v) for v in x])
    assert np.max(np.abs(got / np.exp(x) - 1)) < 4e-16


def _precedes(ka, ia, kb, ib):
    return ka > kb or (ka == kb and ia < ib)


def test_select_topk_against_subset_enumeration():
    """The selected set is the unique k-subset whose every member precedes
    every non-member in (key desc, index asc); members are listed in that
    order. Keys are drawn from a small set so ties are frequent."""
    rng = np.random.default_rng(3)
    for E in range(1, 7):
        for k in range(1, min(E, 3) + 1):
            keys = rng.choice(np.array([-1.0, 0.0, -0.0, 0.5, 2.0], dtype=np.float32),
                              size=(8, E))
            got = oracle.select_topk(oracle.selection_key(keys, "softmax"), k)
            for t in range(8):
                found = []
                for S in itertools.combinations(range(E), k):
                    rest = [j for j in range(E) if j not in S]
                    if all(_precedes(keys[t, a], a, keys[t, b], b) for a in S for b in rest):
                        found.append(S)
                assert len(found) == 1
                S = sorted(found[0], key=lambda j: (-float(keys[t, j]), j))
                assert list(got[t]) == S


def test_nan_ranks_last_and_signed_zero_equal():
    key = np.array([[np.nan, -0.0, 0.0, -np.inf]], dtype=np.float32)
    got = oracle.select_topk(oracle.selection_key(key, "softmax"), 4)
    # -0 and +0 tie -> index order; NaN counts as -inf and ties with index 3
    assert list(got[0]) == [1, 2, 0, 3]


def test_selection_on_logits_equals_selection_on_softmax():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((64, 128)).astype(np.float32)
    w = (rng.standard_normal((16, 128)) / 11.3).astype(np.float32)
    w[3] = w[9]          # exact ties
    r = oracle.route(x, w, 4, "softmax")
    p = softmax(r["logits"].astype(np.float64), axis=1)
    order = np.lexsort((np.broadcast_to(np.arange(16), p.shape), -p), axis=-1)[:, :4]
    assert np.array_equal(order, r["topk_idx"])


def test_weight_closed_forms():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((32, 64)).astype(np.float32)
    w = (rng.standard_normal((6, 64)) / 8).astype(np.float32)
    # k = E: renormalised top-k softmax is the full softmax
    r = oracle.route(x, w, 6, "softmax")
    full = softmax(r["logits"].astype(np.float64), axis=1)
    assert np.allclose(r["topk_w"], np.take_along_axis(full, r["topk_idx"].astype(int), 1),
                       rtol=1e-13, atol=0)
    # k = 1: weight 1
    r1 = oracle.route(x, w, 1, "softmax")
    assert np.all(r1["topk_w"] == 1.0)
    # renormalised softmax = softmax over the selected logits
    r3 = oracle.route(x, w, 3, "softmax")
    sel = np.take_along_axis(r3["logits"].astype(np.float64), r3["topk_idx"].astype(int), 1)
    assert np.allclose(r3["topk_w"], softmax(sel, axis=1), rtol=1e-13, atol=0)
    # sigmoid: selected expit scores over their sum; the selection bias is
    # in the key only
    bias = np.linspace(-0.1, 0.1, 6).astype(np.float32)
    rs = oracle.route(x, w, 3, "sigmoid", sel_bias=bias)
    sel = np.take_along_axis(rs["logits"].astype(np.float64), rs["topk_idx"].astype(int), 1)
    s = expit(sel)
    assert np.allclose(rs["topk_w"], s / s.sum(1, keepdims=True), rtol=1e-13, atol=0)
    key = (oracle.sigmoid_c(rs["logits"]) + bias).astype(np.float32)
    kt = np.take_along_axis(key, rs["topk_idx"].astype(int), 1)
    assert np.all(np.diff(kt, axis=1) <= 0)


def test_adversarial_routing():
    rng = np.random.default_rng(13)
    x = rng.standard_normal((16, 64)).astype(np.float32)
    w = (rng.standard_normal((8, 64)) / 8).astype(np.float32)
    # duplicated rows: exact ties, lowest index first
    w[5] = w[2]
    w[7] = w[2]
    r = oracle.route(x, w, 8, "softmax")
    for t in range(16):
        pos = {int(e): j for j, e in enumerate(r["topk_idx"][t])}
        assert pos[2] < pos[5] < pos[7]
        assert pos[5] == pos[2] + 1 and pos[7] == pos[5] + 1
    # rows one ulp apart: the larger logit wins although its index is higher
    w2 = np.zeros((4, 64), dtype=np.float32)
    w2[:, 0] = 1.0
    w2[3, 0] = np.nextafter(np.float32(1.0), np.float32(2.0))
    xx = np.zeros((1, 64), dtype=np.float32)
    xx[0, 0] = 1.0
    assert oracle.route(xx, w2, 1, "softmax")["topk_idx"][0, 0] == 3
    # x = 0: all logits equal -> experts 0..k-1 (softmax); sigmoid with a
    # selection bias -> the largest biases
    z = np.zeros((2, 64), dtype=np.float32)
    assert list(oracle.route(z, w, 3, "softmax")["topk_idx"][0]) == [0, 1, 2]
    bias = np.array([0.0, 0.05, -0.1, 0.09, 0.01, -0.02, 0.1, 0.0], dtype=np.float32)
    got = oracle.route(z, w, 3, "sigmoid", sel_bias=bias)["topk_idx"][0]
    assert list(got) == [6, 3, 1]


def test_counts_and_map_invariants():
    rng = np.random.default_rng(17)
    x = rng.standard_normal((100, 64)).astype(np.float32)
    w = (rng.standard_normal((12, 64)) / 8).astype(np.float32)
    r = oracle.route(x, w, 4, "softmax")
    assert r["counts"].sum() == 100 * 4
    assert np.all(r["routing_map"].sum(1) == 4)
    for t in range(100):
        assert len(set(r["topk_idx"][t].tolist())) == 4
    assert np.array_equal(r["counts"], np.bincount(r["topk_idx"].ravel(), minlength=12))
