"""Pins of the oracle's routing variants ("emerging-techniques-moe-training"):
capacity-factor token dropping (Capacity Factor Tuning, the DeepSpeed MoE
config) and expert-choice routing (Routing Mechanisms). Each is checked
against a differently written brute force, closed forms and invariants, and
the dropping backward against fp64 finite differences."""
import math

import numpy as np
import pytest

import oracle
from test_oracle_layer import _rand_layer


def test_capacity_formula_matches_the_page():
    """The page's rule int(tokens / experts * factor): 4096 tokens, 8
    experts, top-1, factors 1.25 and 2.0; min_capacity 4 for tiny batches;
    top-k counts the T*k slots."""
    assert oracle.expert_capacity(4096, 8, 1, 1.25) == 640
    assert oracle.expert_capacity(4096, 8, 1, 2.0) == 1024
    assert oracle.expert_capacity(8, 64, 1, 1.25) == 4
    assert oracle.expert_capacity(8, 64, 1, 1.25, min_capacity=0) == 0
    assert oracle.expert_capacity(8192, 128, 8, 1.25) == 640


def _brute_keep(idx, E, C):
    """Sequential counters: walk the pairs in token order, an expert accepts
    a pair while it has taken fewer than C."""
    T, k = idx.shape
    taken = [0] * E
    keep = np.zeros((T, k), dtype=bool)
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if taken[e] < C:
                keep[t, j] = True
                taken[e] += 1
    return keep


@pytest.mark.parametrize("C", [0, 1, 3, 7, 100])
def test_capacity_keep_matches_counters(C):
    rng = np.random.default_rng(C + 5)
    T, E, k = 60, 6, 2
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)])
    keep = oracle.capacity_keep(idx, E, C)
    assert np.array_equal(keep, _brute_keep(idx, E, C))
    counts = np.bincount(idx.reshape(-1), minlength=E)
    kept = np.bincount(idx[keep], minlength=E)
    assert np.array_equal(kept, np.minimum(counts, C))


def _layer(rng, act="swiglu", T=24, h=32, E=6, F=16):
    return _rand_layer(rng, T, h, E, F, act)


def test_dropping_forward_brute_force_and_limits():
    """Per-token loop with counters against the oracle's masked expert loop;
    capacity >= the largest load is the dropless layer bit for bit; capacity
    0 gives zeros; tokens whose pairs are all kept are unchanged."""
    rng = np.random.default_rng(11)
    x, wg, w1, w2, _, _ = _layer(rng)
    T, E, k = x.shape[0], w1.shape[0], 2
    free = oracle.forward(x, wg, w1, w2, k, "softmax", "swiglu")
    C = 5
    r = oracle.forward(x, wg, w1, w2, k, "softmax", "swiglu", capacity=C)
    taken = [0] * E
    brute = np.zeros_like(r["out"])
    for t in range(T):
        for j in range(k):
            e = int(free["topk_idx"][t, j])
            if taken[e] < C:
                taken[e] += 1
                y, _ = oracle.expert_forward(x[t:t + 1].astype(np.float64), w1[e], w2[e], "swiglu")
                brute[t] += free["topk_w"][t, j] * y[0]
    assert np.allclose(r["out"], brute, rtol=1e-13, atol=1e-13)
    assert (~r["keep"]).any()
    full = oracle.forward(x, wg, w1, w2, k, "softmax", "swiglu", capacity=T)
    assert np.array_equal(full["out"], free["out"])
    zero = oracle.forward(x, wg, w1, w2, k, "softmax", "swiglu", capacity=0)
    assert not zero["out"].any()
    whole = r["keep"].all(axis=1)
    assert np.array_equal(r["out"][whole], free["out"][whole])
    sub = oracle.forward(x, wg, w1, w2, k, "softmax", "swiglu", capacity=C, tokens=[3, 0, 17])
    assert np.allclose(sub["out"], r["out"][[3, 0, 17]], rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_dropping_backward_finite_differences(score):
    """Every coordinate of x, w_gate and b_gate and 120 of each expert
    matrix: fp64 central differences of the loss with dropping (the keep
    mask is fixed by the selection, which the steps leave unchanged)."""
    rng = np.random.default_rng(47)
    T, h, E, F, k, C = 12, 32, 4, 16, 2, 4
    x, wg, w1, w2, _, _ = _rand_layer(rng, T, h, E, F, "swiglu")
    G = rng.standard_normal((T, h))
    bg = 0.3 * rng.standard_normal(E)
    p = dict(x=x.astype(np.float64), w_gate=wg.astype(np.float64), w1=w1.astype(np.float64),
             w2=w2.astype(np.float64), b_gate=bg)
    L, idx, logits, w = oracle.loss_fp64(p["x"], p["w_gate"], p["w1"], p["w2"], k, score, "swiglu", G,
                                         b_gate=bg, capacity=C)
    keep = oracle.capacity_keep(idx, E, C)
    assert (~keep).any() and keep.any()
    g = oracle.backward(p["x"], p["w_gate"], p["w1"], p["w2"], k, score, "swiglu", G, b_gate=bg,
                        routing=dict(logits=logits, topk_idx=idx, topk_w=w), capacity=C)
    assert not g["d_topk_w"][~keep].any()
    grads = dict(x=g["dx"], w_gate=g["dw_gate"], b_gate=g["db_gate"],
                 w1=np.stack([g["dw1"][e] for e in range(E)]), w2=np.stack([g["dw2"][e] for e in range(E)]))
    eps = 1e-6
    for name in ["x", "w_gate", "b_gate", "w1", "w2"]:
        coords = list(np.ndindex(p[name].shape))
        if len(coords) > 120:
            coords = [coords[i] for i in rng.choice(len(coords), 120, replace=False)]
        for c in coords:
            def at(delta):
                q = dict(p)
                d = np.zeros_like(p[name])
                d[c] = delta
                q[name] = p[name] + d
                return oracle.loss_fp64(q["x"], q["w_gate"], q["w1"], q["w2"], k, score, "swiglu", G,
                                        b_gate=q["b_gate"], expect_idx=idx, capacity=C)[0]
            fd = (at(eps) - at(-eps)) / (2 * eps)
            assert abs(fd - grads[name][c]) <= 1e-6 * (1 + abs(grads[name][c])), (name, c, fd, grads[name][c])


def test_expert_choice_brute_force_and_ties():
    """Each expert's choice by a plain sort of (−logit, token) pairs;
    repeated logits go to the lower token indices; weights are the softmax
    gate probabilities."""
    rng = np.random.default_rng(13)
    T, E, C = 20, 5, 6
    l = rng.standard_normal((T, E)).astype(np.float32)
    l[3:9, 2] = 1.5            # a tie spanning the cut of expert 2
    l[:, 4] = 0.25             # expert 4: all equal
    chosen, weights = oracle.expert_choice(l, C)
    for e in range(E):
        pairs = sorted((-float(l[t, e]), t) for t in range(T))
        assert chosen[e].tolist() == sorted(t for _, t in pairs[:C])
    assert chosen[4].tolist() == list(range(C))
    ex = np.exp(l.astype(np.float64) - l.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    for e in range(E):
        assert np.allclose(weights[e], p[chosen[e], e], rtol=1e-14, atol=0)


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_expert_choice_every_token_is_the_dense_mixture(act):
    """Capacity T: every expert takes every token, so the layer is the
    softmax-weighted mixture of all experts, evaluated densely."""
    rng = np.random.default_rng(17)
    x, wg, w1, w2, b1, b2 = _rand_layer(rng, 16, 32, 4, 16, act, bias=(act == "gelu"))
    r = oracle.expert_choice_forward(x, wg, w1, w2, 16, act, b1=b1, b2=b2)
    logits = oracle.gate_logits(x, wg)
    ex = np.exp(logits.astype(np.float64) - logits.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    dense = np.zeros((16, 32))
    for e in range(4):
        y, _ = oracle.expert_forward(x.astype(np.float64), w1[e], w2[e], act,
                                     None if b1 is None else b1[e], None if b2 is None else b2[e])
        dense += p[:, e:e + 1] * y
    assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-13)


def test_expert_choice_load_is_exactly_balanced():
    """Every expert takes exactly C tokens; a token may be taken by none."""
    rng = np.random.default_rng(19)
    x, wg, w1, w2, _, _ = _rand_layer(rng, 40, 32, 8, 16, "swiglu")
    r = oracle.expert_choice_forward(x, wg, w1, w2, 10, "swiglu")
    assert r["chosen"].shape == (8, 10)
    assert all(len(set(row.tolist())) == 10 for row in r["chosen"])
    assert all(np.all(np.diff(row) > 0) for row in r["chosen"])
    untaken = np.setdiff1d(np.arange(40), r["chosen"].reshape(-1))
    assert not r["out"][untaken].any()
    sub = oracle.expert_choice_forward(x, wg, w1, w2, 10, "swiglu", tokens=[5, 0, 33])
    assert np.allclose(sub["out"], r["out"][[5, 0, 33]], rtol=1e-13, atol=1e-14)
