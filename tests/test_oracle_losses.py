"""Pins of the oracle's auxiliary router losses (load-balancing loss and
router z-loss, "emerging-techniques-moe-training", section 3 Load Balancing)
and of their gradient: the handbook's single-expert value, closed forms for
uniform and collapsed routers, a hand-worked two-token case, shift
invariances, fp64 central differences, and the layer backward with the
losses added."""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _topk(logits, k):
    """Selection by descending logit, lower index first on ties (the
    softmax router's order)."""
    order = np.lexsort((np.broadcast_to(np.arange(logits.shape[1]), logits.shape), -logits), axis=-1)
    return order[:, :k]


def test_single_expert_aux_loss_is_exactly_one():
    g = json.load(open(os.path.join(GOLDEN, "handbook_single_expert_losses.json")))
    rng = np.random.default_rng(3)
    l = rng.standard_normal((37, g["num_experts"])) * 5
    idx = np.zeros((37, g["topk"]), dtype=np.int64)
    aux, z = oracle.router_losses(l, idx, g["num_experts"])
    assert aux == g["aux_loss"]
    # one expert: logsumexp of one logit is the logit itself
    assert z == pytest.approx(float(np.mean(l[:, 0] ** 2)), rel=1e-14)


def test_hand_worked_two_tokens():
    """T=2, E=2, top-1, both tokens with logits (0, ln 3): each softmax is
    (1/4, 3/4), both tokens choose expert 1, so f = (0, 1), P = (1/4, 3/4),
    aux = 2 * 3/4 = 3/2 and z = (ln 4)^2."""
    l = np.array([[0.0, math.log(3.0)], [0.0, math.log(3.0)]])
    idx = _topk(l, 1)
    assert idx.tolist() == [[1], [1]]
    aux, z = oracle.router_losses(l, idx, 2)
    assert aux == pytest.approx(1.5, rel=1e-15)
    assert z == pytest.approx(math.log(4.0) ** 2, rel=1e-15)


def test_mean_router_probs_hand_worked_and_invariants():
    """Logits (0, ln 3) and (ln 3, 0): softmaxes (1/4, 3/4) and (3/4, 1/4),
    so P = (1/2, 1/2). For any logits P is a distribution; equal logits give
    1/E; an empty batch gives zeros; aux = E <f, P>."""
    l = np.array([[0.0, math.log(3.0)], [math.log(3.0), 0.0]])
    assert oracle.mean_router_probs(l) == pytest.approx([0.5, 0.5], rel=1e-15)
    rng = np.random.default_rng(9)
    l = 4 * rng.standard_normal((50, 7))
    P = oracle.mean_router_probs(l)
    assert P.sum() == pytest.approx(1.0, rel=1e-14) and (P > 0).all()
    assert oracle.mean_router_probs(np.zeros((5, 8))) == pytest.approx(np.full(8, 1 / 8), rel=1e-15)
    assert not oracle.mean_router_probs(np.zeros((0, 3))).any()
    idx = _topk(l, 2)
    aux, _ = oracle.router_losses(l, idx, 7)
    assert aux == pytest.approx(7 * float(oracle.expert_fraction(idx, 7) @ P), rel=1e-14)


def test_uniform_router_gives_one_whatever_the_load():
    """Equal logits within each token: P_e = 1/E, so aux = sum_e f_e = 1 even
    for a skewed selection."""
    rng = np.random.default_rng(5)
    T, E, k = 64, 16, 4
    l = np.repeat(rng.standard_normal((T, 1)), E, axis=1)
    idx = rng.choice(3, size=(T, k))          # only experts 0..2 get load
    aux, z = oracle.router_losses(l, idx, E)
    assert aux == pytest.approx(1.0, rel=1e-14)
    assert z == pytest.approx(float(np.mean((l[:, 0] + math.log(E)) ** 2)), rel=1e-14)


def test_balanced_load_gives_one_whatever_the_logits():
    """f_e = 1/E for every expert: aux = sum_e P_e = 1."""
    rng = np.random.default_rng(7)
    T, E, k = 48, 12, 2
    l = 3 * rng.standard_normal((T, E))
    idx = (np.arange(T * k).reshape(T, k)) % E
    aux, _ = oracle.router_losses(l, idx, E)
    assert aux == pytest.approx(1.0, rel=1e-14)


def test_collapsed_router_approaches_E():
    """Every token sends all its probability to expert 0 and chooses it
    (top-1): f_0 = P_0 = 1, aux = E."""
    T, E = 20, 8
    l = np.zeros((T, E))
    l[:, 0] = 200.0
    aux, z = oracle.router_losses(l, _topk(l, 1), E)
    assert aux == pytest.approx(E, rel=1e-12)
    assert z == pytest.approx(200.0 ** 2, rel=1e-12)


def test_z_loss_is_stable_for_large_logits():
    l = np.full((3, 2), 1000.0)
    _, z = oracle.router_losses(l, np.zeros((3, 1), np.int64), 2)
    assert z == pytest.approx((1000.0 + math.log(2.0)) ** 2, rel=1e-15)


def test_shift_invariances():
    """Adding c_t to every logit of token t leaves every softmax, hence aux,
    unchanged and moves each logsumexp by c_t."""
    rng = np.random.default_rng(11)
    T, E, k = 30, 10, 3
    l = rng.standard_normal((T, E))
    idx = _topk(l, k)
    c = rng.standard_normal((T, 1)) * 4
    a0, _ = oracle.router_losses(l, idx, E)
    a1, z1 = oracle.router_losses(l + c, idx, E)
    assert a1 == pytest.approx(a0, rel=1e-13)
    m = l.max(axis=1)
    lse = m + np.log(np.exp(l - m[:, None]).sum(axis=1))
    assert z1 == pytest.approx(float(np.mean((lse + c[:, 0]) ** 2)), rel=1e-13)


def test_empty_batch_gives_zero():
    aux, z = oracle.router_losses(np.zeros((0, 4)), np.zeros((0, 2), np.int64), 4)
    assert aux == 0.0 and z == 0.0
    assert oracle.router_losses_dlogits(np.zeros((0, 4)), np.zeros((0, 2), np.int64), 4, 1.0,
                                        1.0).shape == (0, 4)


@pytest.mark.parametrize("ca,cz", [(1.0, 0.0), (0.0, 1.0), (0.7, 0.3)])
def test_dlogits_finite_differences(ca, cz):
    """Every coordinate of the logit gradient against fp64 central
    differences of the losses, with the selection (hence f) held fixed."""
    rng = np.random.default_rng(13)
    T, E, k = 6, 5, 2
    l = rng.standard_normal((T, E))
    idx = _topk(l, k)
    g = oracle.router_losses_dlogits(l, idx, E, ca, cz)

    def L(v):
        a, z = oracle.router_losses(v, idx, E)
        return ca * a + cz * z

    eps = 1e-6
    for t in range(T):
        for e in range(E):
            d = np.zeros_like(l)
            d[t, e] = eps
            fd = (L(l + d) - L(l - d)) / (2 * eps)
            assert abs(fd - g[t, e]) <= 1e-8 * (1 + abs(g[t, e])), (t, e, fd, g[t, e])
    # aux is shift invariant per token: its gradient sums to 0 over experts
    ga = oracle.router_losses_dlogits(l, idx, E, 1.0, 0.0)
    assert np.allclose(ga.sum(axis=1), 0.0, atol=1e-15)


def _micro_layer(rng, score):
    T, h, E, F, k = 8, 64, 8, 32, 2
    # x on the fp32 grid: the backward reads activations in fp32
    x = rng.standard_normal((T, h)).astype(np.float32).astype(np.float64)
    wg = rng.standard_normal((E, h)) / math.sqrt(h)
    w1 = rng.standard_normal((E, 2 * F, h)) / math.sqrt(h)
    w2 = rng.standard_normal((E, h, F)) / math.sqrt(F)
    bg = 0.3 * rng.standard_normal(E)
    G = rng.standard_normal((T, h))
    return dict(x=x, w_gate=wg, w1=w1, w2=w2, b_gate=bg, G=G, k=k, score=score)


@pytest.mark.parametrize("score", ["softmax", "sigmoid"])
def test_layer_backward_with_losses_finite_differences(score):
    """The layer backward with both losses added (coefficients far above the
    pages' 0.01 / 0.001 so their terms are visible) against fp64 central
    differences along random directions of x, the router weight and bias."""
    rng = np.random.default_rng(17)
    p = _micro_layer(rng, score)
    ca, cz = 0.9, 0.4
    kw = dict(b_gate=p["b_gate"], coef_aux=ca, coef_z=cz)
    L, idx, logits, w = oracle.loss_fp64(p["x"], p["w_gate"], p["w1"], p["w2"], p["k"], score,
                                         "swiglu", p["G"], **kw)
    routing = dict(logits=logits, topk_idx=idx, topk_w=w)
    g = oracle.backward(p["x"], p["w_gate"], p["w1"], p["w2"], p["k"], score, "swiglu", p["G"],
                        routing=routing, **kw)
    g0 = oracle.backward(p["x"], p["w_gate"], p["w1"], p["w2"], p["k"], score, "swiglu", p["G"],
                         routing=routing, b_gate=p["b_gate"])
    for name, key in [("x", "dx"), ("w_gate", "dw_gate"), ("b_gate", "db_gate")]:
        # the losses change the gradient noticeably
        assert np.abs(g[key] - g0[key]).max() > 1e-3 * np.abs(g0[key]).max()
        for _ in range(3):
            V = rng.standard_normal(p[name].shape)
            eps = 1e-4 * np.linalg.norm(p[name]) / np.linalg.norm(V)
            q1 = dict(p)
            q2 = dict(p)
            q1[name] = p[name] + eps * V
            q2[name] = p[name] - eps * V
            Lp = oracle.loss_fp64(q1["x"], q1["w_gate"], p["w1"], p["w2"], p["k"], score, "swiglu",
                                  p["G"], b_gate=q1["b_gate"], coef_aux=ca, coef_z=cz, expect_idx=idx)[0]
            Lm = oracle.loss_fp64(q2["x"], q2["w_gate"], p["w1"], p["w2"], p["k"], score, "swiglu",
                                  p["G"], b_gate=q2["b_gate"], coef_aux=ca, coef_z=cz, expect_idx=idx)[0]
            fd = (Lp - Lm) / (2 * eps)
            an = float((g[key] * V).sum())
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)
