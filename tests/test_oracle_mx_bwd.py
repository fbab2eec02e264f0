"""Pins of the oracle's MXFP8 training step (expert GEMMs in MXFP8, "Scalable
Training of Mixture-of-Experts Models with Megatron Core", sections 5.3.3 and
5.4) against things other than the functions themselves: hand-derived block
outcomes for the column-wise and per-segment quantisation, the plain fp64
backward (finite-difference pinned) when no quantisation acts, a scalar
brute force of every blocked product on a tiny ragged expert, and the
forward's output through the routing-weight gradients."""
import math

import numpy as np
import pytest

import oracle


def _ones_with_outlier(n, c, row, col, big):
    v = np.ones((n, c))
    v[row, col] = big
    return v


def test_axis0_blocks_are_32_rows_of_one_column():
    """An outlier of 2^20 sets its block's exponent to 12: the other 31 rows
    of that column block (value 1 = 2^-12 after scaling, below half the
    smallest E4M3 subnormal 2^-9) flush to 0; the next 32 rows of the same
    column, and every other column, keep their 1s."""
    v = _ones_with_outlier(70, 3, 5, 1, 2.0 ** 20)
    q = oracle.mx_roundtrip_axis0(v)
    want = np.ones((70, 3))
    want[0:32, 1] = 0.0
    want[5, 1] = 2.0 ** 20
    assert np.array_equal(q, want)


def test_axis0_segments_block_from_their_first_row():
    """Segments [0,10), [10,10) (empty), [10,70): the outlier at row 5 only
    reaches rows 0..9; rows 10..41 are the second segment's first block; a
    second outlier at row 45 reaches rows 42..69 (that segment's partial last
    block, padded with zero rows)."""
    v = _ones_with_outlier(70, 2, 5, 1, 2.0 ** 20)
    v[45, 1] = 2.0 ** 20
    q = oracle.mx_roundtrip_axis0(v, starts=[0, 10, 10, 70])
    want = np.ones((70, 2))
    want[0:10, 1] = 0.0
    want[5, 1] = 2.0 ** 20
    want[42:70, 1] = 0.0
    want[45, 1] = 2.0 ** 20
    assert np.array_equal(q, want)


def test_axis0_partial_block_scale_comes_from_its_rows():
    """A 3-row segment [3, 5, 7] (amax 7, exponent -6): scaled by 64 to 192,
    320, 448, all on the grid, so it is returned unchanged; [1.1, 3] gets
    exponent -7, 1.1 * 128 = 140.8 rounds to 144 on the grid (step 16), i.e.
    1.125."""
    v = np.array([[3.0], [5.0], [7.0], [1.1], [3.0]])
    q = oracle.mx_roundtrip_axis0(v, starts=[0, 3, 5])
    assert np.array_equal(q[:3, 0], [3.0, 5.0, 7.0])
    assert q[3, 0] == 1.125 and q[4, 0] == 3.0


def _mx_exact(rng, shape):
    """Values on the E4M3 grid whose every 32-block along the last axis
    starts with 256 (exponent 0): MXFP8 along the last axis is exact."""
    grid = np.array([0.5, 0.75, 1.0, 1.5, 2.0, 3.0, 5.0, 7.0, 12.0, 40.0, 96.0, 224.0])
    v = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    v[..., ::32] = 256.0
    return v


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_without_quantisation_equals_the_plain_backward(act):
    """x and W1 exact in MXFP8 along h, so the forward's pre-activations are
    the plain ones; with every backward Q switched off the function must be
    the plain fp64 expert backward (itself pinned by finite differences)."""
    rng = np.random.default_rng(3)
    m, h, F = 37, 64, 32
    n1 = 2 if act == "swiglu" else 1
    xe = _mx_exact(rng, (m, h)) / 256.0
    w1 = _mx_exact(rng, (n1 * F, h)) / 2048.0
    w2 = rng.standard_normal((h, F)) / 8.0
    dy = rng.standard_normal((m, h))
    got = oracle.expert_backward_mxfp8(xe, w1, w2, act, dy, quantise=False)
    ref = oracle.expert_backward(xe, w1, w2, act, dy)
    assert np.allclose(got["a"], xe @ w1.T, rtol=0, atol=0)
    for key in ("dx", "dw1", "dw2", "dgu"):
        assert np.allclose(got[key], ref[key], rtol=1e-12, atol=1e-12), key


def _q_block(vals):
    """MXFP8 round trip of one block given as a list (scalar code: shared
    exponent floor(log2 amax) - 8 clamped to [-127, 127], elements rounded on
    the E4M3 grid by oracle.e4m3_round)."""
    amax = max(abs(v) for v in vals)
    e = -127 if amax == 0 else max(-127, min(127, math.floor(math.log2(amax)) - 8))
    return [float(oracle.e4m3_round(v / 2.0 ** e)) * 2.0 ** e for v in vals]


def _q_rows(M):
    """Blocks of 32 along each row."""
    out = np.zeros_like(M)
    for r in range(M.shape[0]):
        for b in range(0, M.shape[1], 32):
            out[r, b:b + 32] = _q_block(list(M[r, b:b + 32]))
    return out


def _q_cols(M):
    """Blocks of 32 consecutive rows of each column, the last block partial."""
    out = np.zeros_like(M)
    for c in range(M.shape[1]):
        for b in range(0, M.shape[0], 32):
            blk = list(M[b:b + 32, c])
            out[b:b + len(blk), c] = _q_block(blk)
    return out


def _dot_loops(A, B):
    """A @ B with one np.dot per output element."""
    C = np.zeros((A.shape[0], B.shape[1]))
    for i in range(A.shape[0]):
        for j in range(B.shape[1]):
            C[i, j] = np.dot(A[i, :], B[:, j])
    return C


def test_blocked_products_against_a_scalar_brute_force():
    """Tiny SwiGLU expert with 37 tokens (one full and one partial token
    block), h = 64, F = 32: every quantised operand rebuilt block by block
    along the axis the reading fixes, products element by element."""
    rng = np.random.default_rng(11)
    m, h, F = 37, 64, 32
    xe = rng.standard_normal((m, h))
    w1 = rng.standard_normal((2 * F, h)) / 8.0
    w2 = rng.standard_normal((h, F)) / 6.0
    dy = rng.standard_normal((m, h)) * np.exp(rng.standard_normal((m, 1)))
    got = oracle.expert_backward_mxfp8(xe, w1, w2, "swiglu", dy)

    a = _dot_loops(_q_rows(xe), _q_rows(w1).T)                 # forward: both along h
    g, u = a[:, :F], a[:, F:]
    sg = 1.0 / (1.0 + np.exp(-g))
    hid = g * sg * u
    dhid = _dot_loops(_q_rows(dy), _q_cols(w2))                # along h: dy rows, W2 columns
    da = np.concatenate([dhid * u * sg * (1.0 + g * (1.0 - sg)), dhid * g * sg], axis=1)
    dx = _dot_loops(_q_rows(da), _q_cols(w1))                  # along 2F
    dw2 = _dot_loops(_q_cols(dy).T, _q_cols(hid))              # along the tokens
    dw1 = _dot_loops(_q_cols(da).T, _q_cols(xe))
    for key, want in (("a", a), ("dgu", da), ("dx", dx), ("dw2", dw2), ("dw1", dw1)):
        assert np.allclose(got[key], want, rtol=1e-11, atol=1e-11), key
    # the blocking matters here: without it the results move by far more
    plain = oracle.expert_backward_mxfp8(xe, w1, w2, "swiglu", dy, quantise=False)
    assert np.abs(plain["dw1"] - dw1).max() > 1e-3 * np.abs(dw1).max()


def test_layer_routing_weight_gradients_use_the_mxfp8_forward():
    """sum_j w_tj dL/dw_tj = <G_t, out_t> with out from forward_mxfp8 (out_t
    = sum_j w_tj y_tj), and the expert gradients are expert_backward_mxfp8's
    over each expert's tokens in ascending order."""
    rng = np.random.default_rng(5)
    T, h, F, E, k = 50, 64, 32, 4, 2
    x = rng.standard_normal((T, h)).astype(np.float32)
    wg = (rng.standard_normal((E, h)) / 8).astype(np.float32)
    w1 = rng.standard_normal((E, 2 * F, h)) / 8.0
    w2 = rng.standard_normal((E, h, F)) / 6.0
    G = rng.standard_normal((T, h))
    f = oracle.forward_mxfp8(x, wg, w1, w2, k, "softmax", "swiglu")
    b = oracle.backward_mxfp8(x, wg, w1, w2, k, "softmax", "swiglu", G)
    lhs = (f["topk_w"] * b["d_topk_w"]).sum(axis=1)
    rhs = (G * f["out"]).sum(axis=1)
    assert np.allclose(lhs, rhs, rtol=1e-10, atol=1e-10)
    e = 2
    tok, slot = np.nonzero(f["topk_idx"] == e)
    order = np.argsort(tok, kind="stable")
    tok, slot = tok[order], slot[order]
    dy = f["topk_w"][tok, slot][:, None] * G[tok]
    ge = oracle.expert_backward_mxfp8(x[tok].astype(np.float64), w1[e], w2[e], "swiglu", dy)
    assert np.array_equal(b["dw1"][e], ge["dw1"]) and np.array_equal(b["dw2"][e], ge["dw2"])
