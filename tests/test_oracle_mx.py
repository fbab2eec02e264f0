"""Pins of the oracle's MXFP8 quantisation ("Scalable Training of
Mixture-of-Experts Models with Megatron Core", section 5.3.3: 1 x 32 blocks,
E8M0 scales, E4M3 elements): the E4M3 grid against its closed-form values
and an exhaustive nearest search, the shared-exponent rule, error bounds,
scale invariance, and the MXFP8 layer against a dense evaluation."""
import numpy as np
import pytest

import oracle


def _grid():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


def test_e4m3_closed_form_values():
    """Format constants: 448 = 1.75 * 2^8 is the largest finite value (code
    0x7e), 2^-6 the smallest normal (0x08), 2^-9 the smallest subnormal
    (0x01); 1.0 is 0x38; 0x7f and 0xff are NaN; 254 finite codes."""
    d = oracle.e4m3_decode(np.array([0x7e, 0x08, 0x01, 0x38, 0xb8, 0x00, 0x80], dtype=np.uint8))
    assert d.tolist()[:5] == [448.0, 2.0 ** -6, 2.0 ** -9, 1.0, -1.0]
    assert d[5] == 0.0 and d[6] == 0.0 and np.signbit(d[6])
    assert np.isnan(oracle.e4m3_decode(np.array([0x7f, 0xff], dtype=np.uint8))).all()
    codes, vals = _grid()
    assert codes.size == 254
    pos = vals[codes < 0x80]
    assert np.all(np.diff(pos) > 0), "positive codes decode in increasing order"
    assert np.array_equal(oracle.e4m3_encode(vals), codes)
    assert np.array_equal(oracle.e4m3_round(vals), vals)


def test_e4m3_round_matches_exhaustive_nearest():
    """Nearest finite grid value by exhaustive search, ties to the even code,
    magnitudes above 448 saturated; includes exact midpoints."""
    codes, vals = _grid()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[1:] + pos[:-1]) / 2
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-500, 500, 3000), rng.standard_normal(3000) * 0.05, mids, -mids,
                        [448.0, 464.0, 479.9, 1e6, -1e6, 0.0]])
    got = oracle.e4m3_round(y)
    for v, g in zip(y, got):
        a = min(abs(v), 448.0)
        d = np.abs(pos - a)
        best = np.nonzero(d == d.min())[0]
        if best.size > 1:   # tie: the even code
            cand = [b for b in best if oracle.e4m3_encode(np.array([pos[b]]))[0] % 2 == 0]
            best = cand
        assert abs(g) == pos[best[0]] and (g == 0 or np.sign(g) == np.sign(v)), (v, g)


def test_mx_shared_exponent_and_exact_blocks():
    """A block whose largest magnitude is 448 * 2^s gets scale code 127 + s
    and round-trips exactly when its elements are on the scaled grid; the
    largest magnitude m of any block lands in [256, 512) before rounding; an
    all-zero block gets scale code 0."""
    codes, vals = _grid()
    rng = np.random.default_rng(5)
    for s in (-20, -3, 0, 7, 30):
        blk = rng.choice(vals, 32) * 2.0 ** s
        blk[5] = 448.0 * 2.0 ** s
        q, sc = oracle.mx_quantize(blk[None, :])
        assert sc[0, 0] == 127 + s
        assert np.array_equal(oracle.mx_dequantize(q, sc)[0], blk)
    v = rng.standard_normal((64, 96)) * 10.0 ** rng.uniform(-6, 6, (64, 1))
    q, sc = oracle.mx_quantize(v)
    amax = np.abs(v.reshape(64, 3, 32)).max(axis=-1)
    scaled = amax / 2.0 ** (sc.astype(np.float64) - 127)
    assert np.all((scaled >= 256) & (scaled < 512))
    zq, zs = oracle.mx_quantize(np.zeros((2, 64)))
    assert not zq.any() and not zs.any()


def test_mx_error_bound_and_scale_invariance():
    """Elements in the normal range are within half a unit of the third
    mantissa bit (relative 2^-4), the rest within half the subnormal step
    times the block scale, saturated ones within 64 * scale; multiplying a
    block by 2^j shifts its scale code by j and keeps its element codes."""
    rng = np.random.default_rng(7)
    v = rng.standard_normal((40, 128)) * np.exp(rng.uniform(-3, 3, (40, 128)))
    q, sc = oracle.mx_quantize(v)
    d = oracle.mx_dequantize(q, sc)
    X = np.repeat(2.0 ** (sc.astype(np.float64) - 127), 32, axis=1)
    a = np.abs(v) / X
    err = np.abs(d - v) / X
    normal = (a >= 2.0 ** -6) & (a <= 448)
    assert np.all(err[normal] <= a[normal] * 2.0 ** -4 * (1 + 1e-12))
    assert np.all(err[a < 2.0 ** -6] <= 2.0 ** -10 * (1 + 1e-12))
    assert np.all(err[a > 448] <= 64)
    q2, sc2 = oracle.mx_quantize(v * 2.0 ** 9)
    assert np.array_equal(q2, q) and np.array_equal(sc2.astype(int), sc.astype(int) + 9)
    assert np.array_equal(oracle.mx_roundtrip(d), d)


def _torch_mx_roundtrip(v):
    """An MXFP8 round trip written independently of the oracle: the block
    exponent from frexp (largest magnitude m = f 2^e with f in [0.5, 1), so
    floor(log2 m) = e - 1), the scaled elements clamped to +-448 and rounded by
    torch's own float8_e4m3fn conversion (nearest-even). torch converts a
    float64 through float32, which can round twice; the function checks that
    no element sits where that could matter (a float32 rounding that lands
    exactly on an E4M3 midpoint while the float64 value does not)."""
    import torch
    v = np.asarray(v, dtype=np.float64)
    blk = v.reshape(v.shape[:-1] + (v.shape[-1] // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    _, e = np.frexp(amax)
    exp = np.where(amax > 0, np.clip(e - 1 - 8, -127, 127), -127)
    scaled = np.clip(np.ldexp(blk, -exp[..., None]), -448.0, 448.0)
    s32 = scaled.astype(np.float32).astype(np.float64)
    grid = np.unique(np.abs(oracle.e4m3_decode(np.arange(256, dtype=np.uint8))))
    grid = grid[np.isfinite(grid)]
    mids = (grid[1:] + grid[:-1]) / 2
    risky = (s32 != scaled) & np.isin(np.abs(s32), mids)
    assert not risky.any(), "double-rounding case in the reference quantiser"
    q = torch.as_tensor(scaled).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    return np.ldexp(q, exp[..., None]).reshape(v.shape)


def test_mx_quantize_matches_an_independent_quantiser():
    """Activation-like rows (SwiGLU values of random projections, several
    magnitudes, zeros, exact E4M3 midpoints at a fixed scale) quantised by the
    oracle equal the independent frexp + torch float8 round trip, element by
    element."""
    rng = np.random.default_rng(13)
    g = rng.standard_normal((200, 256)) * 3
    u = rng.standard_normal((200, 256))
    act = oracle.silu(g) * u * np.exp(rng.uniform(-20, 20, (200, 1)))
    act[3] = 0.0
    act[4, :32] = 0.0
    grid = np.unique(np.abs(oracle.e4m3_decode(np.arange(256, dtype=np.uint8))))
    grid = grid[np.isfinite(grid)]
    mids = (grid[1:] + grid[:-1]) / 2
    act[5] = rng.choice(mids, 256) * rng.choice([-1.0, 1.0], 256)
    act[5, ::32] = 448.0                      # block maximum 448: scale 2^0, midpoints stay midpoints
    assert np.array_equal(oracle.mx_roundtrip(act), _torch_mx_roundtrip(act))


@pytest.mark.parametrize("act", ["swiglu", "gelu"])
def test_mxfp8_layer_identical_experts_is_the_dense_fp8_ffn(act):
    """Identical experts, renormalised weights: the MXFP8 layer equals one
    dense FFN on the quantised token rows, weights and (unrounded)
    activation, evaluated here with torch's float64 SiLU/GELU and the
    independent quantiser; the activation the oracle reports is that dense
    activation in permuted-row order, with its codes."""
    import torch
    rng = np.random.default_rng(9)
    T, h, E, F, k = 24, 64, 4, 64, 2
    n1 = 2 if act == "swiglu" else 1
    x = rng.standard_normal((T, h)).astype(np.float32)
    wg = (rng.standard_normal((E, h)) / 8).astype(np.float32)
    w1 = np.repeat((rng.standard_normal((1, n1 * F, h)) / 8), E, axis=0)
    w2 = np.repeat((rng.standard_normal((1, h, F)) / 8), E, axis=0)
    r = oracle.forward_mxfp8(x, wg, w1, w2, k, "softmax", act, with_act=True)
    a = torch.as_tensor(_torch_mx_roundtrip(x.astype(np.float64)) @ _torch_mx_roundtrip(w1[0]).T)
    if act == "swiglu":
        hid = (torch.nn.functional.silu(a[:, :F]) * a[:, F:]).numpy()
    else:
        hid = torch.nn.functional.gelu(a).numpy()
    dense = _torch_mx_roundtrip(hid) @ _torch_mx_roundtrip(w2[0]).T
    assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-12)
    perm = oracle.permutation(r["topk_idx"], E)
    rows = perm["sorted_token"]
    assert np.allclose(r["act"], hid[rows], rtol=1e-13, atol=1e-13)
    assert np.array_equal(oracle.mx_dequantize(r["act_codes"], r["act_scales"]), _torch_mx_roundtrip(hid[rows]))
    plain = oracle.forward(x, wg, w1, w2, k, "softmax", act)
    rel = np.abs(r["out"] - plain["out"]).max() / np.abs(plain["out"]).max()
    assert 1e-3 < rel < 0.1, rel


def test_roundtrip_equals_the_decoded_codes():
    """mx_roundtrip (no bit codes) gives exactly mx_dequantize(mx_quantize(v))
    on blocks mixing magnitudes (2^-140 .. 2^100), zeros, saturating and
    midpoint values; every finite E4M3 code decodes and re-encodes to
    itself."""
    rng = np.random.default_rng(21)
    v = rng.standard_normal((64, 256)) * 2.0 ** rng.integers(-140, 100, size=(64, 1))
    v[3, :32] = 0.0
    v[5, 40] = 1e30
    v[7, 64:96] = np.arange(32) * 0.0625 + 1.0 / 32     # E4M3 midpoints after scaling
    assert np.array_equal(oracle.mx_roundtrip(v), oracle.mx_dequantize(*oracle.mx_quantize(v)))
    codes = np.array([c for c in range(256) if (c & 0x7f) != 0x7f], dtype=np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes)), codes)
