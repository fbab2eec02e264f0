"""GPU parity of the MXFP8 path ("Scalable Training of Mixture-of-Experts
Models with Megatron Core", section 5.3.3), through the C ABI, against the
oracle: the quantisation bit for bit (codes and scales are integers), the
activation's codes and scales (quantised from fp32 in the first projection's
epilogue) equal to the oracle's wherever the GPU's fp32 activation is too
close to a rounding boundary to decide it, and the MXFP8 layer within 2e-2
of the oracle's MXFP8 layer (products and sums in fp64 on the dequantised
values), per tensor and per token row.

Deciding a code is integer work done on a floating-point value, and the two
sides compute that value differently (fp32 MFMA accumulation against fp64):
a code may differ only where the interval [v - b, v + b] around the fp64
activation v, b the fp32 computation's error bound, holds an E4M3 rounding
boundary (or, for a block scale, a power of two of the block maximum). The
test checks that every difference is of that kind and reports how many
there are."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_06_amd import workloads as wl
from parity import TOL, mfma_gamma, oracle_inputs, rel_err, rel_err_tensor, to_device, to_np32

pytestmark = pytest.mark.gpu


def _hard_rows(rng):
    """Rows that exercise every branch: zeros, ties of the E4M3 grid,
    saturation, subnormal elements, tiny and huge block scales."""
    codes = np.arange(256, dtype=np.uint8)
    grid = oracle.e4m3_decode(codes)
    grid = grid[np.isfinite(grid)]
    pos = np.unique(np.abs(grid))
    mids = (pos[1:] + pos[:-1]) / 2
    rows = []
    rows.append(np.zeros(64))
    r = rng.choice(mids, 64)
    r[0] = 448.0                                   # fixes the block scale at 2^0: ties stay ties
    r[32] = 448.0
    rows.append(r * rng.choice([-1.0, 1.0], 64))
    rows.append(np.concatenate([[480.0, 500.0, 1.0e-3, 2.0 ** -9], rng.standard_normal(60)]))
    rows.append(rng.standard_normal(64) * 2.0 ** -120)
    rows.append(rng.standard_normal(64) * 2.0 ** 100)
    rows.append(rng.standard_normal(64) * np.exp(rng.uniform(-12, 12, 64)))
    return np.stack(rows)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_quantize_bit_exact(moe_lib, dtype):
    rng = np.random.default_rng(21)
    hard = _hard_rows(rng)
    rand = rng.standard_normal((300, 64)) * np.exp(rng.uniform(-8, 8, (300, 1)))
    v = torch.as_tensor(np.concatenate([hard, rand]), dtype=torch.float32).to(dtype)
    codes, scales = moe_lib.moe_mx_quantize(v.cuda())
    rc, rs = oracle.mx_quantize(to_np32(v).astype(np.float64))
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    bad = np.nonzero(got != rc)
    assert bad[0].size == 0, (bad[0][:5], bad[1][:5], got[bad][:5], rc[bad][:5])


@pytest.mark.parametrize("lo", [256.0, 1.0, 2.0 ** -7, 2.0 ** -10])
def test_quantize_whole_binade(moe_lib, lo):
    """Every fp32 value of the binade [lo, 2 lo), both signs, quantised with
    the block scale fixed at 2^0 (each block of 32 holds 31 sweep values and
    the anchor 300): the elements are then the values themselves, so this
    covers every input of the E4M3 rounding in that binade. The binades: the
    top one (saturation of (448, 512) included), one of the normal range,
    the top subnormal one (rounding up into the smallest normal 2^-6) and
    the one rounding to the smallest subnormal 2^-9 or to zero."""
    first = np.float32(lo).view(np.uint32)
    sweep = (first + np.arange(1 << 23, dtype=np.uint32)).view(np.float32)
    n = sweep.size // 31 * 31
    tail = sweep[n:]
    blocks = np.concatenate([sweep[:n].reshape(-1, 31), np.pad(tail, (0, 31 - tail.size))[None]])
    blocks = np.pad(blocks, ((0, -blocks.shape[0] % 8), (0, 0)))
    v = np.concatenate([blocks, np.full((blocks.shape[0], 1), np.float32(300.0))], axis=1)
    v[1::2] *= -1
    v = v.reshape(-1, 256)                          # rows of 8 blocks
    print("case binade", lo, v.shape, flush=True)
    codes, scales = moe_lib.moe_mx_quantize(torch.as_tensor(v).cuda())
    rc, rs = oracle.mx_quantize(v.astype(np.float64))
    assert (rs == 127).all()
    assert np.array_equal(scales.cpu().numpy(), rs)
    got = codes.cpu().numpy()
    bad = np.nonzero(got != rc)
    assert bad[0].size == 0, (v[bad][:5], got[bad][:5], rc[bad][:5])


def test_quantize_weights_bit_exact(moe_lib):
    """The Mixtral-shaped layer's first expert matrix (14336 x 2 rows of
    4096), quantised along h."""
    cfg = wl.CONFIGS[2]
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=False)
    w = inp["w1"][0]
    codes, scales = moe_lib.moe_mx_quantize(w)
    rows = slice(0, 28672, 97)
    rc, rs = oracle.mx_quantize(to_np32(w[rows]).astype(np.float64))
    assert np.array_equal(codes[rows].cpu().numpy(), rc)
    assert np.array_equal(scales[rows].cpu().numpy(), rs)


def _check_act_codes(got_codes, got_scales, ref, o, perm, E, F):
    """Codes and scales of the activation against the oracle's, with every
    difference explained by the fp32 error bound (see the module docstring).
    The bound on the GPU's silu(g) * u: the dot products' error (gamma times
    the sums of absolute products) carried through the derivatives, plus the
    epilogue's own roundings: hardware exp2 and reciprocal (about 1 ulp each,
    the exp2 argument's rounding magnified by |g log2 e|), the add and the two
    multiplies. Returns (differing blocks, differing codes, blocks, codes)."""
    h = o["x"].shape[1]
    xq = oracle.mx_roundtrip(o["x"].astype(np.float64))
    gam = mfma_gamma(h)
    bound = np.zeros_like(ref["act"])
    for e in range(E):
        r0, r1 = int(perm["offsets"][e]), int(perm["offsets"][e + 1])
        if r1 == r0:
            continue
        w1q = oracle.mx_roundtrip(np.asarray(o["w1"][e], dtype=np.float64))
        xs = xq[perm["sorted_token"][r0:r1]]
        a = xs @ w1q.T
        S = np.abs(xs) @ np.abs(w1q).T
        g, u = a[:, :F], a[:, F:]
        sg = 1.0 / (1.0 + np.exp(-g))
        dsilu = np.abs(sg * (1 + g * (1 - sg)))
        bound[r0:r1] = (dsilu * gam * S[:, :F] * np.abs(u) + np.abs(g * sg) * gam * S[:, F:]
                        + (4 + 2 * np.abs(g) + 8) * 2.0 ** -24 * np.abs(ref["act"][r0:r1]))
    P = ref["act"].shape[0]
    blk = ref["act"].reshape(P, F // 32, 32)
    bb = bound.reshape(P, F // 32, 32)
    amax = np.abs(blk).max(axis=-1)
    bmax = bb.max(axis=-1)

    def expo(m):
        return np.where(m > 0, np.clip(np.floor(np.log2(np.where(m > 0, m, 1.0))) - 8, -127, 127), -127)

    ex_ref = ref["act_scales"].astype(np.int64) - 127
    ex_got = got_scales.astype(np.int64) - 127
    lo, hi = expo(np.maximum(amax - bmax, 0.0)), expo(amax + bmax)
    assert np.array_equal(expo(amax), ex_ref)
    sdiff = ex_got != ex_ref
    assert np.all((ex_got >= lo) & (ex_got <= hi)), "a block scale differs beyond the fp32 error bound"
    # codes of the blocks whose scales agree, in scaled units
    same = ~sdiff
    v = blk / 2.0 ** ex_ref[..., None]
    b = bb / 2.0 ** ex_ref[..., None]
    gv = oracle.e4m3_decode(got_codes.reshape(P, F // 32, 32))
    rv = oracle.e4m3_decode(ref["act_codes"].reshape(P, F // 32, 32))
    rlo, rhi = oracle.e4m3_round(v - b), oracle.e4m3_round(v + b)
    cdiff = (gv != rv) & same[..., None]
    ok = (gv >= np.minimum(rlo, rhi)) & (gv <= np.maximum(rlo, rhi))
    bad = ~ok & same[..., None]
    if bad.any():
        # how far the GPU value must have been from the fp64 one: the distance
        # from v to the nearest value that rounds to the GPU's code, in units
        # of the bound b
        vb, gb, bbad = v[bad], gv[bad], b[bad]
        grid = np.unique(oracle.e4m3_decode(np.arange(256, dtype=np.uint8)))
        grid = grid[np.isfinite(grid)]
        idx = np.searchsorted(grid, gb)
        lo_edge = np.where(idx > 0, (grid[np.maximum(idx - 1, 0)] + gb) / 2, gb)
        hi_edge = np.where(idx < grid.size - 1, (grid[np.minimum(idx + 1, grid.size - 1)] + gb) / 2, gb)
        dist = np.where(vb < lo_edge, lo_edge - vb, np.where(vb > hi_edge, vb - hi_edge, 0.0))
        steps = np.abs(np.searchsorted(grid, gb) - np.searchsorted(grid, rv[bad]))
        raise AssertionError("%d codes differ beyond the fp32 error bound; needed / bound: max %.3g, median "
                             "%.3g; grid steps apart: max %d; examples v=%s got=%s ref=%s b=%s"
                             % (bad.sum(), (dist / bbad).max(), np.median(dist / bbad), steps.max(),
                                vb[:4], gb[:4], rv[bad][:4], bbad[:4]))
    nb, nc = int(sdiff.size), int(same.sum() * 32)
    # a bug (a misplaced column, a wrong scale) would move far more codes
    assert sdiff.sum() <= 0.01 * nb and cdiff.sum() <= 0.01 * nc, (int(sdiff.sum()), nb, int(cdiff.sum()), nc)
    return int(sdiff.sum()), int(cdiff.sum()), nb, nc


MX_CASES = {
    "mixtral_small": wl.small_variant(wl.CONFIGS[2], T=600, h=256, F=384),
    "qwen3_small": wl.small_variant(wl.CONFIGS[3], T=1000, h=512, F=256),
    "imbalanced_small": wl.small_variant(wl.CONFIGS[5], T=300, h=256, F=128, E=32),
}


def _random_mx_cases(n=6, seed=20261205):
    """Seeded random sizes (h and F multiples of 128, 1 <= k <= E) on the
    Mixtral, Qwen3, DeepSeek-V3 (sigmoid with a selection bias, no shared
    expert), imbalanced and handbook structures."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        base = (2, 3, 4, 5, 6)[i % 5]
        T = int(rng.integers(1, 600))
        h = 128 * int(rng.integers(1, 7))
        F = 128 * int(rng.integers(1, 5))
        E = int(rng.integers(9 if base == 5 else 1, 65))
        k = int(rng.integers(1, min(E, 12) + 1))
        out["random%d_c%d_T%d_h%d_F%d_E%d_k%d" % (i, base, T, h, F, E, k)] = wl.small_variant(
            wl.CONFIGS[base], T=T, h=h, F=F, E=E, k=k).with_shape(n_shared=0)
    return out


MX_CASES.update(_random_mx_cases())


@pytest.mark.parametrize("name", list(MX_CASES))
def test_mxfp8_layer_parity(moe_lib, name):
    """Layer output of the MXFP8 path against the oracle's MXFP8 layer;
    the routing is the bf16 path's, bit for bit; the distance of both to
    the unquantised layer is reported."""
    from mixture_experts_layer_06_amd import layer
    cfg = MX_CASES[name]
    print("case mxfp8", name, flush=True)
    inp = wl.make_inputs(cfg, device="cpu", with_grad_out=False)
    dinp = to_device(inp)
    wq = layer.quantize_experts_mx(dinp)
    g = layer.forward_mxfp8(dinp, wq, cfg.k, cfg.score)
    torch.cuda.synchronize()
    o = oracle_inputs(inp)
    ref = oracle.forward_mxfp8(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act,
                               b_gate=o["b_gate"], sel_bias=o["sel_bias"], with_act=True)
    assert np.array_equal(g["topk_idx"].cpu().numpy(), ref["topk_idx"])
    # the quantised tokens the first GEMM reads are the oracle's
    xq, xs = oracle.mx_quantize(o["x"].astype(np.float64))
    gxq, gxs = moe_lib.moe_mx_quantize(dinp["x"])
    assert np.array_equal(gxq.cpu().numpy(), xq) and np.array_equal(gxs.cpu().numpy(), xs)
    perm = oracle.permutation(ref["topk_idx"], cfg.E)
    assert np.array_equal(g["offsets"].cpu().numpy(), perm["offsets"])
    nsb, ncd, nb, nc = _check_act_codes(g["act_codes"].cpu().numpy(), g["act_scales"].cpu().numpy(), ref, o,
                                        perm, cfg.E, cfg.F)
    err = rel_err_tensor(to_np32(g["out"]), ref["out"])
    rows = rel_err(to_np32(g["out"]), ref["out"])
    plain = oracle.forward(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act,
                           b_gate=o["b_gate"], sel_bias=o["sel_bias"])
    print("activation: %d of %d block scales and %d of %d codes differ, each within the fp32 error bound; "
          "out vs oracle MXFP8 layer: tensor %.3g, row-wise %.3g; MXFP8 vs unquantised: gpu %.3g, oracle %.3g"
          % (nsb, nb, ncd, nc, err, rows, rel_err_tensor(to_np32(g["out"]), plain["out"]),
             rel_err_tensor(ref["out"], plain["out"])), flush=True)
    assert err <= TOL["bf16"] and rows <= TOL["bf16"], (err, rows)


def test_mxfp8_grouped_ffn_dispatch_copy_equals_gather(moe_lib):
    """Permuted token rows quantised and read directly give the same bits as
    the unpermuted rows gathered inside the first GEMM."""
    from mixture_experts_layer_06_amd import binding as B
    cfg = wl.small_variant(wl.CONFIGS[3], T=700, h=384, F=256)
    inp = to_device(wl.make_inputs(cfg, device="cpu", with_grad_out=False))
    r = B.moe_route(inp["x"], inp["w_gate"], cfg.k, cfg.score)
    p = B.moe_permute(inp["x"], r["topk_idx"], cfg.E)
    w1q, w1s = B.moe_mx_quantize(inp["w1"])
    w2q, w2s = B.moe_mx_quantize(inp["w2"])
    xq, xs = B.moe_mx_quantize(inp["x"])
    a = B.moe_grouped_ffn_mx(xq, xs, p["offsets"], w1q, w1s, w2q, w2s, gather_rows=p["sorted_token"],
                             want_act=True)
    pq, ps = B.moe_mx_quantize(p["x_perm"])
    b = B.moe_grouped_ffn_mx(pq, ps, p["offsets"], w1q, w1s, w2q, w2s, want_act=True)
    torch.cuda.synchronize()
    for key in ("act", "act_codes", "act_scales", "y"):
        assert torch.equal(a[key], b[key]), key


def test_mxfp8_handbook_layer_full_size_sampled(moe_lib):
    """The handbook's layer at full size (32,768 tokens, 64 experts of width
    1024, top-8): sampled tokens against the oracle's MXFP8 layer."""
    from mixture_experts_layer_06_amd import layer
    cfg = wl.CONFIGS[6]
    print("case mxfp8 handbook full size", flush=True)
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=False)
    wq = layer.quantize_experts_mx(inp)
    g = layer.forward_mxfp8(inp, wq, cfg.k, cfg.score)
    torch.cuda.synchronize()

    class Lazy:
        def __init__(self, t):
            self.t = t
            self.shape = tuple(t.shape)

        def __getitem__(self, e):
            return self.t[e].float().cpu().numpy()

    tokens = np.linspace(0, cfg.T - 1, 5).astype(np.int64)
    ref = oracle.forward_mxfp8(to_np32(inp["x"]), to_np32(inp["w_gate"]), Lazy(inp["w1"]), Lazy(inp["w2"]),
                               cfg.k, cfg.score, cfg.act, tokens=tokens)
    assert np.array_equal(g["topk_idx"][torch.as_tensor(tokens, device="cuda")].cpu().numpy(), ref["topk_idx"])
    got = to_np32(g["out"][torch.as_tensor(tokens, device="cuda")])
    err, rows = rel_err_tensor(got, ref["out"]), rel_err(got, ref["out"])
    print("sampled out rel err: tensor %.3g, row-wise %.3g" % (err, rows), flush=True)
    assert err <= TOL["bf16"] and rows <= TOL["bf16"], (err, rows)


def test_mxfp8_split_second_projection(moe_lib):
    """A layer whose second projection leaves a short last round of tiles
    (4096 tokens, top-2 of 8 experts, h = 2048: about 288 tiles of 256 x 256
    for 256 compute units), so its last tiles are split along F into
    pieces: tokens of the last expert (whose tiles are the split ones) and a
    spread of others against the oracle's MXFP8 layer, and the split result
    against the unsplit one (the same products, summed in another order)."""
    from mixture_experts_layer_06_amd import binding as B
    from mixture_experts_layer_06_amd import layer
    cfg = wl.small_variant(wl.CONFIGS[2], T=4096, h=2048, F=1024)
    print("case mxfp8 split", cfg.T, cfg.h, cfg.F, flush=True)
    inp = wl.make_inputs(cfg, device="cpu", with_grad_out=False)
    o = oracle_inputs(inp)
    rt = oracle.route(o["x"], o["w_gate"], cfg.k, cfg.score)
    counts = np.bincount(rt["topk_idx"].reshape(-1), minlength=cfg.E)
    tiles = int(sum((int(c) + 255) // 256 for c in counts)) * (cfg.h // 256)
    rem = tiles % 256
    assert 0 < 2 * rem <= 256, (tiles, rem)   # the split plan's condition on a 256-block grid
    last = np.nonzero((rt["topk_idx"] == cfg.E - 1).any(axis=1))[0]
    tokens = np.unique(np.concatenate([last[:: max(1, len(last) // 24)], np.linspace(0, cfg.T - 1, 8).astype(np.int64)]))
    dinp = to_device(inp)
    wq = layer.quantize_experts_mx(dinp)
    g = layer.forward_mxfp8(dinp, wq, cfg.k, cfg.score)
    torch.cuda.synchronize()
    ref = oracle.forward_mxfp8(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act, tokens=tokens)
    got = to_np32(g["out"][torch.as_tensor(tokens, device="cuda")])
    err, rows = rel_err_tensor(got, ref["out"]), rel_err(got, ref["out"])
    print("sampled out rel err: tensor %.3g, row-wise %.3g" % (err, rows), flush=True)
    assert err <= TOL["bf16"] and rows <= TOL["bf16"], (err, rows)
    xq, xs = B.moe_mx_quantize(dinp["x"])
    args = (xq, xs, g["offsets"], wq["w1_codes"], wq["w1_scales"], wq["w2_codes"], wq["w2_scales"])
    a = B.moe_grouped_ffn_mx(*args, gather_rows=g["sorted_token"], split=True)
    b = B.moe_grouped_ffn_mx(*args, gather_rows=g["sorted_token"], split=False)
    torch.cuda.synchronize()
    assert torch.equal(a["act_codes"], b["act_codes"])
    d = rel_err_tensor(to_np32(a["y"]), to_np32(b["y"]))
    print("split vs unsplit y: %.3g" % d, flush=True)
    assert d <= 1e-2, d
