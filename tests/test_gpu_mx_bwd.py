"""GPU parity of the MXFP8 training step ("Scalable Training of
Mixture-of-Experts Models with Megatron Core", sections 5.1, 5.3.3 and 5.4)
through the C ABI against the oracle's ``backward_mxfp8`` and
``expert_backward_mxfp8`` (pinned in test_oracle_mx_bwd.py).

The transposed weight quantisation is compared bit for bit. The kernels
form every quantised operand from fp32 values (the first projection
recomputed from the forward's codes, dY built from the routing weight and
dL/dout), the oracle from exact ones: only a value within its fp32 error
bound of an E4M3 rounding boundary (or of a change of block exponent) can
round differently. The small layers are held to the bf16 tolerance (2e-2)
plainly: token rows row by row, weight gradients per expert tensor. On the
model-sized layer an expert's weight gradients reduce over few tokens, so
one such rounding moves a whole row: there each element may differ by what
the fp32 bounds allow (computed by the test from the oracle's operands) and
what remains is held to 2e-2 of each row's sum of absolute terms (see
_expert_errs)."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_06_amd import workloads as wl
from parity import TOL, mfma_gamma, oracle_inputs, rel_err, rel_err_tensor, rel_err_terms, to_device, to_np32

pytestmark = pytest.mark.gpu


class _LazyExperts:
    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return self.t[e].float().cpu().numpy()


def _gpu_chain(cfg, dinp):
    from mixture_experts_layer_06_amd import layer
    wq = layer.quantize_experts_mx(dinp, for_backward=True)
    f = layer.forward_mxfp8(dinp, wq, cfg.k, cfg.score, keep_for_backward=True)
    g = layer.backward_mxfp8(dinp, f, wq, dinp["grad_out"], cfg.k, cfg.score)
    torch.cuda.synchronize()
    return wq, f, g


@pytest.mark.parametrize("E,R,C", [(3, 96, 320), (2, 256, 128), (2, 160, 100)])
def test_transposed_weight_quantisation_is_bit_exact(moe_lib, E, R, C):
    """moe_mx_quantize_t of [E, R, C] against oracle.mx_quantize of each
    matrix's transpose (blocks of 32 rows of a column), including an all-zero
    block and a huge outlier: 128-row tiles with a partial last tile (R = 96,
    160), whole tiles, and C not a multiple of 64 (one thread per block)."""
    from mixture_experts_layer_06_amd import binding as B
    g = torch.Generator().manual_seed(3)
    w = (torch.randn(E, R, C, generator=g) * torch.exp(torch.randn(E, 1, C, generator=g) * 3)).to(torch.bfloat16)
    w[1, 32:64, 7] = 0
    w[E - 1, 5, C - 20] = 3.0e38
    for src in (w, w.float()):
        codes, scales = B.moe_mx_quantize_t(src.cuda())
        torch.cuda.synchronize()
        for e in range(E):
            rc, rs = oracle.mx_quantize(src[e].float().numpy().astype(np.float64).T)
            assert np.array_equal(codes[e].cpu().numpy(), rc), e
            assert np.array_equal(scales[e].cpu().numpy(), rs), e


CASES = {
    # Mixtral-shaped routing (8 experts, top-2), ragged segments
    "ragged_top2": wl.small_variant(wl.CONFIGS[2], T=300, h=256, F=256, E=8, k=2),
    # the imbalanced (Zipf) load with a gate bias: empty experts get zero
    # weight gradients
    "empty_experts": wl.small_variant(wl.CONFIGS[5], T=40, h=128, F=128, E=32, k=2),
    # Qwen3-shaped routing (top-8 of 32), several token blocks per expert
    "top8_of_32": wl.small_variant(wl.CONFIGS[3], T=200, h=256, F=128, E=32, k=8),
}


def _random_cases(n=5, seed=20261206):
    """Seeded random sizes (h and F multiples of 128, 1 <= k <= E) on the
    Mixtral, Qwen3, DeepSeek-V3 (sigmoid with a selection bias, no shared
    expert), imbalanced and handbook structures."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        base = (2, 3, 4, 5, 6)[i % 5]
        T = int(rng.integers(1, 400))
        h = 128 * int(rng.integers(1, 5))
        F = 128 * int(rng.integers(1, 4))
        E = int(rng.integers(9 if base == 5 else 1, 49))
        k = int(rng.integers(1, min(E, 12) + 1))
        out["random%d_c%d_T%d_h%d_F%d_E%d_k%d" % (i, base, T, h, F, E, k)] = wl.small_variant(
            wl.CONFIGS[base], T=T, h=h, F=F, E=E, k=k).with_shape(n_shared=0)
    return out


CASES.update(_random_cases())


@pytest.mark.parametrize("name", list(CASES))
def test_mxfp8_training_step_small(moe_lib, name):
    cfg = CASES[name]
    print("case mx backward", name, flush=True)
    inp = wl.make_inputs(cfg, device="cpu", with_grad_out=True)
    dinp = to_device(inp)
    _, f, g = _gpu_chain(cfg, dinp)
    o = oracle_inputs(inp)
    G = to_np32(inp["grad_out"]).astype(np.float64)
    ref = oracle.backward_mxfp8(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act, G,
                                b_gate=o["b_gate"], sel_bias=o["sel_bias"])
    assert np.array_equal(f["topk_idx"].cpu().numpy(), oracle.route(o["x"], o["w_gate"], cfg.k, cfg.score,
                                                                    o["b_gate"], o["sel_bias"])["topk_idx"])
    tol = TOL[cfg.dtype]
    errs = {"grad_x": rel_err(to_np32(g["grad_x"]), ref["dx"]),
            "grad_topk_w": rel_err_tensor(g["grad_topk_w"].cpu().numpy(), ref["d_topk_w"]),
            "grad_w_gate": rel_err_tensor(g["grad_w_gate"].cpu().numpy(), ref["dw_gate"])}
    counts = f["counts"].cpu().numpy()
    for e in range(cfg.E):
        gw1, gw2 = g["grad_w1"][e].cpu().numpy(), g["grad_w2"][e].cpu().numpy()
        if counts[e] == 0:
            assert not gw1.any() and not gw2.any(), "empty expert %d" % e
            continue
        if not name.startswith("random"):
            errs["grad_w1[%d]" % e] = rel_err_tensor(gw1, ref["dw1"][e])
            errs["grad_w2[%d]" % e] = rel_err_tensor(gw2, ref["dw2"][e])
    if name.startswith("random"):
        # every expert over all of its tokens with the code-flip allowance
        # (an E4M3 code may differ where its operand lies within the fp32
        # bound of a rounding boundary): the plain per-tensor bound cannot
        # absorb one flipped code in an expert of a few tokens
        _expert_errs(cfg, o, G, f, g, [e for e in range(cfg.E) if counts[e] > 0], errs)
    if name == "empty_experts":
        assert (counts == 0).any()
    worst = max(errs, key=errs.get)
    print("largest error %s %.3g over %d tensors; grad_topk_w row-wise %.3g (reported)"
          % (worst, errs[worst], len(errs), rel_err(g["grad_topk_w"].cpu().numpy(), ref["d_topk_w"])), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


U = 2.0 ** -24


def _expo(m):
    return np.where(m > 0, np.clip(np.floor(np.log2(np.where(m > 0, m, 1.0))) - 8, -127, 127), -127).astype(np.int64)


def _spread_axis0(v, b):
    """How far the MXFP8 round trip of v along axis 0 (blocks of 32 rows
    from row 0, zero-padded) can move when every element may be off by up to
    b: per element, the largest |Q'(v') - Q(v)| over |v' - v| <= b, for each
    block exponent the perturbed block maximum allows (e4m3_round is
    monotone, so the extremes lie at v - b and v + b)."""
    m, n = v.shape
    mp = -(-m // 32) * 32
    V = np.zeros((mp, n))
    V[:m] = v
    Bb = np.zeros((mp, n))
    Bb[:m] = b
    V = V.reshape(mp // 32, 32, n)
    Bb = Bb.reshape(mp // 32, 32, n)
    amax = np.abs(V).max(axis=1, keepdims=True)
    bmax = Bb.max(axis=1, keepdims=True)
    e = _expo(amax)
    q = np.ldexp(oracle.e4m3_round(np.ldexp(V, -e)), e)
    D = np.zeros_like(V)
    for ec in (_expo(np.maximum(amax - bmax, 0.0)), _expo(amax + bmax)):
        for sgn in (-1.0, 1.0):
            D = np.maximum(D, np.abs(np.ldexp(oracle.e4m3_round(np.ldexp(V + sgn * Bb, -ec)), ec) - q))
    return D.reshape(mp, n)[:m]


def _fp32_bounds(xe, w1e, w2e, dy):
    """Bounds on how far the kernel's fp32 operands of the token-blocked and
    row-blocked quantisations can be from the exact ones: dY (the fp32
    routing weight times dL/dout, a few ulp), the recomputed g and u (the
    MFMA bound on sums of K = h products), act = silu(g) u and dgu (those
    errors carried through the derivatives, plus dact's own: the MFMA bound
    and the spread of Q_h(dY)), each with 16 ulp for exp, division and
    products. Also returns the exact dgu (da) and activation (hid)."""
    h = xe.shape[1]
    F = w2e.shape[1]
    xq, w1q = oracle.mx_roundtrip(xe), oracle.mx_roundtrip(w1e)
    a = xq @ w1q.T
    b_a = mfma_gamma(h) * (np.abs(xq) @ np.abs(w1q).T)
    g, u, bg, bu = a[:, :F], a[:, F:], b_a[:, :F], b_a[:, F:]
    sg = 1.0 / (1.0 + np.exp(-g))
    silu = g * sg
    psi = sg * (1.0 + g * (1.0 - sg))                       # silu'
    dpsi = sg * (1.0 - sg) * (2.0 + g * (1.0 - 2.0 * sg))   # silu''
    hid = silu * u
    fe = 16 * U * (1.0 + np.abs(g))
    b_act = np.abs(psi) * bg * np.abs(u) + np.abs(silu) * bu + fe * np.abs(hid)
    b_dy = 10 * U * np.abs(dy)
    dyq, w2c = oracle.mx_roundtrip(dy), oracle.mx_roundtrip_axis0(w2e)
    dact = dyq @ w2c
    b_dact = mfma_gamma(h) * (np.abs(dyq) @ np.abs(w2c)) + _spread_axis0(dy.T, b_dy.T).T @ np.abs(w2c)
    dg, du = dact * u * psi, dact * silu
    b_dg = np.abs(u * psi) * b_dact + np.abs(dact) * (np.abs(psi) * bu + np.abs(u * dpsi) * bg) + fe * np.abs(dg)
    b_du = np.abs(silu) * b_dact + np.abs(dact) * np.abs(psi) * bg + fe * np.abs(du)
    return dict(a=a, b_a=b_a, dact=dact, b_dact=b_dact, da=np.concatenate([dg, du], axis=1),
                b_da=np.concatenate([b_dg, b_du], axis=1), hid=hid, b_act=b_act, b_dy=b_dy)


def _ws_layout(P, h, F, E):
    """Byte offsets of the backward's workspace buffers, in the order the
    kernel source lays them out (every buffer starts at a 256-byte
    boundary); the token-blocked operands have rows of Pc padded token
    columns and a zero k-step of 128 more."""
    Pc = ((P + 127 * E) + 127) // 128 * 128
    ld = Pc + 128
    sizes = [("poffs", (E + 1) * 4), ("gu", P * 2 * F * 4), ("dy_c", P * h),
             ("dy_s", P * h // 32), ("dyT_c", h * ld), ("dyT_s", h * ld // 32), ("actT_c", F * ld),
             ("actT_s", F * ld // 32), ("dact", P * F * 4), ("dgu_c", P * 2 * F),
             ("dgu_s", P * 2 * F // 32), ("dguT_c", 2 * F * ld), ("dguT_s", 2 * F * ld // 32), ("xT_c", h * ld),
             ("xT_s", h * ld // 32)]
    off, at = {}, 0
    for name, nbytes in sizes:
        off[name] = at
        at += (nbytes + 255) // 256 * 256
    return ld, off, at


def _codes_explained(got_c, got_s, v, b, what):
    """MXFP8 codes and scales of v [m, K] along its last axis (the kernel's
    got_c [m, K], got_s [m, K/32]) against the oracle's, every difference
    explained: the value within its fp32 bound b of an E4M3 rounding
    boundary (or of a change of block exponent). Returns the number of
    differing codes."""
    rc, rs = oracle.mx_quantize(v)
    D = _spread_axis0(v.T, b.T).T
    gv = oracle.mx_dequantize(got_c, got_s)
    rv = oracle.mx_dequantize(rc, rs)
    diff = gv != rv
    assert not (diff & ~(np.abs(gv - rv) <= D)).any(), "%s: a code differs beyond the fp32 bound" % what
    return int(diff.sum())


def _stage_checks(cfg, dinp, f, wq, o, G, experts):
    """The backward's intermediates, read from a workspace the test hands
    to the call, for each listed expert over all of its tokens: the padded
    segment offsets exactly; the recomputed pre-activations and dact within
    their fp32 bounds of the oracle's; x blocked along the tokens bit for
    bit; the codes of dY (along h and along the tokens), of the activation
    (along the tokens) and of dgu (along 2F and along the tokens), which
    only exist quantised, equal but for differences their fp32 bounds
    explain."""
    from mixture_experts_layer_06_amd import binding as B
    P, h = int(f["sorted_token"].numel()), cfg.h
    F, E = cfg.F, cfg.E
    ld, off, total = _ws_layout(P, h, F, E)
    assert total == B.lib().moe_grouped_ffn_bwd_mx_workspace_size(P, h, F, E)
    ws = torch.full((total,), 0x5a, dtype=torch.uint8, device="cuda")
    row_w = B.moe_permute_weights(f["topk_w"], f["row_of"])
    B.moe_grouped_ffn_bwd_mx(dinp["grad_out"], row_w, dinp["x"], f["x_codes"], f["x_scales"], f["sorted_token"],
                             f["offsets"], wq["w1_codes"], wq["w1_scales"], wq["w1t_codes"], wq["w1t_scales"],
                             wq["w2t_codes"], wq["w2t_scales"], workspace=ws)
    torch.cuda.synchronize()

    def buf(name, shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        return ws[off[name]:off[name] + n].view(dtype).view(*shape)

    r = oracle.route(o["x"], o["w_gate"], cfg.k, cfg.score, o["b_gate"])
    counts = np.bincount(r["topk_idx"].ravel(), minlength=E)
    poffs = np.concatenate([[0], np.cumsum((counts + 127) // 128 * 128)])
    assert np.array_equal(buf("poffs", (E + 1,), torch.int32).cpu().numpy(), poffs)
    # the zero k-step after the padded token columns of every token-blocked
    # operand (the workspace starts as 0x5a bytes): codes and scale bytes 0
    for cname, sname, N in (("dyT_c", "dyT_s", h), ("actT_c", "actT_s", F), ("xT_c", "xT_s", h),
                            ("dguT_c", "dguT_s", 2 * F)):
        assert not buf(cname, (N, ld), torch.uint8)[:, ld - 128:].any(), cname
        assert not buf(sname, (N, ld // 32), torch.uint8)[:, ld // 32 - 4:].any(), sname
    offs = f["offsets"].cpu().numpy()
    for e in experts:
        tok, slot = np.nonzero(r["topk_idx"] == e)
        m, r0, r1, p0 = tok.size, int(offs[e]), int(offs[e + 1]), int(poffs[e])
        if m == 0:
            continue
        dy = r["topk_w"][tok, slot][:, None] * G[tok]
        xe = np.asarray(o["x"][tok], dtype=np.float64)
        w1e, w2e = np.asarray(o["w1"][e], dtype=np.float64), np.asarray(o["w2"][e], dtype=np.float64)
        bd = _fp32_bounds(xe, w1e, w2e, dy)
        for name, ref, bound, cols in (("gu", bd["a"], bd["b_a"], 2 * F), ("dact", bd["dact"], bd["b_dact"], F)):
            got = buf(name, (P, cols), torch.float32)[r0:r1].cpu().numpy().astype(np.float64)
            assert np.all(np.abs(got - ref) <= bound + 1e-30), "%s of expert %d beyond its fp32 bound" % (name, e)
        mp = -(-m // 128) * 128

        def tok_codes(cname, sname, N):
            c = buf(cname, (N, ld), torch.uint8)[:, p0:p0 + mp].cpu().numpy()
            sc = buf(sname, (N, ld // 32), torch.uint8)[:, p0 // 32:(p0 + mp) // 32].cpu().numpy()
            return c, sc

        pad = lambda v: np.concatenate([v, np.zeros((mp - m, v.shape[1]))]).T      # [N, mp], zero columns
        xc, xs = tok_codes("xT_c", "xT_s", h)
        rc, rs = oracle.mx_quantize(pad(xe))
        assert np.array_equal(xc, rc) and np.array_equal(xs, rs), "x along the tokens, expert %d" % e
        dc, ds = tok_codes("dyT_c", "dyT_s", h)
        n_t = _codes_explained(dc, ds, pad(dy), pad(bd["b_dy"]), "dY along the tokens")
        n_r = _codes_explained(buf("dy_c", (P, h), torch.uint8)[r0:r1].cpu().numpy(),
                               buf("dy_s", (P, h // 32), torch.uint8)[r0:r1].cpu().numpy(), dy, bd["b_dy"],
                               "dY along h")
        ac, asc = tok_codes("actT_c", "actT_s", F)
        n_a = _codes_explained(ac, asc, pad(bd["hid"]), pad(bd["b_act"]), "act along the tokens")
        gc, gs = tok_codes("dguT_c", "dguT_s", 2 * F)
        n_gt = _codes_explained(gc, gs, pad(bd["da"]), pad(bd["b_da"]), "dgu along the tokens")
        n_gr = _codes_explained(buf("dgu_c", (P, 2 * F), torch.uint8)[r0:r1].cpu().numpy(),
                                buf("dgu_s", (P, 2 * F // 32), torch.uint8)[r0:r1].cpu().numpy(), bd["da"],
                                bd["b_da"], "dgu along 2F")
        print("expert %d stages: gu, dact within bounds; x codes exact; codes differing, each explained: dY %d "
              "(tokens) %d (h) of %d, act %d of %d, dgu %d (tokens) %d (2F) of %d"
              % (e, n_t, n_r, m * h, n_a, m * F, n_gt, n_gr, 2 * m * F), flush=True)


def _beyond(got, ref, allow, terms):
    """Row-wise error left once the deviations the fp32 bounds allow are
    taken off, against each row's sum of absolute terms."""
    return rel_err_terms(np.maximum(np.abs(got - ref) - allow, 0.0), np.zeros_like(ref), terms)


def _expert_errs(cfg, o, G, f, g, experts, errs):
    """Each listed expert over all of its tokens, against
    expert_backward_mxfp8 fed from the seeded inputs: its rows of
    grad_x_perm and its weight gradients. An element may differ where an
    operand of a blocked quantisation lies within its fp32 bound of an E4M3
    rounding boundary (or of a change of block exponent): by at most that
    operand's spread times the other operand (plus the MFMA's own
    accumulation bound). What remains must be within the tolerance of each
    row's sum of absolute terms; the share of elements such a spread touches
    and the plain per-tensor errors are printed."""
    r = oracle.route(o["x"], o["w_gate"], cfg.k, cfg.score, o["b_gate"], o.get("sel_bias"))
    offs = f["offsets"].cpu().numpy()
    for e in experts:
        tok, slot = np.nonzero(r["topk_idx"] == e)        # ascending tokens: the segment's order
        m = tok.size
        assert offs[e + 1] - offs[e] == m
        dy = r["topk_w"][tok, slot][:, None] * G[tok]
        xe = np.asarray(o["x"][tok], dtype=np.float64)
        w1e, w2e = np.asarray(o["w1"][e], dtype=np.float64), np.asarray(o["w2"][e], dtype=np.float64)
        ge = oracle.expert_backward_mxfp8(xe, w1e, w2e, cfg.act, dy)
        bd = _fp32_bounds(xe, w1e, w2e, dy)
        gx = to_np32(g["grad_x_perm"][int(offs[e]):int(offs[e + 1])])
        gw1, gw2 = g["grad_w1"][e].cpu().numpy(), g["grad_w2"][e].cpu().numpy()
        # dx = Q_2F(dgu) Q_2F(W1)
        n2 = bd["da"].shape[1]
        daq, w1c = oracle.mx_roundtrip(bd["da"]), oracle.mx_roundtrip_axis0(w1e)
        D = _spread_axis0(bd["da"].T, bd["b_da"].T).T
        allow = D @ np.abs(w1c) + mfma_gamma(n2) * (np.abs(daq) @ np.abs(w1c))
        errs["grad_x_perm[%d]" % e] = _beyond(gx, ge["dx"], allow, np.abs(bd["da"]) @ np.abs(w1e))
        # dW1 = Q_tok(dgu)^T Q_tok(x), dW2 = Q_tok(dY)^T Q_tok(act)
        gam_t = mfma_gamma(-(-m // 128) * 128)
        xt, dat = oracle.mx_roundtrip_axis0(xe), oracle.mx_roundtrip_axis0(bd["da"])
        Dda = _spread_axis0(bd["da"], bd["b_da"])
        allow1 = Dda.T @ np.abs(xt) + gam_t * (np.abs(dat).T @ np.abs(xt))
        errs["grad_w1[%d]" % e] = _beyond(gw1, ge["dw1"], allow1, np.abs(bd["da"]).T @ np.abs(xe))
        dyt, actt = oracle.mx_roundtrip_axis0(dy), oracle.mx_roundtrip_axis0(bd["hid"])
        Ddy, Dact = _spread_axis0(dy, bd["b_dy"]), _spread_axis0(bd["hid"], bd["b_act"])
        allow2 = Ddy.T @ (np.abs(actt) + Dact) + np.abs(dyt).T @ Dact + gam_t * (np.abs(dyt).T @ np.abs(actt))
        errs["grad_w2[%d]" % e] = _beyond(gw2, ge["dw2"], allow2, np.abs(dy).T @ np.abs(bd["hid"]))
        print("expert %d (%d rows): spread touches %.2g%% of dgu, %.2g%% of dY, %.2g%% of act; plain errors "
              "grad_x_perm row-wise %.3g, grad_w1 %.3g, grad_w2 %.3g (per tensor)"
              % (e, m, 100 * (Dda > 0).mean(), 100 * (Ddy > 0).mean(), 100 * (Dact > 0).mean(),
                 rel_err(gx, ge["dx"]), rel_err_tensor(gw1, ge["dw1"]), rel_err_tensor(gw2, ge["dw2"])),
              flush=True)


def test_mxfp8_training_step_slice_of_mixtral(moe_lib):
    """The first 64 tokens of the Mixtral-shaped layer with its full weights
    (h=4096, F=14336, E=8, top-2): the lightest and the heaviest expert over
    all of their tokens, results and intermediates."""
    cfg = wl.CONFIGS[2].with_shape(T=64)
    print("case mx backward T=64 slice", flush=True)
    full = wl.make_inputs(wl.CONFIGS[2], device="cuda", with_grad_out=True)
    dinp = wl.slice_tokens(full, 64)
    wq, f, g = _gpu_chain(cfg, dinp)
    o = {"x": to_np32(dinp["x"]), "w_gate": to_np32(dinp["w_gate"]), "b_gate": None,
         "w1": _LazyExperts(dinp["w1"]), "w2": _LazyExperts(dinp["w2"])}
    G = to_np32(dinp["grad_out"]).astype(np.float64)
    counts = f["counts"].cpu().numpy()
    order = np.argsort(counts, kind="stable")
    experts = [int(order[0]), int(order[-1])] if counts[order[0]] > 0 else [int(order[-1])]
    errs = {}
    _expert_errs(cfg, o, G, f, g, experts, errs)
    print({k: round(v, 5) for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
    _stage_checks(cfg, dinp, f, wq, o, G, experts)


def test_mxfp8_training_step_full_size_sampled(moe_lib):
    """The full Mixtral-shaped step (T=4096): the lightest expert (about a
    thousand rows) over all of its tokens, results and intermediates; two
    runs bitwise equal."""
    cfg = wl.CONFIGS[2]
    print("case mx backward full size", flush=True)
    dinp = wl.make_inputs(cfg, device="cuda", with_grad_out=True)
    wq, f, g = _gpu_chain(cfg, dinp)
    counts = f["counts"].cpu().numpy()
    e = int(np.argsort(counts, kind="stable")[0])
    o = {"x": to_np32(dinp["x"]), "w_gate": to_np32(dinp["w_gate"]), "b_gate": None,
         "w1": _LazyExperts(dinp["w1"]), "w2": _LazyExperts(dinp["w2"])}
    G = to_np32(dinp["grad_out"]).astype(np.float64)
    errs = {}
    _expert_errs(cfg, o, G, f, g, [e], errs)
    print({k: round(v, 5) for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
    _stage_checks(cfg, dinp, f, wq, o, G, [e])
    from mixture_experts_layer_06_amd import layer
    g2 = layer.backward_mxfp8(dinp, f, wq, dinp["grad_out"], cfg.k, cfg.score)
    torch.cuda.synchronize()
    for key in ("grad_x", "grad_w1", "grad_w2", "grad_w_gate"):
        assert torch.equal(g[key], g2[key]), key


def test_mxfp8_training_step_imbalanced_full_size(moe_lib):
    """The full imbalanced Qwen3-shaped step (T=8192, h=4096, F=1536,
    E=128, top-8, Zipf-skewed gate bias, empty experts): the heaviest expert
    (about 6,300 rows, 50 k-steps in each weight-gradient tile) and the
    lightest expert with tokens (one k-step) over all of their tokens. The
    weight-gradient launches run their tiles heaviest expert first, every
    other round reversed, over many rounds of the persistent grid."""
    cfg = wl.CONFIGS[5]
    print("case mx backward imbalanced full size", flush=True)
    dinp = wl.make_inputs(cfg, device="cuda", with_grad_out=True)
    wq, f, g = _gpu_chain(cfg, dinp)
    counts = f["counts"].cpu().numpy()
    live = np.nonzero(counts > 0)[0]
    experts = [int(live[np.argmax(counts[live])]), int(live[np.argmin(counts[live])])]
    assert counts[experts[0]] > 48 * 128 and counts[experts[1]] <= 128
    o = {"x": to_np32(dinp["x"]), "w_gate": to_np32(dinp["w_gate"]), "b_gate": to_np32(dinp["b_gate"]),
         "w1": _LazyExperts(dinp["w1"]), "w2": _LazyExperts(dinp["w2"])}
    G = to_np32(dinp["grad_out"]).astype(np.float64)
    errs = {}
    _expert_errs(cfg, o, G, f, g, experts, errs)
    print({k: round(v, 5) for k, v in errs.items()}, flush=True)
    assert all(v <= TOL["bf16"] for v in errs.values()), errs
    # an expert without tokens gets zero weight gradients
    dead = int(np.nonzero(counts == 0)[0][0])
    assert not g["grad_w1"][dead].any() and not g["grad_w2"][dead].any()
