"""GPU parity of the backward for the expert kinds beyond bf16 SwiGLU, through
the C ABI, against the oracle's backward (pinned by finite differences):
the tiny fp32 layer of "emerging-techniques-moe-training" (Quick Start:
Linear + GELU + Linear with biases, a biased gate), the same expert in bf16,
fp32 SwiGLU, and the bias gradients of the bf16 SwiGLU kernels; then the
autograd function that chains the calls (MoELayerFn) against the explicit
chain and the oracle.

Tolerances: 1e-4 for fp32, 2e-2 for bf16, under the usual measure (rows for
token tensors, per expert tensor for weight and bias gradients)."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_06_amd import workloads as wl
from parity import TOL, oracle_inputs, rel_err, rel_err_tensor, rel_err_terms, to_device, to_np32

pytestmark = pytest.mark.gpu


def _with_gate_bias(inp, seed):
    g = torch.Generator().manual_seed(seed)
    inp["b_gate"] = torch.randn(inp["w_gate"].shape[0], generator=g) * 0.1
    return inp


def _topk_w_terms(cfg, o, topk_idx, G):
    """Sum of |G_t,i y_tj,i| over i for every pair (t, j): the scale of the
    error of <G_t, y_tj> when y is stored in bf16, whatever the cancellation
    in the dot product (expert outputs from the oracle's expert forward)."""
    terms = np.zeros(topk_idx.shape)
    for e in range(cfg.E):
        tok, slot = np.nonzero(topk_idx == e)
        if tok.size == 0:
            continue
        y, _ = oracle.expert_forward(o["x"][tok], o["w1"][e], o["w2"][e], cfg.act,
                                     None if o["b1"] is None else o["b1"][e], None if o["b2"] is None else o["b2"][e])
        terms[tok, slot] = (np.abs(G[tok]) * np.abs(y)).sum(axis=1)
    return terms


def _check(cfg, inp, g, ref, tol):
    """Token rows against their own scale; for the routing-weight gradients
    (one dot product <dL/dout, y> per pair, y stored in the layer dtype) the
    row scale is the dot products' sum of absolute terms, as for weight
    gradients (the plain row-wise figure is printed)."""
    o = oracle_inputs(inp)
    gw = g["grad_topk_w"].cpu().numpy()
    terms = _topk_w_terms(cfg, o, ref_topk(cfg, o), to_np32(inp["grad_out"]).astype(np.float64))
    errs = {"grad_x": rel_err(to_np32(g["grad_x"]), ref["dx"]),
            "grad_topk_w": max(rel_err_tensor(gw, ref["d_topk_w"]), rel_err_terms(gw, ref["d_topk_w"], terms)),
            "grad_w_gate": rel_err_tensor(g["grad_w_gate"].cpu().numpy(), ref["dw_gate"])}
    if inp.get("b_gate") is not None:
        errs["grad_b_gate"] = rel_err_tensor(g["grad_b_gate"].cpu().numpy(), ref["db_gate"])
    for e in range(cfg.E):
        if not ref["dw1"][e].any():
            assert not g["grad_w1"][e].any() and not g["grad_w2"][e].any()
            continue
        errs["grad_w1[%d]" % e] = rel_err_tensor(g["grad_w1"][e].cpu().numpy(), ref["dw1"][e])
        errs["grad_w2[%d]" % e] = rel_err_tensor(g["grad_w2"][e].cpu().numpy(), ref["dw2"][e])
        if inp.get("b1") is not None:
            errs["grad_b1[%d]" % e] = rel_err_tensor(g["grad_b1"][e].cpu().numpy(), ref["db1"][e])
            errs["grad_b2[%d]" % e] = rel_err_tensor(g["grad_b2"][e].cpu().numpy(), ref["db2"][e])
    worst = max(errs, key=errs.get)
    print("largest error %s %.3g over %d tensors; grad_topk_w plain row-wise %.3g (reported)"
          % (worst, errs[worst], len(errs), rel_err(gw, ref["d_topk_w"])), flush=True)
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, bad


def ref_topk(cfg, o):
    return oracle.route(o["x"], o["w_gate"], cfg.k, cfg.score, o["b_gate"])["topk_idx"]


CASES = {
    # the tiny fp32 layer as it is, with nonzero expert and gate biases
    "tiny_fp32_gelu": (wl.CONFIGS[1], {}),
    "gelu_bf16_ragged": (wl.small_variant(wl.CONFIGS[1], T=333, h=192, F=320, E=16, k=4).with_shape(dtype="bf16"),
                         {}),
    "swiglu_fp32": (wl.small_variant(wl.CONFIGS[1], T=200, h=128, F=192, E=8, k=2).with_shape(act="swiglu"), {}),
    "swiglu_bf16_biases": (wl.small_variant(wl.CONFIGS[5], T=300, h=256, F=128, E=32).with_shape(
        expert_bias=True, gate_bias=False), {}),
}


def _random_cases(n=4, seed=20261207):
    """Seeded random sizes (h and F multiples of 64, 1 <= k <= E) for each
    expert kind with biases: GELU fp32, GELU bf16, SwiGLU fp32, SwiGLU bf16."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(n):
        T = int(rng.integers(1, 400))
        h = 64 * int(rng.integers(1, 7))
        F = 64 * int(rng.integers(1, 7))
        E = int(rng.integers(9, 41))
        k = int(rng.integers(1, min(E, 12) + 1))
        kind = ("gelu", "gelu", "swiglu", "swiglu")[i % 4]
        dt = ("f32", "bf16", "f32", "bf16")[i % 4]
        if kind == "swiglu" and dt == "bf16":
            cfg = wl.small_variant(wl.CONFIGS[5], T=T, h=h, F=F, E=E, k=k).with_shape(
                expert_bias=True, gate_bias=False)
        else:
            cfg = wl.small_variant(wl.CONFIGS[1], T=T, h=h, F=F, E=E, k=k).with_shape(act=kind, dtype=dt)
        out["random%d_%s_%s_T%d_h%d_F%d_E%d_k%d" % (i, kind, dt, T, h, F, E, k)] = (cfg, {})
    return out


CASES.update(_random_cases())


@pytest.mark.parametrize("name", list(CASES))
def test_backward_expert_kinds_with_biases(moe_lib, name):
    from mixture_experts_layer_06_amd import layer
    cfg, _ = CASES[name]
    print("case backward", name, flush=True)
    inp = wl.make_inputs(cfg, device="cpu", nonzero_expert_bias=True, with_grad_out=True)
    if cfg.gate_bias:
        _with_gate_bias(inp, 5)
    dinp = to_device(inp)
    f = layer.forward(dinp, cfg.k, cfg.score, cfg.act, keep_for_backward=True)
    g = layer.backward(dinp, f, dinp["grad_out"], cfg.k, cfg.score, cfg.act)
    torch.cuda.synchronize()
    o = oracle_inputs(inp)
    ref = oracle.backward(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act,
                          to_np32(inp["grad_out"]), b_gate=o["b_gate"], b1=o["b1"], b2=o["b2"])
    assert np.array_equal(f["topk_idx"].cpu().numpy(), oracle.route(o["x"], o["w_gate"], cfg.k, cfg.score,
                                                                    o["b_gate"])["topk_idx"])
    _check(cfg, inp, g, ref, TOL[cfg.dtype])


def test_gelu_backward_empty_batch(moe_lib):
    """T = 0 on the fp32 GELU path: every expert's weight and bias gradients
    are exact zeros."""
    from mixture_experts_layer_06_amd import binding as B
    cfg = wl.CONFIGS[1]
    inp = to_device(wl.make_inputs(cfg, device="cpu", nonzero_expert_bias=True))
    z = torch.zeros((0, cfg.h), dtype=torch.float32, device="cuda")
    offs = torch.zeros(cfg.E + 1, dtype=torch.int32, device="cuda")
    g = B.moe_grouped_ffn_bwd(z, z, torch.zeros((0, cfg.F), device="cuda"), torch.zeros((0, cfg.F), device="cuda"),
                              offs, inp["w1"], inp["w2"], "gelu", want_bias_grads=True)
    torch.cuda.synchronize()
    for key in ("grad_w1", "grad_w2", "grad_b1", "grad_b2"):
        assert g[key].shape[0] == cfg.E and not g[key].any(), key


@pytest.mark.parametrize("name", ["tiny_fp32_gelu", "swiglu_bf16_biases"])
@pytest.mark.parametrize("losses", [False, True])
def test_autograd_function_matches_the_chain(moe_lib, name, losses):
    """MoELayerFn through torch.autograd: the gradients equal, bit for bit,
    those of the explicit forward/backward chain (with the loss coefficients
    as the upstream gradients of the losses), and the oracle's within the
    tolerance."""
    from mixture_experts_layer_06_amd import layer
    cfg, _ = CASES[name]
    print("case autograd", name, "losses" if losses else "", flush=True)
    inp = to_device(wl.make_inputs(cfg, device="cpu", nonzero_expert_bias=True, with_grad_out=True))
    if cfg.gate_bias:
        inp["b_gate"] = (torch.randn(cfg.E, generator=torch.Generator().manual_seed(5)) * 0.1).cuda()
    names = ["x", "w_gate", "w1", "w2", "b_gate", "b1", "b2"]
    leaves = {n: (inp[n].detach().clone().requires_grad_(True) if inp.get(n) is not None else None) for n in names}
    out, ls = layer.MoELayerFn.apply(*[leaves[n] for n in names], None, cfg.k, cfg.score, cfg.act, losses)
    coef_aux, coef_z = (1e-2, 1e-3) if losses else (0.0, 0.0)
    loss = (out.float() * inp["grad_out"].float()).sum() + coef_aux * ls[0] + coef_z * ls[1]
    loss.backward()
    torch.cuda.synchronize()
    f = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=True, router_losses=losses)
    ref = layer.backward(inp, f, inp["grad_out"], cfg.k, cfg.score, cfg.act, coef_aux=coef_aux, coef_z=coef_z)
    torch.cuda.synchronize()
    assert torch.equal(out, f["out"])
    pairs = {"x": "grad_x", "w_gate": "grad_w_gate", "w1": "grad_w1", "w2": "grad_w2", "b_gate": "grad_b_gate",
             "b1": "grad_b1", "b2": "grad_b2"}
    for n, key in pairs.items():
        if leaves[n] is None:
            continue
        assert leaves[n].grad is not None, n
        assert torch.equal(leaves[n].grad, ref[key].to(leaves[n].dtype)), n
    o = {k: to_np32(v) for k, v in inp.items() if isinstance(v, torch.Tensor)}
    ro = oracle.backward(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act, o["grad_out"],
                         b_gate=o.get("b_gate"), b1=o.get("b1"), b2=o.get("b2"), coef_aux=coef_aux, coef_z=coef_z)
    tol = TOL[cfg.dtype]
    assert rel_err(to_np32(leaves["x"].grad), ro["dx"]) <= tol
    assert rel_err_tensor(leaves["w_gate"].grad.float().cpu().numpy(), ro["dw_gate"]) <= tol
