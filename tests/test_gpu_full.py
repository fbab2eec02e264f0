"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times. Routing and permutation indices are compared bit for bit on
every token; the layer output on a sample of tokens that the oracle computes
one by one (routing is per token, so the oracle's result for a token does not
depend on the others)."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_06_amd import workloads as wl
from parity import TOL, rel_err, to_device, to_np32

pytestmark = pytest.mark.gpu


class _LazyExperts:
    """Expert weights left on the GPU; the oracle fetches expert e on use."""

    def __init__(self, t):
        self.t = t
        self.shape = tuple(t.shape)

    def __getitem__(self, e):
        return self.t[e].float().cpu().numpy()


@pytest.mark.parametrize("cid,n_sample", [(2, 12), (3, 12), (4, 5), (5, 8), (6, 8)])
def test_full_size_forward(moe_lib, cid, n_sample):
    from mixture_experts_layer_06_amd import layer
    cfg = wl.CONFIGS[cid]
    print("full-size forward, config", cid, cfg.name, flush=True)
    inp = wl.make_inputs(cfg, device="cuda", with_grad_out=False)
    g = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=True, want_logits=True)
    torch.cuda.synchronize()
    x = to_np32(inp["x"])
    wg = to_np32(inp["w_gate"])
    bg = to_np32(inp.get("b_gate"))
    sb = to_np32(inp.get("sel_bias"))
    ref = oracle.route(x, wg, cfg.k, cfg.score, bg, sb)
    assert np.array_equal(g["logits"].cpu().numpy().view(np.uint32), ref["logits"].view(np.uint32))
    assert np.array_equal(g["topk_idx"].cpu().numpy(), ref["topk_idx"])
    assert np.array_equal(g["counts"].cpu().numpy(), ref["counts"])
    assert rel_err(g["topk_w"].cpu().numpy(), ref["topk_w"]) <= 1e-5
    perm = oracle.permutation(ref["topk_idx"], cfg.E)
    assert np.array_equal(g["offsets"].cpu().numpy(), perm["offsets"])
    assert np.array_equal(g["sorted_token"].cpu().numpy(), perm["sorted_token"])
    assert np.array_equal(g["row_of"].cpu().numpy(), perm["row_of"])
    # x_perm rows are exact copies
    rows = torch.arange(0, cfg.P, max(1, cfg.P // 97), device="cuda")
    st = g["sorted_token"].long()
    assert torch.equal(g["x_perm"][rows], inp["x"][st[rows]])
    # sampled tokens through the whole layer
    tokens = np.linspace(0, cfg.T - 1, n_sample).astype(np.int64)
    w1s = to_np32(inp.get("w1_sh"))
    w2s = to_np32(inp.get("w2_sh"))
    o = oracle.forward(x, wg, _LazyExperts(inp["w1"]), _LazyExperts(inp["w2"]), cfg.k, cfg.score,
                       cfg.act, b_gate=bg, sel_bias=sb, w1_sh=w1s, w2_sh=w2s, tokens=tokens)
    got = to_np32(g["out"][torch.as_tensor(tokens, device="cuda")])
    err = rel_err(got, o["out"])
    print("config", cid, "sampled output rel err", err, flush=True)
    assert err <= TOL[cfg.dtype], err
    # expert outputs of the sampled pairs, in permuted order
    ri = perm["row_of"][tokens]
    y = to_np32(g["y"][torch.as_tensor(ri.ravel(), device="cuda")]).reshape(len(tokens), cfg.k, -1)
    assert rel_err(y.reshape(-1, cfg.h), o["y_pair"].reshape(-1, cfg.h)) <= TOL[cfg.dtype]
    # the inference path the benchmark times (no x_perm; the first GEMM
    # gathers token rows) computes the same numbers bit for bit
    g2 = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=False)
    torch.cuda.synchronize()
    assert g2["x_perm"] is None
    for key in ("topk_idx", "topk_w", "row_of", "act", "y", "out"):
        assert torch.equal(g2[key], g[key]), key


def test_imbalanced_load_profile(moe_lib):
    """The imbalanced workload realises its skew on the GPU path too: empty
    experts exist and the hottest expert holds about 12x the mean load."""
    from mixture_experts_layer_06_amd import binding as B
    cfg = wl.CONFIGS[5]
    inp = wl.make_inputs(cfg, device="cuda", router_only=True)
    r = B.moe_route(inp["x"], inp["w_gate"], cfg.k, cfg.score, b_gate=inp["b_gate"])
    c = r["counts"].cpu().numpy()
    assert c.sum() == cfg.P
    assert (c == 0).sum() >= 4
    assert c.max() > 8 * cfg.P / cfg.E


@pytest.mark.parametrize("memory_efficient", [False, True])
def test_empty_batch_forward_backward(moe_lib, memory_efficient):
    """T = 0: every stage runs on an empty batch without error, the output
    and the input gradient are empty, and the weight gradients are exactly
    zero (no token reaches any expert or the router)."""
    from mixture_experts_layer_06_amd import layer
    cfg = wl.small_variant(wl.CONFIGS[5], T=0, h=128, F=64, E=16)
    print("case empty batch, memory_efficient", memory_efficient, flush=True)
    dinp = to_device(wl.make_inputs(cfg, device="cpu"))
    if memory_efficient:
        dinp.pop("b_gate", None)
    f = layer.forward(dinp, cfg.k, cfg.score, cfg.act, keep_for_backward=True,
                      memory_efficient=memory_efficient, recompute=memory_efficient)
    g = layer.backward(dinp, f, dinp["grad_out"], cfg.k, cfg.score, cfg.act)
    torch.cuda.synchronize()
    assert tuple(f["out"].shape) == (0, cfg.h)
    assert tuple(g["grad_x"].shape) == (0, cfg.h)
    for key in ("grad_w1", "grad_w2", "grad_w_gate"):
        assert not g[key].any(), key
    if g.get("grad_b_gate") is not None:
        assert not g["grad_b_gate"].any()


def test_empty_batch_mxfp8(moe_lib):
    """T = 0 through the MXFP8 layer: empty output, no error."""
    from mixture_experts_layer_06_amd import layer
    cfg = wl.small_variant(wl.CONFIGS[2], T=0, h=256, F=128)
    dinp = to_device(wl.make_inputs(cfg, device="cpu", with_grad_out=False))
    wq = layer.quantize_experts_mx(dinp)
    f = layer.forward_mxfp8(dinp, wq, cfg.k, cfg.score)
    torch.cuda.synchronize()
    assert tuple(f["out"].shape) == (0, cfg.h)
