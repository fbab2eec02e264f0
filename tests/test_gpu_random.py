"""GPU parity of the forward path on a seeded sweep of random small layers.

Each case takes the routing, activation and structure of one of the six
workloads (softmax or sigmoid with a selection bias, gate bias or none,
SwiGLU or GELU with biases, a shared expert, the skewed gate bias, bf16 or
fp32) with sizes drawn at random within the library's limits (h and F
multiples of 64, 1 <= k <= E), so that shapes the hand-picked cases do not
name also meet the oracle: routing and the permutation bit for bit, the
expert outputs and the layer output within 2e-2 (bf16) or 1e-4 (fp32) under
the error measure of tests/parity.py."""
import sys

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_06_amd import workloads as wl
from parity import TOL, oracle_inputs, rel_err, to_device, to_np32

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        base = 1 + i % 6
        T = int(rng.integers(1, 700))
        h = 64 * int(rng.integers(1, 13))
        F = 64 * int(rng.integers(1, 9))
        E = int(rng.integers(1, 97))
        if base == 5:
            E = max(E, 9)          # the skewed gate bias leaves 8 experts dead
        k = int(rng.integers(1, min(E, 8 if i % 2 == 0 else 12) + 1))   # above 8 every other case
        out.append((i, base, T, h, F, E, k))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda c: "r%d_c%d_T%d_h%d_F%d_E%d_k%d" % c)
def test_random_layer_forward(moe_lib, case):
    i, base, T, h, F, E, k = case
    print("case random", case, flush=True)
    sys.stdout.flush()
    cfg = wl.small_variant(wl.CONFIGS[base], T=T, h=h, F=F, E=E, k=k)
    inp = wl.make_inputs(cfg, device="cpu", with_grad_out=False)
    from mixture_experts_layer_06_amd import layer
    g = layer.forward(to_device(inp), cfg.k, cfg.score, cfg.act, keep_for_backward=True, want_logits=True)
    torch.cuda.synchronize()
    o = oracle_inputs(inp)
    ref = oracle.forward(o["x"], o["w_gate"], o["w1"], o["w2"], cfg.k, cfg.score, cfg.act,
                         b_gate=o["b_gate"], sel_bias=o["sel_bias"], b1=o["b1"], b2=o["b2"],
                         w1_sh=o["w1_sh"], w2_sh=o["w2_sh"])
    perm = oracle.permutation(ref["topk_idx"], cfg.E)
    logits = g["logits"].cpu().numpy()
    assert np.array_equal(logits.view(np.uint32), ref["logits"].view(np.uint32)), "gate logits differ bitwise"
    assert np.array_equal(g["topk_idx"].cpu().numpy(), ref["topk_idx"])
    assert np.array_equal(g["counts"].cpu().numpy(), ref["counts"])
    assert rel_err(g["topk_w"].cpu().numpy(), ref["topk_w"]) <= 1e-5
    if cfg.dtype == "bf16" and cfg.E >= 32 and cfg.k <= 8:
        # the same routing through the MFMA-filtered path (taken when no
        # logits are asked for): bitwise the fixed-order result
        from mixture_experts_layer_06_amd import binding as B
        d = to_device(inp)
        r = B.moe_route(d["x"], d["w_gate"], cfg.k, cfg.score, b_gate=d.get("b_gate"), sel_bias=d.get("sel_bias"))
        torch.cuda.synchronize()
        assert np.array_equal(r["topk_idx"].cpu().numpy(), ref["topk_idx"])
        assert np.array_equal(r["topk_w"].cpu().numpy().view(np.uint32),
                              g["topk_w"].cpu().numpy().view(np.uint32))
    assert np.array_equal(g["offsets"].cpu().numpy(), perm["offsets"])
    assert np.array_equal(g["row_of"].cpu().numpy(), perm["row_of"])
    y = to_np32(g["y"])
    y_ref = np.zeros_like(y, dtype=np.float64)
    for t in range(cfg.T):
        for j in range(cfg.k):
            y_ref[perm["row_of"][t, j]] = ref["y_pair"][t, j]
    assert rel_err(y, y_ref) <= TOL[cfg.dtype]
    err = rel_err(to_np32(g["out"]), ref["out"])
    print("  out error %.3g" % err, flush=True)
    assert err <= TOL[cfg.dtype], err
