"""HIP graph capture of the layer's C-ABI calls. The entry points allocate
nothing themselves (outputs and workspaces come from the caller), clear
memory with a fill kernel rather than hipMemsetAsync, and never synchronise
with the host, so a whole step recorded once in a graph replays as the
eager calls run. Each replay follows eager steps of the program's own and
must give bit-identical results to the eager step (every reduction has a
fixed order)."""
import pytest
import torch

from mixture_experts_layer_06_amd import workloads as wl
from parity import to_device

pytestmark = pytest.mark.gpu

CASES = {
    "mixtral_small_forward": wl.small_variant(wl.CONFIGS[2], T=300, h=256, F=256, E=8, k=2),
    "tiny_fp32_gelu_forward": wl.CONFIGS[1],
    "imbalanced_training_step": wl.small_variant(wl.CONFIGS[5], T=300, h=256, F=128, E=32),
    "handbook_training_step": wl.small_variant(wl.CONFIGS[6], T=512, h=256, F=128, E=16),
    "mxfp8_training_step": wl.small_variant(wl.CONFIGS[6], T=512, h=256, F=128, E=16),
}
MX = {"mxfp8_training_step"}


@pytest.mark.parametrize("name", list(CASES))
def test_graph_replay_equals_eager(moe_lib, name):
    from mixture_experts_layer_06_amd import layer
    cfg = CASES[name]
    train = cfg.backward
    print("case graph", name, flush=True)
    inp = to_device(wl.make_inputs(cfg, device="cpu", with_grad_out=train))
    mx = name in MX
    if mx:
        wq = layer.quantize_experts_mx(inp, for_backward=True)

    def step():
        if mx:
            f = layer.forward_mxfp8(inp, wq, cfg.k, cfg.score, keep_for_backward=True)
            return f, layer.backward_mxfp8(inp, f, wq, inp["grad_out"], cfg.k, cfg.score)
        f = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=train)
        g = layer.backward(inp, f, inp["grad_out"], cfg.k, cfg.score, cfg.act) if train else {}
        return f, g

    keys_f = ["out", "topk_idx", "topk_w", "counts"]
    keys_g = ["grad_x", "grad_w1", "grad_w2", "grad_w_gate"] + (["grad_b_gate"] if cfg.gate_bias else [])
    f0, g0 = step()
    torch.cuda.synchronize()
    ref = {k: f0[k].clone() for k in keys_f}
    ref.update({k: g0[k].clone() for k in keys_g if train})
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fg, gg = step()
    for rep in range(3):
        step()                       # eager work of the program between replays
        graph.replay()
        torch.cuda.synchronize()
        for k in keys_f:
            assert torch.equal(fg[k], ref[k]), (rep, k)
        for k in keys_g if train else []:
            assert torch.equal(gg[k], ref[k]), (rep, k)
