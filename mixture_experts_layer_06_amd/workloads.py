"""Layer shapes and seeded synthetic inputs for the sparse MoE layer.

This module is shared by the HIP path's tests and benchmark and by the CPU
oracle's tests. It holds shapes, seeds and random draws only: none of the
layer's arithmetic (routing, permutation, expert FFN, combine) lives here.

The five workloads follow the layer shapes the pages discuss:

* a tiny fp32 layer whose expert is Linear(h->4h) + GELU + Linear(4h->h) with
  biases and whose gate is a biased Linear(h->E) ("emerging-techniques-moe-training",
  Quick Start "Basic MoE Architecture");
* a Mixtral-8x7B-shaped layer (E=8, top-2, SwiGLU 4096->14336->4096;
  "emerging-techniques-moe-training", Advanced Patterns "Mixtral 8x7B Architecture");
* a Qwen3-235B-shaped and a DeepSeek-V3-shaped layer, the two models of the
  performance table in "Scalable Training of Mixture-of-Experts Models with
  Megatron Core" (section 8.2), the latter with sigmoid scoring, an
  aux-loss-free selection bias (section 2.2) and one shared expert;
* an imbalanced training step on the Qwen3 shapes whose gate bias skews the
  expert load towards a Zipf(1.2) profile with several empty experts
  (load imbalance: section 1.3 of the same page).

Weights are drawn N(0, 1/fan_in); activations N(0, 1). bf16 workloads draw in
fp32 and round to bf16 (round-to-nearest-even, torch's conversion). Inputs are
generated with torch on the requested device; the CPU and GPU generators give
different (but each deterministic) streams for the same seed, so a test always
hands the same realised tensors to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import torch

SOFTMAX = "softmax"
SIGMOID = "sigmoid"
GELU = "gelu"
SWIGLU = "swiglu"

# tensor ids used in seeds: seed = 1000 * config_id + tensor_id (+ 100 * variant)
_TID = dict(x=1, w_gate=2, b_gate=3, w1=4, b1=5, w2=6, b2=7, w1_sh=8, w2_sh=9,
            sel_bias=10, grad_out=11, skew_perm=12, logits=13, dlogits=14)


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    cid: int
    name: str
    T: int          # tokens
    h: int          # hidden size
    E: int          # routed experts
    k: int          # top-k
    F: int          # expert intermediate width
    dtype: str      # "f32" or "bf16"
    score: str      # SOFTMAX or SIGMOID
    act: str        # GELU or SWIGLU
    gate_bias: bool = False
    expert_bias: bool = False
    sel_bias: bool = False
    n_shared: int = 0
    skew: bool = False      # Zipf-skewed gate bias, dead experts
    backward: bool = False

    @property
    def n1(self) -> int:
        """Rows of W1 per expert in units of F (SwiGLU stacks gate and up)."""
        return 2 if self.act == SWIGLU else 1

    @property
    def P(self) -> int:
        return self.T * self.k

    def with_shape(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)

    def active_flops_forward(self) -> float:
        """Algorithmic forward FLOPs: router GEMM plus every (token, expert) FFN.

        A SwiGLU expert holds three h x F matrices and a GELU expert two; each
        matrix costs 2*h*F FLOP per token routed to it.
        """
        nmat = 3 if self.act == SWIGLU else 2
        flops = 2.0 * self.T * self.h * self.E
        flops += self.P * nmat * 2.0 * self.h * self.F
        flops += self.n_shared * self.T * nmat * 2.0 * self.h * self.F
        return flops

    def active_flops_backward(self) -> float:
        """Backward FLOPs: dgrad and wgrad of every expert matrix (2x forward),
        the router's weight gradient and its input-gradient term (2 x 2ThE over
        the selected pairs only: 2*2*P*h), and the per-pair dot <G, Y>."""
        nmat = 3 if self.act == SWIGLU else 2
        flops = 2.0 * self.P * nmat * 2.0 * self.h * self.F
        flops += 2.0 * 2.0 * self.P * self.h
        flops += 2.0 * self.P * self.h
        return flops


CONFIGS = {
    1: LayerConfig(1, "tiny_fp32_gelu", T=256, h=128, E=8, k=2, F=512, dtype="f32",
                   score=SOFTMAX, act=GELU, gate_bias=True, expert_bias=True),
    2: LayerConfig(2, "mixtral_8x7b_layer", T=4096, h=4096, E=8, k=2, F=14336,
                   dtype="bf16", score=SOFTMAX, act=SWIGLU),
    3: LayerConfig(3, "qwen3_235b_layer", T=8192, h=4096, E=128, k=8, F=1536,
                   dtype="bf16", score=SOFTMAX, act=SWIGLU),
    4: LayerConfig(4, "deepseek_v3_layer", T=8192, h=7168, E=256, k=8, F=2048,
                   dtype="bf16", score=SIGMOID, act=SWIGLU, sel_bias=True, n_shared=1),
    5: LayerConfig(5, "qwen3_imbalanced_train", T=8192, h=4096, E=128, k=8, F=1536,
                   dtype="bf16", score=SOFTMAX, act=SWIGLU, gate_bias=True, skew=True,
                   backward=True),
    # the MoE layer of the training handbook ("Mixture-of-Experts from
    # Architecture to Large-Scale Training", section 2.5): 64 experts of width
    # 1024, top-8, hidden 2048; one micro-batch of 8 sequences of 4096 tokens
    6: LayerConfig(6, "handbook_moe_train", T=32768, h=2048, E=64, k=8, F=1024,
                   dtype="bf16", score=SOFTMAX, act=SWIGLU, backward=True),
}

# Zipf-skew recipe for the imbalanced step: gate bias b_e = GAMMA * ln(r_e ** -S)
# for the live experts ranked r_e = 1..E-N_DEAD in a seeded random order, and
# DEAD_BIAS for N_DEAD experts, which then never reach the top-k.
SKEW_GAMMA = 0.55
SKEW_S = 1.2
SKEW_N_DEAD = 8
SKEW_DEAD_BIAS = -30.0


def torch_dtype(cfg: LayerConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def _gen(cfg: LayerConfig, name: str, device, variant: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(1000 * cfg.cid + _TID[name] + 100 * variant)
    return g


def _normal(shape, std, cfg, name, device, variant, out_dtype):
    """N(0, std^2) drawn in fp32, then rounded to the layer dtype.

    Large tensors are drawn in slabs along dim 0 so that the fp32 staging
    buffer stays small (the DeepSeek-V3-shaped expert stack is 22.5 GB in bf16).
    """
    g = _gen(cfg, name, device, variant)
    out = torch.empty(shape, dtype=out_dtype, device=device)
    n0 = shape[0]
    row = math.prod(shape[1:]) if len(shape) > 1 else 1
    slab = max(1, (1 << 26) // max(row, 1))
    for s in range(0, n0, slab):
        e = min(n0, s + slab)
        tmp = torch.randn((e - s,) + tuple(shape[1:]), generator=g, device=device,
                          dtype=torch.float32)
        if std != 1.0:
            tmp.mul_(std)
        out[s:e].copy_(tmp)
    return out


def make_inputs(cfg: LayerConfig, device="cpu", variant: int = 0,
                nonzero_expert_bias: bool = False, with_grad_out: Optional[bool] = None,
                router_only: bool = False):
    """Seeded synthetic tensors for one layer invocation.

    Returns a dict of torch tensors on ``device``:
      x[T,h], w_gate[E,h] (layer dtype), b_gate[E] f32 or None, sel_bias[E] f32
      or None, w1[E,n1*F,h], b1[E,n1*F] or None, w2[E,h,F], b2[E,h] or None,
      w1_sh[n1*F,h] / w2_sh[h,F] or None, grad_out[T,h] or None.
    ``router_only`` stops after x, the gate and the biases (expert tensors are
    then absent). For SwiGLU the first F rows of w1[e] are the gate projection and the next F
    rows the up projection.
    """
    dt = torch_dtype(cfg)
    T, h, E, F, n1 = cfg.T, cfg.h, cfg.E, cfg.F, cfg.n1
    inp = {}
    inp["x"] = _normal((T, h), 1.0, cfg, "x", device, variant, dt)
    inp["w_gate"] = _normal((E, h), 1.0 / math.sqrt(h), cfg, "w_gate", device, variant, dt)
    inp["b_gate"] = None
    if cfg.skew:
        inp["b_gate"] = skew_gate_bias(cfg, device, variant)
    elif cfg.gate_bias:
        inp["b_gate"] = torch.zeros(E, dtype=torch.float32, device=device)
    inp["sel_bias"] = None
    if cfg.sel_bias:
        g = _gen(cfg, "sel_bias", device, variant)
        u = torch.rand(E, generator=g, device=device, dtype=torch.float32)
        inp["sel_bias"] = u * 0.2 - 0.1
    if router_only:
        return inp
    inp["w1"] = _normal((E, n1 * F, h), 1.0 / math.sqrt(h), cfg, "w1", device, variant, dt)
    inp["w2"] = _normal((E, h, F), 1.0 / math.sqrt(F), cfg, "w2", device, variant, dt)
    inp["b1"] = inp["b2"] = None
    if cfg.expert_bias:
        if nonzero_expert_bias:
            inp["b1"] = _normal((E, n1 * F), 0.1, cfg, "b1", device, variant, dt)
            inp["b2"] = _normal((E, h), 0.1, cfg, "b2", device, variant, dt)
        else:
            inp["b1"] = torch.zeros((E, n1 * F), dtype=dt, device=device)
            inp["b2"] = torch.zeros((E, h), dtype=dt, device=device)
    inp["w1_sh"] = inp["w2_sh"] = None
    if cfg.n_shared:
        inp["w1_sh"] = _normal((n1 * F, h), 1.0 / math.sqrt(h), cfg, "w1_sh", device, variant, dt)
        inp["w2_sh"] = _normal((h, F), 1.0 / math.sqrt(F), cfg, "w2_sh", device, variant, dt)
    if with_grad_out is None:
        with_grad_out = cfg.backward
    inp["grad_out"] = None
    if with_grad_out:
        inp["grad_out"] = _normal((T, h), 1.0, cfg, "grad_out", device, variant, dt)
    return inp


def router_logit_draw(cfg: LayerConfig, device="cpu", variant: int = 0):
    """Seeded stand-ins for a router's logits and a logit gradient, [T,E] fp32
    each: the logits N(0,1) per element (the spread of x . w_gate for the
    seeded x and w_gate) with the per-expert skew offsets of the imbalanced
    workload added where it has them; the gradient N(0, 1e-4)."""
    T, E = cfg.T, cfg.E
    logits = torch.randn((T, E), generator=_gen(cfg, "logits", "cpu", variant), dtype=torch.float32)
    if cfg.skew:
        logits += skew_gate_bias(cfg, "cpu", variant)[None, :]
    dl = torch.randn((T, E), generator=_gen(cfg, "dlogits", "cpu", variant), dtype=torch.float32) * 1e-2
    return logits.to(device), dl.to(device)


def skew_gate_bias(cfg: LayerConfig, device="cpu", variant: int = 0) -> torch.Tensor:
    """Gate bias giving a Zipf-like expert load with SKEW_N_DEAD empty experts."""
    E = cfg.E
    g = torch.Generator(device="cpu")
    g.manual_seed(1000 * cfg.cid + _TID["skew_perm"] + 100 * variant)
    perm = torch.randperm(E, generator=g)
    n_dead = min(SKEW_N_DEAD, max(E - 1, 0))
    b = torch.empty(E, dtype=torch.float64)
    b[perm[:n_dead]] = SKEW_DEAD_BIAS
    live = perm[n_dead:]
    ranks = torch.arange(1, live.numel() + 1, dtype=torch.float64)
    b[live] = SKEW_GAMMA * torch.log(ranks ** (-SKEW_S))
    return b.to(torch.float32).to(device)


def slice_tokens(inp: dict, T: int) -> dict:
    """The first T tokens of x and grad_out with the same weights."""
    out = dict(inp)
    out["x"] = inp["x"][:T].contiguous()
    if inp.get("grad_out") is not None:
        out["grad_out"] = inp["grad_out"][:T].contiguous()
    return out


def small_variant(cfg: LayerConfig, T: int, h: int, F: int, E: Optional[int] = None,
                  k: Optional[int] = None) -> LayerConfig:
    """A reduced-size layer with the same routing, activation and structure."""
    return cfg.with_shape(T=T, h=h, F=F, E=E if E is not None else cfg.E,
                          k=k if k is not None else cfg.k)
