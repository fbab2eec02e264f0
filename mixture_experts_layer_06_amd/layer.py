"""The whole MoE layer as a chain of C-ABI calls (Route -> Permute -> Grouped
FFN -> Unpermute, and the backward in reverse), on torch's current stream.

Only orchestration lives here: every step runs in libmoe.so's HIP kernels.
The stage order is that of "Scalable Training of Mixture-of-Experts Models
with Megatron Core", section 2.1.
"""
from __future__ import annotations

import torch

from . import binding as B


def _timed(timers, name, fn):
    """Runs fn(); with a timers dict, brackets it with HIP events on the
    current stream and appends the (start, end) pair under name."""
    if timers is None:
        return fn()
    s = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(s)
    r = fn()
    e1.record(s)
    timers.setdefault(name, []).append((e0, e1))
    return r


def forward(inp: dict, k: int, score: str, act: str, keep_for_backward: bool = False,
            timers: dict | None = None, router_losses: bool = False,
            memory_efficient: bool = False, recompute: bool = False, capacity: int | None = None,
            want_logits: bool | None = None):
    """One forward pass. ``inp`` holds device tensors named as in
    ``workloads.make_inputs``. Returns a dict with ``out`` and the
    intermediate results of every stage. With ``timers``, the grouped FFN
    call is bracketed by HIP events (key "grouped_ffn"). With
    ``router_losses``, also ``losses`` = {aux, z} (load-balancing loss and
    router z-loss, "emerging-techniques-moe-training", section 3).

    ``memory_efficient`` ("Scalable Training of Mixture-of-Experts Models
    with Megatron Core", section 4.1.1; experts without output bias): the
    routing weight scales the activation before the second projection and the
    combine is an unweighted sum; the backward then needs neither the expert
    outputs nor the activation, which are not kept. ``recompute`` (section
    4.1.2) alone drops only the activation, which the backward rebuilds from
    the pre-activations.

    ``capacity`` ("emerging-techniques-moe-training", Capacity Factor
    Tuning): every expert takes at most that many of its pairs, the first in
    token order; the rest are dropped. The result then also holds ``kept``,
    the capacity-limited dispatch the expert stages use, while the full one
    stays for the router's backward.

    The router's logits are kept (``logits``) when the losses or the
    backward need them (the losses; the sigmoid router's backward) or when
    ``want_logits`` asks for them; otherwise the route may take its
    MFMA-filtered path, whose selection and weights are the same bits."""
    x = inp["x"]
    E = inp["w_gate"].shape[0]
    if want_logits is None:
        want_logits = router_losses or (keep_for_backward and score == "sigmoid")
    r = B.moe_route(x, inp["w_gate"], k, score, b_gate=inp.get("b_gate"),
                    sel_bias=inp.get("sel_bias"), want_logits=want_logits or router_losses)
    # inference: the first GEMM gathers token rows itself (no dispatch copy);
    # training keeps x_perm for the weight gradient of the first projection
    gather = not keep_for_backward
    p = B.moe_permute(x, r["topk_idx"], E, with_x_perm=not gather and capacity is None)
    d = p
    if capacity is not None:
        d = B.moe_capacity_drop(r["topk_idx"], p["offsets"], p["row_of"], capacity, x=x,
                                with_x_perm=not gather)
    has_sh = inp.get("w1_sh") is not None
    row_w = B.moe_permute_weights(r["topk_w"], d["row_of"]) if memory_efficient else None
    f = _timed(timers, "grouped_ffn", lambda: B.moe_grouped_ffn(
        x if gather else d["x_perm"], d["offsets"], inp["w1"], inp["w2"], act, b1=inp.get("b1"),
        b2=inp.get("b2"), x_sh=x if has_sh else None, w1_sh=inp.get("w1_sh"), w2_sh=inp.get("w2_sh"),
        keep_gu=keep_for_backward, gather_rows=d["sorted_token"] if gather else None,
        row_w=row_w))
    out = B.moe_unpermute(f["y"], d["row_of"], None if memory_efficient else r["topk_w"], y_sh=f["y_sh"])
    if memory_efficient or recompute:
        f["act"] = None          # rebuilt from gu in the backward
    if memory_efficient:
        f["y"] = None            # the backward needs no expert output
    res = dict(out=out, row_w=row_w, recompute=memory_efficient or recompute)
    if router_losses:
        res["losses"], _ = B.moe_router_losses(r["logits"], r["counts"], k)
    res.update(r)
    res.update(p)
    res.update(f)
    if capacity is not None:
        res["kept"] = d
    return res


def capacity_from_factor(T: int, E: int, k: int, capacity_factor: float, min_capacity: int = 4) -> int:
    """Expert capacity int(T*k/E * factor), at least min_capacity
    ("emerging-techniques-moe-training", Capacity Factor Tuning, with the
    T*k routing slots counted as the tokens; min_capacity from the DeepSpeed
    config on that page)."""
    return max(int(min_capacity), int((T * k / E) * capacity_factor))


def forward_expert_choice(inp: dict, capacity: int, act: str, timers: dict | None = None):
    """Forward with expert-choice routing ("emerging-techniques-moe-training",
    Routing Mechanisms): every expert takes the ``capacity`` tokens with its
    largest logits; a chosen pair is weighted by the token's softmax gate
    probability. The experts' rows are gathered from x inside the first
    grouped GEMM, the weight is applied to the activation, and each token
    sums the rows of the experts that chose it."""
    x = inp["x"]
    T = x.shape[0]
    r = B.moe_route(x, inp["w_gate"], 1, "softmax", b_gate=inp.get("b_gate"), want_logits=True)
    c = B.moe_expert_choice(r["logits"], capacity)
    has_sh = inp.get("w1_sh") is not None
    f = _timed(timers, "grouped_ffn", lambda: B.moe_grouped_ffn(
        x, c["offsets"], inp["w1"], inp["w2"], act, b1=inp.get("b1"), x_sh=x if has_sh else None,
        w1_sh=inp.get("w1_sh"), w2_sh=inp.get("w2_sh"), gather_rows=c["sorted_token"], row_w=c["row_w"]))
    out = B.moe_combine_rows(f["y"], c["token_rows"], c["token_nrows"], y_sh=f["y_sh"])
    res = dict(out=out, logits=r["logits"], T=T)
    res.update(c)
    return res


def backward(inp: dict, fwd: dict, grad_out, k: int, score: str, act: str,
             timers: dict | None = None, coef_aux: float = 0.0, coef_z: float = 0.0):
    """Gradients of sum(grad_out * out) + coef_aux * aux + coef_z * z for a
    forward run with keep_for_backward=True (routed experts; no shared
    expert); aux and z are the load-balancing and z-losses of the router's
    logits. With ``timers``, the grouped FFN backward call is bracketed by
    HIP events (key "grouped_ffn_bwd"). A forward with ``capacity`` runs the
    expert stages on its kept dispatch and the router's backward on the full
    one."""
    E = inp["w_gate"].shape[0]
    row_w = fwd.get("row_w")
    d = fwd.get("kept") or fwd        # the dispatch the expert stages used
    if row_w is not None:
        grad_y, _ = B.moe_unpermute_bwd(grad_out, None, d["row_of"], None)
    else:
        grad_y, grad_w = B.moe_unpermute_bwd(grad_out, fwd["y"], d["row_of"], fwd["topk_w"])
    if fwd.get("recompute"):
        g = _timed(timers, "grouped_ffn_bwd", lambda: B.moe_grouped_ffn_bwd_recompute(
            grad_y, d["x_perm"], fwd["gu"], d["offsets"], inp["w1"], inp["w2"], act, row_w=row_w))
    else:
        has_b = inp.get("b1") is not None or inp.get("b2") is not None
        g = _timed(timers, "grouped_ffn_bwd", lambda: B.moe_grouped_ffn_bwd(
            grad_y, d["x_perm"], fwd["act"], fwd["gu"], d["offsets"], inp["w1"], inp["w2"], act,
            want_bias_grads=has_b))
    if row_w is not None:
        grad_w = B.moe_permute_weights_bwd(g["grad_row_w"], d["row_of"])
    r = B.moe_route_bwd(inp["x"], E, fwd["topk_idx"], fwd["topk_w"], grad_w, fwd["offsets"],
                        fwd["sorted_token"], score=score, logits=fwd.get("logits"),
                        want_b_grad=inp.get("b_gate") is not None)
    grad_x = B.moe_permute_bwd(g["grad_x_perm"], d["row_of"], r["grad_logits_sel"],
                               fwd["topk_idx"], inp["w_gate"])
    if coef_aux != 0.0 or coef_z != 0.0:
        if fwd.get("logits") is None:
            raise B.MoeError("the auxiliary losses' backward needs the forward's logits "
                             "(run the forward with router_losses=True)")
        dl = B.moe_router_losses_bwd(fwd["logits"], fwd["counts"], k, coef_aux, coef_z)
        B.moe_router_dense_bwd(inp["x"], inp["w_gate"], dl, grad_w_gate=r["grad_w_gate"],
                               grad_b_gate=r["grad_b_gate"], grad_x=grad_x)
    return dict(grad_x=grad_x, grad_topk_w=grad_w, grad_y=grad_y, grad_w1=g["grad_w1"],
                grad_w2=g["grad_w2"], grad_b1=g.get("grad_b1"), grad_b2=g.get("grad_b2"),
                grad_w_gate=r["grad_w_gate"], grad_b_gate=r["grad_b_gate"],
                grad_logits_sel=r["grad_logits_sel"])


def quantize_experts_mx(inp: dict, for_backward: bool = False) -> dict:
    """MXFP8 codes and scales of the expert weights, each along its reduction
    axis (once per weight update): w1 and w2 along h and F for the forward;
    with ``for_backward`` also along 2F and h, stored transposed (w1t
    [E, h, 2F], w2t [E, F, h]) for the input gradients."""
    w1q, w1s = B.moe_mx_quantize(inp["w1"])
    w2q, w2s = B.moe_mx_quantize(inp["w2"])
    out = dict(w1_codes=w1q, w1_scales=w1s, w2_codes=w2q, w2_scales=w2s)
    if for_backward:
        out["w1t_codes"], out["w1t_scales"] = B.moe_mx_quantize_t(inp["w1"])
        out["w2t_codes"], out["w2t_scales"] = B.moe_mx_quantize_t(inp["w2"])
    return out


def forward_mxfp8(inp: dict, wq: dict, k: int, score: str, timers: dict | None = None,
                  keep_for_backward: bool = False):
    """Forward with the expert GEMMs in MXFP8 ("Scalable Training of
    Mixture-of-Experts Models with Megatron Core", section 5.3.3): the router
    as in ``forward`` (fp32 logits), the token rows quantised along h and
    gathered by the first GEMM, the activation quantised along F in the first
    GEMM's epilogue (from fp32), the weighted combine in fp32. SwiGLU experts
    without bias. The result keeps the token codes (x_codes, x_scales) that
    ``backward_mxfp8`` recomputes the first projection from, and, with
    ``keep_for_backward`` and sigmoid scoring, the logits the router's
    backward needs."""
    x = inp["x"]
    E = inp["w_gate"].shape[0]
    r = B.moe_route(x, inp["w_gate"], k, score, b_gate=inp.get("b_gate"), sel_bias=inp.get("sel_bias"),
                    want_logits=keep_for_backward and score == "sigmoid")
    p = B.moe_permute(x, r["topk_idx"], E, with_x_perm=False)
    xq, xs = B.moe_mx_quantize(x)
    f = _timed(timers, "grouped_ffn", lambda: B.moe_grouped_ffn_mx(
        xq, xs, p["offsets"], wq["w1_codes"], wq["w1_scales"], wq["w2_codes"], wq["w2_scales"],
        gather_rows=p["sorted_token"]))
    out = B.moe_unpermute(f["y"], p["row_of"], r["topk_w"])
    res = dict(out=out, x_codes=xq, x_scales=xs)
    res.update(r)
    res.update(p)
    res.update(f)
    return res


def backward_mxfp8(inp: dict, fwd: dict, wq: dict, grad_out, k: int, score: str, timers: dict | None = None):
    """Gradients of sum(grad_out * out) for a ``forward_mxfp8`` run, the
    expert GEMMs in MXFP8 (``wq`` from quantize_experts_mx(...,
    for_backward=True); the first projection recomputed from the forward's
    codes), the combine, dispatch and router backward as in ``backward``
    (the router keeps fp32, section 5.1). With ``timers``, the expert
    backward call is bracketed by HIP events (key "grouped_ffn_bwd")."""
    E = inp["w_gate"].shape[0]
    _, grad_w = B.moe_unpermute_bwd(grad_out, fwd["y"], fwd["row_of"], fwd["topk_w"])
    row_w = B.moe_permute_weights(fwd["topk_w"], fwd["row_of"])
    g = _timed(timers, "grouped_ffn_bwd", lambda: B.moe_grouped_ffn_bwd_mx(
        grad_out, row_w, inp["x"], fwd["x_codes"], fwd["x_scales"], fwd["sorted_token"], fwd["offsets"],
        wq["w1_codes"], wq["w1_scales"], wq["w1t_codes"], wq["w1t_scales"], wq["w2t_codes"], wq["w2t_scales"]))
    r = B.moe_route_bwd(inp["x"], E, fwd["topk_idx"], fwd["topk_w"], grad_w, fwd["offsets"],
                        fwd["sorted_token"], score=score, logits=fwd.get("logits"),
                        want_b_grad=inp.get("b_gate") is not None)
    grad_x = B.moe_permute_bwd(g["grad_x_perm"], fwd["row_of"], r["grad_logits_sel"], fwd["topk_idx"],
                               inp["w_gate"])
    return dict(grad_x=grad_x, grad_topk_w=grad_w, grad_x_perm=g["grad_x_perm"], grad_w1=g["grad_w1"],
                grad_w2=g["grad_w2"], grad_w_gate=r["grad_w_gate"], grad_b_gate=r["grad_b_gate"],
                grad_logits_sel=r["grad_logits_sel"])


class MoELayerFn(torch.autograd.Function):
    """The layer as a torch autograd function over the C-ABI calls:

        out, losses = MoELayerFn.apply(x, w_gate, w1, w2, b_gate, b1, b2, sel_bias,
                                       k, score, act, router_losses)

    ``out`` [T,h] is the layer output; ``losses`` is the fp32 pair (load-
    balancing loss, router z-loss) of "emerging-techniques-moe-training",
    section 3 when ``router_losses`` is true (then the forward keeps the
    router's logits), else zeros that carry no gradient. The backward runs
    ``backward`` with the upstream gradients of ``losses`` as the loss
    coefficients (read on the host, one synchronisation, only when they
    matter). Optional tensors may be None; ``sel_bias`` (the selection bias)
    gets no gradient. Routed experts only (no shared expert). Weight and bias
    gradients are computed in fp32 and returned in their parameters'
    dtype."""

    @staticmethod
    def forward(ctx, x, w_gate, w1, w2, b_gate, b1, b2, sel_bias, k: int, score: str, act: str,
                router_losses: bool = False):
        inp = dict(x=x.contiguous(), w_gate=w_gate, w1=w1, w2=w2, b_gate=b_gate, b1=b1, b2=b2,
                   sel_bias=sel_bias, w1_sh=None, w2_sh=None)
        f = forward(inp, k, score, act, keep_for_backward=True, router_losses=router_losses)
        ctx.inp, ctx.fwd, ctx.args, ctx.with_losses = inp, f, (k, score, act), router_losses
        losses = f["losses"] if router_losses else torch.zeros(2, dtype=torch.float32, device=x.device)
        if not router_losses:
            ctx.mark_non_differentiable(losses)
        return f["out"], losses

    @staticmethod
    def backward(ctx, grad_out, grad_losses):
        inp, f = ctx.inp, ctx.fwd
        coef_aux = coef_z = 0.0
        if ctx.with_losses and grad_losses is not None:
            coef_aux, coef_z = (float(v) for v in grad_losses.detach().cpu())
        if grad_out is None:
            grad_out = torch.zeros_like(f["out"])
        g = backward(inp, f, grad_out.contiguous(), *ctx.args, coef_aux=coef_aux, coef_z=coef_z)

        def cast(t, like):
            return None if t is None or like is None else t.to(like.dtype)

        return (g["grad_x"], cast(g["grad_w_gate"], inp["w_gate"]), cast(g["grad_w1"], inp["w1"]),
                cast(g["grad_w2"], inp["w2"]), cast(g["grad_b_gate"], inp["b_gate"]),
                cast(g["grad_b1"], inp["b1"]), cast(g["grad_b2"], inp["b2"]), None, None, None, None, None)
