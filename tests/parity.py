"""Helpers shared by the GPU parity tests: converting seeded inputs for the
oracle and the error measure.

Error measure (the pages only say "max relative error"): for an output with
rows (tokens), the largest of
  * max |got - ref| / max |ref| over the whole tensor, and
  * max over rows t of ||got_t - ref_t||_inf / max(||ref_t||_inf, 1e-6 * max|ref|),
which stays meaningful where single elements of ref are near zero.

Weight gradients are sums over an expert's tokens; their rows can cancel to
near zero, so their row-wise measure is taken against the row's sum of
absolute terms (``rel_err_terms``): the error a correct fp32/bf16 kernel
makes on a sum is bounded by a multiple of that sum, not of its result.
"""
import numpy as np
import torch

TOL = {"bf16": 2e-2, "f32": 1e-4}


def to_np32(t):
    """Exact fp32 copy of a (bf16 or fp32) tensor on any device."""
    if t is None:
        return None
    return t.detach().to("cpu").float().numpy()


def rel_err(got, ref) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    if got.ndim == 1:
        got, ref = got[None], ref[None]
    got = got.reshape(got.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    d = np.abs(got - ref)
    amax = np.abs(ref).max()
    if amax == 0:
        return float(d.max())
    whole = d.max() / amax
    rows = d.max(axis=1) / np.maximum(np.abs(ref).max(axis=1), 1e-6 * amax)
    return float(max(whole, rows.max()))


def rel_err_tensor(got, ref) -> float:
    """max |got - ref| / max |ref| over the whole tensor."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    amax = np.abs(ref).max() if ref.size else 0.0
    d = np.abs(got - ref).max() if ref.size else 0.0
    return float(d / amax) if amax > 0 else float(d)


def oracle_inputs(inp: dict) -> dict:
    """numpy fp32 views of the seeded tensors, named as the oracle's arguments."""
    return dict(x=to_np32(inp["x"]), w_gate=to_np32(inp["w_gate"]),
                b_gate=to_np32(inp.get("b_gate")), sel_bias=to_np32(inp.get("sel_bias")),
                w1=to_np32(inp.get("w1")), w2=to_np32(inp.get("w2")),
                b1=to_np32(inp.get("b1")), b2=to_np32(inp.get("b2")),
                w1_sh=to_np32(inp.get("w1_sh")), w2_sh=to_np32(inp.get("w2_sh")))


def to_device(inp: dict, device="cuda") -> dict:
    return {k: (v.to(device) if isinstance(v, torch.Tensor) else v) for k, v in inp.items()}


def rel_err_terms(got, ref, terms) -> float:
    """max over rows f of max_i |got - ref|[f, i] / max_i terms[f, i], where
    terms[f, i] = sum over the summed index of |the products| (for a weight
    gradient dW = sum_t a_t^T b_t: |a|^T |b|)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    terms = np.asarray(terms, dtype=np.float64)
    assert got.shape == ref.shape == terms.shape
    d = np.abs(got - ref).max(axis=1)
    t = terms.max(axis=1)
    floor = 1e-30 + 1e-9 * t.max()
    return float((d / np.maximum(t, floor)).max())


def expert_grad_terms(oracle, x_rows, w1e, w2e, act, dy):
    """Sums of absolute terms of an expert's weight gradients over its rows
    (x_rows [m,h], dy [m,h] = routing weight times dL/dout): |dgu|^T |x| for
    dW1 and |dy|^T |act| for dW2, from the oracle's own expert backward."""
    gb = oracle.expert_backward(x_rows, w1e, w2e, act, dy)
    x64 = np.abs(np.asarray(x_rows, dtype=np.float64))
    return np.abs(gb["dgu"]).T @ x64, np.abs(dy).T @ np.abs(gb["hid"])


def mfma_gamma(K):
    """Relative error bound (times sum |products|) of an fp32 dot product of
    K exact products summed by the scaled fp8 MFMA. How one instruction adds
    its 64 products is not specified (order, internal width, rounding or
    truncation), so the bound is the classical one for any order: every
    product added with its own error of at most 2u (u = 2^-24; truncation as
    well as rounding), plus the K/64 accumulations into C and a margin of 8.
    A tighter model, (K/64 + 8) roundings per element, was measured to be
    exceeded by up to 3.75 times on the device."""
    return (K + K / 64 + 8) * 2.0 ** -23
