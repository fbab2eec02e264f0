"""Helpers shared by the GPU parity tests: converting seeded inputs for the
oracle and the error measure.

Error measure (the pages only say "max relative error"): for an output with
rows (tokens), the largest of
  * max |got - ref| / max |ref| over the whole tensor, and
  * max over rows t of ||got_t - ref_t||_inf / max(||ref_t||_inf, 1e-6 * max|ref|),
which stays meaningful where single elements of ref are near zero.
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
