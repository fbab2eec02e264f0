"""ctypes binding of libmoe.so: the C entry points under the same names.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, outputs are allocated with torch on the input's device, and the
call goes to the C ABI on torch's current stream. Every step of the layer
runs in the library's HIP kernels; there is no fallback. If the library is
not built, ``load()`` raises.
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

_lib = None
_lock = threading.Lock()

DTYPE = {torch.float32: 0, torch.bfloat16: 1}
SCORE = {"softmax": 0, "sigmoid": 1}
ACT = {"gelu": 0, "swiglu": 1}

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_sz = ctypes.c_size_t

_SIGS = {
    "moe_abi_version": ([], _int),
    "moe_status_string": ([_int], ctypes.c_char_p),
    "moe_last_error": ([], ctypes.c_char_p),
    "moe_route_workspace_size": ([_i64, _int], _sz),
    "moe_route": ([_vp, _int, _i64, _i64, _vp, _vp, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp,
                   _vp, _sz, _vp], _int),
    "moe_permute_workspace_size": ([_i64, _int, _int], _sz),
    "moe_permute": ([_vp, _int, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_permute_noalloc": ([_vp, _int, _i64, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp], _int),
    "moe_grouped_ffn_workspace_size": ([_int], _sz),
    "moe_grouped_ffn": ([_vp, _vp, _i64, _int, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp, _vp, _vp, _vp,
                         _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_unpermute": ([_vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp], _int),
    "moe_unpermute_bwd": ([_vp, _vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp], _int),
    "moe_grouped_ffn_bwd": ([_vp, _vp, _vp, _vp, _int, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp,
                             _vp, _vp, _vp, _vp, _vp, _vp, _vp], _int),
    "moe_route_bwd_workspace_size": ([_i64, _i64, _int, _int], _sz),
    "moe_route_bwd": ([_vp, _int, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                       _vp, _vp, _vp, _sz, _vp], _int),
    "moe_permute_bwd": ([_vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _vp, _int, _vp, _vp], _int),
    "moe_router_losses_workspace_size": ([_i64, _int], _sz),
    "moe_router_losses": ([_vp, _vp, _i64, _int, _int, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_router_losses_bwd": ([_vp, _vp, _i64, _int, _int, ctypes.c_float, ctypes.c_float, _vp, _vp],
                              _int),
    "moe_router_dense_bwd_workspace_size": ([_i64, _i64, _int], _sz),
    "moe_grouped_ffn_weighted": ([_vp, _vp, _i64, _int, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp, _vp,
                                  _vp, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_permute_weights": ([_vp, _i64, _int, _vp, _vp, _vp], _int),
    "moe_permute_weights_bwd": ([_vp, _i64, _int, _vp, _vp, _vp], _int),
    "moe_grouped_ffn_bwd_recompute_workspace_size": ([_i64, _i64, _int], _sz),
    "moe_capacity_drop": ([_vp, _vp, _vp, _vp, _int, _i64, _i64, _int, _int, _int, _vp, _vp, _vp, _vp, _vp],
                          _int),
    "moe_expert_choice_workspace_size": ([_i64, _int], _sz),
    "moe_mx_quantize": ([_vp, _int, _i64, _i64, _vp, _vp, _vp], _int),
    "moe_grouped_ffn_mx_workspace_size": ([_i64, _i64, _i64, _int], _sz),
    "moe_grouped_ffn_mx": ([_vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp, _vp, _vp, _vp,
                            _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_mx_quantize_t": ([_vp, _int, _i64, _i64, _i64, _vp, _vp, _vp], _int),
    "moe_grouped_ffn_bwd_mx_workspace_size": ([_i64, _i64, _i64, _int], _sz),
    "moe_grouped_ffn_bwd_mx": ([_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp,
                                _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_expert_choice": ([_vp, _i64, _int, _int, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_combine_rows": ([_vp, _int, _i64, _i64, _int, _i64, _vp, _vp, _vp, _vp, _vp], _int),
    "moe_grouped_ffn_bwd_recompute": ([_vp, _vp, _vp, _int, _i64, _i64, _i64, _int, _vp, _int, _vp, _vp,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp], _int),
    "moe_router_dense_bwd": ([_vp, _vp, _int, _i64, _i64, _int, _vp, _vp, _vp, _vp, _vp, _sz, _vp],
                             _int),
}


class MoeError(RuntimeError):
    pass


def load(path: Optional[str] = None):
    """Load libmoe.so (built in-tree by build.py); raise if it is absent."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise MoeError("libmoe.so is not built (%s); run "
                           "`python -m mixture_experts_layer_06_amd.build`" % p)
        lib = ctypes.CDLL(p)
        for name, (args, res) in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = res
        _lib = lib
        return lib


def lib():
    return _lib if _lib is not None else load()


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else _vp(t.data_ptr())


def _stream(t: torch.Tensor):
    return _vp(torch.cuda.current_stream(t.device).cuda_stream)


def _check(rc: int, name: str):
    if rc != 0:
        L = lib()
        raise MoeError("%s: %s: %s" % (name, L.moe_status_string(rc).decode(),
                                       L.moe_last_error().decode()))


def _req(t: torch.Tensor, name: str, dtype=None, shape=None, device=None):
    if t is None:
        raise MoeError("%s is required" % name)
    if not t.is_cuda:
        raise MoeError("%s must be a device tensor" % name)
    if device is not None and t.device != device:
        raise MoeError("%s is on %s, expected %s" % (name, t.device, device))
    if not t.is_contiguous():
        raise MoeError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise MoeError("%s has dtype %s, expected %s" % (name, t.dtype, dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise MoeError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    return t


def _opt(t, name, **kw):
    return None if t is None else _req(t, name, **kw)


def abi_version() -> int:
    return lib().moe_abi_version()


# ----------------------------------------------------------------- forward

def moe_route(x, w_gate, k: int, score: str = "softmax", b_gate=None, sel_bias=None,
              want_logits: bool = False, want_map: bool = False, use_workspace: bool = True):
    """Route stage. Without want_logits the library may take its MFMA-filtered
    path (given a workspace); its outputs are bitwise those of the fixed-order
    pass."""
    _req(x, "x")
    dev = x.device
    T, h = x.shape
    E = w_gate.shape[0]
    _req(w_gate, "w_gate", dtype=x.dtype, shape=(E, h), device=dev)
    _opt(b_gate, "b_gate", dtype=torch.float32, shape=(E,), device=dev)
    _opt(sel_bias, "sel_bias", dtype=torch.float32, shape=(E,), device=dev)
    out = dict(
        topk_idx=torch.empty((T, k), dtype=torch.int32, device=dev),
        topk_w=torch.empty((T, k), dtype=torch.float32, device=dev),
        counts=torch.empty((E,), dtype=torch.int32, device=dev),
        logits=torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None,
        routing_map=torch.empty((T, E), dtype=torch.uint8, device=dev) if want_map else None,
    )
    nws = lib().moe_route_workspace_size(T, E) if (use_workspace and not want_logits) else 0
    ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    rc = lib().moe_route(_ptr(x), DTYPE[x.dtype], T, h, _ptr(w_gate), _ptr(b_gate), E, k,
                         SCORE[score], _ptr(sel_bias), _ptr(out["logits"]), _ptr(out["topk_idx"]),
                         _ptr(out["topk_w"]), _ptr(out["routing_map"]), _ptr(out["counts"]),
                         _ptr(ws), nws, _stream(x))
    _check(rc, "moe_route")
    return out


def moe_permute(x, topk_idx, E: int, with_x_perm: bool = True):
    _req(x, "x")
    dev = x.device
    T, h = x.shape
    k = topk_idx.shape[1]
    _req(topk_idx, "topk_idx", dtype=torch.int32, shape=(T, k), device=dev)
    P = T * k
    ws_bytes = lib().moe_permute_workspace_size(T, E, k)
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    out = dict(
        offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
        sorted_token=torch.empty((P,), dtype=torch.int32, device=dev),
        row_of=torch.empty((T, k), dtype=torch.int32, device=dev),
        x_perm=torch.empty((P, h), dtype=x.dtype, device=dev) if with_x_perm else None,
    )
    rc = lib().moe_permute(_ptr(x), DTYPE[x.dtype], T, h, E, k, _ptr(topk_idx), _ptr(out["offsets"]),
                           _ptr(out["sorted_token"]), _ptr(out["row_of"]), _ptr(out["x_perm"]),
                           _ptr(ws), ws.numel(), _stream(x))
    _check(rc, "moe_permute")
    return out


def moe_permute_noalloc(x, topk_idx, E: int, with_x_perm: bool = True, out: dict | None = None):
    """moe_permute with the library's static scratch instead of a workspace.
    ``out`` (optional): preallocated offsets, sorted_token, row_of (and
    x_perm) tensors to write, so that the call itself allocates nothing."""
    _req(x, "x")
    dev = x.device
    T, h = x.shape
    k = topk_idx.shape[1]
    _req(topk_idx, "topk_idx", dtype=torch.int32, shape=(T, k), device=dev)
    P = T * k
    if out is None:
        out = dict(
            offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
            sorted_token=torch.empty((P,), dtype=torch.int32, device=dev),
            row_of=torch.empty((T, k), dtype=torch.int32, device=dev),
            x_perm=torch.empty((P, h), dtype=x.dtype, device=dev) if with_x_perm else None,
        )
    _req(out["offsets"], "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(out["sorted_token"], "sorted_token", dtype=torch.int32, shape=(P,), device=dev)
    _req(out["row_of"], "row_of", dtype=torch.int32, shape=(T, k), device=dev)
    _opt(out.get("x_perm"), "x_perm", dtype=x.dtype, shape=(P, h), device=dev)
    rc = lib().moe_permute_noalloc(_ptr(x), DTYPE[x.dtype], T, h, E, k, _ptr(topk_idx), _ptr(out["offsets"]),
                                   _ptr(out["sorted_token"]), _ptr(out["row_of"]), _ptr(out.get("x_perm")),
                                   _stream(x))
    _check(rc, "moe_permute_noalloc")
    return out


def moe_grouped_ffn(x_perm, offsets, w1, w2, act: str = "swiglu", b1=None, b2=None, x_sh=None,
                    w1_sh=None, w2_sh=None, keep_gu: bool = False, use_workspace: bool = True,
                    workspace=None, gather_rows=None, row_w=None):
    """Grouped expert FFN. With gather_rows (the sorted_token of
    moe_permute), x_perm is the unpermuted x [T,h] and the first GEMM reads
    its rows in permuted order itself. With row_w ([P] fp32, from
    moe_permute_weights) the activation of permuted row r is scaled by
    row_w[r] (moe_grouped_ffn_weighted; no b2)."""
    _req(x_perm, "x_perm")
    dev = x_perm.device
    dt = x_perm.dtype
    x_rows, h = x_perm.shape
    if gather_rows is not None:
        _req(gather_rows, "gather_rows", dtype=torch.int32, device=dev)
        P = gather_rows.numel()
    else:
        P = x_rows
    E = w1.shape[0]
    n1 = 2 if act == "swiglu" else 1
    F = w2.shape[2]
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(w1, "w1", dtype=dt, shape=(E, n1 * F, h), device=dev)
    _req(w2, "w2", dtype=dt, shape=(E, h, F), device=dev)
    _opt(b1, "b1", dtype=dt, shape=(E, n1 * F), device=dev)
    _opt(b2, "b2", dtype=dt, shape=(E, h), device=dev)
    T_sh = 0
    if x_sh is not None:
        T_sh = x_sh.shape[0]
        _req(x_sh, "x_sh", dtype=dt, shape=(T_sh, h), device=dev)
        _req(w1_sh, "w1_sh", dtype=dt, shape=(n1 * F, h), device=dev)
        _req(w2_sh, "w2_sh", dtype=dt, shape=(h, F), device=dev)
    out = dict(
        act=torch.empty((P + T_sh, F), dtype=dt, device=dev),
        gu=torch.empty((P + T_sh, n1 * F), dtype=dt, device=dev) if keep_gu else None,
        y=torch.empty((P, h), dtype=dt, device=dev),
        y_sh=torch.empty((T_sh, h), dtype=dt, device=dev) if T_sh else None,
    )
    if workspace is not None:
        _req(workspace, "workspace", dtype=torch.uint8, device=dev)
        ws, nws = workspace, workspace.numel()
    else:
        nws = lib().moe_grouped_ffn_workspace_size(DTYPE[dt]) if use_workspace else 0
        ws = torch.empty(nws, dtype=torch.uint8, device=dev) if nws else None
    if row_w is not None:
        _req(row_w, "row_w", dtype=torch.float32, shape=(P,), device=dev)
        if b2 is not None:
            raise MoeError("moe_grouped_ffn: row weights need an expert without output bias")
        rc = lib().moe_grouped_ffn_weighted(_ptr(x_perm), _ptr(gather_rows), x_rows, DTYPE[dt], P, h, F,
                                            E, _ptr(offsets), ACT[act], _ptr(w1), _ptr(b1), _ptr(w2),
                                            _ptr(x_sh), T_sh, _ptr(w1_sh), _ptr(w2_sh), _ptr(row_w),
                                            _ptr(out["act"]), _ptr(out["gu"]), _ptr(out["y"]),
                                            _ptr(out["y_sh"]), _ptr(ws), nws, _stream(x_perm))
        _check(rc, "moe_grouped_ffn_weighted")
        return out
    rc = lib().moe_grouped_ffn(_ptr(x_perm), _ptr(gather_rows), x_rows, DTYPE[dt], P, h, F, E,
                               _ptr(offsets), ACT[act],
                               _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(x_sh), T_sh,
                               _ptr(w1_sh), _ptr(w2_sh), _ptr(out["act"]), _ptr(out["gu"]),
                               _ptr(out["y"]), _ptr(out["y_sh"]), _ptr(ws), nws, _stream(x_perm))
    _check(rc, "moe_grouped_ffn")
    return out


def moe_unpermute(y, row_of, topk_w, y_sh=None, out=None):
    """Weighted combine; topk_w None: weights 1 (rows already weighted)."""
    _req(y, "y")
    dev = y.device
    T, k = row_of.shape
    h = y.shape[1]
    _req(row_of, "row_of", dtype=torch.int32, device=dev)
    _opt(topk_w, "topk_w", dtype=torch.float32, shape=(T, k), device=dev)
    _opt(y_sh, "y_sh", dtype=y.dtype, shape=(T, h), device=dev)
    if out is None:
        out = torch.empty((T, h), dtype=y.dtype, device=dev)
    _req(out, "out", dtype=y.dtype, shape=(T, h), device=dev)
    rc = lib().moe_unpermute(_ptr(y), DTYPE[y.dtype], T, h, k, _ptr(row_of), _ptr(topk_w),
                             _ptr(y_sh), _ptr(out), _stream(y))
    _check(rc, "moe_unpermute")
    return out


# ---------------------------------------------------------------- backward

def moe_unpermute_bwd(grad_out, y, row_of, topk_w):
    """(grad_y, grad_topk_w). topk_w None (unweighted combine): y is not
    used, grad_y rows are copies of grad_out and grad_topk_w is None."""
    _req(grad_out, "grad_out")
    dev = grad_out.device
    T, h = grad_out.shape
    k = row_of.shape[1]
    _req(row_of, "row_of", dtype=torch.int32, shape=(T, k), device=dev)
    if topk_w is not None:
        _req(y, "y", dtype=grad_out.dtype, shape=(T * k, h), device=dev)
        _req(topk_w, "topk_w", dtype=torch.float32, shape=(T, k), device=dev)
    else:
        y = None
    grad_y = torch.empty((T * k, h), dtype=grad_out.dtype, device=dev)
    grad_w = torch.empty((T, k), dtype=torch.float32, device=dev) if topk_w is not None else None
    rc = lib().moe_unpermute_bwd(_ptr(grad_out), _ptr(y), DTYPE[grad_out.dtype], T, h, k, _ptr(row_of),
                                 _ptr(topk_w), _ptr(grad_y), _ptr(grad_w), _stream(grad_out))
    _check(rc, "moe_unpermute_bwd")
    return grad_y, grad_w


def moe_grouped_ffn_bwd(grad_y, x_perm, act_out, gu, offsets, w1, w2, act: str = "swiglu",
                        want_bias_grads: bool = False):
    """Expert gradients; with want_bias_grads also grad_b1 [E, n1 F] and
    grad_b2 [E, h] (fp32)."""
    _req(grad_y, "grad_y")
    dev = grad_y.device
    dt = grad_y.dtype
    P, h = grad_y.shape
    E = w1.shape[0]
    F = w2.shape[2]
    n1 = 2 if act == "swiglu" else 1
    _req(x_perm, "x_perm", dtype=dt, shape=(P, h), device=dev)
    _req(act_out, "act", dtype=dt, device=dev)
    _req(gu, "gu", dtype=dt, device=dev)
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(w1, "w1", dtype=dt, shape=(E, n1 * F, h), device=dev)
    _req(w2, "w2", dtype=dt, shape=(E, h, F), device=dev)
    grad_gu = torch.empty((P, n1 * F), dtype=dt, device=dev)
    grad_x_perm = torch.empty((P, h), dtype=dt, device=dev)
    grad_w1 = torch.empty((E, n1 * F, h), dtype=torch.float32, device=dev)
    grad_w2 = torch.empty((E, h, F), dtype=torch.float32, device=dev)
    grad_b1 = torch.empty((E, n1 * F), dtype=torch.float32, device=dev) if want_bias_grads else None
    grad_b2 = torch.empty((E, h), dtype=torch.float32, device=dev) if want_bias_grads else None
    rc = lib().moe_grouped_ffn_bwd(_ptr(grad_y), _ptr(x_perm), _ptr(act_out), _ptr(gu), DTYPE[dt], P,
                                   h, F, E, _ptr(offsets), ACT[act], _ptr(w1), _ptr(w2),
                                   _ptr(grad_gu), _ptr(grad_x_perm), _ptr(grad_w1), _ptr(grad_w2),
                                   _ptr(grad_b1), _ptr(grad_b2), _stream(grad_y))
    _check(rc, "moe_grouped_ffn_bwd")
    return dict(grad_gu=grad_gu, grad_x_perm=grad_x_perm, grad_w1=grad_w1, grad_w2=grad_w2,
                grad_b1=grad_b1, grad_b2=grad_b2)


def moe_grouped_ffn_bwd_recompute(grad_y, x_perm, gu, offsets, w1, w2, act: str = "swiglu",
                                  row_w=None):
    """Grouped FFN backward with the activation rebuilt from gu; with row_w
    (memory-efficient permutation) also grad_row_w [P] = dL/d row_w."""
    _req(grad_y, "grad_y")
    dev = grad_y.device
    dt = grad_y.dtype
    P, h = grad_y.shape
    E = w1.shape[0]
    F = w2.shape[2]
    n1 = 2 if act == "swiglu" else 1
    _req(x_perm, "x_perm", dtype=dt, shape=(P, h), device=dev)
    _req(gu, "gu", dtype=dt, device=dev)
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(w1, "w1", dtype=dt, shape=(E, n1 * F, h), device=dev)
    _req(w2, "w2", dtype=dt, shape=(E, h, F), device=dev)
    _opt(row_w, "row_w", dtype=torch.float32, shape=(P,), device=dev)
    out = dict(grad_gu=torch.empty((P, n1 * F), dtype=dt, device=dev),
               grad_x_perm=torch.empty((P, h), dtype=dt, device=dev),
               grad_w1=torch.empty((E, n1 * F, h), dtype=torch.float32, device=dev),
               grad_w2=torch.empty((E, h, F), dtype=torch.float32, device=dev),
               grad_row_w=torch.empty((P,), dtype=torch.float32, device=dev) if row_w is not None else None)
    nws = lib().moe_grouped_ffn_bwd_recompute_workspace_size(P, F, int(row_w is not None))
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=dev)
    rc = lib().moe_grouped_ffn_bwd_recompute(
        _ptr(grad_y), _ptr(x_perm), _ptr(gu), DTYPE[dt], P, h, F, E, _ptr(offsets), ACT[act], _ptr(w1),
        _ptr(w2), _ptr(row_w), _ptr(out["grad_gu"]), _ptr(out["grad_x_perm"]), _ptr(out["grad_w1"]),
        _ptr(out["grad_w2"]), _ptr(out["grad_row_w"]), _ptr(ws), ws.numel(), _stream(grad_y))
    _check(rc, "moe_grouped_ffn_bwd_recompute")
    return out


def moe_permute_weights(topk_w, row_of):
    """row_w [T*k] fp32 with row_w[row_of[t,j]] = topk_w[t,j]."""
    _req(topk_w, "topk_w", dtype=torch.float32)
    dev = topk_w.device
    T, k = topk_w.shape
    _req(row_of, "row_of", dtype=torch.int32, shape=(T, k), device=dev)
    row_w = torch.empty((T * k,), dtype=torch.float32, device=dev)
    rc = lib().moe_permute_weights(_ptr(topk_w), T, k, _ptr(row_of), _ptr(row_w), _stream(topk_w))
    _check(rc, "moe_permute_weights")
    return row_w


def moe_permute_weights_bwd(grad_row_w, row_of):
    """grad_topk_w [T,k] with grad_topk_w[t,j] = grad_row_w[row_of[t,j]]."""
    _req(grad_row_w, "grad_row_w", dtype=torch.float32)
    dev = grad_row_w.device
    T, k = row_of.shape
    _req(row_of, "row_of", dtype=torch.int32, shape=(T, k), device=dev)
    _req(grad_row_w, "grad_row_w", dtype=torch.float32, shape=(T * k,), device=dev)
    g = torch.empty((T, k), dtype=torch.float32, device=dev)
    rc = lib().moe_permute_weights_bwd(_ptr(grad_row_w), T, k, _ptr(row_of), _ptr(g), _stream(grad_row_w))
    _check(rc, "moe_permute_weights_bwd")
    return g


def moe_route_bwd(x, E: int, topk_idx, topk_w, grad_topk_w, offsets, sorted_token,
                  score: str = "softmax", logits=None, want_b_grad: bool = False):
    _req(x, "x")
    dev = x.device
    T, h = x.shape
    k = topk_idx.shape[1]
    _req(topk_idx, "topk_idx", dtype=torch.int32, shape=(T, k), device=dev)
    _req(topk_w, "topk_w", dtype=torch.float32, shape=(T, k), device=dev)
    _req(grad_topk_w, "grad_topk_w", dtype=torch.float32, shape=(T, k), device=dev)
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(sorted_token, "sorted_token", dtype=torch.int32, shape=(T * k,), device=dev)
    _opt(logits, "logits", dtype=torch.float32, shape=(T, E), device=dev)
    ws_bytes = lib().moe_route_bwd_workspace_size(T, h, E, k)
    ws = torch.empty((max(ws_bytes, 16),), dtype=torch.uint8, device=dev)
    out = dict(
        grad_logits_sel=torch.empty((T, k), dtype=torch.float32, device=dev),
        grad_w_gate=torch.empty((E, h), dtype=torch.float32, device=dev),
        grad_b_gate=torch.empty((E,), dtype=torch.float32, device=dev) if want_b_grad else None,
    )
    rc = lib().moe_route_bwd(_ptr(x), DTYPE[x.dtype], T, h, E, k, SCORE[score], _ptr(logits),
                             _ptr(topk_idx), _ptr(topk_w), _ptr(grad_topk_w), _ptr(offsets),
                             _ptr(sorted_token), _ptr(out["grad_logits_sel"]),
                             _ptr(out["grad_w_gate"]), _ptr(out["grad_b_gate"]), _ptr(ws),
                             ws.numel(), _stream(x))
    _check(rc, "moe_route_bwd")
    return out


def moe_permute_bwd(grad_x_perm, row_of, grad_logits_sel=None, topk_idx=None, w_gate=None):
    _req(grad_x_perm, "grad_x_perm")
    dev = grad_x_perm.device
    T, k = row_of.shape
    h = grad_x_perm.shape[1]
    _req(row_of, "row_of", dtype=torch.int32, device=dev)
    E = 0
    if grad_logits_sel is not None:
        _req(grad_logits_sel, "grad_logits_sel", dtype=torch.float32, shape=(T, k), device=dev)
        _req(topk_idx, "topk_idx", dtype=torch.int32, shape=(T, k), device=dev)
        _req(w_gate, "w_gate", dtype=grad_x_perm.dtype, device=dev)
        E = w_gate.shape[0]
    grad_x = torch.empty((T, h), dtype=grad_x_perm.dtype, device=dev)
    rc = lib().moe_permute_bwd(_ptr(grad_x_perm), DTYPE[grad_x_perm.dtype], T, h, k, _ptr(row_of),
                               _ptr(grad_logits_sel), _ptr(topk_idx), _ptr(w_gate), E,
                               _ptr(grad_x), _stream(grad_x_perm))
    _check(rc, "moe_permute_bwd")
    return grad_x


# ------------------------------------------------- auxiliary router losses

def moe_router_losses(logits, counts, k: int, want_probs_mean: bool = False):
    """(losses [2] fp32 = {aux, z}, probs_mean [E] or None) on the device."""
    _req(logits, "logits", dtype=torch.float32)
    dev = logits.device
    T, E = logits.shape
    _req(counts, "counts", dtype=torch.int32, shape=(E,), device=dev)
    losses = torch.empty((2,), dtype=torch.float32, device=dev)
    pmean = torch.empty((E,), dtype=torch.float32, device=dev) if want_probs_mean else None
    nws = lib().moe_router_losses_workspace_size(T, E)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=dev)
    rc = lib().moe_router_losses(_ptr(logits), _ptr(counts), T, E, k, _ptr(losses), _ptr(pmean),
                                 _ptr(ws), ws.numel(), _stream(logits))
    _check(rc, "moe_router_losses")
    return losses, pmean


def moe_router_losses_bwd(logits, counts, k: int, coef_aux: float, coef_z: float):
    """Dense d(coef_aux * aux + coef_z * z)/d logits, [T,E] fp32."""
    _req(logits, "logits", dtype=torch.float32)
    dev = logits.device
    T, E = logits.shape
    _req(counts, "counts", dtype=torch.int32, shape=(E,), device=dev)
    grad = torch.empty((T, E), dtype=torch.float32, device=dev)
    rc = lib().moe_router_losses_bwd(_ptr(logits), _ptr(counts), T, E, k, float(coef_aux),
                                     float(coef_z), _ptr(grad), _stream(logits))
    _check(rc, "moe_router_losses_bwd")
    return grad


def moe_router_dense_bwd(x, w_gate, grad_logits, grad_w_gate=None, grad_b_gate=None, grad_x=None):
    """Accumulate a dense logit gradient into the router's gradients in place:
    grad_w_gate += D^T x, grad_b_gate += sum_t D, grad_x += D w_gate (each
    skipped when None)."""
    _req(x, "x")
    dev = x.device
    T, h = x.shape
    E = w_gate.shape[0]
    _req(w_gate, "w_gate", dtype=x.dtype, shape=(E, h), device=dev)
    _req(grad_logits, "grad_logits", dtype=torch.float32, shape=(T, E), device=dev)
    _opt(grad_w_gate, "grad_w_gate", dtype=torch.float32, shape=(E, h), device=dev)
    _opt(grad_b_gate, "grad_b_gate", dtype=torch.float32, shape=(E,), device=dev)
    _opt(grad_x, "grad_x", dtype=x.dtype, shape=(T, h), device=dev)
    nws = lib().moe_router_dense_bwd_workspace_size(T, h, E)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=dev)
    rc = lib().moe_router_dense_bwd(_ptr(x), _ptr(w_gate), DTYPE[x.dtype], T, h, E, _ptr(grad_logits),
                                    _ptr(grad_w_gate), _ptr(grad_b_gate), _ptr(grad_x), _ptr(ws),
                                    ws.numel(), _stream(x))
    _check(rc, "moe_router_dense_bwd")



# -------------------------------------------------------- routing variants

def moe_capacity_drop(topk_idx, offsets, row_of, capacity: int, x=None, with_x_perm: bool = False):
    """Capacity-limited permutation from moe_permute's outputs: offsets_kept,
    row_of_kept (-1 = dropped), sorted_token_kept and optionally x_perm_kept."""
    _req(topk_idx, "topk_idx", dtype=torch.int32)
    dev = topk_idx.device
    T, k = topk_idx.shape
    E = offsets.numel() - 1
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(row_of, "row_of", dtype=torch.int32, shape=(T, k), device=dev)
    h, dt = 64, torch.bfloat16
    if with_x_perm:
        _req(x, "x", shape=(T, x.shape[1]), device=dev)
        h, dt = x.shape[1], x.dtype
    out = dict(offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
               row_of=torch.empty((T, k), dtype=torch.int32, device=dev),
               sorted_token=torch.empty((T * k,), dtype=torch.int32, device=dev),
               x_perm=torch.empty((T * k, h), dtype=dt, device=dev) if with_x_perm else None)
    rc = lib().moe_capacity_drop(_ptr(topk_idx), _ptr(offsets), _ptr(row_of), _ptr(x if with_x_perm else None),
                                 DTYPE[dt], T, h, E, k, int(capacity), _ptr(out["offsets"]), _ptr(out["row_of"]),
                                 _ptr(out["sorted_token"]), _ptr(out["x_perm"]), _stream(topk_idx))
    _check(rc, "moe_capacity_drop")
    return out


def moe_expert_choice(logits, capacity: int):
    """Expert-choice selection from router logits [T,E] fp32."""
    _req(logits, "logits", dtype=torch.float32)
    dev = logits.device
    T, E = logits.shape
    C = int(capacity)
    out = dict(offsets=torch.empty((E + 1,), dtype=torch.int32, device=dev),
               sorted_token=torch.empty((E * C,), dtype=torch.int32, device=dev),
               row_w=torch.empty((E * C,), dtype=torch.float32, device=dev),
               token_rows=torch.empty((T, E), dtype=torch.int32, device=dev),
               token_nrows=torch.empty((T,), dtype=torch.int32, device=dev))
    nws = lib().moe_expert_choice_workspace_size(T, E)
    ws = torch.empty((max(nws, 16),), dtype=torch.uint8, device=dev)
    rc = lib().moe_expert_choice(_ptr(logits), T, E, C, _ptr(out["offsets"]), _ptr(out["sorted_token"]),
                                 _ptr(out["row_w"]), _ptr(out["token_rows"]), _ptr(out["token_nrows"]), _ptr(ws),
                                 ws.numel(), _stream(logits))
    _check(rc, "moe_expert_choice")
    return out


def moe_combine_rows(y, token_rows, token_nrows, y_sh=None):
    _req(y, "y")
    dev = y.device
    P, h = y.shape
    T, E = token_rows.shape
    _req(token_rows, "token_rows", dtype=torch.int32, device=dev)
    _req(token_nrows, "token_nrows", dtype=torch.int32, shape=(T,), device=dev)
    _opt(y_sh, "y_sh", dtype=y.dtype, shape=(T, h), device=dev)
    out = torch.empty((T, h), dtype=y.dtype, device=dev)
    rc = lib().moe_combine_rows(_ptr(y), DTYPE[y.dtype], T, h, E, P, _ptr(token_rows), _ptr(token_nrows),
                                _ptr(y_sh), _ptr(out), _stream(y))
    _check(rc, "moe_combine_rows")
    return out



# ------------------------------------------------------------------ MXFP8

def moe_mx_quantize(src):
    """(codes uint8 [..., K], scales uint8 [..., K/32]) of src (bf16/fp32),
    quantised along its last axis."""
    _req(src, "src")
    dev = src.device
    K = src.shape[-1]
    rows = src.numel() // K if K else 0
    codes = torch.empty(src.shape, dtype=torch.uint8, device=dev)
    scales = torch.empty(tuple(src.shape[:-1]) + (K // 32,), dtype=torch.uint8, device=dev)
    rc = lib().moe_mx_quantize(_ptr(src), DTYPE[src.dtype], rows, K, _ptr(codes), _ptr(scales), _stream(src))
    _check(rc, "moe_mx_quantize")
    return codes, scales


def moe_grouped_ffn_mx(x_codes, x_scales, offsets, w1_codes, w1_scales, w2_codes, w2_scales,
                       gather_rows=None, act: str = "swiglu", split: bool = True, want_act: bool = False):
    """The grouped SwiGLU FFN in MXFP8. ``split``: pass a workspace, so that
    the second projection may split its last round of tiles along F.
    ``want_act``: also return the bf16 activation (the codes and scales of
    the activation are always returned)."""
    _req(x_codes, "x_codes", dtype=torch.uint8)
    dev = x_codes.device
    x_rows, h = x_codes.shape
    P = gather_rows.numel() if gather_rows is not None else x_rows
    E = w1_codes.shape[0]
    F = w2_codes.shape[2]
    _req(x_scales, "x_scales", dtype=torch.uint8, shape=(x_rows, h // 32), device=dev)
    _opt(gather_rows, "gather_rows", dtype=torch.int32, device=dev)
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(w1_codes, "w1_codes", dtype=torch.uint8, shape=(E, 2 * F, h), device=dev)
    _req(w1_scales, "w1_scales", dtype=torch.uint8, shape=(E, 2 * F, h // 32), device=dev)
    _req(w2_codes, "w2_codes", dtype=torch.uint8, shape=(E, h, F), device=dev)
    _req(w2_scales, "w2_scales", dtype=torch.uint8, shape=(E, h, F // 32), device=dev)
    out = dict(act=torch.empty((P, F), dtype=torch.bfloat16, device=dev) if want_act else None,
               act_codes=torch.empty((P, F), dtype=torch.uint8, device=dev),
               act_scales=torch.empty((P, F // 32), dtype=torch.uint8, device=dev),
               y=torch.empty((P, h), dtype=torch.bfloat16, device=dev))
    nws = lib().moe_grouped_ffn_mx_workspace_size(P, h, F, E) if split else 0
    ws = torch.empty((nws,), dtype=torch.uint8, device=dev) if nws else None
    rc = lib().moe_grouped_ffn_mx(_ptr(x_codes), _ptr(x_scales), _ptr(gather_rows), x_rows, P, h, F, E,
                                  _ptr(offsets), ACT[act], _ptr(w1_codes), _ptr(w1_scales), _ptr(w2_codes),
                                  _ptr(w2_scales), _ptr(out["act"]), _ptr(out["act_codes"]),
                                  _ptr(out["act_scales"]), _ptr(out["y"]), _ptr(ws), nws, _stream(x_codes))
    _check(rc, "moe_grouped_ffn_mx")
    return out


def moe_mx_quantize_t(src):
    """(codes uint8 [B, C, R], scales uint8 [B, C, R/32]) of src [B, R, C]
    (bf16/fp32): each matrix quantised along R (its columns) and stored
    transposed."""
    _req(src, "src")
    if src.dim() != 3:
        raise MoeError("moe_mx_quantize_t: src must be [B, R, C]")
    Bn, R, C = src.shape
    dev = src.device
    codes = torch.empty((Bn, C, R), dtype=torch.uint8, device=dev)
    scales = torch.empty((Bn, C, R // 32), dtype=torch.uint8, device=dev)
    rc = lib().moe_mx_quantize_t(_ptr(src), DTYPE[src.dtype], Bn, R, C, _ptr(codes), _ptr(scales), _stream(src))
    _check(rc, "moe_mx_quantize_t")
    return codes, scales


def moe_grouped_ffn_bwd_mx(grad_out, row_w, x, x_codes, x_scales, sorted_token, offsets, w1_codes, w1_scales,
                           w1t_codes, w1t_scales, w2t_codes, w2t_scales, act: str = "swiglu", workspace=None):
    """Expert gradients with every GEMM in MXFP8 (the first projection
    recomputed from the forward's codes): grad_x_perm [P, h] bf16, grad_w1
    [E, 2F, h] and grad_w2 [E, h, F] fp32. grad_out [T, h] and x [T, h]
    unpermuted (rows gathered by sorted_token), row_w [P] the routing weight
    of each permuted row. ``workspace``: a uint8 device tensor of at least
    moe_grouped_ffn_bwd_mx_workspace_size bytes to use (else one is
    allocated)."""
    _req(grad_out, "grad_out", dtype=torch.bfloat16)
    dev = grad_out.device
    T, h = grad_out.shape
    P = sorted_token.numel()
    E, F2, _ = w1_codes.shape
    F = F2 // 2
    _req(row_w, "row_w", dtype=torch.float32, shape=(P,), device=dev)
    _req(x, "x", dtype=torch.bfloat16, shape=(T, h), device=dev)
    _req(x_codes, "x_codes", dtype=torch.uint8, shape=(T, h), device=dev)
    _req(x_scales, "x_scales", dtype=torch.uint8, shape=(T, h // 32), device=dev)
    _req(sorted_token, "sorted_token", dtype=torch.int32, shape=(P,), device=dev)
    _req(offsets, "offsets", dtype=torch.int32, shape=(E + 1,), device=dev)
    _req(w1_codes, "w1_codes", dtype=torch.uint8, shape=(E, 2 * F, h), device=dev)
    _req(w1_scales, "w1_scales", dtype=torch.uint8, shape=(E, 2 * F, h // 32), device=dev)
    _req(w1t_codes, "w1t_codes", dtype=torch.uint8, shape=(E, h, 2 * F), device=dev)
    _req(w1t_scales, "w1t_scales", dtype=torch.uint8, shape=(E, h, 2 * F // 32), device=dev)
    _req(w2t_codes, "w2t_codes", dtype=torch.uint8, shape=(E, F, h), device=dev)
    _req(w2t_scales, "w2t_scales", dtype=torch.uint8, shape=(E, F, h // 32), device=dev)
    out = dict(grad_x_perm=torch.empty((P, h), dtype=torch.bfloat16, device=dev),
               grad_w1=torch.empty((E, 2 * F, h), dtype=torch.float32, device=dev),
               grad_w2=torch.empty((E, h, F), dtype=torch.float32, device=dev))
    nws = lib().moe_grouped_ffn_bwd_mx_workspace_size(P, h, F, E)
    if workspace is None:
        ws = torch.empty((nws,), dtype=torch.uint8, device=dev)
    else:
        _req(workspace, "workspace", dtype=torch.uint8, device=dev)
        if workspace.numel() < nws:
            raise MoeError("moe_grouped_ffn_bwd_mx: workspace smaller than %d bytes" % nws)
        ws, nws = workspace, workspace.numel()
    rc = lib().moe_grouped_ffn_bwd_mx(_ptr(grad_out), _ptr(row_w), _ptr(x), _ptr(x_codes), _ptr(x_scales),
                                      _ptr(sorted_token), T, P, h, F, E, _ptr(offsets), ACT[act], _ptr(w1_codes),
                                      _ptr(w1_scales), _ptr(w1t_codes), _ptr(w1t_scales), _ptr(w2t_codes),
                                      _ptr(w2t_scales), _ptr(out["grad_x_perm"]), _ptr(out["grad_w1"]),
                                      _ptr(out["grad_w2"]), _ptr(ws), nws, _stream(grad_out))
    _check(rc, "moe_grouped_ffn_bwd_mx")
    return out
