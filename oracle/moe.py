"""CPU oracle for one sparse MoE layer: forward (Route, Dispatch, Expert
computation, Combine) and backward.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import or call anything under
``oracle/``. The HIP library never links, loads or calls it, and this module
never imports the HIP package: the two share no code. Inputs come from the
seeded generators (``workloads``) as numpy arrays.

Precision: the router runs in fp32 with a fixed summation order ("Scalable
Training of Mixture-of-Experts Models with Megatron Core", section 5.1 keeps
the router in FP32; the order itself is spelled out in ``gate.c``). Every
other floating-point step runs in fp64, so the oracle is the exact result of
the definitions up to fp64 rounding.

Definitions followed (page titles are the pages' own):

* Router, "Scalable Training ... with Megatron Core", section 2.2: logits
  l = W_r^T x; softmax scores p_i = e^{l_i} / sum_j e^{l_j} or sigmoid scores;
  top-k selection. "emerging-techniques-moe-training", Quick Start and the
  Mixtral block: softmax over all experts, torch.topk, then division by the
  sum of the k selected scores.
* Selection ties, silent on the pages: the total order is (key descending,
  expert index ascending); -0 and +0 are equal; a NaN key ranks as -inf.
* Sigmoid scoring (DeepSeek-V3, section 2.2): the printed normaliser sums over
  all experts; the workload normalises over the selected experts, which is
  the reading taken. The aux-loss-free bias (same section) enters only the
  selection key sigma(l) + bias, never the weights.
* Dispatch, section 2.1 stage 2: tokens regrouped into expert-contiguous
  order. Within an expert the order is ascending token index (the pages give
  none; ascending is the plainest reading of "restore the original order" in
  stage 4).
* Expert computation, section 2.1 stage 3. GELU expert: Linear + GELU(erf) +
  Linear with biases ("emerging-techniques-moe-training", Quick Start).
  SwiGLU expert without bias: three matrices, gate and up then down ("Mixture
  -of-Experts from Architecture to Large-Scale Training", section 2.5; the
  formula itself is lost in the extracted page, the standard
  silu(x W_g^T) * (x W_u^T) W_d^T is used).
* Combine, section 2.1 stage 4 and section 1.1's MoE(x) = sum_{i in TopK}
  p_i E_i(x): out[t] = sum_j w[t,j] y_{e_j}(x_t), plus the shared expert's
  output with weight 1 (the shared expert is named in the handbook page's
  introduction; its weight is not given, 1 is taken).
* Auxiliary router losses ("emerging-techniques-moe-training", section 3
  Load Balancing): the load-balancing loss E * sum_e f_e P_e, with f_e the
  share of the T*k routing slots that chose expert e and P_e the mean over
  tokens of the softmax over all E logits, and the router z-loss, the mean
  over tokens of logsumexp(l)^2. Readings: both read the router's raw logits
  (gate bias included, aux-loss-free selection bias excluded) whatever the
  scoring function; f_e counts the selection actually made, a piecewise
  constant function of the logits, so it carries no gradient; an empty batch
  (T = 0) gives 0 for both.

* Capacity and token dropping ("emerging-techniques-moe-training", Capacity
  Factor Tuning and the DeepSpeed config): capacity = int(T*k/E * factor),
  at least min_capacity; pairs past an expert's capacity, in ascending token
  order, are dropped and the kept pairs keep their weights (the pages say
  neither which pairs go nor whether weights are renormalised).
* Expert-choice routing (same page, Routing Mechanisms): each expert takes
  the `capacity` tokens with the largest logits (ties: lower token index);
  a chosen pair is weighted by the token's softmax gate probability.

* MXFP8 ("Scalable Training ... with Megatron Core", section 5.3.3: 1 x 32
  blocks, E8M0 scales; E4M3 elements as in the page's FP8 recipes). The
  page does not say how a block's scale is chosen: the shared exponent is
  floor(log2(max |v|)) - 8, so the largest element lands in [256, 512) and
  is rounded to nearest-even on the E4M3 grid with saturation at 448.
  Training in MXFP8 (same page, sections 5.1 and 5.3.3; 5.4 for the
  alignment to 32): the pages say only that the expert GEMMs run in low
  precision while the router keeps fp32. The reading taken: every expert
  GEMM, forward and backward, takes both operands in MXFP8 with the 1 x 32
  blocks along that GEMM's own reduction axis. The input gradients then use
  dY blocked along h against W2 blocked along h (column-wise), and the
  gradient of the pre-activations blocked along 2F against W1 blocked along
  2F; the weight gradients reduce over an expert's tokens, so both of their
  operands are blocked along the tokens, each expert's segment on its own
  from its first row, its last block padded with zero rows (the pages pad
  the routing map to a multiple of 32 rather than the tokens; zero rows are
  that padding). The SwiGLU backward itself runs in fp64 on the forward's
  exact pre-activations.

Parity status: every function here is pinned by tests/test_oracle_*.py
against closed forms, invariants, brute force and finite differences; the
absolute output values of the four model-shaped workloads rest on those pins
(the pages print no worked example).
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle_gate.so")
_lib = None
_lib_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile gate.c into liboracle_gate.so with gcc (no GPU toolchain)."""
    src = os.path.join(_HERE, "gate.c")
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-march=x86-64-v3", "-ffp-contract=off", "-fno-fast-math",
           "-fopenmp", "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            fp = ctypes.POINTER(ctypes.c_float)
            lib.oracle_gate_logits.argtypes = [fp, fp, fp, ctypes.c_long, ctypes.c_long,
                                               ctypes.c_long, fp]
            lib.oracle_gate_logits.restype = None
            lib.oracle_exp_c.argtypes = [ctypes.c_double]
            lib.oracle_exp_c.restype = ctypes.c_double
            lib.oracle_sigmoid_c.argtypes = [ctypes.c_float]
            lib.oracle_sigmoid_c.restype = ctypes.c_float
            lib.oracle_sigmoid_c_array.argtypes = [fp, ctypes.c_long, fp]
            lib.oracle_sigmoid_c_array.restype = None
            lib.oracle_sigmoid_c_sweep.argtypes = [
                ctypes.c_float, ctypes.c_float, ctypes.POINTER(ctypes.c_double),
                ctypes.POINTER(ctypes.c_long), ctypes.POINTER(ctypes.c_long)]
            lib.oracle_sigmoid_c_sweep.restype = None
            _lib = lib
    return _lib


def _fptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


# --------------------------------------------------------------------- router

def gate_logits(x: np.ndarray, w_gate: np.ndarray, b_gate=None) -> np.ndarray:
    """fp32 router logits in gate order G (see gate.c). x[T,h], w_gate[E,h]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    w = np.ascontiguousarray(w_gate, dtype=np.float32)
    T, h = x.shape
    E = w.shape[0]
    assert w.shape[1] == h
    out = np.empty((T, E), dtype=np.float32)
    b = None
    if b_gate is not None:
        b = np.ascontiguousarray(b_gate, dtype=np.float32)
    _load().oracle_gate_logits(_fptr(x), _fptr(w), _fptr(b) if b is not None else None,
                               T, h, E, _fptr(out))
    return out


def exp_c(y: float) -> float:
    """The fp64 exponential used inside sigma_c (gate.c)."""
    return float(_load().oracle_exp_c(float(y)))


def sigmoid_c(l: np.ndarray) -> np.ndarray:
    """Canonical fp32 sigmoid (gate.c), elementwise."""
    l = np.ascontiguousarray(l, dtype=np.float32)
    out = np.empty_like(l)
    _load().oracle_sigmoid_c_array(_fptr(l), l.size, _fptr(out))
    return out


def sigmoid_c_sweep(lo: float, hi: float):
    mu = ctypes.c_double()
    nd = ctypes.c_long()
    nc = ctypes.c_long()
    _load().oracle_sigmoid_c_sweep(lo, hi, ctypes.byref(mu), ctypes.byref(nd), ctypes.byref(nc))
    return mu.value, nd.value, nc.value


def selection_key(logits: np.ndarray, score: str, sel_bias=None) -> np.ndarray:
    """fp32 key the top-k ranks on.

    Softmax: the logit itself. Softmax is strictly increasing in each logit, so
    ranking logits ranks the probabilities the pages select on, and equal
    logits give equal probabilities. Sigmoid: sigma_c(l) + bias (fp32 add).
    """
    logits = np.asarray(logits, dtype=np.float32)
    if score == "softmax":
        key = logits.copy()
    elif score == "sigmoid":
        key = sigmoid_c(logits)
        if sel_bias is not None:
            key = (key + np.asarray(sel_bias, dtype=np.float32)[None, :]).astype(np.float32)
    else:
        raise ValueError(score)
    key = np.where(np.isnan(key), np.float32(-np.inf), key).astype(np.float32)
    key = key + np.float32(0.0)   # -0 -> +0
    return key


def select_topk(key: np.ndarray, k: int) -> np.ndarray:
    """First k experts of each row in the order (key desc, index asc)."""
    T, E = key.shape
    idx = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((idx, -key.astype(np.float64)), axis=-1)
    return order[:, :k].astype(np.int32)


def routing_weights(logits_sel: np.ndarray, logits_all: np.ndarray, score: str) -> np.ndarray:
    """fp64 weights of the k selected experts (rows of logits_sel).

    softmax: p = softmax over all E logits, then p_sel / sum(p_sel).
    sigmoid: s = sigma(l) of the selected logits, then s / sum(s).
    """
    ls = logits_sel.astype(np.float64)
    if score == "softmax":
        la = logits_all.astype(np.float64)
        m = la.max(axis=1, keepdims=True)
        z = np.exp(la - m).sum(axis=1, keepdims=True)
        p_sel = np.exp(ls - m) / z
        return p_sel / p_sel.sum(axis=1, keepdims=True)
    s = 1.0 / (1.0 + np.exp(-ls))
    return s / s.sum(axis=1, keepdims=True)


def route(x, w_gate, k: int, score: str = "softmax", b_gate=None, sel_bias=None,
          logits=None):
    """Router stage. Returns logits (fp32), key (fp32), topk_idx [T,k] int32,
    topk_w [T,k] fp64, routing_map [T,E] uint8, counts [E] int64."""
    if logits is None:
        logits = gate_logits(x, w_gate, b_gate)
    T, E = logits.shape
    key = selection_key(logits, score, sel_bias)
    topk_idx = select_topk(key, k)
    sel_logits = np.take_along_axis(logits, topk_idx.astype(np.int64), axis=1)
    topk_w = routing_weights(sel_logits, logits, score)
    routing_map = np.zeros((T, E), dtype=np.uint8)
    np.put_along_axis(routing_map, topk_idx.astype(np.int64), 1, axis=1)
    counts = routing_map.sum(axis=0).astype(np.int64)
    return dict(logits=logits, key=key, topk_idx=topk_idx, topk_w=topk_w,
                routing_map=routing_map, counts=counts)


# ------------------------------------------------------------------ dispatch

def permutation(topk_idx: np.ndarray, E: int):
    """Expert-contiguous order of the (token, expert) pairs.

    Pairs are listed expert by expert; inside an expert, tokens ascend. Returns
    offsets [E+1] (exclusive prefix of the counts), sorted_token [T*k] (the
    token of each permuted row) and row_of [T,k] (the permuted row of pair
    (t, topk_idx[t,j])).
    """
    T, k = topk_idx.shape
    routing_map = np.zeros((T, E), dtype=bool)
    np.put_along_axis(routing_map, topk_idx.astype(np.int64), True, axis=1)
    e_of_row, t_of_row = np.nonzero(routing_map.T)     # row-major over (e, t)
    counts = routing_map.sum(axis=0)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    row_index = np.full((E, T), -1, dtype=np.int64)
    row_index[e_of_row, t_of_row] = np.arange(e_of_row.size)
    row_of = row_index[topk_idx.astype(np.int64), np.arange(T)[:, None]]
    return dict(offsets=offsets, sorted_token=t_of_row.astype(np.int64),
                row_of=row_of, counts=counts.astype(np.int64))


# ------------------------------------------------------------------- experts

def silu(a):
    return a / (1.0 + np.exp(-a))


def gelu_erf(a):
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * a * (1.0 + erf(a / math.sqrt(2.0)))


def expert_forward(xe, w1e, w2e, act: str, b1e=None, b2e=None):
    """One expert on the rows xe [m,h] in fp64. w1e [n1*F,h] (SwiGLU: gate rows
    then up rows), w2e [h,F]. Returns y [m,h] and the cached pre-activations."""
    xe = np.asarray(xe, dtype=np.float64)
    w1e = np.asarray(w1e, dtype=np.float64)
    w2e = np.asarray(w2e, dtype=np.float64)
    F = w2e.shape[1]
    a = xe @ w1e.T
    if b1e is not None:
        a = a + np.asarray(b1e, dtype=np.float64)[None, :]
    if act == "swiglu":
        g, u = a[:, :F], a[:, F:]
        hid = silu(g) * u
    elif act == "gelu":
        hid = gelu_erf(a)
    else:
        raise ValueError(act)
    y = hid @ w2e.T
    if b2e is not None:
        y = y + np.asarray(b2e, dtype=np.float64)[None, :]
    return y, dict(a=a, hid=hid)


def expert_capacity(T: int, E: int, k: int, capacity_factor: float, min_capacity: int = 4) -> int:
    """Tokens an expert may take ("emerging-techniques-moe-training",
    Capacity Factor Tuning: int(tokens / experts * capacity_factor); the
    DeepSpeed config on that page adds min_capacity 4). Reading: with top-k
    routing the tokens counted are the T*k routing slots, so a factor of 1
    is the mean load and 1.25 a 25 % buffer, as the page describes it."""
    return max(int(min_capacity), int((T * k / E) * capacity_factor))


def capacity_keep(topk_idx, E: int, capacity: int) -> np.ndarray:
    """keep[t,j]: pair (t, topk_idx[t,j]) is among the first `capacity`
    pairs of its expert in ascending token order ("drop_tokens": pairs past
    an expert's capacity are dropped; the pages do not say which, the
    plainest reading is arrival order)."""
    idx = np.asarray(topk_idx)
    T, k = idx.shape
    keep = np.zeros((T, k), dtype=bool)
    for e in range(E):
        tok, slot = np.nonzero(idx == e)          # ascending t
        keep[tok[:capacity], slot[:capacity]] = True
    return keep


def forward(x, w_gate, w1, w2, k: int, score: str, act: str, b_gate=None, sel_bias=None,
            b1=None, b2=None, w1_sh=None, w2_sh=None, tokens=None, routing=None, capacity=None):
    """Whole layer in fp64 (router fp32). All arrays numpy; x [T,h].

    ``tokens`` restricts the evaluation to those token indices (routing is
    per-token, so this equals the full computation on those rows; with
    ``capacity`` the kept pairs are found from the routing of every token
    first). With ``capacity``, pairs
    past an expert's capacity (``capacity_keep``) contribute nothing; the
    kept pairs keep their weights. Returns the route dict plus out [n,h]
    fp64, y_pair [n,k,h] (expert outputs per selected pair, zero for dropped
    pairs), keep [n,k] and y_shared [n,h] or None.
    """
    x = np.asarray(x, dtype=np.float32)
    E = w1.shape[0]
    keep = None
    if tokens is not None:
        tokens = np.asarray(tokens, dtype=np.int64)
        if capacity is not None:
            # which pairs an expert keeps depends on every token before them
            if routing is not None:
                raise ValueError("pass the full routing without tokens")
            full = route(x, w_gate, k, score, b_gate, sel_bias)
            keep = capacity_keep(full["topk_idx"], E, capacity)[tokens]
        x = x[tokens]
    if routing is None:
        routing = route(x, w_gate, k, score, b_gate, sel_bias)
    topk_idx = routing["topk_idx"]
    topk_w = routing["topk_w"]
    n, h = x.shape
    out = np.zeros((n, h), dtype=np.float64)
    y_pair = np.zeros((n, k, h), dtype=np.float64)
    # Per expert, as in the pages' loop over experts: gather the tokens that
    # chose it, run the expert, weight and add back.
    if keep is None:
        keep = np.ones(topk_idx.shape, dtype=bool) if capacity is None else capacity_keep(topk_idx, E, capacity)
    for e in range(E):
        tok, slot = np.nonzero((topk_idx == e) & keep)
        if tok.size == 0:
            continue
        y, _ = expert_forward(x[tok], w1[e], w2[e], act,
                              None if b1 is None else b1[e], None if b2 is None else b2[e])
        y_pair[tok, slot] = y
    for j in range(k):
        out += topk_w[:, j:j + 1] * y_pair[:, j]
    y_sh = None
    if w1_sh is not None:
        y_sh, _ = expert_forward(x, w1_sh, w2_sh, act)
        out += y_sh
    res = dict(routing)
    res.update(out=out, y_pair=y_pair, y_shared=y_sh, keep=keep)
    return res


# ----------------------------------------------------------------- MXFP8

E4M3_MAX = 448.0          # largest finite E4M3 value (1.75 * 2^8)
E4M3_EMAX = 8             # exponent of the largest E4M3 binade
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_SUB_STEP = 2.0 ** -9  # spacing of the subnormals


def e4m3_round(y):
    """Round float64 values to the E4M3 grid, nearest with ties to the even
    mantissa, magnitudes above 448 saturated to 448 (fp64 arithmetic on the
    grid's definition: 3 mantissa bits, exponent bias 7, subnormal step
    2^-9, no infinities). With |y| = m 2^E, m in [0.5, 1), the grid step at
    |y| is 2^(E-4) in the normal range and 2^-9 below 2^-6, i.e. 2^max(E-4, -9);
    scaling by powers of two is exact, so the only rounding is np.rint's
    (half to even)."""
    y = np.asarray(y, dtype=np.float64)
    a = np.abs(y)
    _, E = np.frexp(a)
    s = np.maximum(E - 4, -9)
    out = np.minimum(np.ldexp(np.rint(np.ldexp(a, -s)), s), E4M3_MAX)
    return np.copysign(out, y)


def e4m3_encode(v):
    """Bit codes (uint8) of values already on the E4M3 grid."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    m, E = np.frexp(a)                      # a = m 2^E; normal values: exponent E - 1, mantissa 16 m - 8
    sub = a < E4M3_MIN_NORMAL
    code = np.where(sub, np.rint(a / E4M3_SUB_STEP), (E - 1 + 7) * 8 + np.rint(m * 16 - 8)).astype(np.int64)
    code |= np.where(np.signbit(v), 0x80, 0)
    return code.astype(np.uint8)


def e4m3_decode(code):
    """float64 values of E4M3 bit codes (0x7f / 0xff, the NaN codes, decode
    as NaN)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * E4M3_SUB_STEP, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    val = np.where((c & 0x7f) == 0x7f, np.nan, val)
    return s * val


def _mx_block_exponent(amax):
    """Shared exponent of blocks with largest magnitude amax: floor(log2
    amax) - 8 (= frexp exponent - 9), clamped to [-127, 127]; -127 for an
    all-zero block."""
    _, E = np.frexp(amax)
    return np.where(amax > 0, np.clip(E - 1 - E4M3_EMAX, -127, 127), -127)


def mx_quantize(v):
    """MXFP8 quantisation along the last axis ("Scalable Training of
    Mixture-of-Experts Models with Megatron Core", section 5.3.3: 1 x 32
    blocks, E8M0 scales, E4M3 elements). Per block of 32: the shared
    exponent is floor(log2 of the block's largest magnitude) - 8 (the E4M3
    exponent of its largest binade), clamped to [-127, 127]; elements are
    v / 2^exponent rounded by ``e4m3_round``. An all-zero block gets
    exponent -127. Returns (codes uint8 [..., K], scale codes uint8
    [..., K/32] = exponent + 127)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // 32, 32))
    exp = _mx_block_exponent(np.abs(blk).max(axis=-1))
    q = e4m3_round(np.ldexp(blk, -exp[..., None]))
    codes = e4m3_encode(q).reshape(v.shape)
    return codes, (exp + 127).astype(np.uint8)


def mx_dequantize(codes, scales):
    """float64 values of MXFP8 data: element * 2^(scale - 127)."""
    c = np.asarray(codes)
    K = c.shape[-1]
    val = e4m3_decode(c).reshape(c.shape[:-1] + (K // 32, 32))
    val = val * 2.0 ** (np.asarray(scales, dtype=np.float64) - 127)[..., None]
    return val.reshape(c.shape)


def mx_roundtrip(v):
    """v quantised to MXFP8 along the last axis and back (float64): the
    values mx_dequantize(*mx_quantize(v)) gives, without the bit codes
    (each element e4m3_round(v 2^-exp) 2^exp with its block's exponent)."""
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    blk = v.reshape(v.shape[:-1] + (K // 32, 32))
    exp = _mx_block_exponent(np.abs(blk).max(axis=-1))[..., None]
    return np.ldexp(e4m3_round(np.ldexp(blk, -exp)), exp).reshape(v.shape)


def forward_mxfp8(x, w_gate, w1, w2, k: int, score: str, act: str, b_gate=None, sel_bias=None,
                  routing=None, tokens=None, with_act: bool = False):
    """The layer with the expert GEMMs in MXFP8: routing as ``forward``; the
    token rows, both weight matrices (along their reduction axes: h for W1,
    F for W2) and the activation (along F) quantised by ``mx_quantize``;
    products and sums in fp64 on the dequantised values. The activation is
    quantised as computed (fp64 here), with no intermediate rounding: the
    page's recipe quantises the activations themselves. SwiGLU or GELU
    without biases, no shared expert.

    With ``with_act``, the result also holds the activation in permuted-row
    order (expert-major, tokens ascending, as ``permutation``): ``act``
    [P, F] fp64 and its quantisation ``act_codes``, ``act_scales``."""
    x = np.asarray(x, dtype=np.float32)
    if tokens is not None:
        x = x[np.asarray(tokens, dtype=np.int64)]
    if routing is None:
        routing = route(x, w_gate, k, score, b_gate, sel_bias)
    topk_idx, topk_w = routing["topk_idx"], routing["topk_w"]
    n, h = x.shape
    E = w1.shape[0]
    xq = mx_roundtrip(x)
    out = np.zeros((n, h), dtype=np.float64)
    acts = []
    for e in range(E):
        tok, slot = np.nonzero(topk_idx == e)
        if tok.size == 0:
            continue
        order = np.argsort(tok, kind="stable")
        tok, slot = tok[order], slot[order]
        w1q = mx_roundtrip(np.asarray(w1[e], dtype=np.float64))
        w2q = mx_roundtrip(np.asarray(w2[e], dtype=np.float64))
        a = xq[tok] @ w1q.T
        if act == "swiglu":
            F = w2q.shape[1]
            hid = silu(a[:, :F]) * a[:, F:]
        else:
            hid = gelu_erf(a)
        codes, scales = mx_quantize(hid)
        y = mx_dequantize(codes, scales) @ w2q.T
        out[tok] += topk_w[tok, slot][:, None] * y
        if with_act:
            acts.append((hid, codes, scales))
    res = dict(routing)
    res.update(out=out)
    if with_act:
        F = w2.shape[2]
        res.update(act=np.concatenate([a_[0] for a_ in acts]) if acts else np.zeros((0, F)),
                   act_codes=np.concatenate([a_[1] for a_ in acts]) if acts else np.zeros((0, F), np.uint8),
                   act_scales=np.concatenate([a_[2] for a_ in acts]) if acts else np.zeros((0, F // 32), np.uint8))
    return res


def mx_roundtrip_axis0(v, starts=None):
    """v [n, c] quantised to MXFP8 along axis 0 and back: blocks of 32
    consecutive rows of one column share a scale. With ``starts`` (ascending
    segment boundaries s_0 = 0 < ... < s_m = n, empty segments allowed), each
    segment [s_i, s_{i+1}) is blocked on its own from its first row and its
    last block is completed with zero rows, which set no scale and are not
    returned."""
    v = np.asarray(v, dtype=np.float64)
    n = v.shape[0]
    bounds = [0, n] if starts is None else [int(b) for b in starts]
    out = np.zeros_like(v)
    for lo, hi in zip(bounds[:-1], bounds[1:]):
        m = hi - lo
        if m <= 0:
            continue
        mp = -(-m // 32) * 32
        pad = np.zeros((mp,) + v.shape[1:], dtype=np.float64)
        pad[:m] = v[lo:hi]
        out[lo:hi] = mx_roundtrip(pad.T).T[:m]
    return out


def expert_backward_mxfp8(xe, w1e, w2e, act, dy, quantise=True):
    """Gradients of one expert with its GEMMs in MXFP8 (reading above), fp64
    on dequantised operands. xe [m,h]: the expert's token rows in segment
    order (tokens ascending); dy [m,h]: the gradient of its weighted outputs
    in the same order. The forward's pre-activations are those of
    ``forward_mxfp8`` (x and W1 blocked along h). SwiGLU or GELU, no biases.

      dhid = Q_h(dy) Q_h(W2)                 (reduction over h)
      da   = activation backward of dhid at the forward's pre-activations
      dx   = Q_2F(da) Q_2F(W1)               (reduction over 2F, or F)
      dW2  = Q_tok(dy)^T Q_tok(hid)          (reduction over the tokens)
      dW1  = Q_tok(da)^T Q_tok(x)

    With quantise=False every Q is the identity: the result is then the
    plain fp64 backward of the same expert (``expert_backward``) evaluated at
    the MXFP8 forward's pre-activations."""
    xe = np.asarray(xe, dtype=np.float64)
    w1e = np.asarray(w1e, dtype=np.float64)
    w2e = np.asarray(w2e, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    rows = mx_roundtrip if quantise else (lambda v: np.asarray(v, dtype=np.float64))
    cols = mx_roundtrip_axis0 if quantise else (lambda v: np.asarray(v, dtype=np.float64))
    F = w2e.shape[1]
    a = mx_roundtrip(xe) @ mx_roundtrip(w1e).T          # the forward's pre-activations (always MXFP8)
    if act == "swiglu":
        g, u = a[:, :F], a[:, F:]
        hid = silu(g) * u
    else:
        hid = gelu_erf(a)
    dhid = rows(dy) @ cols(w2e)                         # [m,F]
    if act == "swiglu":
        da = np.concatenate([dhid * u * _dsilu(g), dhid * silu(g)], axis=1)
    else:
        da = dhid * _dgelu(a)
    dx = rows(da) @ cols(w1e)                           # [m,h]
    dw2 = cols(dy).T @ cols(hid)                        # [h,F]
    dw1 = cols(da).T @ cols(xe)                         # [n1F,h]
    return dict(dx=dx, dw1=dw1, dw2=dw2, dgu=da, hid=hid, a=a)


def backward_mxfp8(x, w_gate, w1, w2, k, score, act, grad_out, b_gate=None, sel_bias=None,
                   routing=None, experts=None):
    """``backward`` for the layer whose expert GEMMs run in MXFP8: the
    routing-weight gradients use the MXFP8 forward's expert outputs, the
    expert gradients ``expert_backward_mxfp8`` (each expert over all of its
    tokens, ascending), the router's gradients stay as in ``backward``.
    dw1/dw2 are keyed by expert (all, or those in ``experts``)."""
    x = np.asarray(x, dtype=np.float32)
    T, h = x.shape
    E = w1.shape[0]
    if routing is None:
        routing = route(x, w_gate, k, score, b_gate, sel_bias)
    topk_idx, topk_w = routing["topk_idx"], routing["topk_w"]
    G = np.asarray(grad_out, dtype=np.float64)
    x64 = x.astype(np.float64)
    want = set(range(E)) if experts is None else set(int(e) for e in experts)
    dx = np.zeros((T, h), dtype=np.float64)
    d_topk_w = np.zeros((T, k), dtype=np.float64)
    dw1, dw2 = {}, {}
    for e in range(E):
        tok, slot = np.nonzero(topk_idx == e)
        if tok.size == 0:
            if e in want:
                dw1[e] = np.zeros((w1.shape[1], h))
                dw2[e] = np.zeros((h, w2.shape[2]))
            continue
        order = np.argsort(tok, kind="stable")
        tok, slot = tok[order], slot[order]
        w1e = np.asarray(w1[e], dtype=np.float64)
        w2e = np.asarray(w2[e], dtype=np.float64)
        dy = topk_w[tok, slot][:, None] * G[tok]
        gb = expert_backward_mxfp8(x64[tok], w1e, w2e, act, dy)
        # the forward's expert outputs: activation quantised along F
        y = mx_roundtrip(gb["hid"]) @ mx_roundtrip(w2e).T
        d_topk_w[tok, slot] = (G[tok] * y).sum(axis=1)
        np.add.at(dx, tok, gb["dx"])
        if e in want:
            dw1[e] = gb["dw1"]
            dw2[e] = gb["dw2"]
    logits_sel = np.take_along_axis(routing["logits"], topk_idx.astype(np.int64), axis=1)
    dl = router_backward_dlogits(topk_w, d_topk_w, score, logits_sel)
    dlogits = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dlogits, topk_idx.astype(np.int64), dl, axis=1)
    rg = router_grads(x64, w_gate, dlogits)
    dx += rg["dx"]
    return dict(dx=dx, d_topk_w=d_topk_w, d_logits_sel=dl, dw_gate=rg["dw_gate"], db_gate=rg["db_gate"],
                dw1=dw1, dw2=dw2)


def expert_choice(logits, capacity: int):
    """Expert-choice selection ("emerging-techniques-moe-training", Routing
    Mechanisms, Expert Choice Routing: the router's scores transposed to
    [experts, tokens], then each expert takes its top-`capacity` tokens).
    Order: logit descending, then token index ascending. Returns chosen
    [E, capacity] (each expert's tokens in ascending token order) and the
    weights [E, capacity] = softmax over all E logits of the token, at the
    choosing expert (the page gives no weights; the gate probability is the
    weight used everywhere else on it)."""
    l = np.asarray(logits, dtype=np.float32)
    T, E = l.shape
    C = int(capacity)
    chosen = np.zeros((E, C), dtype=np.int64)
    t_idx = np.arange(T)
    for e in range(E):
        order = np.lexsort((t_idx, -l[:, e].astype(np.float64)))
        chosen[e] = np.sort(order[:C])
    p, _ = _log_softmax_parts(l)
    weights = np.take_along_axis(p.T, chosen, axis=1)
    return chosen, weights


def expert_choice_forward(x, w_gate, w1, w2, capacity: int, act: str, b_gate=None, b1=None, b2=None,
                          logits=None, tokens=None):
    """out[t] = sum over the experts that chose token t (ascending) of
    softmax(l_t)_e * E_e(x_t), fp64 (logits fp32 in gate order G). A token
    no expert chose gets 0. ``tokens``: evaluate the output of those tokens
    only (the selection still sees every token)."""
    x = np.asarray(x, dtype=np.float32)
    if logits is None:
        logits = gate_logits(x, w_gate, b_gate)
    chosen, weights = expert_choice(logits, capacity)
    T, h = x.shape
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)
    where = {int(t): i for i, t in enumerate(rows)}
    out = np.zeros((rows.size, h), dtype=np.float64)
    x64 = x.astype(np.float64)
    for e in range(chosen.shape[0]):
        sel = [i for i, t in enumerate(chosen[e]) if int(t) in where]
        if not sel:
            continue
        tok = chosen[e][sel]
        y, _ = expert_forward(x64[tok], w1[e], w2[e], act,
                              None if b1 is None else b1[e], None if b2 is None else b2[e])
        np.add.at(out, [where[int(t)] for t in tok], weights[e][sel][:, None] * y)
    return dict(logits=logits, chosen=chosen, weights=weights, out=out)


def combine(y_perm, row_of, topk_w, y_shared=None):
    """Combine stage on its own (fp64): out[t] = sum_j w[t,j] y_perm[row_of[t,j]]
    (+ y_shared[t]), j ascending."""
    y_perm = np.asarray(y_perm, dtype=np.float64)
    T, k = row_of.shape
    out = np.zeros((T, y_perm.shape[1]), dtype=np.float64)
    for j in range(k):
        out += np.asarray(topk_w, dtype=np.float64)[:, j:j + 1] * y_perm[np.asarray(row_of)[:, j]]
    if y_shared is not None:
        out += np.asarray(y_shared, dtype=np.float64)
    return out


# ------------------------------------------------------------------ backward

def _dsilu(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def _dgelu(a):
    erf = np.vectorize(math.erf, otypes=[np.float64])
    cdf = 0.5 * (1.0 + erf(a / math.sqrt(2.0)))
    pdf = np.exp(-0.5 * a * a) / math.sqrt(2.0 * math.pi)
    return cdf + a * pdf


def expert_backward(xe, w1e, w2e, act, dy, b1e=None, b2e=None):
    """Gradients of sum(dy * expert(xe)) w.r.t. xe, w1e, w2e, b1e, b2e (fp64)."""
    xe = np.asarray(xe, dtype=np.float64)
    w1e = np.asarray(w1e, dtype=np.float64)
    w2e = np.asarray(w2e, dtype=np.float64)
    F = w2e.shape[1]
    _, c = expert_forward(xe, w1e, w2e, act, b1e, b2e)
    a, hid = c["a"], c["hid"]
    dw2 = dy.T @ hid                      # [h,F]
    dhid = dy @ w2e                       # [m,F]
    if act == "swiglu":
        g, u = a[:, :F], a[:, F:]
        da = np.concatenate([dhid * u * _dsilu(g), dhid * silu(g)], axis=1)
    else:
        da = dhid * _dgelu(a)
    dw1 = da.T @ xe                       # [n1F,h]
    dx = da @ w1e                         # [m,h]
    db1 = da.sum(axis=0) if b1e is not None else None
    db2 = dy.sum(axis=0) if b2e is not None else None
    return dict(dx=dx, dw1=dw1, dw2=dw2, db1=db1, db2=db2, dgu=da, hid=hid)


def router_backward_dlogits(topk_w, d_topk_w, score, logits_sel=None):
    """d L / d logit of each selected expert (fp64), [T,k].

    softmax renormalised over the selection: w_j = e^{l_j} / sum_sel e^{l_i},
    so dl_j = w_j (g_j - sum_i w_i g_i). Unselected logits do not reach the
    output and get 0. sigmoid normalised over the selection: w_j = s_j / S with
    s = sigma(l), so dl_j = s_j (1 - s_j) / S * (g_j - sum_i w_i g_i).
    """
    w = np.asarray(topk_w, dtype=np.float64)
    g = np.asarray(d_topk_w, dtype=np.float64)
    centred = g - (w * g).sum(axis=1, keepdims=True)
    if score == "softmax":
        return w * centred
    s = 1.0 / (1.0 + np.exp(-np.asarray(logits_sel, dtype=np.float64)))
    S = s.sum(axis=1, keepdims=True)
    return s * (1.0 - s) / S * centred


def _log_softmax_parts(logits):
    """Per-token softmax over all experts and logsumexp (fp64), both with
    the row maximum taken out before exponentiating."""
    l = np.asarray(logits, dtype=np.float64)
    m = l.max(axis=1, keepdims=True)
    ex = np.exp(l - m)
    s = ex.sum(axis=1, keepdims=True)
    return ex / s, (m + np.log(s))[:, 0]


def expert_fraction(topk_idx, E: int) -> np.ndarray:
    """f_e: routing slots that chose expert e over all T*k slots (fp64)."""
    idx = np.asarray(topk_idx).reshape(-1).astype(np.int64)
    if idx.size == 0:
        return np.zeros(E)
    return np.bincount(idx, minlength=E)[:E].astype(np.float64) / idx.size


def router_losses(logits, topk_idx, E: int):
    """(aux, z) in fp64 ("emerging-techniques-moe-training", section 3 Load
    Balancing):

        aux = E * sum_e f_e * P_e,  P_e = mean_t softmax(l_t)_e
        z   = mean_t logsumexp(l_t)^2
    """
    l = np.asarray(logits, dtype=np.float64)
    T = l.shape[0]
    if T == 0:
        return 0.0, 0.0
    p, lse = _log_softmax_parts(l)
    f = expert_fraction(topk_idx, E)
    aux = E * float((f * p.mean(axis=0)).sum())
    z = float((lse * lse).mean())
    return aux, z


def mean_router_probs(logits) -> np.ndarray:
    """P_e = mean over tokens of softmax(l_t)_e, [E] fp64 (zeros for T = 0)."""
    l = np.asarray(logits, dtype=np.float64)
    if l.shape[0] == 0:
        return np.zeros(l.shape[1])
    p, _ = _log_softmax_parts(l)
    return p.mean(axis=0)


def router_losses_dlogits(logits, topk_idx, E: int, coef_aux: float, coef_z: float):
    """d(coef_aux * aux + coef_z * z) / d logits, [T,E] fp64.

    With p = softmax(l_t), dP_e/dl_{t,j} = p_{t,e} (delta_ej - p_{t,j}) / T,
    so the load-balancing term is (E/T) p_{t,j} (f_j - sum_e f_e p_{t,e});
    d lse_t / d l_{t,j} = p_{t,j}, so the z term is (2/T) lse_t p_{t,j}.
    f_e is held fixed (see the header).
    """
    l = np.asarray(logits, dtype=np.float64)
    T = l.shape[0]
    if T == 0:
        return np.zeros((0, E))
    p, lse = _log_softmax_parts(l)
    f = expert_fraction(topk_idx, E)
    a = (p * f[None, :]).sum(axis=1, keepdims=True)
    d_aux = (E / T) * p * (f[None, :] - a)
    d_z = (2.0 / T) * lse[:, None] * p
    return coef_aux * d_aux + coef_z * d_z


def router_grads(x, w_gate, dlogits):
    """Gradients through l = W_r x + b of a logit gradient D [T,E] (fp64):
    dW_r = D^T x [E,h], db = sum_t D_t [E], dx = D W_r [T,h]."""
    D = np.asarray(dlogits, dtype=np.float64)
    x64 = np.asarray(x, dtype=np.float64)
    wg = np.asarray(w_gate, dtype=np.float64)
    return dict(dw_gate=D.T @ x64, db_gate=D.sum(axis=0), dx=D @ wg)


def backward(x, w_gate, w1, w2, k, score, act, grad_out, b_gate=None, sel_bias=None,
             b1=None, b2=None, routing=None, experts=None, coef_aux=0.0, coef_z=0.0, capacity=None):
    """Gradients of L = sum(grad_out * out) + coef_aux * aux + coef_z * z
    for the routed layer (no shared expert); aux and z as in
    ``router_losses``. Top-k indices carry no gradient.

    Returns dx [T,h], d_topk_w [T,k], d_logits_sel [T,k], dw_gate [E,h],
    db_gate [E], and dicts dw1/dw2/db1/db2 keyed by expert (all experts, or
    those listed in ``experts``; an expert with no tokens gets exact zeros).
    With ``capacity``, dropped pairs (``capacity_keep``) reach no expert and
    get d_topk_w = 0; the router's gradient still runs over every selected
    pair, since the kept weights depend on all selected logits.
    """
    x = np.asarray(x, dtype=np.float32)
    T, h = x.shape
    E = w1.shape[0]
    if routing is None:
        routing = route(x, w_gate, k, score, b_gate, sel_bias)
    topk_idx = routing["topk_idx"]
    topk_w = routing["topk_w"]
    G = np.asarray(grad_out, dtype=np.float64)
    x64 = x.astype(np.float64)
    want = set(range(E)) if experts is None else set(int(e) for e in experts)
    dx = np.zeros((T, h), dtype=np.float64)
    d_topk_w = np.zeros((T, k), dtype=np.float64)
    dw1, dw2, db1, db2 = {}, {}, {}, {}
    keep = np.ones(topk_idx.shape, dtype=bool) if capacity is None else capacity_keep(topk_idx, E, capacity)
    for e in range(E):
        tok, slot = np.nonzero((topk_idx == e) & keep)
        n1F = w1.shape[1]
        if tok.size == 0:
            if e in want:
                dw1[e] = np.zeros((n1F, h))
                dw2[e] = np.zeros((h, w2.shape[2]))
                if b1 is not None:
                    db1[e] = np.zeros(n1F)
                    db2[e] = np.zeros(h)
            continue
        b1e = None if b1 is None else b1[e]
        b2e = None if b2 is None else b2[e]
        y, _ = expert_forward(x64[tok], w1[e], w2[e], act, b1e, b2e)
        d_topk_w[tok, slot] = (G[tok] * y).sum(axis=1)
        dy = topk_w[tok, slot][:, None] * G[tok]
        gb = expert_backward(x64[tok], w1[e], w2[e], act, dy, b1e, b2e)
        np.add.at(dx, tok, gb["dx"])
        if e in want:
            dw1[e] = gb["dw1"]
            dw2[e] = gb["dw2"]
            if b1 is not None:
                db1[e] = gb["db1"]
                db2[e] = gb["db2"]
    logits_sel = np.take_along_axis(routing["logits"], topk_idx.astype(np.int64), axis=1)
    dl = router_backward_dlogits(topk_w, d_topk_w, score, logits_sel)
    dlogits = np.zeros((T, E), dtype=np.float64)
    np.put_along_axis(dlogits, topk_idx.astype(np.int64), dl, axis=1)
    if coef_aux != 0.0 or coef_z != 0.0:
        dlogits += router_losses_dlogits(routing["logits"], topk_idx, E, coef_aux, coef_z)
    rg = router_grads(x64, w_gate, dlogits)
    dw_gate, db_gate = rg["dw_gate"], rg["db_gate"]
    dx += rg["dx"]
    return dict(dx=dx, d_topk_w=d_topk_w, d_logits_sel=dl, d_logits=dlogits,
                dw_gate=dw_gate, db_gate=db_gate, dw1=dw1, dw2=dw2, db1=db1, db2=db2)


# ----------------------------------------------------- fp64 forward for FD

def loss_fp64(x, w_gate, w1, w2, k, score, act, grad_out, b_gate=None, sel_bias=None,
              b1=None, b2=None, expect_idx=None, coef_aux=0.0, coef_z=0.0, capacity=None):
    """L = sum(grad_out * out) + coef_aux * aux + coef_z * z with every
    step, logits included, in fp64.

    Used only to check the backward by finite differences: the fp32 gate order
    would quantise small perturbations of the router weights. Selection uses
    the fp64 logits; ``expect_idx`` asserts that a perturbation left it
    unchanged (top-k is piecewise constant, so the derivative exists only
    there).
    """
    x = np.asarray(x, dtype=np.float64)
    logits = x @ np.asarray(w_gate, dtype=np.float64).T
    if b_gate is not None:
        logits = logits + np.asarray(b_gate, dtype=np.float64)[None, :]
    if score == "softmax":
        key = logits
    else:
        key = 1.0 / (1.0 + np.exp(-logits))
        if sel_bias is not None:
            key = key + np.asarray(sel_bias, dtype=np.float64)[None, :]
    T, E = logits.shape
    order = np.lexsort((np.broadcast_to(np.arange(E), (T, E)), -key), axis=-1)
    topk_idx = order[:, :k]
    if expect_idx is not None and not np.array_equal(topk_idx, expect_idx):
        raise RuntimeError("selection changed under the perturbation")
    sel = np.take_along_axis(logits, topk_idx, axis=1)
    w = routing_weights(sel, logits, score)
    out = np.zeros_like(x)
    keep = np.ones(topk_idx.shape, dtype=bool) if capacity is None else capacity_keep(topk_idx, E, capacity)
    for e in range(w1.shape[0]):
        tok, slot = np.nonzero((topk_idx == e) & keep)
        if tok.size == 0:
            continue
        y, _ = expert_forward(x[tok], w1[e], w2[e], act,
                              None if b1 is None else b1[e], None if b2 is None else b2[e])
        np.add.at(out, tok, w[tok, slot][:, None] * y)
    L = float((np.asarray(grad_out, dtype=np.float64) * out).sum())
    if coef_aux != 0.0 or coef_z != 0.0:
        aux, z = router_losses(logits, topk_idx, E)
        L += coef_aux * aux + coef_z * z
    return L, topk_idx, logits, w
