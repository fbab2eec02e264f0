"""Benchmark of the sparse MoE layer on one MI355X.

One step = one pass of the whole forward hot path over one batch of synthetic
input: Route -> Permute -> Grouped FFN (two grouped GEMMs with the fused
SwiGLU) -> Unpermute, all through libmoe.so's C ABI on one stream. The
default workload is the Mixtral-8x7B-shaped layer (T=4096 tokens, h=4096,
E=8, top-2, SwiGLU 14336, bf16 with fp32 accumulation).

Prints one JSON line: active TFLOP/s (router GEMM plus every routed
token's expert FLOPs, no padding credited) and tokens/s; the roofline of the
dominant call (the grouped FFN, or its backward in a training step), timed
with HIP events around that call inside the timed steps; per-stage times with
their roofline fractions (stages timed separately with HIP events after an
eviction of the 256 MB last-level cache); and the CPU oracle timed on a
bounded sample of the same workload.

The default run (the Mixtral-shaped layer, no variant flags) adds one
sub-record per other workload under "configs": the tiny fp32 GELU layer, the
Qwen3-235B and DeepSeek-V3 inference layers, the imbalanced Qwen3 training
step and the handbook training step, each timed over a few steps with its
dominant call's MFMA fraction from HIP events and the oracle timed on a few
of its tokens; then the Mixtral-shaped forward and the imbalanced training
step again with MXFP8 expert GEMMs (fractions of the fp8 peak). The GPU clock is sampled while the headline step is repeated
for about three seconds after the timed steps (the driver's metrics table
refreshes about once a second, too slowly for the timed steps alone).

``--copy-calibration`` runs only a plain elementwise copy of 1 GiB (fp32
negation, 1 GiB read and 1 GiB written per launch): the HBM byte counters
read for it give the scale factor applied to the counters of the GEMMs.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MoE layer active TFLOP/s + tokens/s at 1 MI355X; % of MFMA/HBM roofline"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 2.4 GHz x 4096 FLOP/clk (dense)
PEAK_F32_MFMA_TFLOPS = 157.3
PEAK_FP8_TFLOPS = 5033.2       # dense fp8 MFMA: twice the bf16 rate
PEAK_HBM_GBS = 8000.0
# fp32 FMA on the vector ALUs without packed instructions (which this library
# does not emit): 256 CU x 4 SIMD x 16 lanes x 2 FLOP x 2.4 GHz
PEAK_F32_VALU_TFLOPS = 78.6
COEF_AUX, COEF_Z = 1e-2, 1e-3
# measured HBM traffic of the grouped FFN (rocprofv3 FETCH_SIZE / WRITE_SIZE,
# scaled by the same counters on a plain copy); valid while the GEMM sources
# hash to the recorded value
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "grouped_ffn_mixtral_8x7b_layer_hbm_traffic.md")
GEMM_SOURCES = ["ffn.hip", "gemm_common.hpp", "common.hpp"]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--stage-reps", type=int, default=10)
    p.add_argument("--cpu-tokens", type=int, default=4096,
                   help="tokens of the workload the CPU oracle is timed on")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-stages", action="store_true")
    p.add_argument("--memory-efficient", action="store_true",
                   help="apply the routing weight before the second projection (experts without "
                        "output bias) and rebuild the activation in the backward")
    p.add_argument("--capacity-factor", type=float, default=None,
                   help="drop pairs past int(T*k/E * factor) per expert (min 4), in token order")
    p.add_argument("--expert-choice", action="store_true",
                   help="expert-choice routing, capacity T*k/E per expert (forward only)")
    p.add_argument("--mxfp8", action="store_true",
                   help="expert GEMMs in MXFP8 (1x32 blocks, E8M0 scales; weights quantised before "
                        "timing, tokens and activation inside the step); forward only")
    p.add_argument("--router-losses", action="store_true",
                   help="add the load-balancing loss (coefficient 1e-2) and router z-loss "
                        "(1e-3) to a training step, and time their kernels as stages")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB elementwise copy (counter calibration)")
    p.add_argument("--graph-steps", type=int, default=20,
                   help="also time this many replays of one step captured in a HIP graph (0: none)")
    p.add_argument("--hipblaslt-reference", action="store_true",
                   help="time only torch.matmul (hipBLASLt) on the dense shapes of the Mixtral-shaped "
                        "layer's two projections, as a reference for the grouped GEMM")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the sub-records of the other workloads")
    p.add_argument("--config-steps", type=int, default=5, help="timed steps per sub-record")
    p.add_argument("--config-cpu-tokens", type=int, default=8,
                   help="tokens of each sub-record's workload the oracle is timed on")
    p.add_argument("--clock-seconds", type=float, default=3.0,
                   help="length of the clock-sampling loop after the timed steps (0: none)")
    return p.parse_args()


def gemm_source_hash():
    h = hashlib.sha256()
    for name in GEMM_SOURCES:
        with open(os.path.join(ROOT, "mixture_experts_layer_06_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(workload: str):
    """HBM bytes per grouped-FFN call from the committed counter summary, or
    None when it is missing, for another workload, or for other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
    except OSError:
        return None
    start = text.find("```json")
    if start < 0:
        return None
    end = text.find("```", start + 7)
    rec = json.loads(text[start + 7:end])
    if rec.get("workload") != workload or rec.get("gemm_source_sha256") != gemm_source_hash():
        return None
    return rec


class ClockSampler:
    """Samples the GPU core clock (MHz) on a background thread while the timed
    steps run: the mean over XCDs of amdsmi's GPU-metrics current_gfxclks,
    else the active level of sysfs pp_dpm_sclk (a DPM level, coarser than
    the real clock). The driver refreshes these values on its own schedule,
    so short runs get few distinct readings."""

    def __init__(self, period_s=0.002):
        import glob
        import threading
        self.period = period_s
        self.smi = None
        self.source = None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            h = amdsmi.amdsmi_get_processor_handles()[0]
            amdsmi.amdsmi_get_gpu_metrics_info(h)["current_gfxclks"]
            self.smi = (amdsmi, h)
            self.source = "amdsmi gpu metrics current_gfxclks, mean over XCDs"
        except Exception:
            self.smi = None
        self.files = [] if self.smi else sorted(glob.glob("/sys/class/drm/card*/device/pp_dpm_sclk"))
        if self.files:
            self.source = "sysfs pp_dpm_sclk active level"
        self.samples = []
        self.stop = threading.Event()
        self.thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        if self.smi:
            amdsmi, h = self.smi
            try:
                v = [c for c in amdsmi.amdsmi_get_gpu_metrics_info(h)["current_gfxclks"]
                     if isinstance(c, (int, float)) and 0 < c < 10000]
                return float(sum(v) / len(v)) if v else None
            except Exception:
                return None
        for f in self.files:
            try:
                with open(f) as fh:
                    for line in fh:
                        if line.strip().endswith("*"):
                            return float(line.split(":")[1].strip().rstrip("*").strip().lower().rstrip("mhz"))
            except OSError:
                continue
        return None

    def _run(self):
        while not self.stop.is_set():
            v = self._read()
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        self.thread.start()
        return self

    def __exit__(self, *exc):
        self.stop.set()
        self.thread.join()

    def summary(self):
        # the metrics table is refreshed by the driver on its own schedule and
        # often holds idle-state values during short bursts of work; readings
        # below 500 MHz are not a loaded GPU's clock and are dropped
        v = np.asarray([x for x in self.samples if x >= 500.0])
        if v.size == 0:
            return {"mhz_median": None, "samples": len(self.samples), "source": self.source,
                    "note": "no plausible reading (all below 500 MHz)" if self.samples else "no reading"}
        return {"mhz_median": float(np.median(v)), "mhz_min": float(v.min()), "mhz_max": float(v.max()),
                "samples": int(v.size), "distinct_readings": int(np.unique(v).size),
                "samples_below_500mhz": len(self.samples) - int(v.size), "source": self.source}


def sample_clock(torch, step, seconds):
    """Repeats step() for about `seconds` while the clock sampler runs; a
    barrier every 20 steps keeps the queue short."""
    with ClockSampler() as clock:
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            step()
            n += 1
            if n % 20 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
    out = clock.summary()
    out["loop"] = "%d repeated steps over %.1f s after the timed steps" % (n, time.perf_counter() - t0)
    return out


def host_info():
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
        with open("/proc/meminfo") as f:
            for line in f:
                if line.startswith("MemTotal"):
                    info["host_ram_gib"] = round(int(line.split()[1]) / 2 ** 20, 1)
                    break
    except OSError:
        pass
    info["visible_cpus"] = os.cpu_count()
    return info


def copy_bandwidth(torch, reps=5):
    """Plain 1 GiB fp32 elementwise copy (read 1 GiB, write 1 GiB), best of reps."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    torch.neg(src, out=dst)
    best = None
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.neg(src, out=dst)
        e1.record()
        e1.synchronize()
        t = e0.elapsed_time(e1) * 1e-3
        best = t if best is None else min(best, t)
    del src, dst
    return 2.0 * 4 * n / best / 1e9


def copy_calibration():
    import torch
    n = 1 << 28                                   # fp32 elements: 1 GiB
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": 4 * n, "bytes_written": 4 * n,
                                           "launches": 3}}), flush=True)


def hipblaslt_reference(torch, reps=20):
    """torch.matmul in bf16 (hipBLASLt) on the dense equivalents of the
    Mixtral-shaped layer's two projections over all 8192 routed rows:
    [8192, 4096] x [4096, 28672] and [8192, 14336] x [14336, 4096], best and
    mean of `reps` HIP-event timings; the GPU clock sampled over a 3 s loop
    of the first product."""
    out = {}
    g = torch.Generator(device="cuda:0").manual_seed(7)
    for name, (M, K, N) in (("first projection", (8192, 4096, 28672)), ("second projection", (8192, 14336, 4096))):
        a = torch.randn(M, K, device="cuda:0", generator=g).to(torch.bfloat16)
        b = torch.randn(K, N, device="cuda:0", generator=g).to(torch.bfloat16)
        for _ in range(3):
            torch.matmul(a, b)
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            torch.matmul(a, b)
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        fl = 2.0 * M * K * N
        out[name] = {"shape_mkn": [M, K, N], "tflops_best": fl / min(ts) / 1e12,
                     "tflops_mean": fl / float(np.mean(ts)) / 1e12, "ms_mean": float(np.mean(ts)) * 1e3}
        if name == "first projection":
            out["gpu_clock"] = sample_clock(torch, lambda: torch.matmul(a, b), 3.0)
        del a, b
    return out


def stage_bytes(cfg, P, es):
    """Algorithmic HBM bytes of the memory-bound stages (index traffic included).
    Inference permutes indices only (the first GEMM gathers rows); training
    also writes x_perm."""
    T, h, k, E = cfg.T, cfg.h, cfg.k, cfg.E
    route = T * h * es + E * h * es + T * k * 8 + E * 4
    permute = T * k * 4 * 3 + P * 4
    if cfg.backward:
        permute += T * h * es + P * h * es
    unpermute = P * h * es + T * h * es + T * k * 8 + (T * h * es if cfg.n_shared else 0)
    return dict(route=route, permute=permute, unpermute=unpermute)


def ffn_flops(cfg):
    nmat = 3 if cfg.act == "swiglu" else 2
    return (cfg.P + cfg.n_shared * cfg.T) * nmat * 2.0 * cfg.h * cfg.F


def ffn_weight_bytes(cfg, es):
    n1 = 2 if cfg.act == "swiglu" else 1
    return (cfg.E + cfg.n_shared) * (n1 + 1) * cfg.h * cfg.F * es


def cpu_baseline(cfg, inp, n_tok):
    """The oracle as it stands, on the first n_tok tokens of the workload."""
    import oracle
    from threadpoolctl import threadpool_info

    class Lazy:
        def __init__(self, t):
            self.t = t
            self.shape = tuple(t.shape)

        def __getitem__(self, e):
            return self.t[e].float().cpu().numpy()

    x = inp["x"][:n_tok].float().cpu().numpy()
    wg = inp["w_gate"].float().cpu().numpy()
    sel = None if inp.get("sel_bias") is None else inp["sel_bias"].cpu().numpy()
    bg = None if inp.get("b_gate") is None else inp["b_gate"].cpu().numpy()
    w1, w2 = Lazy(inp["w1"]), Lazy(inp["w2"])
    # stage the needed experts' weights on the host outside the timed region
    r = oracle.route(x, wg, cfg.k, cfg.score, bg, sel)
    used = sorted(set(int(e) for e in np.unique(r["topk_idx"])))
    W1 = {e: w1[e] for e in used}
    W2 = {e: w2[e] for e in used}

    class Dict:
        def __init__(self, d, shape):
            self.d = d
            self.shape = shape

        def __getitem__(self, e):
            return self.d[e]

    W1o, W2o = Dict(W1, w1.shape), Dict(W2, w2.shape)
    w1s = None if inp.get("w1_sh") is None else inp["w1_sh"].float().cpu().numpy()
    w2s = None if inp.get("w2_sh") is None else inp["w2_sh"].float().cpu().numpy()
    t0 = time.perf_counter()
    ref = oracle.forward(x, wg, W1o, W2o, cfg.k, cfg.score, cfg.act, b_gate=bg, sel_bias=sel,
                         w1_sh=w1s, w2_sh=w2s)
    dt = time.perf_counter() - t0
    sub = cfg.with_shape(T=n_tok)
    flops = sub.active_flops_forward()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [os.cpu_count() or 1])
    del ref
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "tokens_per_s": n_tok / dt,
            "seconds": dt, "cores": int(threads), "kind": "oracle",
            "sample": "oracle forward (fp32 router, fp64 experts) on the first %d of %d tokens "
                      "of the same seeded workload; expert weights staged on the host beforehand"
                      % (n_tok, cfg.T)}


SUB_CONFIGS = (1, 3, 4, 5, 6)
MX_SUB_CONFIGS = (2, 5)   # the same workloads with MXFP8 expert GEMMs


def sub_record(torch, layer, wl, cid, steps, warmup, cpu_tokens, with_cpu, mx=False):
    """One other workload's step: forward (plus backward for training
    workloads), timed over `steps` steps after `warmup`, with the dominant
    call's MFMA fraction from HIP events on its stream; the oracle's forward
    on the first cpu_tokens tokens as its CPU baseline. With mx, the expert
    GEMMs in MXFP8 (weights quantised once, before timing; fractions of the
    fp8 peak)."""
    cfg = wl.CONFIGS[cid]
    inp = wl.make_inputs(cfg, device="cuda:0")
    train = cfg.backward
    wq = layer.quantize_experts_mx(inp, for_backward=train) if mx else None

    def step(timers=None):
        if mx:
            f = layer.forward_mxfp8(inp, wq, cfg.k, cfg.score, timers=timers, keep_for_backward=train)
            if train:
                layer.backward_mxfp8(inp, f, wq, inp["grad_out"], cfg.k, cfg.score, timers=timers)
            return f
        f = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=train, timers=timers)
        if train:
            layer.backward(inp, f, inp["grad_out"], cfg.k, cfg.score, cfg.act, timers=timers)
        return f

    for _ in range(warmup):
        step()
    timers = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step(timers)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    flops = cfg.active_flops_forward() + (cfg.active_flops_backward() if train else 0.0)
    live = {name: float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e-3
            for name, pairs in timers.items()}
    nmat = 3 if cfg.act == "swiglu" else 2
    call_flops = {"grouped_ffn": ffn_flops(cfg), "grouped_ffn_bwd": 2.0 * cfg.P * nmat * 2.0 * cfg.h * cfg.F}
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    if mx:
        peak = PEAK_FP8_TFLOPS
    dom = max(live, key=lambda n: live[n])
    rec = {
        "value": flops / dt / 1e12, "unit": "TFLOP/s", "tokens_per_s": cfg.T / dt,
        "ms_per_step": dt * 1e3, "steps": steps, "warmup": warmup,
        "dtype": "mxfp8 (e4m3, e8m0 1x32)" if mx else cfg.dtype,
        "step": "forward + backward" if train else "forward",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.h, "experts": cfg.E,
                   "topk": cfg.k, "expert_ffn": cfg.F, "score": cfg.score, "act": cfg.act,
                   "shared_experts": cfg.n_shared},
        "frac_of_peak": flops / dt / 1e12 / peak,
        "dominant_call": {"call": dom, "ms": live[dom] * 1e3,
                          "achieved_tflops": call_flops[dom] / live[dom] / 1e12, "peak_tflops": peak,
                          "frac": call_flops[dom] / live[dom] / 1e12 / peak,
                          "timing": "HIP events around the call on its stream, mean over the timed steps"},
        "calls_ms": {n: v * 1e3 for n, v in live.items()},
    }
    if mx and train:
        rec["dominant_call"]["flops_note"] = "algorithmic backward FLOPs only, the recomputation not credited"
    if dom == "grouped_ffn":
        # the forward expert call's roof: the slower of its MFMA work at peak
        # and one read of every expert weight at the nominal HBM rate
        w_bytes = ffn_weight_bytes(cfg, 1) * 33 / 32 if mx else ffn_weight_bytes(cfg, 2 if cfg.dtype == "bf16" else 4)
        t_mfma = call_flops[dom] / (peak * 1e12)
        t_w = w_bytes / (PEAK_HBM_GBS * 1e9)
        rec["dominant_call"].update({
            "bound": "hbm (weight bytes)" if t_w > t_mfma else "mfma",
            "roof_ms": max(t_mfma, t_w) * 1e3, "roof_frac": max(t_mfma, t_w) / live[dom]})
    if with_cpu:
        try:
            rec["cpu_baseline"] = cpu_baseline(cfg, inp, min(cpu_tokens, cfg.T))
        except Exception as exc:
            rec["cpu_baseline"] = {"error": repr(exc)}
    del inp, wq
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: the layer is built and timed on a single MI355X "
              "(no collectives or sharding in this build); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    import torch
    if args.hipblaslt_reference:
        print(json.dumps({"hipblaslt_reference": hipblaslt_reference(torch)}), flush=True)
        return
    from mixture_experts_layer_06_amd import binding as B
    from mixture_experts_layer_06_amd import layer
    from mixture_experts_layer_06_amd import workloads as wl

    B.load()
    cfg = wl.CONFIGS[args.config]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = wl.make_inputs(cfg, device=dev)
    es = 2 if cfg.dtype == "bf16" else 4
    train = cfg.backward
    flops = cfg.active_flops_forward() + (cfg.active_flops_backward() if train else 0.0)

    losses = args.router_losses and train
    coefs = dict(coef_aux=COEF_AUX, coef_z=COEF_Z) if losses else {}
    meff = args.memory_efficient
    if meff and inp.get("b2") is not None:
        if inp["b2"].any():
            sys.exit("--memory-efficient needs experts without output bias")
        inp["b2"] = None

    cap = None
    if args.capacity_factor is not None:
        cap = layer.capacity_from_factor(cfg.T, cfg.E, cfg.k, args.capacity_factor)
    if args.expert_choice:
        if train:
            sys.exit("--expert-choice runs the forward only; pick a forward workload")
        ec_cap = cfg.T * cfg.k // cfg.E
    if args.mxfp8:
        if cfg.act != "swiglu" or cfg.n_shared or cfg.dtype != "bf16" or inp.get("b1") is not None:
            sys.exit("--mxfp8 runs bf16 SwiGLU layers without expert biases or a shared expert")
        if losses or meff or cap is not None or args.expert_choice:
            sys.exit("--mxfp8 combines with no other variant flag")
        # weights quantised once per weight update, outside the timed steps
        wq = layer.quantize_experts_mx(inp, for_backward=train)

    def step(timers=None):
        if args.mxfp8:
            f = layer.forward_mxfp8(inp, wq, cfg.k, cfg.score, timers=timers, keep_for_backward=train)
            if train:
                layer.backward_mxfp8(inp, f, wq, inp["grad_out"], cfg.k, cfg.score, timers=timers)
            return f
        if args.expert_choice:
            return layer.forward_expert_choice(inp, ec_cap, cfg.act, timers=timers)
        f = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=train, timers=timers,
                          router_losses=losses, memory_efficient=meff, capacity=cap)
        if train:
            layer.backward(inp, f, inp["grad_out"], cfg.k, cfg.score, cfg.act, timers=timers, **coefs)
        return f

    for _ in range(args.warmup):
        step()
    timers = {}
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        res = step(timers)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    clock = sample_clock(torch, step, args.clock_seconds) if args.clock_seconds > 0 else None
    graph_rec = None
    if args.graph_steps > 0 and cap is None and not args.expert_choice:
        # the same step captured once in a HIP graph and replayed: the C-ABI
        # calls allocate nothing themselves and record no memset
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        tg = time.perf_counter()
        for _ in range(args.graph_steps):
            graph.replay()
        torch.cuda.synchronize()
        dtg = (time.perf_counter() - tg) / args.graph_steps
        graph_rec = {"ms_per_step": dtg * 1e3, "value": flops / dtg / 1e12, "steps": args.graph_steps,
                     "note": "one captured step replayed; the headline value is the eager steps'"}
        del graph
    if args.expert_choice:
        counts = np.full(cfg.E, ec_cap)
    else:
        counts = res["counts"].cpu().numpy()
    if cap is not None:
        # only the kept pairs reach an expert
        kept = int(res["kept"]["offsets"][-1].item())
        dropped_frac = 1.0 - kept / cfg.P
        nmat = 3 if cfg.act == "swiglu" else 2
        flops -= (cfg.P - kept) * nmat * 2.0 * cfg.h * cfg.F * (3.0 if train else 1.0)
    live = {name: float(np.mean([a.elapsed_time(b) for a, b in pairs])) * 1e-3
            for name, pairs in timers.items()}

    out = {
        "metric": METRIC,
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": dt * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8 (e4m3, e8m0 1x32)" if args.mxfp8 else cfg.dtype,
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "hidden": cfg.h, "experts": cfg.E,
                   "topk": cfg.k, "expert_ffn": cfg.F, "score": cfg.score, "act": cfg.act,
                   "shared_experts": cfg.n_shared,
                   "step": "forward + backward" if train else "forward",
                   "router_losses": {"coef_aux": COEF_AUX, "coef_z": COEF_Z} if losses else None,
                   "memory_efficient_permutation": meff,
                   "routing": ("expert_choice, capacity %d per expert" % ec_cap if args.expert_choice else
                               "top-k, capacity %d per expert (factor %g)" % (cap, args.capacity_factor)
                               if cap is not None else "top-k, dropless")},
        "tokens_per_s": cfg.T / dt,
        "frac_of_bf16_peak": flops / dt / 1e12 / PEAK_BF16_TFLOPS,
        "active_gflop_per_step": flops / 1e9,
        "expert_load": {"min": int(counts.min()), "max": int(counts.max())},
        "dropped_pair_fraction": dropped_frac if cap is not None else None,
        # activations the forward keeps for the backward (training step only)
        "saved_for_backward_bytes": int(sum(res[n].numel() * res[n].element_size()
                                            for n in ("x_perm", "gu", "act", "y", "row_w", "logits")
                                            if res.get(n) is not None)) if train else None,
        "gpu_clock": clock,
        "hip_graph": graph_rec,
    }

    # roofline of the dominant call, from the events inside the timed steps
    peak = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_MFMA_TFLOPS
    if args.mxfp8:
        peak = PEAK_FP8_TFLOPS
    nmat = 3 if cfg.act == "swiglu" else 2
    bwd_flops = 2.0 * cfg.P * nmat * 2.0 * cfg.h * cfg.F
    call_flops = {"grouped_ffn": ffn_flops(cfg), "grouped_ffn_bwd": bwd_flops}
    dom = max(live, key=lambda n: live[n])
    rec = recorded_traffic(cfg.name) if dom == "grouped_ffn" and not args.mxfp8 else None
    gk = "grouped_gemm_bf16" if cfg.dtype == "bf16" else "grouped_gemm_f32"
    if args.mxfp8:
        gk = "grouped_gemm_mx (MXFP8)"
    kernels = {"grouped_ffn": "%s %s launch + %s plain launch (one moe_grouped_ffn call)"
                              % (gk, "SwiGLU" if cfg.act == "swiglu" else "GELU", gk),
               "grouped_ffn_bwd": "moe_grouped_ffn_bwd call (SwiGLU backward, data and weight "
                                  "gradient launches)"}
    if args.mxfp8:
        kernels["grouped_ffn"] = ("grouped_gemm_mx SwiGLU launch with the activation quantised in its "
                                  "epilogue + grouped_gemm_mx plain launch (one moe_grouped_ffn_mx call)")
        kernels["grouped_ffn_bwd"] = ("moe_grouped_ffn_bwd_mx call (first projection recomputed, five "
                                      "MXFP8 GEMM launches: three by token segments, two by k-segments; quantisation and SwiGLU-backward passes); "
                                      "algorithmic backward FLOPs only, the recomputation not credited")
    out["roofline"] = {
        "kernel": kernels[dom], "bound": "mfma",
        "achieved": call_flops[dom] / live[dom] / 1e12, "peak": peak, "unit": "TFLOP/s",
        "frac": call_flops[dom] / live[dom] / 1e12 / peak,
        "traffic": rec["traffic_bytes_per_call"] if rec else None,
        "flops_per_call": call_flops[dom], "ms_per_call": live[dom] * 1e3,
        "timing": "HIP events around the call on its stream, mean over the %d timed steps"
                  % args.steps,
    }
    if rec:
        out["roofline"]["traffic_note"] = rec["note"]

    # the stage-by-stage timings cover the top-k dropless chain
    if not args.no_stages and not args.expert_choice and cap is None and not args.mxfp8:
        stream = torch.cuda.current_stream(dev)
        flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        E = cfg.E
        r = B.moe_route(inp["x"], inp["w_gate"], cfg.k, cfg.score, b_gate=inp.get("b_gate"),
                        sel_bias=inp.get("sel_bias"))
        # as layer.forward runs them: inference gathers token rows inside the
        # first GEMM (no dispatch copy); training materialises x_perm
        p = B.moe_permute(inp["x"], r["topk_idx"], E, with_x_perm=train)
        has_sh = inp.get("w1_sh") is not None
        a_in = p["x_perm"] if train else inp["x"]
        g_rows = None if train else p["sorted_token"]
        row_w = B.moe_permute_weights(r["topk_w"], p["row_of"]) if meff else None
        f = B.moe_grouped_ffn(a_in, p["offsets"], inp["w1"], inp["w2"], cfg.act,
                              b1=inp.get("b1"), b2=inp.get("b2"), x_sh=inp["x"] if has_sh else None,
                              w1_sh=inp.get("w1_sh"), w2_sh=inp.get("w2_sh"), gather_rows=g_rows,
                              row_w=row_w)
        calls = {
            "route": lambda: B.moe_route(inp["x"], inp["w_gate"], cfg.k, cfg.score,
                                         b_gate=inp.get("b_gate"), sel_bias=inp.get("sel_bias")),
            "permute": lambda: B.moe_permute(inp["x"], r["topk_idx"], E, with_x_perm=train),
            "grouped_ffn": lambda: B.moe_grouped_ffn(
                a_in, p["offsets"], inp["w1"], inp["w2"], cfg.act, b1=inp.get("b1"),
                b2=inp.get("b2"), x_sh=inp["x"] if has_sh else None, w1_sh=inp.get("w1_sh"),
                w2_sh=inp.get("w2_sh"), gather_rows=g_rows, row_w=row_w),
            "unpermute": lambda: B.moe_unpermute(f["y"], p["row_of"], None if meff else r["topk_w"],
                                                 y_sh=f["y_sh"]),
        }
        if train:
            f2 = layer.forward(inp, cfg.k, cfg.score, cfg.act, keep_for_backward=True,
                               memory_efficient=meff, router_losses=losses)
            if meff:
                gy, _ = B.moe_unpermute_bwd(inp["grad_out"], None, f2["row_of"], None)
                gf = B.moe_grouped_ffn_bwd_recompute(gy, f2["x_perm"], f2["gu"], f2["offsets"],
                                                     inp["w1"], inp["w2"], cfg.act, row_w=f2["row_w"])
                gw = B.moe_permute_weights_bwd(gf["grad_row_w"], f2["row_of"])
                calls["unpermute_bwd"] = lambda: B.moe_unpermute_bwd(inp["grad_out"], None,
                                                                     f2["row_of"], None)
                calls["grouped_ffn_bwd"] = lambda: B.moe_grouped_ffn_bwd_recompute(
                    gy, f2["x_perm"], f2["gu"], f2["offsets"], inp["w1"], inp["w2"], cfg.act,
                    row_w=f2["row_w"])
            else:
                gy, gw = B.moe_unpermute_bwd(inp["grad_out"], f2["y"], f2["row_of"], f2["topk_w"])
                gf = B.moe_grouped_ffn_bwd(gy, f2["x_perm"], f2["act"], f2["gu"], f2["offsets"],
                                           inp["w1"], inp["w2"], cfg.act)
                calls["unpermute_bwd"] = lambda: B.moe_unpermute_bwd(inp["grad_out"], f2["y"],
                                                                     f2["row_of"], f2["topk_w"])
                calls["grouped_ffn_bwd"] = lambda: B.moe_grouped_ffn_bwd(
                    gy, f2["x_perm"], f2["act"], f2["gu"], f2["offsets"], inp["w1"], inp["w2"], cfg.act)
            gr = B.moe_route_bwd(inp["x"], E, f2["topk_idx"], f2["topk_w"], gw, f2["offsets"],
                                 f2["sorted_token"], score=cfg.score, logits=f2["logits"],
                                 want_b_grad=inp.get("b_gate") is not None)
            calls["route_bwd"] = lambda: B.moe_route_bwd(
                inp["x"], E, f2["topk_idx"], f2["topk_w"], gw, f2["offsets"], f2["sorted_token"],
                score=cfg.score, logits=f2["logits"], want_b_grad=inp.get("b_gate") is not None)
            calls["permute_bwd"] = lambda: B.moe_permute_bwd(gf["grad_x_perm"], f2["row_of"],
                                                             gr["grad_logits_sel"], f2["topk_idx"],
                                                             inp["w_gate"])
            if losses:
                gx = torch.zeros_like(inp["x"])
                dl = B.moe_router_losses_bwd(f2["logits"], f2["counts"], cfg.k, COEF_AUX, COEF_Z)
                calls["router_losses"] = lambda: B.moe_router_losses(f2["logits"], f2["counts"], cfg.k)
                calls["router_losses_bwd"] = lambda: B.moe_router_losses_bwd(
                    f2["logits"], f2["counts"], cfg.k, COEF_AUX, COEF_Z)
                calls["router_dense_bwd"] = lambda: B.moe_router_dense_bwd(
                    inp["x"], inp["w_gate"], dl, grad_w_gate=gr["grad_w_gate"],
                    grad_b_gate=gr["grad_b_gate"], grad_x=gx)
        stages = {}
        for name, fn in calls.items():
            fn()
            ts = []
            for _ in range(args.stage_reps):
                flush.fill_(1)     # evict the last-level cache
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn()
                e1.record(stream)
                e1.synchronize()
                ts.append(e0.elapsed_time(e1) * 1e-3)
            stages[name] = {"s_median": float(np.median(ts)), "s_min": float(np.min(ts))}
        sb = stage_bytes(cfg, cfg.P, es)
        hbm_stages = ("route", "permute", "unpermute") if train else ("route", "unpermute")
        if not train:
            # the inference permute moves index arrays only (the first GEMM
            # gathers the token rows): launch latency, not a bandwidth figure
            stages["permute"].update(latency_us=stages["permute"]["s_median"] * 1e6,
                                     index_bytes=sb["permute"],
                                     note="index-only (histogram scan and stable rank): latency-bound")
        for name in hbm_stages:
            t = stages[name]["s_median"]
            stages[name]["gb_per_s"] = sb[name] / t / 1e9
            stages[name]["hbm_frac"] = sb[name] / t / 1e9 / PEAK_HBM_GBS
            stages[name]["algorithmic_bytes"] = sb[name]
        t = stages["grouped_ffn"]["s_median"]
        ff = ffn_flops(cfg)
        stages["grouped_ffn"]["tflops"] = ff / t / 1e12
        stages["grouped_ffn"]["mfma_frac"] = ff / t / 1e12 / peak
        stages["grouped_ffn"]["weight_gb_per_s"] = ffn_weight_bytes(cfg, es) / t / 1e9
        if train:
            tb = stages["grouped_ffn_bwd"]["s_median"]
            stages["grouped_ffn_bwd"]["tflops"] = bwd_flops / tb / 1e12
            stages["grouped_ffn_bwd"]["mfma_frac"] = bwd_flops / tb / 1e12 / peak
        if "router_losses" in stages:
            lb = cfg.T * cfg.E * 4 + cfg.E * 4 + 8       # logits and counts read, losses written
            for name, nbytes in (("router_losses", lb), ("router_losses_bwd", lb + cfg.T * cfg.E * 4)):
                t = stages[name]["s_median"]
                stages[name].update(algorithmic_bytes=nbytes, gb_per_s=nbytes / t / 1e9,
                                    hbm_frac=nbytes / t / 1e9 / PEAK_HBM_GBS)
            # D^T x and D w_gate: 2 T E h FLOP each; with bf16 tokens and a
            # multiple of 32 experts they run as bf16 MFMA products on D split
            # into two bf16 halves (twice the FLOP executed), else as fp32 FMA
            # on the vector ALUs
            fl = 4.0 * cfg.T * cfg.E * cfg.h
            t = stages["router_dense_bwd"]["s_median"]
            st = stages["router_dense_bwd"]
            st.update(flops=fl, tflops=fl / t / 1e12)
            if cfg.dtype == "bf16" and cfg.E % 32 == 0:
                st.update(path="mfma, D as bf16 high + low parts", executed_flops=2 * fl,
                          mfma_frac=2 * fl / t / 1e12 / PEAK_BF16_TFLOPS)
            else:
                st.update(path="vector ALU, fp32", valu_frac=fl / t / 1e12 / PEAK_F32_VALU_TFLOPS)
        out["stages"] = stages
        del flush

    out["hbm_copy_gbs"] = copy_bandwidth(torch)
    if not args.no_cpu_baseline:
        try:
            out["cpu_baseline"] = cpu_baseline(cfg, inp, min(args.cpu_tokens, cfg.T))
            out["cpu_baseline"].update(host_info())
        except Exception as exc:   # report, never hide, a failing baseline
            out["cpu_baseline"] = {"error": repr(exc)}
    variant = (args.memory_efficient or args.capacity_factor is not None or args.expert_choice or args.mxfp8
               or args.router_losses)
    if args.config == 2 and not variant and not args.no_configs:
        del inp, res
        torch.cuda.empty_cache()
        out["configs"] = {}
        for cid in SUB_CONFIGS:
            print("sub-record %s" % wl.CONFIGS[cid].name, file=sys.stderr, flush=True)
            out["configs"][wl.CONFIGS[cid].name] = sub_record(
                torch, layer, wl, cid, args.config_steps, 2, args.config_cpu_tokens, not args.no_cpu_baseline)
        for cid in MX_SUB_CONFIGS:
            name = wl.CONFIGS[cid].name + "_mxfp8"
            print("sub-record %s" % name, file=sys.stderr, flush=True)
            out["configs"][name] = sub_record(torch, layer, wl, cid, args.config_steps, 2, 0, False, mx=True)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
