#!/usr/bin/env python3
"""Benchmark of the fused MoE layer on one MI355X.

One step = one forward + backward pass of the whole layer (router, counting
sort, dispatch, grouped SwiGLU GEMMs, combine, and the mirrored backward) over
one batch of synthetic tokens already resident in HBM.  Default workload:
T=8192 tokens, d=4096, E=128 experts, top-8, F=1536, Zipf(1.2) expert
popularity, bf16 with fp32 accumulation.

Prints one JSON line: tokens/s for the whole job, the roofline position of the
dominant kernel (timed with HIP events recorded by the library around each of
its stages, on the stream the kernels run on), grouped-GEMM TFLOP/s per GEMM,
and the CPU oracle timed on a bounded sample of the same workload."""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer tokens/s fwd+bwd (BF16, MXFP8) + grouped-GEMM % MFMA peak, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "mxfp8": 5000.0, "mxfp4": 10100.0, "f32": 157.3}
PEAK_HBM_GBS = 8000.0


class HipEvents:
    """hipEvent_t handles through the HIP runtime (the library records them)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = (ctypes.c_void_p * n)()
        for i in range(n):
            ev = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(ev)) == 0
            out[i] = ev
        return out

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventSynchronize(b) == 0
        r = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        return ms.value if r == 0 else float("nan")


def stage_work(w, P, U, save_for_backward=True, mxfp8_wgrad=False):
    """Algorithmic work of one launch of each stage: FLOPs for the GEMMs,
    HBM bytes for every stage (each operand read once, each output written
    once; a GEMM's weights are those of the E_loc local experts).  With
    mxfp8_wgrad the weight gradients read MXFP8 operands quantised along the
    rows, which the regather stage writes from dout (dY rebuilt with the
    gates), the bf16 H and [dA | dB], and the x rows."""
    d, F, E, k, T = w.d, w.F, w.E, w.k, U
    El = w.e_end - w.expert_begin
    s = 4 if w.precision == "f32" else 2
    flops = {"gemm_up": 4.0 * P * d * F, "gemm_down": 2.0 * P * F * d, "gemm_dh": 2.0 * P * d * F,
             "gemm_dx": 4.0 * P * F * d, "gemm_dw2": 2.0 * P * d * F, "gemm_dw13": 4.0 * P * F * d}
    nbytes = {"router": T * E * 4 + T * k * 8 * 2 + T * 4,
              "dispatch": (U + P) * d * s, "regather": (U + P) * d * s,
              "combine": P * d * s + T * d * s + P * 8,
              "bwd_gate": T * d * s + 2 * P * d * s + 2 * T * E * 4 + P * 8,
              "reduce_dx": P * d * s + T * d * s + P * 4,
              "sort": T * k * 4 * 4 + P * 4}
    # GEMM operands: bf16 (or fp32) elements, or MXFP8 codes (MXFP4: half a
    # byte) plus one E8M0 scale per 32; fp32 weight gradients.
    mx = w.precision in ("mxfp8", "mxfp4")
    q = (0.5 if w.precision == "mxfp4" else 1) + 1 / 32 if mx else s
    # MXFP8: the dispatch writes MXFP8 rows; UP also saves H before its
    # quantisation; the reverse-combine also writes dY in MXFP8; DH and DX read
    # MXFP8 operands, and DH writes [dA | dB] both as bf16 (for the weight
    # gradients) and as MXFP8 (for DX)
    saved_up = (3 if mx else 2) * P * F * s if save_for_backward else 0
    if mx:
        nbytes["bwd_gate"] += P * d * q
        nbytes["dispatch"] = U * d * s + P * d * q
    gemm_bytes = {
        "gemm_up": P * d * q + 2 * El * F * d * q + P * F * q + saved_up,
        "gemm_down": P * F * q + El * d * F * q + P * d * s,
        "gemm_dh": P * d * q + El * d * F * q + 2 * P * F * s + 2 * P * F * s + (2 * P * F * q if mx else 0),
        "gemm_dx": 2 * P * F * q + 2 * El * F * d * q + P * d * s,
        "gemm_dw2": P * d * s + P * F * s + El * d * F * 4,
        "gemm_dw13": 2 * P * F * s + P * d * s + 2 * El * F * d * 4,
    }
    if mx and mxfp8_wgrad:
        gemm_bytes["gemm_dw2"] = P * d * q + P * F * q + El * d * F * 4
        gemm_bytes["gemm_dw13"] = 2 * P * F * q + P * d * q + 2 * El * F * d * 4
        # dY is formed again from dout (U token rows) and the gates, so the
        # reverse-combine writes no bf16 dY rows
        nbytes["regather"] = (P * F + 2 * P * F) * s + 2 * U * d * s + (2 * d + 3 * F) * P * q
        nbytes["bwd_gate"] -= P * d * s
    nbytes.update(gemm_bytes)
    return flops, nbytes


def gemm_peak(precision: str, name: str, mxfp8_wgrad: bool = False) -> float:
    """Dense MFMA peak of one GEMM: in an MXFP8 layer the forward GEMMs and
    the two backward products that lead to dx run on scaled MFMA (MXFP8
    peak); the weight-gradient GEMMs stay bf16 unless mxfp8_wgrad."""
    if precision == "mxfp8":
        if name in ("gemm_dw2", "gemm_dw13") and not mxfp8_wgrad:
            return PEAK_TFLOPS["bf16"]
        return PEAK_TFLOPS["mxfp8"]
    return PEAK_TFLOPS[precision]  # MXFP4: forward only, both products on E2M1 operands


def roof_of(flops_n, bytes_n, ms, peak_tflops):
    """Roofline position of one launch: the bound is whichever of the MFMA
    time (FLOPs / peak) and the HBM time (bytes / 8 TB/s) is longer."""
    t_mfma = flops_n / (peak_tflops * 1e12) if flops_n else 0.0
    t_hbm = bytes_n / (PEAK_HBM_GBS * 1e9)
    if t_mfma >= t_hbm:
        ach = flops_n / (ms * 1e-3) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": peak_tflops, "unit": "TFLOP/s",
                "frac": round(ach / peak_tflops, 4)}
    ach = bytes_n / (ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(ach / PEAK_HBM_GBS, 4)}


TRAFFIC_FILES = {"bf16_train": os.path.join(ROOT, "profiles", "grouped_gemm_bf16_train_hbm_traffic.md"),
                 "mxfp8_train": os.path.join(ROOT, "profiles", "grouped_gemm_mxfp8_train_hbm_traffic.md")}


def measured_traffic(workload: str, stage: str):
    """HBM bytes per launch of `stage` from the committed FETCH_SIZE/WRITE_SIZE
    record of this workload (calibrated counter passes on the same inputs), or
    None when there is no record for this workload and kernel or the kernel
    sources changed since it was taken."""
    import hashlib
    import re
    if workload not in TRAFFIC_FILES:
        return None
    try:
        text = open(TRAFFIC_FILES[workload]).read()
        rec = json.loads(re.search(r"```json\n(.*?)\n```", text, re.S).group(1))
    except (OSError, AttributeError, ValueError):
        return None
    if rec.get("workload") != workload or stage not in rec.get("per_launch", {}):
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        try:
            h.update(open(os.path.join(ROOT, src), "rb").read())
        except OSError:
            return None
    if h.hexdigest()[:16] != rec["source_sha256_16"]:
        return None
    return rec["per_launch"][stage]["traffic_bytes"]


def cpu_baseline(w, inp, sample_tokens: int):
    """The oracle (float64 numpy) on the first `sample_tokens` tokens with
    their full routing, forward + backward; tokens/s = sample / seconds."""
    import numpy as np
    from oracle import mok_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        cores = os.cpu_count() or 1
    S = min(sample_tokens, inp["x"].shape[0])
    x = inp["x"][:S].float().cpu().numpy()
    lg = inp["logits"][:S].cpu().numpy()
    g = inp["dout"][:S].float().cpu().numpy() if "dout" in inp else None
    W1 = inp["W1"].float().cpu().numpy()
    W3 = inp["W3"].float().cpu().numpy()
    W2 = inp["W2"].float().cpu().numpy()
    t0 = time.perf_counter()
    fw = O.forward(x, lg, W1, W3, W2, w.k, w.expert_begin, w.e_end)
    if g is not None:
        O.backward(g, x, lg, W1, W3, W2, w.k, fw, w.expert_begin, w.e_end)
    dt = time.perf_counter() - t0
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": S / dt, "unit": "tokens/s", "cores": int(cores), "kind": "oracle",
            "nproc": os.cpu_count(), "cpu_model": model,
            "scaling": "the oracle's work is linear in the tokens (each token's pairs, plus the per-expert "
                       "weight gradients over the sampled rows), so tokens/s carries over to the full step",
            "sample": f"first {S} of {inp['x'].shape[0]} tokens with all their top-{w.k} pairs, "
                      f"{'forward+backward' if g is not None else 'forward'}, float64 numpy oracle, "
                      f"{dt:.1f} s"}


def router_gemm_bench(w, x, K, Wm, ev, sh):
    """The router GEMM logits = x Wr^T and its backward (dx, dWr) at this
    workload's T, d, E with a synthetic Wr and dlogits, timed apart from the
    layer step (the layer takes the logits as an input).  Roofline per call:
    algorithmic bytes = each operand read once and each output written once;
    flops = 2 T d E per product; bound = the longer of HBM and bf16 MFMA time."""
    import torch

    import workloads as W
    from mixture_experts_layer_34_amd import mok

    T, d = x.shape
    E = w.E
    r = W.make_router_inputs(w.seed, 1, d, E, device=x.device)
    Wr = r["Wr"]
    g = W.normal(w.seed, W.S_DLOGIT, torch.arange(T, device=x.device), E)
    logits = torch.empty((T, E), dtype=torch.float32, device=x.device)
    dx = torch.empty((T, d), dtype=torch.float32, device=x.device)
    dWr = torch.empty((E, d), dtype=torch.float32, device=x.device)
    fwd = lambda: mok.mok_router_logits(x, Wr, T, d, E, logits, sh)
    bwd = lambda: mok.mok_router_logits_backward(x, Wr, g, T, d, E, dx, dWr, sh)
    out = {"shape": f"T={T} d={d} E={E}"}
    for name, fn, flops, nbytes in (
            ("forward", fwd, 2.0 * T * d * E, T * d * 2 + E * d * 2 + T * E * 4),
            ("backward", bwd, 4.0 * T * d * E, T * E * 4 + E * d * 2 + T * d * 2 + T * d * 4 + E * d * 4)):
        for _ in range(Wm):
            fn()
        a, b = ev.create(2)
        ev.record(a, sh)
        for _ in range(K):
            fn()
        ev.record(b, sh)
        ms = ev.elapsed_ms(a, b) / K
        roof = roof_of(flops, nbytes, ms, PEAK_TFLOPS["bf16"])
        out[name] = {"ms": round(ms, 4), "bound": roof["bound"], "achieved": roof["achieved"], "unit": roof["unit"],
                     "frac": roof["frac"], "per_call": f"{flops / 1e9:.2f} GFLOP, {nbytes / 1e6:.1f} MB"}
    torch.cuda.synchronize()
    return out


def fused_router_bench(w, inp, K, Wm, ev, sh):
    """The layer's forward (nothing saved) with the router GEMM in front, at
    this workload's shape: mok_router_logits followed by mok_moe_forward,
    against mok_moe_forward_router (for E <= 128 the GEMM and the router
    step in one kernel).  Milliseconds per call, eager launches."""
    import torch

    import workloads as W
    from mixture_experts_layer_34_amd.layer import MoeBuffers, MoeShape, router_logits

    x = inp["x"]
    T, d = x.shape
    Wr = W.make_router_inputs(w.seed, 1, w.d, w.E, device=x.device)["Wr"]
    buf = MoeBuffers(MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision=w.precision), device=x.device)
    logits = torch.empty((T, w.E), dtype=torch.float32, device=x.device)

    def separate():
        router_logits(x, Wr, out=logits)
        buf.forward(x, logits, inp["W1"], inp["W3"], inp["W2"], stream=sh)

    def fused():
        buf.forward_router(x, Wr, inp["W1"], inp["W3"], inp["W2"], logits=logits, stream=sh)

    out = {"shape": f"T={T} d={w.d} E={w.E} k={w.k} F={w.F}, {w.precision}, forward only"}
    for name, fn in (("router_gemm_then_forward", separate), ("forward_router", fused)):
        for _ in range(Wm):
            fn()
        torch.cuda.synchronize()
        a, b = ev.create(2)
        ev.record(a, sh)
        for _ in range(K):
            fn()
        ev.record(b, sh)
        out[name] = {"ms": round(ev.elapsed_ms(a, b) / K, 4)}
    out["saved_ms"] = round(out["router_gemm_then_forward"]["ms"] - out["forward_router"]["ms"], 4)
    del buf
    torch.cuda.synchronize()
    return out


def measure(name: str, args, extras: bool):
    """Times `steps` layer steps of one workload (after `warmup` untimed
    ones); `extras` adds the copy calibration and the graph-replay timing.
    Returns the result record, the workload, its inputs and the timing
    handles (for the router GEMM and the CPU baseline)."""
    import torch

    import workloads as W
    from mixture_experts_layer_34_amd import mok
    from mixture_experts_layer_34_amd.layer import (MoeBuffers, MoeShape, quantize_mxfp4, quantize_mxfp8,
                                                    quantize_mxfp8_backward_weights)

    w = W.get(name)
    backward = w.backward and not args.forward_only
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = W.make_inputs(w, device=dev)
    T = inp["x"].shape[0]
    mxw = w.precision == "mxfp8" and backward and getattr(args, "mxfp8_wgrad", False)
    shape = MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision=w.precision, expert_begin=w.expert_begin,
                     expert_end=w.e_end, save_for_backward=backward, minibatch_rows=args.minibatch_rows,
                     ring_bytes=(args.ring_mib << 20) if args.minibatch_rows else 0, mxfp8_wgrad=mxw,
                     mover_cus=getattr(args, "mover_cus", 0) if args.minibatch_rows else 0)
    buf = MoeBuffers(shape, device=dev)
    W1, W3, W2, scales = inp["W1"], inp["W3"], inp["W2"], None
    if w.precision in ("mxfp8", "mxfp4"):
        quant = quantize_mxfp8 if w.precision == "mxfp8" else quantize_mxfp4
        q1, s1 = quant(W1)
        q3, s3 = quant(W3)
        q2, s2 = quant(W2)
        W1, W3, W2 = q1, q3, q2
        scales = torch.cat([s1.reshape(-1), s3.reshape(-1), s2.reshape(-1)])
    wt = (quantize_mxfp8_backward_weights(inp["W1"], inp["W3"], inp["W2"])
          if w.precision == "mxfp8" and backward else None)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    if args.copy_calibration_mib and extras:
        n = args.copy_calibration_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    ev = HipEvents()
    K, Wm = args.steps, args.warmup
    stage_ev = [ev.create(2 * mok.MOK_NUM_STAGES) for _ in range(K)]
    start, stop = ev.create(2)

    def bwd(stream=None):
        if wt is not None:
            buf.backward_mxfp8(inp["dout"], inp["x"], inp["logits"], wt, stream=stream)
        else:
            buf.backward(inp["dout"], inp["x"], inp["logits"], inp["W1"], inp["W3"], inp["W2"], stream=stream)

    def step(events=None):
        buf.cfg.stage_events = ctypes.cast(events, ctypes.c_void_p) if events is not None else None
        buf.forward(inp["x"], inp["logits"], W1, W3, W2, scales, stream=sh)
        if backward:
            bwd(sh)

    for _ in range(Wm):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(start, sh)
    for i in range(K):
        step(stage_ev[i])
    ev.record(stop, sh)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = ev.elapsed_ms(start, stop)
    buf.cfg.stage_events = None
    ms_step = ms_total / K

    # The same step captured once into a HIP graph and replayed K times (the
    # library only enqueues kernels, so it captures as is): the launch gaps
    # between the layer's kernels are gone.
    graph_res = None
    if not args.no_graph:
        side = torch.cuda.Stream(dev)
        side.wait_stream(torch.cuda.current_stream(dev))
        with torch.cuda.stream(side):
            buf.cfg.stage_events = None
            buf.forward(inp["x"], inp["logits"], W1, W3, W2, scales)
            if backward:
                bwd()
        torch.cuda.current_stream(dev).wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            buf.forward(inp["x"], inp["logits"], W1, W3, W2, scales)
            if backward:
                bwd()
        graph.replay()
        torch.cuda.synchronize()
        g0, g1 = ev.create(2)
        tg = time.perf_counter()
        ev.record(g0, sh)
        for _ in range(K):
            graph.replay()
        ev.record(g1, sh)
        g_ms = ev.elapsed_ms(g0, g1)
        torch.cuda.synchronize()
        graph_res = {"ms_per_step": round(g_ms / K, 4), "tokens_per_s": round(T * K / (g_ms * 1e-3), 1),
                     "wall_s": round(time.perf_counter() - tg, 3)}
        del graph

    # Cold steps: a 512 MiB device write before each step evicts the 256 MB
    # last-level cache (MALL), so weights and activations come from HBM; each
    # step timed alone, the median reported.
    cold_res = None
    if extras and not args.no_cold:
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        ce = [ev.create(2) for _ in range(K)]
        for i in range(K):
            flush.fill_(i & 0xFF)
            ev.record(ce[i][0], sh)
            step()
            ev.record(ce[i][1], sh)
        vals = sorted(ev.elapsed_ms(a, b) for a, b in ce)
        med = vals[len(vals) // 2]
        cold_res = {"ms_per_step_median": round(med, 4), "tokens_per_s": round(T / (med * 1e-3), 1),
                    "flush": "512 MiB device write before each step, outside the timed events"}
        del flush
        torch.cuda.synchronize()

    # per-stage averages over the timed steps
    stages = {}
    ran = mok.STAGES if backward else mok.STAGES[:mok.STAGES.index("combine") + 1]
    for s, name in enumerate(mok.STAGES):
        if name not in ran:
            continue  # never recorded: asking for its time would be an error
        vals = [ev.elapsed_ms(stage_ev[i][2 * s], stage_ev[i][2 * s + 1]) for i in range(K)]
        stages[name] = sum(vals) / len(vals)
    P = int(buf.offsets[-1].item())
    U = int((buf.topk_idx.ge(w.expert_begin) & buf.topk_idx.lt(w.e_end)).any(dim=1).sum().item())
    flops, nbytes = stage_work(w, P, U, save_for_backward=backward, mxfp8_wgrad=mxw)
    if w.precision == "bf16" and not args.minibatch_rows and T * w.d * 2 < (1 << 31):
        # the library fuses the dispatch into the UP GEMM's loads (pull
        # dispatch): the stage is recorded empty and moves no bytes of its own
        nbytes.pop("dispatch", None)
    dom = max(stages, key=stages.get)
    roof = roof_of(flops.get(dom, 0.0), nbytes[dom], stages[dom], gemm_peak(w.precision, dom, mxw))
    roof.update({"traffic": measured_traffic(w.name, dom) if dom in flops and not args.minibatch_rows else None,
                 "kernel": dom, "avg_ms": round(stages[dom], 4),
                 "per_launch": (f"{flops[dom] / 1e9:.1f} GFLOP, " if dom in flops else "")
                 + f"{nbytes[dom] / 1e6:.1f} MB"})
    gemm = {n: {"ms": round(stages[n], 4), "tflops": round(flops[n] / (stages[n] * 1e-3) / 1e12, 1),
                "frac_peak": round(flops[n] / (stages[n] * 1e-3) / 1e12 / gemm_peak(w.precision, n, mxw), 4),
                "roof": {k_: v for k_, v in roof_of(flops[n], nbytes[n], stages[n],
                                                    gemm_peak(w.precision, n, mxw)).items()
                         if k_ in ("bound", "frac")}}
            for n in flops if n in stages}
    gemm_ms = sum(stages[n] for n in flops if n in stages)
    gemm_flops = sum(flops[n] for n in flops if n in stages)
    # the GEMMs' combined peak: their FLOPs over the time they would take,
    # each at its own peak
    gemm_peak_all = gemm_flops / sum(flops[n] / gemm_peak(w.precision, n, mxw) for n in flops if n in stages)
    hbm = {n: {"ms": round(stages[n], 4), "gbs": round(nbytes[n] / (stages[n] * 1e-3) / 1e9, 1)}
           for n in nbytes if n in stages and n not in flops}

    eager = {"ms_per_step": round(ms_step, 4), "tokens_per_s": round(T * K / (ms_total * 1e-3), 1),
             "wall_s": round(wall, 3)}
    # the faster of the two launch modes is the headline (both run the same
    # work): the replay wins on the training step, eager launches on the short
    # forward-only steps, where the replay adds gaps between the kernels
    use_graph = graph_res is not None and graph_res["ms_per_step"] < eager["ms_per_step"]
    head = graph_res if use_graph else eager
    result = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1, "steps": K, "warmup": Wm,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.precision, "data": "synthetic",
        "config": {"workload": f"{w.name}: T={T} d={w.d} E={w.E} k={w.k} F={w.F} "
                               f"local experts [{w.expert_begin},{w.e_end}) pairs P={P}, "
                               f"{'forward+backward' if backward else 'forward'}"
                               + (f", ring pipeline R={args.minibatch_rows} rows, {args.ring_mib} MiB ring"
                                  + (f", {args.mover_cus} copy-only CUs" if getattr(args, "mover_cus", 0) else "")
                                  if args.minibatch_rows else ""),
                   "global_batch": T, "parallelism": "none (1 GPU)",
                   "launch": "the whole step replayed from a HIP graph" if use_graph
                   else "eager launches on one stream"},
        "roofline": roof,
        "grouped_gemm": {"tflops": round(gemm_flops / (gemm_ms * 1e-3) / 1e12, 1),
                         "frac_peak": round(gemm_flops / (gemm_ms * 1e-3) / 1e12 / gemm_peak_all, 4),
                         "per_gemm": gemm},
        "data_movement": hbm,
        "stages_ms": {k_: round(v, 4) for k_, v in stages.items()},
        "graph_replay": graph_res,
        "eager": eager,
        "cold": cold_res,
        "wall_s": round(wall, 3),
    }
    return result, w, inp, (K, Wm, ev, sh)


def decode_latency(w, inp, K, ev, sh, Ts=(1, 16, 64, 256)):
    """Forward-only calls of a few tokens on the training layer's weights (a
    decode step), microseconds per call, eagerly and replayed from a HIP
    graph: the small-call path (router and sort in one launch up to T 32,
    weight-streaming UP and DOWN up to 4096 pairs) against the tiled GEMMs
    with separate router and sort launches; the same calls with the weights
    in MXFP8 (eager).  For the small-call path also
    the per-stage times (library stage events) and the HBM roofline of the
    two GEMMs: the weights of the experts the call touches, read once, plus
    their activation rows, over 8 TB/s."""
    import torch

    import workloads as W
    from mixture_experts_layer_34_amd import mok
    from mixture_experts_layer_34_amd.layer import MoeBuffers, MoeShape

    dev = inp["x"].device
    n = max(K, 50)
    out = {}
    mx_w = {}
    if w.d % 256 == 0 and w.F % 256 == 0:
        from mixture_experts_layer_34_amd.layer import quantize_mxfp4, quantize_mxfp8
        for prec, quant in (("mxfp8", quantize_mxfp8), ("mxfp4", quantize_mxfp4)):
            q = [quant(inp[nm]) for nm in ("W1", "W3", "W2")]
            mx_w[prec] = (q[0][0], q[1][0], q[2][0], torch.cat([sc.reshape(-1) for _, sc in q]))
    for T in Ts:
        wT = W.scaled(w.name, T=T)
        small = W.make_inputs(wT, device=dev, weights=False)
        row = {"pairs": T * w.k}
        for tag, tiled in (("small_path", False), ("tiled", True)):
            buf = MoeBuffers(MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision=w.precision,
                                      separate_route_sort=tiled, gemm_path="tiled" if tiled else "auto"),
                             device=dev)

            def fwd(events=None, stream=sh):
                buf.cfg.stage_events = ctypes.cast(events, ctypes.c_void_p) if events is not None else None
                buf.forward(small["x"], small["logits"], inp["W1"], inp["W3"], inp["W2"], stream=stream)

            for _ in range(5):
                fwd()
            torch.cuda.synchronize()
            a, b = ev.create(2)
            ev.record(a, sh)
            for _ in range(n):
                fwd()
            ev.record(b, sh)
            rec = {"us": round(ev.elapsed_ms(a, b) * 1e3 / n, 2)}
            if not tiled:
                st = [ev.create(2 * mok.MOK_NUM_STAGES) for _ in range(n)]
                for i in range(n):
                    fwd(st[i])
                torch.cuda.synchronize()
                ran = ["router", "gemm_up", "gemm_down", "combine"] + (["sort"] if T > 32 else [])
                stage_us = {g: round(sum(ev.elapsed_ms(st[i][2 * mok.STAGES.index(g)],
                                                       st[i][2 * mok.STAGES.index(g) + 1])
                                         for i in range(n)) * 1e3 / n, 2) for g in ran}
                rec["stages_us"] = stage_us
                buf.cfg.stage_events = None
                counts = buf.counts.cpu()
                ne = int((counts > 0).sum())
                P = int(counts.sum())
                up_b = ne * 2 * w.F * w.d * 2 + T * w.d * 2 + P * w.F * 2
                dn_b = ne * w.d * w.F * 2 + P * w.F * 2 + P * w.d * 2
                rec["experts_touched"] = ne
                rec["gemm_hbm"] = {
                    "up": {"bytes": up_b, "gbs": round(up_b / (stage_us["gemm_up"] * 1e-6) / 1e9, 1),
                           "frac": round(up_b / (stage_us["gemm_up"] * 1e-6) / (PEAK_HBM_GBS * 1e9), 4)},
                    "down": {"bytes": dn_b, "gbs": round(dn_b / (stage_us["gemm_down"] * 1e-6) / 1e9, 1),
                             "frac": round(dn_b / (stage_us["gemm_down"] * 1e-6) / (PEAK_HBM_GBS * 1e9), 4)}}
                floor = (ne * 3 * w.F * w.d * 2 + 2 * T * w.d * 2) / (PEAK_HBM_GBS * 1e9) * 1e6
                rec["floor_us"] = round(floor, 2)
            side = torch.cuda.Stream(dev)
            side.wait_stream(torch.cuda.current_stream(dev))
            with torch.cuda.stream(side):
                fwd(stream=side.cuda_stream)
            torch.cuda.current_stream(dev).wait_stream(side)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                fwd(stream=torch.cuda.current_stream(dev).cuda_stream)
            graph.replay()
            torch.cuda.synchronize()
            a, b = ev.create(2)
            ev.record(a, sh)
            for _ in range(n):
                graph.replay()
            ev.record(b, sh)
            rec["graph_us"] = round(ev.elapsed_ms(a, b) * 1e3 / n, 2)
            del graph, buf
            row[tag] = rec
        row["speedup"] = round(row["tiled"]["us"] / row["small_path"]["us"], 3)
        for prec, mw in mx_w.items():
            # the same calls with MXFP8 or MXFP4 weights (inference: nothing
            # saved); for the small path also the two GEMMs' stage times and
            # their HBM bytes (codes of half a byte or one byte per weight,
            # plus one scale byte per 32)
            qb = (0.5 if prec == "mxfp4" else 1.0) + 1 / 32
            for tag, tiled in ((f"{prec}_small_path", False), (f"{prec}_tiled", True)):
                buf = MoeBuffers(MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision=prec,
                                          separate_route_sort=tiled, gemm_path="tiled" if tiled else "auto"),
                                 device=dev)

                def fwd_mx(events=None, stream=sh):
                    buf.cfg.stage_events = ctypes.cast(events, ctypes.c_void_p) if events is not None else None
                    buf.forward(small["x"], small["logits"], mw[0], mw[1], mw[2], mw[3], stream=stream)

                for _ in range(5):
                    fwd_mx()
                torch.cuda.synchronize()
                a, b = ev.create(2)
                ev.record(a, sh)
                for _ in range(n):
                    fwd_mx()
                ev.record(b, sh)
                rec = {"us": round(ev.elapsed_ms(a, b) * 1e3 / n, 2)}
                if not tiled:
                    st = [ev.create(2 * mok.MOK_NUM_STAGES) for _ in range(n)]
                    for i in range(n):
                        fwd_mx(st[i])
                    torch.cuda.synchronize()
                    ran = ["router", "dispatch", "gemm_up", "gemm_down", "combine"] + (["sort"] if T > 32 else [])
                    stage_us = {g: round(sum(ev.elapsed_ms(st[i][2 * mok.STAGES.index(g)],
                                                           st[i][2 * mok.STAGES.index(g) + 1])
                                             for i in range(n)) * 1e3 / n, 2) for g in ran}
                    buf.cfg.stage_events = None
                    rec["stages_us"] = stage_us
                    counts = buf.counts.cpu()
                    ne = int((counts > 0).sum())
                    P = int(counts.sum())
                    up_b = ne * 2 * w.F * w.d * qb + P * w.d * qb + P * w.F * qb
                    dn_b = ne * w.d * w.F * qb + P * w.F * qb + P * w.d * 2
                    rec["gemm_hbm"] = {
                        "up": {"bytes": int(up_b), "gbs": round(up_b / (stage_us["gemm_up"] * 1e-6) / 1e9, 1),
                               "frac": round(up_b / (stage_us["gemm_up"] * 1e-6) / (PEAK_HBM_GBS * 1e9), 4)},
                        "down": {"bytes": int(dn_b), "gbs": round(dn_b / (stage_us["gemm_down"] * 1e-6) / 1e9, 1),
                                 "frac": round(dn_b / (stage_us["gemm_down"] * 1e-6) / (PEAK_HBM_GBS * 1e9), 4)}}
                row[tag] = rec
                del buf
            row[f"{prec}_speedup"] = round(row[f"{prec}_tiled"]["us"] / row[f"{prec}_small_path"]["us"], 3)
        out[str(T)] = row
    return {"workload": f"{w.name} weights (d={w.d} E={w.E} k={w.k} F={w.F}), forward only, T tokens per call",
            "calls": n, "per_T": out}


def inference_legs(args):
    """The training layer's forward alone (nothing saved, T 8192) with the
    weights in MXFP8 and in MXFP4: throughput, stage times and the GEMMs'
    MFMA fractions of their own peaks."""
    import torch
    out = {}
    for name in ("mxfp8_infer", "mxfp4_infer"):
        a2 = argparse.Namespace(**vars(args))
        a2.forward_only = True
        a2.no_cold = True
        r, _, _, _ = measure(name, a2, extras=False)
        out[name] = {k_: r[k_] for k_ in ("value", "unit", "ms_per_step", "dtype", "roofline", "grouped_gemm",
                                          "stages_ms")}
        out[name]["config"] = r["config"]["workload"]
        torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="bf16_train")
    ap.add_argument("--forward-only", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=512)
    ap.add_argument("--minibatch-rows", type=int, default=0,
                    help="ring pipeline minibatch rows R (0 = whole layer at once)")
    ap.add_argument("--ring-mib", type=int, default=256, help="ring buffer size with --minibatch-rows")
    ap.add_argument("--mover-cus", type=int, default=0,
                    help="with --minibatch-rows: workgroups that only copy rows (0 = one shared task queue)")
    ap.add_argument("--mover-sweep", type=lambda v: [int(x) for x in v.split(",") if x], default=[16, 32],
                    help="mover_cus values timed at R = 1024 in the ring sweep (comma list; empty: none)")
    ap.add_argument("--ring-sweep", type=lambda v: [int(x) for x in v.split(",") if x], default=[512, 1024, 2048],
                    help="minibatch sizes R of the ring-pipeline sweep after the headline (comma list; empty: none)")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the extra timing of the same step captured in a HIP graph")
    ap.add_argument("--no-cold", action="store_true",
                    help="skip the extra timing of steps that start with the last-level cache flushed")
    ap.add_argument("--no-mxfp8", action="store_true",
                    help="skip the MXFP8 forward+backward leg after the bf16 training workload")
    ap.add_argument("--mxfp8-wgrad", action="store_true",
                    help="with --workload mxfp8_train: MXFP8 weight gradients (MOK_FLAG_MXFP8_WGRAD)")
    ap.add_argument("--no-mxfp8-bf16-wgrad", action="store_true",
                    help="skip the comparison run of the MXFP8 step with bf16 weight gradients")
    ap.add_argument("--no-inference", action="store_true",
                    help="skip the forward-only MXFP8 / MXFP4 legs at the training shape")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip the forward-only few-token latency leg after the bf16 training workload")
    ap.add_argument("--decode-tokens", type=lambda v: [int(x) for x in v.split(",") if x], default=[1, 16, 64, 256],
                    help="tokens per call of the few-token latency leg (comma list)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this size first (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.minibatch_rows >= 4096 or any(r >= 4096 for r in args.ring_sweep):
        # a run of the training layer at R = 4096 faulted the GPU under an
        # earlier, withdrawn ring kernel with no cause shown: not run
        print("bench.py: ring minibatches of 4096 rows or more are not run", file=sys.stderr)
        sys.exit(2)

    import torch

    result, w, inp, (K, Wm, ev, sh) = measure(args.workload, args, extras=True)
    if inp["x"].dtype == torch.bfloat16 and not args.minibatch_rows:
        result["router_gemm"] = router_gemm_bench(w, inp["x"], K, Wm, ev, sh)
        if w.precision == "bf16":
            result["router_gemm"]["fused_into_layer"] = fused_router_bench(w, inp, K, Wm, ev, sh)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_sample_tokens)
    else:
        result["cpu_baseline"] = None
    if args.workload == "bf16_train" and args.ring_sweep and not (args.minibatch_rows or args.forward_only):
        # the same training step with the forward as the ring pipeline (one
        # persistent kernel over minibatches of at most R rows drawn from a
        # fixed ring buffer of --ring-mib MiB), per R
        sweep = {}
        for R in args.ring_sweep:
            a2 = argparse.Namespace(**vars(args))
            a2.minibatch_rows = R
            a2.no_cold = True
            rr, _, _, _ = measure("bf16_train", a2, extras=False)
            sweep[str(R)] = {"ms_per_step": rr["ms_per_step"], "tokens_per_s": rr["value"],
                             "vs_whole_layer": round(result["ms_per_step"] / rr["ms_per_step"], 4),
                             "forward_pipeline_ms": rr["stages_ms"].get("gemm_up"),
                             "launch": rr["config"]["launch"]}
            torch.cuda.empty_cache()
        split = {}
        if 1024 in args.ring_sweep:
            # an explicit split of the compute units between copying and the
            # tiles, against the shared queue (mover_cus = 0) at the same R
            for mc in args.mover_sweep:
                a2 = argparse.Namespace(**vars(args))
                a2.minibatch_rows, a2.mover_cus, a2.no_cold = 1024, mc, True
                rr, _, _, _ = measure("bf16_train", a2, extras=False)
                split[str(mc)] = {"ms_per_step": rr["ms_per_step"],
                                  "forward_pipeline_ms": rr["stages_ms"].get("gemm_up")}
                torch.cuda.empty_cache()
        result["ring_sweep"] = {"ring_mib": args.ring_mib, "per_R": sweep,
                                "mover_split_R1024": split,
                                "whole_layer_forward_ms": round(sum(result["stages_ms"].get(n, 0.0) for n in
                                                                    ("dispatch", "gemm_up", "gemm_down",
                                                                     "combine")), 4)}
    if args.workload == "bf16_train" and not (args.no_decode or args.minibatch_rows or args.forward_only):
        result["decode_latency"] = decode_latency(w, inp, K, ev, sh, args.decode_tokens)
        torch.cuda.empty_cache()
    if args.workload == "bf16_train" and not (args.no_inference or args.minibatch_rows or args.forward_only):
        result["inference"] = inference_legs(args)
    if args.workload == "bf16_train" and not (args.no_mxfp8 or args.minibatch_rows or args.forward_only):
        # the MXFP8 leg of the metric: the same layer, inputs and routing with
        # MXFP8 forward GEMMs and MXFP8 dx products in the backward
        del inp
        torch.cuda.empty_cache()
        a2 = argparse.Namespace(**vars(args))
        a2.mxfp8_wgrad = True
        mx, _, _, _ = measure("mxfp8_train", a2, extras=False)
        result["mxfp8_train"] = {k_: mx[k_] for k_ in ("value", "unit", "ms_per_step", "dtype", "roofline",
                                                        "grouped_gemm", "data_movement", "stages_ms", "eager")}
        result["mxfp8_train"]["config"] = mx["config"]["workload"] + ", MXFP8 weight gradients"
        torch.cuda.empty_cache()
        if not args.no_mxfp8_bf16_wgrad:
            # the same MXFP8 step with the weight gradients in bf16 (the
            # backward's products that lead to dx stay MXFP8)
            a2.mxfp8_wgrad = False
            mb, _, _, _ = measure("mxfp8_train", a2, extras=False)
            result["mxfp8_train"]["bf16_weight_gradients"] = {
                "ms_per_step": mb["ms_per_step"], "tokens_per_s": mb["value"],
                "stages_ms": {k_: v for k_, v in mb["stages_ms"].items() if k_ in ("gemm_dw2", "regather", "gemm_dw13")}}
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
