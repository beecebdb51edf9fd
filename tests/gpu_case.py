"""Helpers of the GPU tests: run the HIP layer on a seeded workload and read
back what the oracle is compared against.  (Not a test module.)"""
from __future__ import annotations

import numpy as np
import torch

import workloads as W
from mixture_experts_layer_34_amd.layer import (MoeBuffers, MoeShape, quantize_mxfp4, quantize_mxfp8,
                                                quantize_mxfp8_backward_weights)


def note(msg: str):
    print(f"[gpu-test] {msg}", flush=True)


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        t = t.float()
    return t.detach().cpu().numpy()


def rel_inf(gpu, ref) -> float:
    """max |gpu - ref| / max |ref| (infinity-norm relative error)."""
    g = np.asarray(gpu, np.float64)
    r = np.asarray(ref, np.float64)
    den = np.abs(r).max() if r.size else 0.0
    return float(np.abs(g - r).max() / (den if den > 0 else 1.0)) if r.size else 0.0


class LazyExperts:
    """Expert weights copied to the host one expert at a time (float64)."""

    def __init__(self, w: torch.Tensor, cache: int = 16):
        self.w = w
        self.cache = {}
        self.order = []
        self.max = cache

    def __getitem__(self, i):
        i = int(i)
        if i not in self.cache:
            self.cache[i] = self.w[i].double().cpu().numpy()
            self.order.append(i)
            if len(self.order) > self.max:
                self.cache.pop(self.order.pop(0))
        return self.cache[i]


def shape_of(w: W.Workload, T: int, backward: bool) -> MoeShape:
    """Whole-layer shape of a workload (no ring; tests set ring fields themselves)."""
    return MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision=w.precision, expert_begin=w.expert_begin,
                    expert_end=w.e_end, save_for_backward=backward)


def run_layer(w: W.Workload, inp: dict, backward: bool = False, buf: MoeBuffers | None = None):
    T = inp["x"].shape[0]
    if buf is None:
        buf = MoeBuffers(shape_of(w, T, backward))
    W1, W3, W2, scales = inp["W1"], inp["W3"], inp["W2"], None
    if w.precision == "mxfp8":
        if "W1q" not in inp:
            q1, s1 = quantize_mxfp8(inp["W1"])
            q3, s3 = quantize_mxfp8(inp["W3"])
            q2, s2 = quantize_mxfp8(inp["W2"])
            inp["W1q"], inp["W3q"], inp["W2q"] = q1, q3, q2
            inp["w_scales"] = torch.cat([s1.reshape(-1), s3.reshape(-1), s2.reshape(-1)])
        W1, W3, W2, scales = inp["W1q"], inp["W3q"], inp["W2q"], inp["w_scales"]
    elif w.precision == "mxfp4":
        if "W1q4" not in inp:
            q1, s1 = quantize_mxfp4(inp["W1"])
            q3, s3 = quantize_mxfp4(inp["W3"])
            q2, s2 = quantize_mxfp4(inp["W2"])
            inp["W1q4"], inp["W3q4"], inp["W2q4"] = q1, q3, q2
            inp["w_scales4"] = torch.cat([s1.reshape(-1), s3.reshape(-1), s2.reshape(-1)])
        W1, W3, W2, scales = inp["W1q4"], inp["W3q4"], inp["W2q4"], inp["w_scales4"]
    buf.forward(inp["x"], inp["logits"], W1, W3, W2, scales)
    if backward and w.precision == "mxfp8":
        if "wt" not in inp:
            inp["wt"] = quantize_mxfp8_backward_weights(inp["W1"], inp["W3"], inp["W2"])
        buf.backward_mxfp8(inp["dout"], inp["x"], inp["logits"], inp["wt"])
    elif backward:
        buf.backward(inp["dout"], inp["x"], inp["logits"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    return buf


def saved_arrays(buf: MoeBuffers) -> dict:
    s = buf.shape
    Tk = s.T * s.k
    act = s.act_dtype
    return dict(
        lse=to_np(buf.saved_view("lse", torch.float32, (s.T,))),
        row_of_pair=to_np(buf.saved_view("row_of_pair", torch.int32, (Tk,))),
        pair_of_row=to_np(buf.saved_view("pair_of_row", torch.int32, (Tk,))),
        A=lambda P: to_np(buf.saved_view("A", act, (Tk, s.F))[:P]),
        B=lambda P: to_np(buf.saved_view("B", act, (Tk, s.F))[:P]),
        H=lambda P: to_np(buf.saved_view("H", act, (Tk, s.F))[:P]),
        Y=lambda P: to_np(buf.saved_view("Y", act, (Tk, s.d))[:P]),
    )


def host_inputs(inp: dict) -> dict:
    """Host copies (numpy) of the small tensors; weights stay lazy."""
    out = {k: to_np(v) for k, v in inp.items() if k in ("x", "logits", "dout", "token_ids")}
    return out
