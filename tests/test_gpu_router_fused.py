"""The forward with the router GEMM in front (mok_moe_forward_router) on the
GPU: bit for bit every output of mok_router_logits followed by
mok_moe_forward on the same inputs (the logits, the routing, every saved
array, out, and the backward that follows), for E <= 128 (the fused kernel:
the router GEMM's tile routes its own tokens from LDS), E > 128 (two
launches), calls of at most 32 tokens (the one-launch router and sort
behind the GEMM), a local expert range, the router variants, MXFP8 and
MXFP4.  The logits themselves are checked against the oracle's router GEMM
(tests/test_gpu_router_gemm.py bounds) and the routing against the oracle's
top-k of the device's logits."""
import numpy as np
import pytest
import torch

import workloads as W
from mixture_experts_layer_34_amd import mok
from mixture_experts_layer_34_amd.layer import (MoeBuffers, MoeShape, quantize_mxfp4, quantize_mxfp8,
                                                router_logits)
from oracle import mok_oracle as O
from tests.gpu_case import note, rel_inf, to_np

pytestmark = pytest.mark.gpu


def _inputs(T, d, E, F, seed):
    w = W.scaled("bf16_fwd", T=T, d=d, E=E, k=1, F=F)
    inp = W.make_inputs(w, device="cuda")
    r = W.make_router_inputs(seed, T, d, E, device="cuda")
    inp["Wr"] = r["Wr"]
    inp["dout"] = torch.randn((T, d), generator=torch.Generator().manual_seed(seed), dtype=torch.float32).to(
        torch.bfloat16).cuda()
    return inp


def _weights(inp, precision):
    if precision == "bf16":
        return inp["W1"], inp["W3"], inp["W2"], None
    quant = quantize_mxfp8 if precision == "mxfp8" else quantize_mxfp4
    q = [quant(inp[n]) for n in ("W1", "W3", "W2")]
    return q[0][0], q[1][0], q[2][0], torch.cat([s.reshape(-1) for _, s in q])


def _pair(T, d, E, k, F, precision="bf16", eb=0, ee=-1, gating="softmax", renorm=False, save=False, seed=3):
    inp = _inputs(T, d, E, F, seed)
    W1, W3, W2, sc = _weights(inp, precision)
    bufs = []
    for fused in (False, True):
        shape = MoeShape(T=T, d=d, E=E, k=k, F=F, precision=precision, expert_begin=eb, expert_end=ee,
                         gating=gating, renorm=renorm, save_for_backward=save)
        b = MoeBuffers(shape)
        b.saved.fill_(0x5A)
        b.workspace.fill_(0xA5)
        if fused:
            b.forward_router(inp["x"], inp["Wr"], W1, W3, W2, sc)
        else:
            b.logits = router_logits(inp["x"], inp["Wr"])
            b.forward(inp["x"], b.logits, W1, W3, W2, sc)
        if save:
            b.backward(inp["dout"], inp["x"], b.logits, inp["W1"], inp["W3"], inp["W2"])
        torch.cuda.synchronize()
        assert b.device_status() == (mok.MOK_OK, 0)
        bufs.append(b)
    return inp, bufs


def _same(a, b, save):
    assert torch.equal(a.logits, b.logits), "logits differ"
    for n in ("out", "topk_idx", "topk_gate", "counts", "offsets"):
        assert torch.equal(getattr(a, n), getattr(b, n)), f"{n} differs"
    assert torch.equal(a.saved, b.saved), "saved arrays differ"
    if save:
        for n in a.grads:
            assert torch.equal(a.grads[n], b.grads[n]), f"{n} differs"


CASES = [
    # name, T, d, E, k, F, extra
    ("fused-E128-ragged", 300, 256, 128, 8, 256, {}),
    ("fused-E64", 100, 512, 64, 4, 256, {}),
    ("fused-E5", 77, 128, 5, 2, 128, {}),
    ("fused-E1", 40, 64, 1, 1, 64, {}),
    ("two-launch-E256", 200, 256, 256, 8, 256, {}),
    ("two-launch-E1024", 1000, 128, 1024, 8, 128, {}),
    ("two-launch-E129", 64, 128, 129, 4, 128, {}),
    ("small-T", 5, 256, 128, 8, 256, {}),
    ("local", 256, 256, 64, 4, 256, dict(eb=8, ee=20)),
    ("sigmoid-renorm", 150, 256, 96, 6, 256, dict(gating="sigmoid", renorm=True)),
    ("train-save", 300, 256, 128, 8, 256, dict(save=True)),
    ("mxfp8", 200, 256, 64, 4, 256, dict(precision="mxfp8")),
    ("mxfp4", 200, 256, 64, 4, 256, dict(precision="mxfp4")),
]


@pytest.mark.parametrize("name,T,d,E,k,F,extra", CASES, ids=[c[0] for c in CASES])
def test_forward_router_equals_separate_calls(name, T, d, E, k, F, extra):
    note(f"forward_router {name} T={T} d={d} E={E} k={k} F={F} {extra}")
    inp, (sep, fus) = _pair(T, d, E, k, F, **extra)
    _same(sep, fus, extra.get("save", False))
    # the logits against the oracle's router GEMM, the routing against the
    # oracle's top-k of the device's logits
    xh, wh = to_np(inp["x"]).astype(np.float64), to_np(inp["Wr"]).astype(np.float64)
    lg = to_np(fus.logits)
    err = np.abs(lg - O.router_logits(xh, wh))
    assert np.all(err <= d * 2.0 ** -24 * (np.abs(xh) @ np.abs(wh).T)), "logits outside the rounding bound"
    idx = O.route(lg, k, extra.get("gating", "softmax"), extra.get("renorm", False))[0]
    assert np.array_equal(to_np(fus.topk_idx), idx)
    note(f"  logits rel_inf {rel_inf(lg, O.router_logits(xh, wh)):.2e}; bitwise equal to the separate calls")


def test_forward_router_zero_tokens_and_reruns():
    note("forward_router T=0")
    inp, (sep, fus) = _pair(0, 128, 16, 2, 128)
    assert int(fus.counts.sum()) == 0
    note("forward_router reruns")
    T, d, E, k, F = 333, 256, 128, 8, 256
    inp = _inputs(T, d, E, F, 9)
    b = MoeBuffers(MoeShape(T=T, d=d, E=E, k=k, F=F))
    first = [t.clone() for t in (b.forward_router(inp["x"], inp["Wr"], inp["W1"], inp["W3"], inp["W2"]),
                                 b.topk_idx, b.topk_gate)] + [b.logits.clone()]
    for rep in range(9):
        b.workspace.fill_(0xFF)
        again = [b.forward_router(inp["x"], inp["Wr"], inp["W1"], inp["W3"], inp["W2"]).clone(), b.topk_idx,
                 b.topk_gate, b.logits]
        for a_, b_ in zip(first, again):
            assert torch.equal(a_, b_), f"rerun {rep} differs"


def test_forward_router_nonfinite_logit_is_reported():
    """A router vector of infinities makes that expert's logits non-finite:
    the fused kernel reports it on the status word like the router step."""
    T, d, E, k, F = 64, 128, 32, 2, 128
    inp = _inputs(T, d, E, F, 5)
    inp["Wr"][3] = float("inf")
    b = MoeBuffers(MoeShape(T=T, d=d, E=E, k=k, F=F))
    b.forward_router(inp["x"], inp["Wr"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    st, bits = b.device_status()
    assert st == mok.MOK_ERR_DEVICE and bits & 1
