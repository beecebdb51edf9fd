"""Ring-buffer minibatch pipeline on the GPU (the forward as one launch per
minibatch: the copy of minibatch m+1 into its ring slot, UP on m and DOWN on
m-1; the backward of a ring configuration reads x rows through the row map).

Every output element is still produced by one workgroup over the full K loop
in the same order, whatever the minibatch cut, so the pipeline's results must
equal the whole-layer mode's bit for bit (forward and backward).  At the
training size the ring path is also compared with the oracle directly:
sampled tokens for out, dx, dgate and d(logits), and the weight gradients of
the lightest, the median and the heaviest expert."""
import numpy as np
import pytest
import torch

import workloads as W
from mixture_experts_layer_34_amd import mok
from mixture_experts_layer_34_amd.layer import MoeBuffers
from oracle import mok_oracle as O
from tests.gpu_case import LazyExperts, host_inputs, note, rel_inf, run_layer, shape_of, to_np

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


def _outputs(buf):
    s = buf.shape
    P = int(buf.offsets[-1].item())
    outs = {"out": buf.out, "idx": buf.topk_idx, "offsets": buf.offsets,
            "H": buf.saved_view("H", torch.bfloat16, (s.T * s.k, s.F))[:P],
            "Y": buf.saved_view("Y", torch.bfloat16, (s.T * s.k, s.d))[:P]}
    if buf.grads:
        outs.update({k: v for k, v in buf.grads.items()})
    return {k: v.clone() for k, v in outs.items()}


def _ring_buffers(w, T, backward, R, ring_slots):
    shape = shape_of(w, T, backward)
    shape.minibatch_rows = R
    shape.ring_bytes = ring_slots * R * w.d * 2
    return MoeBuffers(shape)


def _ring_vs_whole(w, R, ring_slots, backward=True):
    inp = W.make_inputs(w, device="cuda")
    T = inp["x"].shape[0]
    ref = _outputs(run_layer(w, inp, backward=backward))
    buf = run_layer(w, inp, backward=backward, buf=_ring_buffers(w, T, backward, R, ring_slots))
    assert buf.device_status() == (mok.MOK_OK, 0)
    got = _outputs(buf)
    for k in ref:
        assert torch.equal(ref[k], got[k]), f"{k} differs (R={R}, slots={ring_slots})"
    return buf


@pytest.mark.parametrize("R,slots", [(64, 2), (200, 2), (333, 3), (1000, 4), (4096, 2)])
def test_ring_pipeline_bitwise_equals_whole_layer(R, slots):
    """T 777, k 4 (3,108 rows): two slots reused for many minibatches at R 64."""
    w = W.scaled("bf16_train", T=777, d=128, E=16, k=4, F=320)
    note(f"ring R={R} slots={slots}")
    _ring_vs_whole(w, R, slots)


def test_ring_pipeline_local_expert_range():
    w = W.scaled("bf16_fwd", T=900, d=192, E=12, k=3, F=128, expert_begin=4, expert_end=9, backward=True)
    note("ring local range")
    _ring_vs_whole(w, 256, 2)


def test_ring_pipeline_one_hot_large_expert():
    """One expert with nearly every row: it spans many minibatches."""
    w = W.scaled("bf16_train", T=700, d=128, E=6, k=1, F=192, notes={"zipf": 4.0})
    note("ring one-hot")
    _ring_vs_whole(w, 256, 2)


@pytest.fixture(scope="module")
def train_reference():
    """The whole layer's outputs and the oracle's sampled-token and
    per-expert references at the training size, computed once for every R."""
    w = W.get("bf16_train")
    inp = W.make_inputs(w, device="cuda")
    whole = _outputs(run_layer(w, inp, backward=True))
    h = host_inputs(inp)
    idx, gate, _, _ = O.route(h["logits"], w.k)
    counts, offsets, _, por = O.layout(idx, w.E)
    toks = sorted(set(np.random.default_rng(21).choice(w.T, size=6, replace=False).tolist()) | {0, w.T - 1})
    W1, W3, W2 = LazyExperts(inp["W1"]), LazyExperts(inp["W3"]), LazyExperts(inp["W2"])
    ref = {"toks": toks, "out": [], "dx": [], "dgate": [], "dlogits": [], "whole": whole}
    for t in toks:
        ref["out"].append(O.forward_token(t, h["x"][t], h["logits"][t], W1, W3, W2, w.k)[2])
        a, b, c = O.backward_token(h["x"][t], h["logits"][t], h["dout"][t], W1, W3, W2, w.k)
        ref["dx"].append(a); ref["dgate"].append(b); ref["dlogits"].append(c)
    order = np.argsort(counts, kind="stable")
    ref["experts"] = {}
    for e in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        rows = por[offsets[e]:offsets[e + 1]]
        tok, slot = rows // w.k, rows % w.k
        ref["experts"][e] = O.expert_weight_grads(h["x"][tok], gate[tok, slot], h["dout"][tok], W1[e], W3[e], W2[e])
    return w, inp, ref


@pytest.mark.parametrize("R", [512, 1024, 2048, pytest.param(4096, marks=pytest.mark.skip(
    reason="a benchmark run of the training layer at R = 4096 faulted the GPU while a ring-kernel rewrite (since "
           "withdrawn, its source not kept) was under test; no cause was shown, so the training size at R = 4096 "
           "stays off the GPU"))])
def test_ring_pipeline_train_full_size(train_reference, R):
    """bf16_train with the 256 MiB ring (R = 512: 128 minibatches over 64
    slots, each slot used twice): bitwise equal to the whole layer, and the
    oracle on sampled tokens and three experts' weight gradients."""
    w, inp, ref = train_reference
    note(f"ring full size R={R}")
    buf = run_layer(w, inp, backward=True, buf=_ring_buffers(w, w.T, True, R, w.ring_bytes // (R * w.d * 2)))
    assert buf.device_status() == (mok.MOK_OK, 0)
    got = _outputs(buf)
    for k in ref["whole"]:
        assert torch.equal(ref["whole"][k], got[k]), f"{k} differs from the whole layer (R={R})"
    h = host_inputs(inp)
    assert np.array_equal(to_np(buf.topk_idx), O.route(h["logits"], w.k)[0])
    toks = ref["toks"]
    g = buf.grads
    errs = {"out": rel_inf(to_np(buf.out)[toks], np.stack(ref["out"])),
            "dx": rel_inf(to_np(g["dx"])[toks], np.stack(ref["dx"])),
            "dgate": rel_inf(to_np(g["dgate"])[toks], np.stack(ref["dgate"])),
            "dlogits": rel_inf(to_np(g["dlogits"])[toks], np.stack(ref["dlogits"]))}
    for e, (r1, r3, r2) in ref["experts"].items():
        errs[f"dW1[{e}]"] = rel_inf(to_np(g["dW1"][e]), r1)
        errs[f"dW3[{e}]"] = rel_inf(to_np(g["dW3"][e]), r3)
        errs[f"dW2[{e}]"] = rel_inf(to_np(g["dW2"][e]), r2)
    note("  errors " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if v > TOL_BF16}
    assert not bad, bad


@pytest.mark.parametrize("movers", [1, 8, 32, 255])
def test_ring_pipeline_mover_split_bitwise(movers):
    """The explicit split of the workgroups between row copies and tiles:
    which workgroup runs a task never changes what it computes, so every
    mover_cus gives the whole layer's bits (1: one copier; 255: one tile
    workgroup for every UP and DOWN tile)."""
    w = W.scaled("bf16_train", T=777, d=128, E=16, k=4, F=320)
    inp = W.make_inputs(w, device="cuda")
    ref = _outputs(run_layer(w, inp, backward=True))
    note(f"ring mover_cus={movers}")
    shape = shape_of(w, w.T, True)
    shape.minibatch_rows, shape.ring_bytes, shape.mover_cus = 200, 3 * 200 * w.d * 2, movers
    buf = run_layer(w, inp, backward=True, buf=MoeBuffers(shape))
    assert buf.device_status() == (mok.MOK_OK, 0)
    got = _outputs(buf)
    for k in ref:
        assert torch.equal(ref[k], got[k]), f"{k} differs (mover_cus={movers})"


def test_ring_pipeline_mover_split_train_full_size(train_reference):
    """bf16_train at R = 1024 with 32 copy-only workgroups: the whole layer's bits."""
    w, inp, ref = train_reference
    note("ring full size R=1024 mover_cus=32")
    shape = shape_of(w, w.T, True)
    shape.minibatch_rows = 1024
    shape.ring_bytes = w.ring_bytes
    shape.mover_cus = 32
    buf = run_layer(w, inp, backward=True, buf=MoeBuffers(shape))
    assert buf.device_status() == (mok.MOK_OK, 0)
    got = _outputs(buf)
    for k in ref["whole"]:
        assert torch.equal(ref["whole"][k], got[k]), f"{k} differs from the whole layer (mover_cus=32)"
