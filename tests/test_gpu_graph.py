"""The layer's launches can be captured into a HIP graph and replayed.

The library enqueues only kernels on the caller's stream (no allocation, no
memset, no host synchronisation, tile counts read on the device), so a
captured forward + backward replays to the eager result bit for bit: whole
layer (bf16 and MXFP8) and ring pipeline.  Between replays the outputs and the workspace are
overwritten by eager work, so each replay has to produce everything again."""
import pytest
import torch

import workloads as W
from mixture_experts_layer_34_amd.layer import MoeBuffers, quantize_mxfp8, quantize_mxfp8_backward_weights
from tests.gpu_case import note, shape_of

pytestmark = pytest.mark.gpu


def _outputs(buf):
    outs = {"out": buf.out, "idx": buf.topk_idx, "gate": buf.topk_gate, "offsets": buf.offsets}
    outs.update(buf.grads)
    return {k: v.clone() for k, v in outs.items()}


def _poison(buf):
    for t in [buf.out, buf.topk_gate, buf.workspace] + list(buf.grads.values()):
        t.fill_(float("nan") if t.is_floating_point() else 0x7F)
    buf.topk_idx.fill_(-1)
    buf.offsets.fill_(-1)


@pytest.mark.parametrize("name,over,R", [
    ("bf16-layer", dict(T=777, d=128, E=16, k=4, F=320), 0),
    ("bf16-ring", dict(T=777, d=128, E=16, k=4, F=320), 200),
    ("bf16-local", dict(T=600, d=192, E=12, k=3, F=128, expert_begin=2, expert_end=9), 0),
    ("mxfp8-layer", dict(T=777, d=256, E=16, k=4, F=384, precision="mxfp8"), 0),
])
def test_graph_replay_equals_eager(name, over, R):
    w = W.scaled("bf16_train", **over)
    note(f"graph {name}")
    inp = W.make_inputs(w, device="cuda")
    T = inp["x"].shape[0]
    shape = shape_of(w, T, True)
    if R:
        shape.minibatch_rows = R
        shape.ring_bytes = 3 * R * w.d * 2
    buf = MoeBuffers(shape)
    buf.alloc_grads()
    if w.precision == "mxfp8":
        q = [quantize_mxfp8(inp[n]) for n in ("W1", "W3", "W2")]
        scales = torch.cat([sc.reshape(-1) for _, sc in q])
        wt = quantize_mxfp8_backward_weights(inp["W1"], inp["W3"], inp["W2"])

        def step():
            buf.forward(inp["x"], inp["logits"], q[0][0], q[1][0], q[2][0], scales)
            buf.backward_mxfp8(inp["dout"], inp["x"], inp["logits"], wt)
    else:
        def step():
            buf.forward(inp["x"], inp["logits"], inp["W1"], inp["W3"], inp["W2"])
            buf.backward(inp["dout"], inp["x"], inp["logits"], inp["W1"], inp["W3"], inp["W2"])

    step()
    torch.cuda.synchronize()
    ref = _outputs(buf)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        _poison(buf)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = _outputs(buf)
        for k in ref:
            assert torch.equal(ref[k], got[k]), f"replay {rep}: {k} differs"
