"""The weight-streaming forward GEMMs of small BF16 calls (at most 4096
token-expert pairs, d and F multiples of 128) on the GPU.

Against the oracle, whole layer: out, the saved H and Y rows and, where the
forward saves for backward, A, B and every gradient of the backward that
follows (which reads what the streaming kernels saved).  The shapes cover
each K split of the kernels (UP: d / 128 multiple of 4, 2 or 1; DOWN: F),
experts of 0, 1-16, 17-31, exactly 32 and several 32-row tiles, a local
expert range, and the largest streaming call; the same inputs through the
tiled kernels (MOK_FLAG_TILED_GEMMS) must meet the same bar, and reruns must
be bitwise identical."""
import numpy as np
import pytest
import torch

import workloads as W
from mixture_experts_layer_34_amd import mok
from mixture_experts_layer_34_amd.layer import MoeBuffers, MoeShape
from oracle import mok_oracle as O
from tests.gpu_case import host_inputs, note, rel_inf, saved_arrays, to_np

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
STREAM_MAX_PAIRS = 4096


def _ksplit(K):
    return 4 if K % 512 == 0 else (2 if K % 256 == 0 else (1 if K % 128 == 0 else 0))


def _run(w, inp, backward, path="stream"):
    T = inp["x"].shape[0]
    shape = MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision="bf16", expert_begin=w.expert_begin,
                     expert_end=w.e_end, save_for_backward=backward, gemm_path=path)
    buf = MoeBuffers(shape)
    buf.saved.fill_(0xAB)
    buf.forward(inp["x"], inp["logits"], inp["W1"], inp["W3"], inp["W2"])
    if backward:
        buf.backward(inp["dout"], inp["x"], inp["logits"], inp["W1"], inp["W3"], inp["W2"])
    torch.cuda.synchronize()
    assert buf.device_status() == (mok.MOK_OK, 0)
    return buf


def _errors(w, inp, buf, backward):
    h = host_inputs(inp)
    W1, W3, W2 = (to_np(inp[n]).astype(np.float64) for n in ("W1", "W3", "W2"))
    fw = O.forward(h["x"], h["logits"], W1, W3, W2, w.k, w.expert_begin, w.e_end)
    idx = O.route(h["logits"], w.k)[0]
    assert np.array_equal(to_np(buf.topk_idx), idx)
    P = int(to_np(buf.offsets)[w.e_end] - to_np(buf.offsets)[w.expert_begin])
    sv = saved_arrays(buf)
    errs = {"out": rel_inf(to_np(buf.out), fw["out"]), "H": rel_inf(sv["H"](P), fw["H"]),
            "Y": rel_inf(sv["Y"](P), fw["Y"])}
    if backward:
        bw = O.backward(h["dout"], h["x"], h["logits"], W1, W3, W2, w.k, fw, w.expert_begin, w.e_end)
        errs["A"] = rel_inf(sv["A"](P), fw["A"])
        errs["B"] = rel_inf(sv["B"](P), fw["B"])
        g = buf.grads
        for n in ("dx", "dgate", "dlogits"):
            errs[n] = rel_inf(to_np(g[n]), bw[n])
        for n in ("dW1", "dW3", "dW2"):
            gw = to_np(g[n])
            errs[n] = max(rel_inf(gw[i], bw[n][i]) for i in range(w.E_loc))
    return errs


CASES = [
    # name, workload overrides, backward
    ("ks4-ks2", dict(T=200, d=512, E=16, k=4, F=768), True),           # UP K split 4, DOWN 2
    ("ks2-ks4", dict(T=96, d=256, E=8, k=2, F=1024), False),           # UP 2, DOWN 4 (run as 2)
    ("ks1-ks1", dict(T=300, d=128, E=12, k=3, F=128), True),           # both unsplit
    ("one-token", dict(T=1, d=1024, E=64, k=8, F=512), True),          # eight experts of one row
    ("tiles-ragged", dict(T=333, d=384, E=6, k=2, F=640, notes={"zipf": 1.5}), True),   # many 32-row tiles
    ("one-hot", dict(T=400, d=256, E=5, k=1, F=256, notes={"zipf": 5.0}), False),       # one expert, ~13 tiles
    ("local-range", dict(T=256, d=512, E=32, k=4, F=256, expert_begin=8, expert_end=20), True),
    ("max-pairs", dict(T=512, d=256, E=64, k=8, F=384), False),        # 4096 pairs: the largest streaming call
]


@pytest.mark.parametrize("name,over,backward", CASES, ids=[c[0] for c in CASES])
def test_stream_gemms_match_oracle(name, over, backward):
    base = "bf16_train" if "zipf" in over.get("notes", {}) else "bf16_fwd"
    w = W.scaled(base, backward=backward, **over)
    assert w.T * w.k <= STREAM_MAX_PAIRS and _ksplit(w.d) and _ksplit(w.F)
    note(f"stream {name} {over} backward={backward}")
    inp = W.make_inputs(w, device="cuda")
    buf = _run(w, inp, backward)
    counts = to_np(buf.counts)[w.expert_begin:w.e_end]
    note(f"  rows per local expert: max {counts.max()}, empty {(counts == 0).sum()}")
    errs = _errors(w, inp, buf, backward)
    note(f"  streaming: max error {max(errs.values()):.3e} ({max(errs, key=errs.get)})")
    bad = {k: v for k, v in errs.items() if v > TOL_BF16}
    assert not bad, bad
    tiled = _run(w, inp, backward, path="tiled")
    errs_t = _errors(w, inp, tiled, backward)
    note(f"  tiled:     max error {max(errs_t.values()):.3e} ({max(errs_t, key=errs_t.get)})")
    bad = {k: v for k, v in errs_t.items() if v > TOL_BF16}
    assert not bad, bad
    # the two paths differ only in summation order: the routing state is the same
    assert torch.equal(buf.topk_idx, tiled.topk_idx) and torch.equal(buf.offsets, tiled.offsets)


def test_stream_gemms_rerun_bitwise():
    w = W.scaled("bf16_train", T=256, d=512, E=16, k=8, F=768)
    note("stream determinism")
    inp = W.make_inputs(w, device="cuda")
    a = _run(w, inp, True)
    for rep in range(3):
        b = _run(w, inp, True)
        assert torch.equal(a.out, b.out), f"rerun {rep}: out differs"
        for n in a.grads:
            assert torch.equal(a.grads[n], b.grads[n]), f"rerun {rep}: {n} differs"


def test_stream_not_used_past_its_range():
    """4097 pairs, or F not a multiple of 128: the tiled kernels run even when
    streaming is asked for, so the flag changes nothing, bit for bit."""
    for over in (dict(T=513, d=256, E=64, k=8, F=256), dict(T=64, d=256, E=8, k=2, F=192)):
        w = W.scaled("bf16_fwd", **over)
        note(f"stream range {over}")
        inp = W.make_inputs(w, device="cuda")
        a, b = _run(w, inp, False), _run(w, inp, False, path="tiled")
        assert torch.equal(a.out, b.out)


@pytest.mark.parametrize("T,expect", [(16, "stream"), (64, "stream"), (65, "tiled"), (128, "tiled")])
def test_auto_choice(T, expect):
    """Without a GEMM flag: streaming up to four rows per local expert on
    average (T * k <= 4 E_loc), the tiled kernels past that; the default
    call's output is bitwise that of the path it chose."""
    w = W.scaled("bf16_train", T=T, d=256, F=256, E=32, k=2)
    note(f"auto choice T={T} pairs={T * w.k} E_loc={w.E_loc}")
    inp = W.make_inputs(w, device="cuda")
    auto, chosen = _run(w, inp, False, path="auto"), _run(w, inp, False, path=expect)
    assert torch.equal(auto.out, chosen.out)


# ------------------------------------------------------------------ MXFP8 weight streaming (inference)

TOL_MX = 3e-2

MX_CASES = [
    ("mx-one-token", dict(T=1, d=512, E=16, k=4, F=256)),
    ("mx-tiles-ragged", dict(T=100, d=256, E=8, k=2, F=384)),           # up to ~50 rows: two 32-row tiles
    ("mx-local", dict(T=64, d=512, E=32, k=4, F=256, expert_begin=8, expert_end=20)),
    ("mx-k-eq-E", dict(T=40, d=256, E=4, k=4, F=128)),                  # every expert 40 rows
]


def _run_mx(w, inp, path):
    from tests.gpu_case import run_layer
    T = inp["x"].shape[0]
    shape = MoeShape(T=T, d=w.d, E=w.E, k=w.k, F=w.F, precision="mxfp8", expert_begin=w.expert_begin,
                     expert_end=w.e_end, save_for_backward=False, gemm_path=path)
    buf = run_layer(w, inp, backward=False, buf=MoeBuffers(shape))
    assert buf.device_status() == (mok.MOK_OK, 0)
    return buf


@pytest.mark.parametrize("name,over", MX_CASES, ids=[c[0] for c in MX_CASES])
def test_stream_mxfp8_forward_matches_oracle(name, over):
    """MXFP8 forward without saving (inference): the streaming UP and DOWN
    against the oracle's MXFP8 forward (out and Y rows), next to the tiled
    MXFP8 kernels on the same inputs."""
    w = W.scaled("bf16_fwd", precision="mxfp8", backward=False, **over)
    note(f"stream mxfp8 {name} {over}")
    inp = W.make_inputs(w, device="cuda")
    h = host_inputs(inp)
    W1, W3, W2 = (to_np(inp[n]).astype(np.float64) for n in ("W1", "W3", "W2"))
    fw = O.forward(h["x"], h["logits"], W1, W3, W2, w.k, w.expert_begin, w.e_end, mxfp8=True)
    for path in ("stream", "tiled"):
        buf = _run_mx(w, inp, path)
        assert np.array_equal(to_np(buf.topk_idx), fw["idx"])
        P = int(to_np(buf.offsets)[w.e_end])
        Y = to_np(buf.saved_view("Y", torch.bfloat16, (w.T * w.k, w.d))[:P])
        errs = {"out": rel_inf(to_np(buf.out), fw["out"]), "Y": rel_inf(Y, fw["Y"])}
        note(f"  {path}: " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
        bad = {k: v for k, v in errs.items() if v > TOL_MX}
        assert not bad, (path, bad)


@pytest.mark.parametrize("T", [1, 16, 64])
def test_stream_mxfp8_train_shape_sampled(T):
    """d 4096, E 128, k 8, F 1536 in MXFP8, forward only, the default choice
    (streaming up to four rows per expert): sampled tokens against the
    oracle's per-token MXFP8 forward; reruns bitwise."""
    from tests.gpu_case import LazyExperts
    w = W.scaled("bf16_train", precision="mxfp8", backward=False, T=T)
    note(f"stream mxfp8 train shape T={T}")
    inp = W.make_inputs(w, device="cuda")
    buf = _run_mx(w, inp, "auto")
    out = to_np(buf.out).copy()
    again = _run_mx(w, inp, "auto")
    assert np.array_equal(out, to_np(again.out)), "rerun differs"
    h = host_inputs(inp)
    W1, W3, W2 = LazyExperts(inp["W1"]), LazyExperts(inp["W3"]), LazyExperts(inp["W2"])
    toks = sorted(set(np.random.default_rng(T).choice(T, size=min(T, 3), replace=False).tolist()) | {T - 1})
    ref = np.stack([O.forward_token(t, h["x"][t], h["logits"][t], W1, W3, W2, w.k, mxfp8=True)[2] for t in toks])
    err = rel_inf(out[toks], ref)
    note(f"  out sampled {err:.2e}")
    assert err <= TOL_MX
