"""GPU parity of the HIP layer against the CPU oracle, through the C ABI.

Bars: indices, counts, offsets and the row maps bit-exact; gates within 1e-5;
float outputs within an infinity-norm relative error of 1e-4 (fp32 path) or
2e-2 (bf16 path, fp32 accumulation); repeated runs bitwise identical."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import mok_oracle as O
from tests.gpu_case import LazyExperts, host_inputs, note, rel_inf, run_layer, saved_arrays, to_np

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_F32 = 1e-4
TOL_GATE = 1e-5


def _check_routing(buf, logits_np, k, eb, ee):
    """Routing and placement: bit-exact against the oracle."""
    E = logits_np.shape[1]
    idx, gate, lse, _ = O.route(logits_np, k)
    counts, offsets, rop, por = O.layout(idx, E, eb, ee)
    g_idx = to_np(buf.topk_idx)
    assert np.array_equal(g_idx, idx), "top-k indices differ"
    assert np.array_equal(to_np(buf.counts), counts), "expert counts differ"
    assert np.array_equal(to_np(buf.offsets), offsets), "expert offsets differ"
    sv = saved_arrays(buf)
    P = int(offsets[-1])
    assert np.array_equal(sv["row_of_pair"], rop), "row_of_pair differs"
    assert np.array_equal(sv["pair_of_row"][:P], por), "pair_of_row differs"
    g_gate = to_np(buf.topk_gate)
    assert np.abs(g_gate - gate).max() <= TOL_GATE * max(1.0, np.abs(gate).max())
    assert np.abs(sv["lse"] - lse).max() <= 1e-5 * max(1.0, np.abs(lse).max())
    return P


def _inputs(w, device="cuda"):
    return W.make_inputs(w, device=device)


# ------------------------------------------------------------------ routing + placement

ROUTING_CASES = [
    ("tiny", dict(T=256, E=8, k=2)),
    ("one-expert", dict(T=100, E=1, k=1)),
    ("k-equals-E", dict(T=50, E=6, k=6)),
    ("E1000", dict(T=97, E=1000, k=8)),
    ("three-chunks-ragged", dict(T=3001, E=64, k=3)),
    ("local-range", dict(T=2000, E=32, k=4, expert_begin=8, expert_end=12)),
    ("one-token", dict(T=1, E=16, k=4)),
]


@pytest.mark.parametrize("name,over", ROUTING_CASES, ids=[c[0] for c in ROUTING_CASES])
def test_routing_and_placement_bit_exact(name, over):
    w = W.scaled("bf16_fwd", d=64, F=64, **over)
    note(f"routing {name} {over}")
    inp = _inputs(w)
    buf = run_layer(w, inp)
    _check_routing(buf, to_np(inp["logits"]), w.k, w.expert_begin, w.e_end)


def test_routing_ties_and_signed_zero():
    """Integer-valued logits (many ties) and +-0 entries: lowest index wins."""
    w = W.scaled("bf16_fwd", T=512, d=64, F=64, E=24, k=5)
    note("routing ties")
    inp = _inputs(w)
    g = torch.Generator().manual_seed(5)
    lg = torch.randint(-2, 3, (512, 24), generator=g).float()
    lg[::7, 3] = -0.0
    lg[::5, 0] = 0.0
    inp["logits"] = lg.cuda()
    buf = run_layer(w, inp)
    _check_routing(buf, to_np(inp["logits"]), w.k, 0, w.E)


def test_zero_tokens():
    w = W.scaled("bf16_fwd", T=0, d=64, F=64, E=8, k=2)
    note("zero tokens")
    inp = _inputs(w)
    buf = run_layer(w, inp)
    assert to_np(buf.counts).sum() == 0 and (to_np(buf.offsets) == 0).all()


@pytest.mark.parametrize("name", ["bf16_fwd", "bf16_train", "ep_share"])
def test_routing_full_size(name):
    w = W.get(name)
    note(f"routing full size {name}")
    inp = W.make_inputs(w, device="cuda", weights=False)
    T = inp["x"].shape[0]
    # routing does not depend on the weights: tiny stand-in FFN sizes
    ws = W.scaled(name, d=64, F=64)
    small = dict(x=inp["x"][:, :64].contiguous(), logits=inp["logits"])
    small.update(W.make_weights(ws, device="cuda"))
    buf = run_layer(ws, small)
    P = _check_routing(buf, to_np(inp["logits"]), w.k, w.expert_begin, w.e_end)
    note(f"  T={T} P={P}")
    if name == "ep_share":
        assert abs(P - 16384) <= 0.1 * 16384


# ------------------------------------------------------------------ whole layer, small sizes

def _oracle_fwd_bwd(w, inp, backward):
    h = host_inputs(inp)
    W1, W3, W2 = (to_np(inp[n]).astype(np.float64) for n in ("W1", "W3", "W2"))
    fw = O.forward(h["x"], h["logits"], W1, W3, W2, w.k, w.expert_begin, w.e_end, mxfp8=w.precision == "mxfp8")
    bw = O.backward(h["dout"], h["x"], h["logits"], W1, W3, W2, w.k, fw, w.expert_begin, w.e_end) if backward else None
    return fw, bw


SMALL_CASES = [
    # name, workload overrides, backward
    ("tiny_fp32", dict(), True),
    ("bf16-ragged", dict(T=512, d=256, E=8, k=2, F=192), True),
    ("bf16-skewed", dict(T=777, d=128, E=16, k=4, F=320, notes={"zipf": 1.2}), True),
    ("bf16-local", dict(T=600, d=192, E=12, k=3, F=128, expert_begin=4, expert_end=9), True),
    # smallest dimensions: K loops of 2 stages, shorter than the stage ring
    ("bf16-min", dict(T=37, d=64, E=4, k=2, F=64), True),
    ("bf16-one-token", dict(T=1, d=64, E=8, k=3, F=128), True),
    # every token on every expert (k = E)
    ("bf16-k-eq-E", dict(T=130, d=128, E=4, k=4, F=128), True),
    # one expert takes nearly every row (several row tiles), others few or none
    ("bf16-one-hot", dict(T=700, d=128, E=6, k=1, F=192, notes={"zipf": 4.0}), True),
]


@pytest.mark.parametrize("name,over,backward", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_layer_small_matches_oracle(name, over, backward):
    base = "tiny_fp32" if name == "tiny_fp32" else ("bf16_train" if "zipf" in over.get("notes", {}) else "bf16_fwd")
    w = W.scaled(base, backward=backward, **over)
    note(f"layer {name} {over}")
    inp = _inputs(w)
    buf = run_layer(w, inp, backward=backward)
    tol = TOL_F32 if w.precision == "f32" else TOL_BF16
    fw, bw = _oracle_fwd_bwd(w, inp, backward)
    P = _check_routing(buf, to_np(inp["logits"]), w.k, w.expert_begin, w.e_end)
    sv = saved_arrays(buf)
    errs = {
        "out": rel_inf(to_np(buf.out), fw["out"]),
        "H": rel_inf(sv["H"](P), fw["H"]),
        "Y": rel_inf(sv["Y"](P), fw["Y"]),
    }
    if backward:
        errs["A"] = rel_inf(sv["A"](P), fw["A"])
        errs["B"] = rel_inf(sv["B"](P), fw["B"])
        g = buf.grads
        errs["dx"] = rel_inf(to_np(g["dx"]), bw["dx"])
        errs["dgate"] = rel_inf(to_np(g["dgate"]), bw["dgate"])
        errs["dlogits"] = rel_inf(to_np(g["dlogits"]), bw["dlogits"])
        counts = to_np(buf.counts)
        for n in ("dW1", "dW3", "dW2"):
            gw = to_np(g[n])
            for i in range(w.E_loc):
                errs[f"{n}[{i}]"] = rel_inf(gw[i], bw[n][i])
                if counts[w.expert_begin + i] == 0:
                    # an expert without rows has an exactly zero gradient
                    assert not gw[i].any(), f"{n}[{i}] of an empty expert is not zero"
    note(f"  max errors: {max(errs.values()):.3e} ({max(errs, key=errs.get)})")
    bad = {k: v for k, v in errs.items() if v > tol}
    assert not bad, bad


# ------------------------------------------------------------------ whole layer, full sizes (sampled)

def _sample_tokens(idx, counts, eb, ee, n, seed):
    """A few tokens of the lightest, median and heaviest local experts plus random ones."""
    rng = np.random.default_rng(seed)
    loc = np.arange(eb, ee)
    nz = loc[counts[loc] > 0]
    order = nz[np.argsort(counts[nz], kind="stable")]
    picks = set()
    for e in (order[0], order[len(order) // 2], order[-1]):
        toks = np.nonzero((idx == e).any(axis=1))[0]
        picks.update(toks[:2].tolist())
    picks.update(rng.choice(idx.shape[0], size=n, replace=False).tolist())
    return sorted(picks)


@pytest.mark.parametrize("name", ["bf16_fwd", "ep_share"])
def test_forward_full_size_sampled(name):
    w = W.get(name)
    note(f"forward full size {name}")
    inp = _inputs(w)
    buf = run_layer(w, inp)
    h = host_inputs(inp)
    P = _check_routing(buf, h["logits"], w.k, w.expert_begin, w.e_end)
    idx = to_np(buf.topk_idx)
    counts = to_np(buf.counts)
    toks = _sample_tokens(idx, counts, w.expert_begin, w.e_end, 12, 1)
    W1, W3, W2 = LazyExperts(inp["W1"]), LazyExperts(inp["W3"]), LazyExperts(inp["W2"])
    out = to_np(buf.out)
    ref = np.stack([O.forward_token(t, h["x"][t], h["logits"][t], W1, W3, W2, w.k, w.expert_begin, w.e_end)[2]
                    for t in toks])
    err = rel_inf(out[toks], ref)
    note(f"  P={P} sampled {len(toks)} tokens, out error {err:.3e}")
    assert err <= TOL_BF16


def test_train_full_size_sampled():
    """bf16_train (T 8192, d 4096, E 128, k 8, F 1536) forward + backward, as
    the benchmark runs it: sampled tokens for out/dx/dgate/dlogits, and the
    weight gradients of the lightest, the median and the heaviest expert."""
    w = W.get("bf16_train")
    note("train full size forward+backward")
    inp = _inputs(w)
    buf = run_layer(w, inp, backward=True)
    h = host_inputs(inp)
    P = _check_routing(buf, h["logits"], w.k, 0, w.E)
    idx = to_np(buf.topk_idx)
    counts = to_np(buf.counts)
    toks = _sample_tokens(idx, counts, 0, w.E, 6, 2)
    W1, W3, W2 = LazyExperts(inp["W1"]), LazyExperts(inp["W3"]), LazyExperts(inp["W2"])
    out, g = to_np(buf.out), buf.grads
    dx, dgate, dlog = to_np(g["dx"]), to_np(g["dgate"]), to_np(g["dlogits"])
    ref_out, ref_dx, ref_dg, ref_dl = [], [], [], []
    for t in toks:
        ref_out.append(O.forward_token(t, h["x"][t], h["logits"][t], W1, W3, W2, w.k)[2])
        a, b, c = O.backward_token(h["x"][t], h["logits"][t], h["dout"][t], W1, W3, W2, w.k)
        ref_dx.append(a); ref_dg.append(b); ref_dl.append(c)
    errs = {"out": rel_inf(out[toks], np.stack(ref_out)), "dx": rel_inf(dx[toks], np.stack(ref_dx)),
            "dgate": rel_inf(dgate[toks], np.stack(ref_dg)), "dlogits": rel_inf(dlog[toks], np.stack(ref_dl))}
    _, gate, _, _ = O.route(h["logits"], w.k)
    _, offsets, _, por = O.layout(idx, w.E)
    order = np.argsort(counts, kind="stable")
    # the lightest, the median and the heaviest expert (its tiles run the
    # longest K loops and its run is shared among several XCD queues)
    for e in (int(order[0]), int(order[len(order) // 2]), int(order[-1])):
        rows = por[offsets[e]:offsets[e + 1]]
        tok, slot = rows // w.k, rows % w.k
        r1, r3, r2 = O.expert_weight_grads(h["x"][tok], gate[tok, slot], h["dout"][tok], W1[e], W3[e], W2[e])
        errs[f"dW1[{e}]"] = rel_inf(to_np(g["dW1"][e]), r1)
        errs[f"dW3[{e}]"] = rel_inf(to_np(g["dW3"][e]), r3)
        errs[f"dW2[{e}]"] = rel_inf(to_np(g["dW2"][e]), r2)
    note(f"  P={P} errors " + ", ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if v > TOL_BF16}
    assert not bad, bad


# ------------------------------------------------------------------ determinism

def _all_outputs(buf):
    outs = [buf.out, buf.topk_idx, buf.topk_gate, buf.counts, buf.offsets]
    if buf.grads:
        outs += [buf.grads[n] for n in ("dx", "dW1", "dW3", "dW2", "dgate", "dlogits")]
    return [o.clone() for o in outs]


@pytest.mark.parametrize("name,over", [("bf16-skewed", dict(T=777, d=128, E=16, k=4, F=320)),
                                       ("bf16_train", dict())])
def test_reruns_bitwise_identical(name, over):
    w = W.scaled("bf16_train", **over)
    note(f"determinism {name}")
    inp = _inputs(w)
    buf = run_layer(w, inp, backward=True)
    first = _all_outputs(buf)
    for rep in range(9):            # ten runs in all
        buf.workspace.fill_(0xFF)   # poison the scratch between runs
        buf = run_layer(w, inp, backward=True, buf=buf)
        again = _all_outputs(buf)
        for a, b in zip(first, again):
            assert torch.equal(a, b), f"rerun {rep} differs"
