"""How sensitive the MXFP8 layer's d(router logits) is to the rounding of the
scaled matrix products, at the shapes of the MXFP8 parity tests (CPU only).

The gfx950 scaled MFMA does not return the exactly rounded fp32 sum of its
products: tests/test_gpu_mfma_probe.py measures errors of about 2^-16 of an
element's sum of magnitudes, up to 1.3e-4.  Here the oracle's own MXFP8
forward is run twice, once as written and once with every pre-activation
a = Q(x) Q(W1)^T and b = Q(x) Q(W3)^T scaled by (1 + u), u uniform in
[-2^-16, 2^-16].  Such a perturbation flips about 0.01 % of the E4M3 codes
of H = silu(a) b.  At d 128, F 256, k 1 with one expert taking nearly every
row, that alone moves d(logits) by up to 4e-2 (infinity-norm relative), past
the 3e-2 bar; that is the size of the GPU's measured deviation there.  At
d 256, F 512 it stays near 5e-3.  The small shape is therefore kept as an
expected failure on the GPU, and the MXFP8 parity cases use the larger one."""
import numpy as np

import workloads as W
from oracle import mok_oracle as O


def _dlogits(w, inp, eps, seed):
    x = inp["x"].float().numpy().astype(np.float64)
    dout = inp["dout"].float().numpy().astype(np.float64)
    W1, W3, W2 = (inp[n].float().numpy().astype(np.float64) for n in ("W1", "W3", "W2"))
    idx, gate, _, p = O.route(inp["logits"].numpy(), w.k)
    rng = np.random.default_rng(seed)
    y = np.zeros((w.T, w.d))
    for e in range(w.E):
        toks = np.nonzero(idx[:, 0] == e)[0]
        if not len(toks):
            continue
        xq = O.mxfp8_qdq(x[toks])
        a = xq @ O.mxfp8_qdq(W1[e]).T
        b = xq @ O.mxfp8_qdq(W3[e]).T
        a = a * (1 + eps * rng.uniform(-1, 1, a.shape))
        b = b * (1 + eps * rng.uniform(-1, 1, b.shape))
        y[toks] = O.mxfp8_qdq(O.silu(a) * b) @ O.mxfp8_qdq(W2[e]).T
    dgate = np.einsum("td,td->t", dout, y)[:, None]        # k = 1: one slot
    return O.route_backward(p, idx, gate, dgate)


def _worst_move(d, F):
    w = W.scaled("bf16_train", precision="mxfp8", backward=True, T=520, d=d, E=6, k=1, F=F, notes={"zipf": 4.0})
    inp = W.make_inputs(w, device="cpu")
    ref = _dlogits(w, inp, 0.0, 0)
    moves = [np.abs(_dlogits(w, inp, 2.0 ** -16, s) - ref).max() / np.abs(ref).max() for s in range(3)]
    return max(moves), ref


def test_dlogits_sensitivity_small_shape_over_the_bar():
    move, ref = _worst_move(128, 256)
    assert np.isfinite(ref).all()
    assert move > 3e-2, move


def test_dlogits_sensitivity_tested_shape_under_the_bar():
    move, _ = _worst_move(256, 512)
    assert move < 1e-2, move
