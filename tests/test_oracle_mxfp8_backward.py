"""Pins of the oracle's MXFP8 backward (no GPU).

The oracle's backward(mxfp8=True) is checked against a second implementation
written with pure-Python scalar loops on a tiny layer: its E4M3 rounding
enumerates every value the OCP OFP8 E4M3 format can hold (bias 7, three
mantissa bits, subnormals m * 2^-9, largest 448) and takes the nearest, ties to
the even code, instead of the oracle's frexp arithmetic; its MX block scale is
2^(floor(log2 amax) - 8) from math.frexp (OCP Microscaling v1.0); its products
are explicit sums.  Each product quantises its two operands along the axis it
contracts (dh: dy and W2 along d; dx: da, db and W1, W3 along F); the weight
gradients use the unquantised operands.  A quantisation along the wrong axis,
a missing quantisation, a transposed weight or a swapped gradient moves the
result by far more than the 1e-9 tolerance.
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import mok_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _e4m3_values():
    """(code, value) for every finite non-negative E4M3 code, by enumeration."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue  # NaN
            code = (e << 3) | m
            v = m * 2.0 ** -9 if e == 0 else (1.0 + m / 8.0) * 2.0 ** (e - 7)
            out.append((code, v))
    return out


_VALUES = _e4m3_values()


def test_enumeration_matches_the_ofp8_table():
    table = {}
    with open(os.path.join(GOLDEN, "e4m3_ocp_ofp8.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()[:2]
            if v.lower() != "nan":
                table[int(c, 16)] = float(v)
    mine = dict(_VALUES)
    for c, v in table.items():
        if c < 0x80:
            assert mine[c] == v, hex(c)
    assert max(mine.values()) == 448.0 and len(mine) == 127


def _round_e4m3(x: float) -> float:
    """Nearest E4M3 value to x (ties to the even code), saturating at 448."""
    a = min(abs(x), 448.0)
    best = None
    for code, v in _VALUES:
        dist = abs(v - a)
        key = (dist, code & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return math.copysign(best[1], x)


def _qdq_row(row):
    """MX quantise-dequantise of a list along its length, blocks of 32."""
    out = []
    for b0 in range(0, len(row), 32):
        blk = row[b0:b0 + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out.extend(0.0 * v for v in blk)
            continue
        _, ex = math.frexp(amax)           # amax = m 2^ex, m in [0.5, 1)
        se = max(-127, min(127, ex - 1 - 8))
        X = 2.0 ** se
        out.extend(_round_e4m3(v / X) * X for v in blk)
    return out


def _qdq_rows(M):
    return [_qdq_row(list(r)) for r in M]


def _transpose(M):
    return [list(c) for c in zip(*M)]


def _matmul_nt(A, B):
    """A [m, K] times B [n, K]^T by explicit sums."""
    return [[sum(a * b for a, b in zip(ra, rb)) for rb in B] for ra in A]


def _silu(z):
    return z / (1.0 + math.exp(-z))


def _sig(z):
    return 1.0 / (1.0 + math.exp(-z))


def _brute(x, logits, g, W1, W3, W2, k):
    T, d = x.shape
    E, F = W1.shape[0], W1.shape[1]
    out = {"dx": np.zeros((T, d)), "dgate": np.zeros((T, k)), "dW1": np.zeros((E, F, d)),
           "dW3": np.zeros((E, F, d)), "dW2": np.zeros((E, d, F))}
    # weights quantised once per product axis
    w1q = [_qdq_rows(W1[e].tolist()) for e in range(E)]          # along d (forward)
    w3q = [_qdq_rows(W3[e].tolist()) for e in range(E)]
    w2q = [_qdq_rows(W2[e].tolist()) for e in range(E)]          # along F (forward)
    w2tq = [_qdq_rows(_transpose(W2[e].tolist())) for e in range(E)]   # [F, d] along d
    w1tq = [_qdq_rows(_transpose(W1[e].tolist())) for e in range(E)]   # [d, F] along F
    w3tq = [_qdq_rows(_transpose(W3[e].tolist())) for e in range(E)]
    for t in range(T):
        lt = [float(v) for v in logits[t]]
        m = max(lt)
        z = sum(math.exp(v - m) for v in lt)
        p = [math.exp(v - m) / z for v in lt]
        # top-k: larger logit first, lower index on ties
        order = sorted(range(E), key=lambda e: (-lt[e], e))[:k]
        xq = _qdq_row(list(x[t]))
        dg = []
        for j, e in enumerate(order):
            a = _matmul_nt([xq], w1q[e])[0]
            b = _matmul_nt([xq], w3q[e])[0]
            h = [_silu(ai) * bi for ai, bi in zip(a, b)]
            y = _matmul_nt([_qdq_row(h)], w2q[e])[0]
            gt = [float(v) for v in g[t]]
            dgj = sum(gi * yi for gi, yi in zip(gt, y))
            dg.append(dgj)
            dy = [p[e] * gi for gi in gt]
            dh = _matmul_nt([_qdq_row(dy)], w2tq[e])[0]
            da = [dh[f] * b[f] * _sig(a[f]) * (1.0 + a[f] * (1.0 - _sig(a[f]))) for f in range(F)]
            db = [dh[f] * _silu(a[f]) for f in range(F)]
            dxa = _matmul_nt([_qdq_row(da)], w1tq[e])[0]
            dxb = _matmul_nt([_qdq_row(db)], w3tq[e])[0]
            for c in range(d):
                out["dx"][t, c] += dxa[c] + dxb[c]
            for f in range(F):
                for c in range(d):
                    out["dW1"][e, f, c] += da[f] * float(x[t, c])
                    out["dW3"][e, f, c] += db[f] * float(x[t, c])
            for c in range(d):
                for f in range(F):
                    out["dW2"][e, c, f] += dy[c] * h[f]
        out["dgate"][t] = dg
    return out


def test_mxfp8_backward_matches_scalar_loops():
    rng = np.random.default_rng(11)
    T, d, F, E, k = 3, 64, 64, 3, 2
    x = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    W1 = (0.3 * rng.standard_normal((E, F, d))).astype(np.float32).astype(np.float64)
    W3 = (0.3 * rng.standard_normal((E, F, d))).astype(np.float32).astype(np.float64)
    W2 = (0.3 * rng.standard_normal((E, d, F))).astype(np.float32).astype(np.float64)
    g = rng.standard_normal((T, d))
    fwd = O.forward(x, logits, W1, W3, W2, k, mxfp8=True)
    bw = O.backward(g, x, logits, W1, W3, W2, k, fwd=fwd, mxfp8=True)
    ref = _brute(x, logits, g, W1, W3, W2, k)
    for name in ("dx", "dgate", "dW1", "dW3", "dW2"):
        got, exp = bw[name], ref[name]
        err = np.abs(got - exp).max() / max(np.abs(exp).max(), 1e-300)
        assert err < 1e-9, (name, err)
    # the quantisation is not a no-op here: the plain backward differs
    plain = O.backward(g, x, logits, W1, W3, W2, k)
    assert np.abs(plain["dx"] - bw["dx"]).max() > 1e-3 * np.abs(bw["dx"]).max()


def test_mxfp8_token_and_expert_views_match_the_layer():
    """backward_token and expert_weight_grads (the sampled checks at full size)
    agree with the whole-layer MXFP8 backward."""
    rng = np.random.default_rng(5)
    T, d, F, E, k = 16, 64, 128, 4, 2
    x = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    W1 = (0.1 * rng.standard_normal((E, F, d))).astype(np.float64)
    W3 = (0.1 * rng.standard_normal((E, F, d))).astype(np.float64)
    W2 = (0.1 * rng.standard_normal((E, d, F))).astype(np.float64)
    g = rng.standard_normal((T, d))
    bw = O.backward(g, x, logits, W1, W3, W2, k, mxfp8=True)
    for t in (0, 7, 15):
        dx, dgate, dl = O.backward_token(x[t], logits[t], g[t], W1, W3, W2, k, mxfp8=True)
        np.testing.assert_allclose(dx, bw["dx"][t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dgate, bw["dgate"][t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dl, bw["dlogits"][t], rtol=1e-12, atol=1e-12)
    fwd = O.forward(x, logits, W1, W3, W2, k, mxfp8=True)
    rop = fwd["row_of_pair"].reshape(T, k)
    for e in range(E):
        toks, slots = np.nonzero(fwd["idx"] == e)
        if toks.size == 0:
            continue
        dW1, dW3, dW2 = O.expert_weight_grads(x[toks], fwd["gate"][toks, slots], g[toks], W1[e], W3[e], W2[e],
                                              mxfp8=True)
        np.testing.assert_allclose(dW1, bw["dW1"][e], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dW3, bw["dW3"][e], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(dW2, bw["dW2"][e], rtol=1e-10, atol=1e-12)
    assert (rop >= 0).all()


def _bf16(vals):
    """bfloat16 rounding of a float32 computation, by torch's own conversion."""
    return torch.tensor(vals, dtype=torch.float64).to(torch.bfloat16).double().tolist()


def _brute_wgrad_rows(x, logits, g, W1, W3, W2, k):
    """MXFP8 weight gradients by scalar loops, each operand quantised along
    the rows of its expert's segment: the segment lists the expert's (token,
    slot) pairs in ascending pair index t*k + j (the counting sort's stable
    order), blocks of 32 rows from its first row, the last block partial."""
    T, d = x.shape
    E, F = W1.shape[0], W1.shape[1]
    w1q = [_qdq_rows(W1[e].tolist()) for e in range(E)]
    w3q = [_qdq_rows(W3[e].tolist()) for e in range(E)]
    w2q = [_qdq_rows(W2[e].tolist()) for e in range(E)]
    w2tq = [_qdq_rows(_transpose(W2[e].tolist())) for e in range(E)]
    seg = {e: [] for e in range(E)}   # per expert: rows of (x, dy, h, da, db)
    for t in range(T):
        lt = [float(v) for v in logits[t]]
        m = max(lt)
        z = sum(math.exp(v - m) for v in lt)
        p = [math.exp(v - m) / z for v in lt]
        order = sorted(range(E), key=lambda e: (-lt[e], e))[:k]
        xq = _qdq_row(list(x[t]))
        for e in order:           # slot j ascending: pair index t*k + j ascending
            a = _matmul_nt([xq], w1q[e])[0]
            b = _matmul_nt([xq], w3q[e])[0]
            h = [_silu(ai) * bi for ai, bi in zip(a, b)]
            dy = [p[e] * float(gi) for gi in g[t]]
            dh = _matmul_nt([_qdq_row(dy)], w2tq[e])[0]
            da = [dh[f] * b[f] * _sig(a[f]) * (1.0 + a[f] * (1.0 - _sig(a[f]))) for f in range(F)]
            db = [dh[f] * _silu(a[f]) for f in range(F)]
            # the operands as the layer holds them: bf16 (x already is)
            seg[e].append((list(map(float, x[t])), _bf16(dy), _bf16(h), _bf16(da), _bf16(db)))
    out = {"dW1": np.zeros((E, F, d)), "dW3": np.zeros((E, F, d)), "dW2": np.zeros((E, d, F))}
    for e in range(E):
        if not seg[e]:
            continue
        # quantise every column along the segment's rows
        cols = [_qdq_rows(_transpose([r[i] for r in seg[e]])) for i in range(5)]   # [col][row]
        X, DY, H, DA, DB = cols
        n = len(seg[e])
        for f in range(F):
            for c in range(d):
                out["dW1"][e, f, c] = sum(DA[f][r] * X[c][r] for r in range(n))
                out["dW3"][e, f, c] = sum(DB[f][r] * X[c][r] for r in range(n))
        for c in range(d):
            for f in range(F):
                out["dW2"][e, c, f] = sum(DY[c][r] * H[f][r] for r in range(n))
    return out


def test_mxfp8_row_quantised_weight_grads_match_scalar_loops():
    rng = np.random.default_rng(23)
    T, d, F, E, k = 41, 32, 32, 3, 2
    x = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 1] += 1.5    # expert 1 takes more than one block of rows
    W1 = (0.3 * rng.standard_normal((E, F, d))).astype(np.float32).astype(np.float64)
    W3 = (0.3 * rng.standard_normal((E, F, d))).astype(np.float32).astype(np.float64)
    W2 = (0.3 * rng.standard_normal((E, d, F))).astype(np.float32).astype(np.float64)
    g = rng.standard_normal((T, d))
    fwd = O.forward(x, logits, W1, W3, W2, k, mxfp8=True)
    sizes = np.diff(fwd["offsets"])
    # segments longer than one block, starting off a 32-row boundary
    assert sizes.max() > 32 and any(o % 32 for o in fwd["offsets"][1:-1])
    bw = O.backward(g, x, logits, W1, W3, W2, k, fwd=fwd, mxfp8=True, mxfp8_wgrad=True)
    ref = _brute_wgrad_rows(x, logits, g, W1, W3, W2, k)
    for name in ("dW1", "dW3", "dW2"):
        err = np.abs(bw[name] - ref[name]).max() / np.abs(ref[name]).max()
        assert err < 1e-9, (name, err)
    # the row quantisation is not a no-op, and blocks aligned to the buffer's
    # row 0 instead of each expert's first row give another result
    plain = O.backward(g, x, logits, W1, W3, W2, k, fwd=fwd, mxfp8=True)
    assert np.abs(plain["dW1"] - bw["dW1"]).max() > 1e-3 * np.abs(bw["dW1"]).max()
    e = int(np.argmax([o % 32 != 0 for o in fwd["offsets"][:-1]]))
    r0, r1 = fwd["offsets"][e], fwd["offsets"][e + 1]
    glob = O.mxfp8_qdq_rows(bw["dA"])[r0:r1].T @ O.mxfp8_qdq_rows(O.permute(x, fwd["pair_of_row"], k))[r0:r1]
    assert np.abs(glob - bw["dW1"][e]).max() > 1e-3 * np.abs(bw["dW1"][e]).max()
    # the other backward outputs are those of the bf16-weight-gradient reading
    for name in ("dx", "dgate", "dlogits"):
        np.testing.assert_array_equal(plain[name], bw[name])


def test_row_quantisation_partial_block():
    """A partial last block takes its scale from its own rows: a segment of
    33 rows whose last row is tiny keeps that row to E4M3 precision, and the
    first 32 rows quantise as a block of their own."""
    rng = np.random.default_rng(3)
    M = rng.standard_normal((33, 4))
    M[32] = 1e-6 * rng.standard_normal(4)
    q = O.mxfp8_qdq_rows(M)
    np.testing.assert_array_equal(q[:32], O.mxfp8_qdq_rows(M[:32]))
    assert np.all(np.abs(q[32] - M[32]) <= 2.0 ** -4 * np.abs(M[32]))
    assert np.all(q[32] != 0)


def test_expert_view_row_quantised():
    rng = np.random.default_rng(8)
    T, d, F, E, k = 48, 64, 64, 2, 2
    x = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    W1 = (0.1 * rng.standard_normal((E, F, d))).astype(np.float64)
    W3 = (0.1 * rng.standard_normal((E, F, d))).astype(np.float64)
    W2 = (0.1 * rng.standard_normal((E, d, F))).astype(np.float64)
    g = rng.standard_normal((T, d))
    fwd = O.forward(x, logits, W1, W3, W2, k, mxfp8=True)
    bw = O.backward(g, x, logits, W1, W3, W2, k, fwd=fwd, mxfp8=True, mxfp8_wgrad=True)
    por = fwd["pair_of_row"]
    for e in range(E):
        r0, r1 = fwd["offsets"][e], fwd["offsets"][e + 1]
        toks, slots = por[r0:r1] // k, por[r0:r1] % k
        got = O.expert_weight_grads(x[toks], fwd["gate"][toks, slots], g[toks], W1[e], W3[e], W2[e],
                                    mxfp8=True, mxfp8_wgrad=True)
        for gv, name in zip(got, ("dW1", "dW3", "dW2")):
            np.testing.assert_allclose(gv, bw[name][e], rtol=1e-10, atol=1e-12)


def test_bf16_round_matches_torch_and_hand_cases():
    """bf16_round: torch's bfloat16 conversion of the same values (float64 to
    float32 to bfloat16, nearest-even at each step), ties to even by hand,
    subnormal spacing, idempotence."""
    rng = np.random.default_rng(17)
    v = np.concatenate([rng.standard_normal(20000) * np.exp(rng.uniform(-60, 60, 20000)),
                        rng.standard_normal(1000) * 1e-39, [0.0, -0.0, 1.0, -3.5]])
    ref = torch.tensor(v, dtype=torch.float64).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(O.bf16_round(v), ref)
    # spacing 2^-7 at 1: halfway cases go to the even mantissa
    assert O.bf16_round(1 + 2.0 ** -8) == 1.0
    assert O.bf16_round(1 + 3 * 2.0 ** -8) == 1 + 2.0 ** -6
    assert O.bf16_round(-(1 + 3 * 2.0 ** -8)) == -(1 + 2.0 ** -6)
    assert O.bf16_round(1 + 2.0 ** -8 + 2.0 ** -20) == 1 + 2.0 ** -7
    # below 2^-126 the spacing is 2^-133
    assert O.bf16_round(3 * 2.0 ** -134) == 2 * 2.0 ** -133
    r = O.bf16_round(v)
    np.testing.assert_array_equal(O.bf16_round(r), r)
