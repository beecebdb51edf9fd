"""Pins of the oracle's MXFP4 functions (no GPU).

E2M1 against the OCP Microscaling v1.0 table of the FP4 element format
(tests/golden/e2m1_ocp_mx.txt, every code) and against an encoder written by
enumeration (nearest of the eight magnitudes, ties to the even code, above 6
saturating); the MXFP4 block scale 2^(floor(log2 amax) - 2) on hand blocks;
and the oracle's MXFP4 forward against a second implementation in
pure-Python scalar loops on a tiny layer (enumerated rounding, math.frexp
scales, explicit sums).  A wrong exponent offset in the scale, a rounding
that goes up on ties, a missing saturation, a quantisation along the wrong
axis or a missing one fails one of these.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

from oracle import mok_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

_MAGS = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]   # code c (0..7) holds _MAGS[c]


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()[:2]
            rows.append((int(c, 16), float(v)))
    return rows


def _enum_code(x: float) -> int:
    """E2M1 code of x by enumeration: the nearest magnitude (ties to the even
    code, i.e. mantissa bit 0), saturating at 6; sign bit from x's sign."""
    a = min(abs(x), 6.0)
    best = min(range(8), key=lambda c: (abs(_MAGS[c] - a), c & 1))
    return best | (8 if math.copysign(1.0, x) < 0 else 0)


def test_e2m1_table_from_the_mx_spec():
    rows = _golden()
    assert len(rows) == 16 and sorted(c for c, _ in rows) == list(range(16))
    codes = np.array([c for c, _ in rows])
    vals = np.array([v for _, v in rows])
    np.testing.assert_array_equal(O.e2m1_decode(codes), vals)
    np.testing.assert_array_equal(np.signbit(O.e2m1_decode(codes)), np.signbit(vals))
    np.testing.assert_array_equal(O.e2m1_encode(vals), codes.astype(np.uint8))
    assert [v for c, v in rows if c < 8] == _MAGS


def test_e2m1_rounding_hand_cases():
    enc = lambda v: int(O.e2m1_encode(np.array([v]))[0])
    # exact midpoints go to the even code
    for v, code in [(0.25, 0x0), (0.75, 0x2), (1.25, 0x2), (1.75, 0x4), (2.5, 0x4), (3.5, 0x6), (5.0, 0x6)]:
        assert enc(v) == code, v
        assert enc(-v) == code | 8, -v
    # just past a midpoint rounds away from the even code
    for v, code in [(0.2500001, 0x1), (0.7499999, 0x1), (1.2500001, 0x3), (2.5000001, 0x5), (5.0000001, 0x7)]:
        assert enc(v) == code, v
    # saturation, signed zeros
    for v in (6.0, 6.5, 7.99, 1e30):
        assert enc(v) == 0x7 and enc(-v) == 0xF
    assert enc(0.0) == 0x0 and enc(-0.0) == 0x8 and enc(-0.1) == 0x8 and enc(0.1) == 0x0
    with pytest.raises(ValueError):
        O.e2m1_encode(np.array([np.inf]))


def test_e2m1_encoder_matches_enumeration():
    rng = np.random.default_rng(4)
    v = np.concatenate([rng.uniform(-8, 8, 20000), rng.standard_normal(5000) * 0.3,
                        np.array([m for a, b in zip(_MAGS, _MAGS[1:]) for m in ((a + b) / 2, -(a + b) / 2)])])
    got = O.e2m1_encode(v)
    exp = np.array([_enum_code(float(x)) for x in v], dtype=np.uint8)
    np.testing.assert_array_equal(got, exp)
    np.testing.assert_array_equal(O.e2m1_encode(O.e2m1_decode(np.arange(16))), np.arange(16, dtype=np.uint8))


def test_mxfp4_quantize_hand_blocks_and_invariants():
    # all-zero block: scale byte 0, codes 0
    c0, s0 = O.mxfp4_quantize(np.zeros((1, 32)))
    assert s0.tolist() == [[0]] and not c0.any()
    # amax = 2^5 exactly: X = 2^3, that element is 4 (code 6)
    blk = np.zeros((1, 32)); blk[0, 3] = 32.0; blk[0, 7] = -3.0
    c1, s1 = O.mxfp4_quantize(blk)
    assert s1[0, 0] == 127 + 3 and c1[0, 3] == 0x6
    assert c1[0, 7] == 0x8 | 0x1            # -3 / 8 = -0.375 -> -0.5
    # amax = 15: X = 2 (floor(log2 15) = 3), 15 / 2 = 7.5 saturates to 6 -> 12
    blk2 = np.full((1, 32), 0.25); blk2[0, 0] = 15.0
    c2, s2 = O.mxfp4_quantize(blk2)
    assert s2[0, 0] == 128 and c2[0, 0] == 0x7
    dq = O.mxfp4_dequantize(c2, s2)
    assert dq[0, 0] == 12.0 and dq[0, 1] == 0.0   # 0.25 / 2 = 0.125 -> 0
    # two blocks per row get their own scales
    v = np.concatenate([np.full(32, 1.0), np.full(32, 1e-3)])[None, :]
    _, s3 = O.mxfp4_quantize(v)
    assert s3[0, 0] == 127 - 2 and s3[0, 1] == 127 + (-10) - 2
    # invariants: idempotent, error at most a quarter of the block's top binade
    # below saturation, sign kept
    rng = np.random.default_rng(9)
    v = rng.standard_normal((64, 128)) * np.exp(rng.uniform(-6, 6, (64, 1)))
    q = O.mxfp4_qdq(v)
    np.testing.assert_array_equal(O.mxfp4_qdq(q), q)
    codes, scales = O.mxfp4_quantize(v)
    X = np.repeat(np.ldexp(1.0, scales.astype(np.int64) - 127), 32, axis=-1)
    under = np.abs(v) <= 6 * X
    assert np.all(np.abs(q - v)[under] <= X[under])         # half the spacing 2 X of [4 X, 6 X]
    assert np.all(np.abs(q - v)[np.abs(v) <= X] <= 0.25 * X[np.abs(v) <= X])
    assert np.all(np.sign(q) * np.sign(v) >= 0)
    with pytest.raises(ValueError):
        O.mxfp4_quantize(np.zeros((2, 40)))


def _qdq_row(row):
    out = []
    for b0 in range(0, len(row), 32):
        blk = row[b0:b0 + 32]
        amax = max(abs(v) for v in blk)
        if amax == 0.0:
            out.extend(0.0 * v for v in blk)
            continue
        _, ex = math.frexp(amax)
        X = 2.0 ** max(-127, min(127, ex - 1 - 2))
        out.extend(math.copysign(_MAGS[_enum_code(v / X) & 7], v) * X for v in blk)
    return out


def _silu(z):
    return z / (1.0 + math.exp(-z))


def test_mxfp4_forward_matches_scalar_loops():
    rng = np.random.default_rng(21)
    T, d, F, E, k = 4, 64, 96, 3, 2
    x = rng.standard_normal((T, d)).astype(np.float32).astype(np.float64)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    W1 = 0.3 * rng.standard_normal((E, F, d))
    W3 = 0.3 * rng.standard_normal((E, F, d))
    W2 = 0.3 * rng.standard_normal((E, d, F))
    fw = O.forward(x, logits, W1, W3, W2, k, mxfp4=True)
    out = np.zeros((T, d))
    for t in range(T):
        lt = [float(v) for v in logits[t]]
        m = max(lt)
        z = sum(math.exp(v - m) for v in lt)
        order = sorted(range(E), key=lambda e: (-lt[e], e))[:k]
        xq = _qdq_row(list(x[t]))
        for e in order:
            w1 = [_qdq_row(list(r)) for r in W1[e]]
            w3 = [_qdq_row(list(r)) for r in W3[e]]
            w2 = [_qdq_row(list(r)) for r in W2[e]]
            a = [sum(p * q for p, q in zip(xq, w)) for w in w1]
            b = [sum(p * q for p, q in zip(xq, w)) for w in w3]
            h = _qdq_row([_silu(ai) * bi for ai, bi in zip(a, b)])
            y = [sum(p * q for p, q in zip(h, w)) for w in w2]
            g = math.exp(lt[e] - m) / z
            for c in range(d):
                out[t, c] += g * y[c]
    err = np.abs(fw["out"] - out).max() / np.abs(out).max()
    assert err < 1e-12, err
    # the quantisation is not a no-op, and not MXFP8's
    plain = O.forward(x, logits, W1, W3, W2, k)["out"]
    m8 = O.forward(x, logits, W1, W3, W2, k, mxfp8=True)["out"]
    assert np.abs(plain - fw["out"]).max() > 1e-2 * np.abs(plain).max()
    assert np.abs(m8 - fw["out"]).max() > 1e-2 * np.abs(plain).max()


def test_mxfp4_token_view_matches_the_layer_and_backward_refuses():
    rng = np.random.default_rng(6)
    T, d, F, E, k = 12, 64, 64, 4, 2
    x = rng.standard_normal((T, d))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    W1, W3 = (0.2 * rng.standard_normal((E, F, d)) for _ in range(2))
    W2 = 0.2 * rng.standard_normal((E, d, F))
    W1l, W3l, W2l = W1[1:3], W3[1:3], W2[1:3]
    fw = O.forward(x, logits, W1l, W3l, W2l, k, expert_begin=1, expert_end=3, mxfp4=True)
    for t in (0, 5, 11):
        _, _, out_t, _ = O.forward_token(t, x[t], logits[t], W1l, W3l, W2l, k, 1, 3, mxfp4=True)
        np.testing.assert_allclose(out_t, fw["out"][t], rtol=1e-12, atol=1e-12)
    with pytest.raises(ValueError):
        O.backward(np.ones((T, d)), x, logits, W1l, W3l, W2l, k, fwd=fw, expert_begin=1, expert_end=3)
    with pytest.raises(ValueError):
        O.forward(x, logits, W1, W3, W2, k, mxfp8=True, mxfp4=True)
