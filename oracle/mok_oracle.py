"""Plain, slow, obviously-correct CPU oracle of the fused deterministic MoE layer.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  The GPU library never uses
it, shares no code with it, and must fail loudly rather than fall back to it.

Everything is float64 numpy.  Inputs arrive as numpy arrays (bf16 values are
widened exactly through float32).  Library primitives used as steps: stable
argsort, bincount, cumsum and dense matmul.  No blocking, no fusion and no
reordering beyond the definitions below.

Pages followed (cited by title and section):
  [kucoin]  kucoin.com, «Cursor's MoK réalise une amélioration des performances
            de 2,37x sur NVIDIA GB300 NVL72», sections 01, 02 and 03.
  [fluid]   fluidifia.com, «Cursor ouvre MoK, un mégakernel qui accélère
            l'entraînement MoE», sections «Quand la communication devient le
            vrai problème» and «Comment MoK tente de gratter des millisecondes
            partout».
  [martel]  laura-martel.com post on Cursor's Mixture-of-Kittens, section «Le
            déterminisme est la partie sous-estimée».

What the layer computes (the method reaches exactly this result, only fused and
faster; [kucoin §03] says the benchmarked layer covers routing, expert FFNs,
combine and the final weighted sum):
  1. router: each token picks k experts from its router logits [kucoin §01];
  2. layout: count the pairs per expert, place every pair in an expert-
     contiguous buffer [kucoin §01, §02 (pull dispatch places rows locally)];
  3. expert FFN (SwiGLU, [kucoin §02 on MXFP8 fused into SwiGLU]) per expert
     over its contiguous rows (a grouped GEMM [kucoin §01]);
  4. combine: send every expert output back to its token and take the
     gate-weighted sum [kucoin §01, §03];
  5. backward: the same steps mirrored (reverse-combine, expert backward,
     reverse-dispatch) [kucoin §01, §02].

Readings taken where the pages are silent:
  * gates: softmax over all E logits, then top-k, no renormalisation (the
    default).  Router variants, for the DeepSeek-V3-type models the pages
    name as the target ([fluid], «Comment MoK…»): sigmoid affinities instead
    of softmax, and/or gates renormalised over the k chosen experts
    (gate_j = a_j / sum_i a_i).  The selection is the same in every variant
    (sigmoid is monotonic, so the top-k of the logits is the top-k of the
    affinities);
  * top-k compares the raw float32 logits; ties go to the lower expert index;
    slot j = 0 is the largest;
  * expert rows are stable: within an expert, ascending pair id p = t*k + j;
  * offsets: unpadded exclusive prefix sum with E+1 entries;
  * dropless (no capacity) [fluid, «Comment MoK…»: the ring buffer avoids
    throwing tokens away];
  * FFN: h = silu(x W1^T) * (x W3^T), y = h W2^T, W1 = gate, W3 = up, no bias;
  * the gate multiplies y in the combine; combine sums over j = 0..k-1 in
    ascending order (any fixed order gives run-to-run identical results, which
    is what [martel] claims; j order is the plainest);
  * MXFP8 follows the OCP Microscaling v1.0 conversion (blocks of 32 along the
    contraction axis, E8M0 shared scale 2^(floor(log2 amax) - 8), elements
    rounded to nearest-even E4M3 with saturation at +-448).
  * MXFP4, the analogue on this hardware of the NVFP4 kernels the pages say
    were tried before the megakernel ([fluid], «Quand la communication devient
    le vrai problème»; the pages give no recipe): the MXFP8 forward with E2M1
    elements instead of E4M3 (OCP Microscaling v1.0 MXFP4: blocks of 32, E8M0
    scale 2^(floor(log2 amax) - 2), elements rounded to nearest-even E2M1 with
    saturation at +-6) for x, the three weights and h; forward only.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "route", "route_backward", "router_logits", "router_logits_backward",
    "layout", "permute", "unpermute_sum", "silu", "expert_ffn",
    "forward", "backward", "combine", "loss",
    "bf16_round", "e4m3_encode", "e4m3_decode", "mxfp8_quantize", "mxfp8_dequantize", "mxfp8_qdq", "mxfp8_qdq_rows",
    "e2m1_encode", "e2m1_decode", "mxfp4_quantize", "mxfp4_dequantize", "mxfp4_qdq",
    "forward_token", "backward_token", "expert_weight_grads",
]


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ------------------------------------------------------------------ router

GATINGS = ("softmax", "sigmoid")


def route(logits, k: int, gating: str = "softmax", renorm: bool = False):
    """Routing with stable top-k.

    The router decides per step and per token which experts it goes to, and each
    token selects several experts [kucoin §01].  Order of experts for token t:
    a precedes b iff logit_a > logit_b, or the logits are equal and a < b.  The
    comparison uses the raw float32 logits (so the GPU and CPU agree exactly on
    the selection); the affinities are float64.

    Affinities a: softmax over the E logits ("softmax", the default) or the
    sigmoid of each logit ("sigmoid").  gate_j = a[idx_j], or with renorm
    a[idx_j] / sum_i a[idx_i] (i over the k chosen experts).

    Returns idx [T,k] int32, gate [T,k] float64, lse [T] float64 (log-sum-exp
    of the logits, whatever the gating), p [T,E] float64 (the affinities).
    """
    if gating not in GATINGS:
        raise ValueError(f"gating must be one of {GATINGS}")
    l32 = np.asarray(logits, dtype=np.float32)
    if l32.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = l32.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if not np.isfinite(l32).all():
        raise ValueError("router logits must be finite")
    # stable sort of the negated logits keeps equal logits in index order;
    # -0.0 and +0.0 compare equal, as in the comparison above.
    order = np.argsort(-l32, axis=1, kind="stable")
    idx = order[:, :k].astype(np.int32)
    l = l32.astype(np.float64)
    m = l.max(axis=1, keepdims=True) if E else np.zeros((T, 1))
    ex = np.exp(l - m)
    s = ex.sum(axis=1, keepdims=True)
    lse = (m + np.log(s))[:, 0]
    p = ex / s if gating == "softmax" else sigmoid(l)
    gate = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        gate = gate / gate.sum(axis=1, keepdims=True)
    return idx, gate, lse, p


def route_backward(p, idx, gate, dgate, gating: str = "softmax", renorm: bool = False):
    """d(logits) from d(gate), by the chain rule through route().

    p [T,E] affinities, idx [T,k], gate [T,k] (as route() returns them),
    dgate [T,k].  Two steps:
      1. d(affinity) of the chosen experts: dgate itself, or with renorm
         (gate_j = a_j / S, S = sum_i a_i) da_i = (dgate_i - sum_j gate_j dgate_j) / S;
         the other experts' affinities do not reach the gates (0);
      2. d(logit) through the affinity: softmax Jacobian p * (DA - <p, DA>),
         or the sigmoid's a (1 - a) DA, with DA [T,E] holding step 1.
    The selection itself has zero gradient.
    """
    p = _f64(p); gate = _f64(gate); dgate = _f64(dgate)
    i64 = np.asarray(idx).astype(np.int64)
    a_sel = np.take_along_axis(p, i64, axis=1)
    if renorm:
        S = a_sel.sum(axis=1, keepdims=True)
        da = (dgate - (gate * dgate).sum(axis=1, keepdims=True)) / S
    else:
        da = dgate
    DA = np.zeros_like(p)
    np.put_along_axis(DA, i64, da, axis=1)
    if gating == "softmax":
        return p * (DA - (p * DA).sum(axis=1, keepdims=True))
    return p * (1.0 - p) * DA


def router_logits(x, Wr):
    """Router GEMM: logits [T,E] = x [T,d] . Wr^T, Wr [E,d] one row per expert
    (the router's linear layer).  The benchmarked layer covers routing as
    well as the expert FFNs [kucoin §03]; float64."""
    return _f64(x) @ _f64(Wr).T


def router_logits_backward(x, Wr, dlogits):
    """Gradients through router_logits: dx = dlogits . Wr [T,d] and
    dWr = dlogits^T . x [E,d]; float64."""
    g = _f64(dlogits)
    return g @ _f64(Wr), g.T @ _f64(x)


# ------------------------------------------------------------------ layout

def layout(idx, E: int, expert_begin: int = 0, expert_end: int | None = None):
    """Counting-sort placement of token-expert pairs into expert-contiguous rows.

    First count the pairs per expert, then decide where each pair goes, keeping
    one expert's rows together so a grouped GEMM sees structured input
    [kucoin §01]; the receiver chooses its own local placement [kucoin §02].
    Only experts in [expert_begin, expert_end) are local; other pairs get no row.

    Pair id p = t*k + j.  Rows are ordered by (expert, p): stable within an
    expert.  Returns counts [E] int64 (0 for non-local experts), offsets [E+1]
    (exclusive prefix sum, offsets[E] = P), row_of_pair [T*k] int64 (-1 where
    non-local) and pair_of_row [P] int64.
    """
    idx = np.asarray(idx)
    if expert_end is None:
        expert_end = E
    e = idx.reshape(-1).astype(np.int64)
    local = (e >= expert_begin) & (e < expert_end)
    counts = np.bincount(e[local], minlength=E).astype(np.int64)
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    local_pairs = np.nonzero(local)[0]
    pair_of_row = local_pairs[np.argsort(e[local], kind="stable")]
    row_of_pair = np.full(e.shape[0], -1, dtype=np.int64)
    row_of_pair[pair_of_row] = np.arange(pair_of_row.shape[0], dtype=np.int64)
    return counts, offsets, row_of_pair, pair_of_row


def permute(x, pair_of_row, k: int):
    """Dispatch: row r of the expert-contiguous buffer is the activation of the
    token of pair pair_of_row[r] (token = pair // k) [kucoin §01, §02]."""
    return _f64(x)[np.asarray(pair_of_row) // k]


def unpermute_sum(rows, row_of_pair, T: int, k: int, weights=None):
    """out[t] = sum over j = 0..k-1 (ascending) of weights[t,j] * rows[row(t,j)],
    skipping pairs with no row.  weights None means all ones."""
    rows = _f64(rows)
    rop = np.asarray(row_of_pair).reshape(T, k)
    out = np.zeros((T,) + rows.shape[1:], dtype=np.float64)
    for j in range(k):
        sel = rop[:, j]
        m = sel >= 0
        w = 1.0 if weights is None else _f64(weights)[m, j][:, None]
        out[m] += w * rows[sel[m]]
    return out


def combine(Y, gate, row_of_pair, T: int, k: int):
    """Combine and the final weighted sum: out_t = sum_j gate[t,j] * y_(t,j),
    j ascending [kucoin §01, §03; martel on determinism]."""
    return unpermute_sum(Y, row_of_pair, T, k, weights=gate)


# ------------------------------------------------------------------ expert FFN

def silu(z):
    z = _f64(z)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def sigmoid(z):
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def expert_ffn(Xe, W1e, W3e, W2e):
    """SwiGLU expert [kucoin §02 names SwiGLU as the activation]:
    a = X W1^T, b = X W3^T, h = silu(a) * b, y = h W2^T."""
    Xe = _f64(Xe)
    a = Xe @ _f64(W1e).T
    b = Xe @ _f64(W3e).T
    h = silu(a) * b
    y = h @ _f64(W2e).T
    return a, b, h, y


# ------------------------------------------------------------------ MXFP8

E4M3_MAX = 448.0
_E4M3_EMAX = 8          # exponent of the largest power of two <= 448


def e4m3_encode(v):
    """Round float64 values to OCP E4M3 (bias 7, no infinities) codes.

    Round to nearest, ties to even; magnitudes above 448 saturate to 448; the
    sign of zero is kept.  Normal values have 3 fraction bits, so the spacing in
    [2^e, 2^(e+1)) is 2^(e-3); below 2^-6 the spacing is 2^-9 (subnormals)."""
    v = _f64(v)
    if not np.isfinite(v).all():
        raise ValueError("e4m3_encode expects finite values")
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, -6)                # floor(log2 a), at least -6
    q = np.ldexp(1.0, e - 3)                  # spacing of representable values
    n = np.rint(a / q)                        # exact division by a power of 2; RNE
    val = n * q                               # representable (may move up a binade)
    _, ex2 = np.frexp(val)
    e2 = ex2 - 1
    normal = val >= 2.0 ** -6
    code_norm = ((e2 + 7) << 3) | (np.rint(np.ldexp(val, -e2) * 8).astype(np.int64) - 8)
    code_sub = np.rint(val / 2.0 ** -9).astype(np.int64)
    code = np.where(normal, code_norm, code_sub)
    return (code | (sign.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(codes):
    """Value of E4M3 codes (S.EEEE.MMM, bias 7; S.1111.111 is NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return s * val


def bf16_round(v):
    """A float32 computation stored as bfloat16: each value is rounded to
    float32, then to the nearest bfloat16 (8 significant bits; spacing
    2^(e-7) in [2^e, 2^(e+1)), 2^-133 below 2^-126), ties to even.  Finite
    inputs."""
    f = np.asarray(_f64(v), np.float32).astype(np.float64)
    _, ex = np.frexp(f)
    e = np.maximum(ex - 1, -126)
    q = np.ldexp(1.0, e - 7)
    return np.rint(f / q) * q


def mxfp8_quantize(v, block: int = 32):
    """MX block quantisation along the last axis [kucoin §02: MXFP8 activation
    quantisation fused into the dispatch, grouped GEMM and SwiGLU paths].

    Per block of 32: X = 2^(floor(log2 amax) - 8), stored as E8M0 byte
    (unbiased exponent + 127, exponent clamped to [-127, 127]); an all-zero block
    stores byte 0.  Elements become E4M3(v / X).  Returns (codes uint8 of v's
    shape, scales uint8 of shape [..., K/32])."""
    v = _f64(v)
    K = v.shape[-1]
    if K % block:
        raise ValueError("last axis must be a multiple of the block size")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.abs(vb).max(axis=-1)
    _, ex = np.frexp(amax)
    sexp = np.clip(ex - 1 - _E4M3_EMAX, -127, 127)
    sexp = np.where(amax == 0, -127, sexp)
    codes = e4m3_encode(vb / np.ldexp(1.0, sexp)[..., None])
    return codes.reshape(v.shape), (sexp + 127).astype(np.uint8)


def mxfp8_dequantize(codes, scales, block: int = 32):
    c = e4m3_decode(codes)
    K = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (K // block, block))
    x = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)[..., None]
    return (cb * x).reshape(c.shape)


def mxfp8_qdq(v, block: int = 32):
    return mxfp8_dequantize(*mxfp8_quantize(v, block), block)


def mxfp8_qdq_rows(M, block: int = 32):
    """MX quantise-dequantise of a [rows, cols] matrix along its rows: each
    column is cut into blocks of 32 consecutive rows starting at row 0, and
    a last partial block takes its scale from the rows it has (zero rows
    appended to fill it change no block maximum)."""
    M = _f64(M)
    R = M.shape[0]
    pad = (-R) % block
    Mp = np.concatenate([M, np.zeros((pad,) + M.shape[1:])], axis=0) if pad else M
    return mxfp8_qdq(Mp.T, block).T[:R]


# ------------------------------------------------------------------ MXFP4

E2M1_MAX = 6.0
_E2M1_EMAX = 2          # exponent of the largest power of two <= 6


def e2m1_encode(v):
    """Round float64 values to OCP E2M1 codes (S.EE.M, exponent bias 1, no
    infinities or NaN; OCP Microscaling v1.0, FP4 element format).

    Round to nearest, ties to even; magnitudes above 6 saturate to 6; the sign
    of zero is kept.  Normal values (from 1 up) have one fraction bit, so the
    spacing in [2^e, 2^(e+1)) is 2^(e-1); below 1 the spacing is 0.5 (the one
    subnormal, 0.5).  The eight magnitudes: 0, 0.5, 1, 1.5, 2, 3, 4, 6."""
    v = _f64(v)
    if not np.isfinite(v).all():
        raise ValueError("e2m1_encode expects finite values")
    sign = np.signbit(v)
    a = np.minimum(np.abs(v), E2M1_MAX)
    _, ex = np.frexp(a)                       # a = m * 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, 0)                 # floor(log2 a), at least 0
    q = np.ldexp(1.0, e - 1)                  # spacing of representable values
    val = np.rint(a / q) * q                  # exact division by a power of 2; RNE
    _, ex2 = np.frexp(val)
    e2 = ex2 - 1
    normal = val >= 1.0
    code_norm = ((e2 + 1) << 1) | (np.rint(np.ldexp(val, -e2) * 2).astype(np.int64) - 2)
    code_sub = np.rint(val / 0.5).astype(np.int64)
    code = np.where(normal, code_norm, code_sub)
    return (code | (sign.astype(np.int64) << 3)).astype(np.uint8)


def e2m1_decode(codes):
    """Value of E2M1 codes (S.EE.M, bias 1; exponent field 0 is the subnormal
    M * 0.5)."""
    c = np.asarray(codes, dtype=np.int64)
    s = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 3
    m = c & 1
    val = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.ldexp(1.0, e - 1))
    return s * val


def mxfp4_quantize(v, block: int = 32):
    """MXFP4 block quantisation along the last axis (OCP Microscaling v1.0).

    Per block of 32: X = 2^(floor(log2 amax) - 2), stored as E8M0 byte
    (unbiased exponent + 127, exponent clamped to [-127, 127]); an all-zero
    block stores byte 0.  Elements become E2M1(v / X), one code (0..15) per
    element.  Returns (codes uint8 of v's shape, scales uint8 [..., K/32])."""
    v = _f64(v)
    K = v.shape[-1]
    if K % block:
        raise ValueError("last axis must be a multiple of the block size")
    vb = v.reshape(v.shape[:-1] + (K // block, block))
    amax = np.abs(vb).max(axis=-1)
    _, ex = np.frexp(amax)
    sexp = np.clip(ex - 1 - _E2M1_EMAX, -127, 127)
    sexp = np.where(amax == 0, -127, sexp)
    codes = e2m1_encode(vb / np.ldexp(1.0, sexp)[..., None])
    return codes.reshape(v.shape), (sexp + 127).astype(np.uint8)


def mxfp4_dequantize(codes, scales, block: int = 32):
    c = e2m1_decode(codes)
    K = c.shape[-1]
    cb = c.reshape(c.shape[:-1] + (K // block, block))
    x = np.ldexp(1.0, np.asarray(scales, dtype=np.int64) - 127)[..., None]
    return (cb * x).reshape(c.shape)


def mxfp4_qdq(v, block: int = 32):
    return mxfp4_dequantize(*mxfp4_quantize(v, block), block)


# ------------------------------------------------------------------ forward

def forward(x, logits, W1, W3, W2, k: int, expert_begin: int = 0, expert_end: int | None = None,
            mxfp8: bool = False, gating: str = "softmax", renorm: bool = False, mxfp4: bool = False):
    """Whole-layer forward in float64.

    x [T,d]; logits [T,E] float32; W1, W3 [E_loc,F,d]; W2 [E_loc,d,F] with
    E_loc = expert_end - expert_begin (weights of expert e at e - expert_begin).
    In MXFP8 mode x rows and W1/W3 rows are quantised along d, W2 rows along F,
    and h along F before the second product (gates, softmax and the combine stay
    float64).  MXFP4 mode quantises the same operands along the same axes to
    MXFP4 (mxfp4_qdq) instead.  Returns a dict with idx, gate, lse, p, counts,
    offsets, row_of_pair, pair_of_row, A, B, H, Y (per row, unscaled) and out
    [T,d].
    """
    if mxfp8 and mxfp4:
        raise ValueError("one of mxfp8, mxfp4")
    qdq = mxfp8_qdq if mxfp8 else (mxfp4_qdq if mxfp4 else None)
    x = _f64(x)
    T, d = x.shape
    E = np.asarray(logits).shape[1]
    if expert_end is None:
        expert_end = E
    idx, gate, lse, p = route(logits, k, gating, renorm)
    counts, offsets, row_of_pair, pair_of_row = layout(idx, E, expert_begin, expert_end)
    Xp = permute(x, pair_of_row, k)
    F = np.asarray(W1).shape[1]
    P = pair_of_row.shape[0]
    A = np.zeros((P, F)); B = np.zeros((P, F)); H = np.zeros((P, F)); Y = np.zeros((P, d))
    for e in range(expert_begin, expert_end):
        r0, r1 = offsets[e], offsets[e + 1]
        if r0 == r1:
            continue
        w1, w3, w2 = W1[e - expert_begin], W3[e - expert_begin], W2[e - expert_begin]
        Xe = Xp[r0:r1]
        if qdq is not None:
            Xe, w1, w3, w2 = qdq(Xe), qdq(w1), qdq(w3), qdq(w2)
            a = Xe @ _f64(w1).T
            b = Xe @ _f64(w3).T
            h = qdq(silu(a) * b)
            y = h @ _f64(w2).T
        else:
            a, b, h, y = expert_ffn(Xe, w1, w3, w2)
        A[r0:r1], B[r0:r1], H[r0:r1], Y[r0:r1] = a, b, h, y
    out = combine(Y, gate, row_of_pair, T, k)
    return dict(idx=idx, gate=gate, lse=lse, p=p, counts=counts, offsets=offsets,
                row_of_pair=row_of_pair, pair_of_row=pair_of_row, A=A, B=B, H=H, Y=Y, out=out,
                gating=gating, renorm=renorm, mxfp8=mxfp8, mxfp4=mxfp4)


def forward_token(t: int, x_t, logits_t, W1, W3, W2, k: int, expert_begin: int = 0,
                  expert_end: int | None = None, mxfp8: bool = False, gating: str = "softmax",
                  renorm: bool = False, mxfp4: bool = False):
    """Output of one token alone (for sampled checks at full size): its top-k
    experts from its own logits, the FFN of each local one, the gate-weighted
    sum in slot order.  Returns (idx [k], gate [k], out [d], y per slot)."""
    if mxfp8 and mxfp4:
        raise ValueError("one of mxfp8, mxfp4")
    qdq = mxfp8_qdq if mxfp8 else (mxfp4_qdq if mxfp4 else None)
    idx, gate, _, _ = route(np.asarray(logits_t, dtype=np.float32)[None, :], k, gating, renorm)
    E = np.asarray(logits_t).shape[0]
    if expert_end is None:
        expert_end = E
    xt = _f64(x_t)[None, :]
    out = np.zeros(xt.shape[1])
    ys = []
    for j in range(k):
        e = int(idx[0, j])
        if not expert_begin <= e < expert_end:
            ys.append(None)
            continue
        w1, w3, w2 = W1[e - expert_begin], W3[e - expert_begin], W2[e - expert_begin]
        if qdq is not None:
            xq = qdq(xt)
            h = qdq(silu(xq @ qdq(w1).T) * (xq @ qdq(w3).T))
            y = (h @ qdq(w2).T)[0]
        else:
            y = expert_ffn(xt, w1, w3, w2)[3][0]
        ys.append(y)
        out += gate[0, j] * y
    return idx[0], gate[0], out, ys


# ------------------------------------------------------------------ backward

def backward(dout, x, logits, W1, W3, W2, k: int, fwd: dict | None = None,
             expert_begin: int = 0, expert_end: int | None = None, gating: str = "softmax",
             renorm: bool = False, mxfp8: bool = False, mxfp8_wgrad: bool = False):
    """Gradients of L = sum(out * dout) in float64.

    The backward pass mirrors the forward: reverse-combine, expert backward,
    reverse-dispatch [kucoin §01: two more communication steps in the reverse
    direction; §02: pull reverse-combine, push reverse-dispatch].  The gradient
    through the top-k selection itself is zero.

      dgate[t,j]  = <dout_t, y_(t,j)>                       (0 for non-local pairs)
      dlogits     = route_backward(p, idx, gate, dgate)     (softmax, no renorm:
                    p * (G - <p, G>), G[t,e] = dgate at the chosen e, else 0)
      dy_r        = gate_r * dout_t(r)                      (reverse-combine)
      dh          = dy W2_e
      da          = dh * b * sigmoid(a) * (1 + a (1 - sigmoid(a)))
      db          = dh * silu(a)
      dx_r        = da W1_e + db W3_e
      dx_t        = sum_j dx_(t,j), j ascending              (reverse-dispatch)
      dW2_e = dy_e^T h_e,  dW1_e = da_e^T x_e,  dW3_e = db_e^T x_e

    MXFP8 mode (the pages report MXFP8 backward timings, [kucoin §03], but give
    no recipe; this is the reading taken): the forward is the MXFP8 one
    (fwd computed with mxfp8=True, so a, b and y come from quantised x, W1,
    W3, h and W2), and each backward product whose result flows on to dx
    quantises both operands along its own contraction axis:
      dh   = Q(dy) Q(W2_e^T)^T            (dy rows and W2_e columns along d)
      dx_r = Q(da) Q(W1_e^T)^T + Q(db) Q(W3_e^T)^T   (along F)
    where Q is mxfp8_qdq over the last axis.  The weight gradients take the
    unquantised operands: dW2_e = dy_e^T h_e with h = silu(a) * b before its
    quantisation, dW1_e = da_e^T x_e, dW3_e = db_e^T x_e.

    mxfp8_wgrad (with mxfp8) also runs the weight gradients in MXFP8: their
    contraction runs over the expert's rows, so each operand is quantised
    along the rows of the expert's segment (mxfp8_qdq_rows, blocks of 32 rows
    from the expert's first row in the placement order).  The operands
    quantised are the tensors as the layer holds them, at the precision of
    its activations: dy, h, da and db rounded to bfloat16 (bf16_round; x
    already is), the reading taken where the pages give no recipe:
      dW2_e = Qr(bf16(dy_e))^T Qr(bf16(h_e)),
      dW1_e = Qr(bf16(da_e))^T Qr(x_e),  dW3_e = Qr(bf16(db_e))^T Qr(x_e).
    """
    x = _f64(x)
    g = _f64(dout)
    T, d = x.shape
    E = np.asarray(logits).shape[1]
    if expert_end is None:
        expert_end = E
    if fwd is None:
        fwd = forward(x, logits, W1, W3, W2, k, expert_begin, expert_end, mxfp8=mxfp8, gating=gating,
                      renorm=renorm)
    gating, renorm = fwd.get("gating", gating), fwd.get("renorm", renorm)
    if mxfp8 != fwd.get("mxfp8", False):
        raise ValueError("backward(mxfp8=...) needs the forward of the same precision")
    if fwd.get("mxfp4", False):
        raise ValueError("the MXFP4 mode is forward only")
    if mxfp8_wgrad and not mxfp8:
        raise ValueError("mxfp8_wgrad needs mxfp8")
    gate, p, Y = fwd["gate"], fwd["p"], fwd["Y"]
    rop = fwd["row_of_pair"].reshape(T, k)
    offsets, pair_of_row = fwd["offsets"], fwd["pair_of_row"]
    A, B, H = fwd["A"], fwd["B"], fwd["H"]

    dgate = np.zeros((T, k))
    for j in range(k):
        m = rop[:, j] >= 0
        dgate[m, j] = np.einsum("td,td->t", g[m], Y[rop[m, j]])
    dlogits = route_backward(p, fwd["idx"], gate, dgate, gating, renorm)

    tok = pair_of_row // k
    slot = pair_of_row % k
    dY = gate[tok, slot][:, None] * g[tok]
    Xp = permute(x, pair_of_row, k)
    F = np.asarray(W1).shape[1]
    P = pair_of_row.shape[0]
    dXp = np.zeros((P, d))
    dA = np.zeros((P, F)); dB = np.zeros((P, F))
    E_loc = expert_end - expert_begin
    dW1 = np.zeros((E_loc, F, d)); dW3 = np.zeros((E_loc, F, d)); dW2 = np.zeros((E_loc, d, F))
    for e in range(expert_begin, expert_end):
        r0, r1 = offsets[e], offsets[e + 1]
        if r0 == r1:
            continue
        i = e - expert_begin
        a, b, h, dy = A[r0:r1], B[r0:r1], H[r0:r1], dY[r0:r1]
        if mxfp8:
            h = silu(a) * b
            dh = mxfp8_qdq(dy) @ mxfp8_qdq(_f64(W2[i]).T).T
        else:
            dh = dy @ _f64(W2[i])
        s = sigmoid(a)
        da = dh * b * s * (1.0 + a * (1.0 - s))
        db = dh * silu(a)
        if mxfp8:
            dXp[r0:r1] = (mxfp8_qdq(da) @ mxfp8_qdq(_f64(W1[i]).T).T
                          + mxfp8_qdq(db) @ mxfp8_qdq(_f64(W3[i]).T).T)
        else:
            dXp[r0:r1] = da @ _f64(W1[i]) + db @ _f64(W3[i])
        if mxfp8_wgrad:
            xq = mxfp8_qdq_rows(Xp[r0:r1])
            dW2[i] = mxfp8_qdq_rows(bf16_round(dy)).T @ mxfp8_qdq_rows(bf16_round(h))
            dW1[i] = mxfp8_qdq_rows(bf16_round(da)).T @ xq
            dW3[i] = mxfp8_qdq_rows(bf16_round(db)).T @ xq
        else:
            dW2[i] = dy.T @ h
            dW1[i] = da.T @ Xp[r0:r1]
            dW3[i] = db.T @ Xp[r0:r1]
        dA[r0:r1], dB[r0:r1] = da, db
    dx = unpermute_sum(dXp, fwd["row_of_pair"], T, k)
    return dict(dx=dx, dW1=dW1, dW3=dW3, dW2=dW2, dgate=dgate, dlogits=dlogits,
                dY=dY, dA=dA, dB=dB, dXp=dXp)


def loss(out, dout) -> float:
    """L = sum(out * dout): the scalar whose gradients backward() returns."""
    return float((_f64(out) * _f64(dout)).sum())


def backward_token(x_t, logits_t, dout_t, W1, W3, W2, k: int, expert_begin: int = 0,
                   expert_end: int | None = None, gating: str = "softmax", renorm: bool = False,
                   mxfp8: bool = False):
    """Backward of one token alone (sampled checks at full size): the pair
    gradients of its local experts summed in slot order, and its router
    gradient.  Same equations as backward(), restricted to one token; every
    pair's backward depends only on that pair.  Returns (dx [d], dgate [k],
    dlogits [E])."""
    l32 = np.asarray(logits_t, dtype=np.float32)[None, :]
    E = l32.shape[1]
    if expert_end is None:
        expert_end = E
    idx, gate, _, p = route(l32, k, gating, renorm)
    xt = _f64(x_t)[None, :]
    g = _f64(dout_t)
    dx = np.zeros(xt.shape[1])
    dgate = np.zeros(k)
    for j in range(k):
        e = int(idx[0, j])
        if not expert_begin <= e < expert_end:
            continue
        i = e - expert_begin
        if mxfp8:
            a, b, y = _mx_expert_forward(xt, W1[i], W3[i], W2[i])
        else:
            a, b, h, y = expert_ffn(xt, W1[i], W3[i], W2[i])
        dgate[j] = float(np.dot(g, y[0]))
        dy = gate[0, j] * g[None, :]
        dh = (mxfp8_qdq(dy) @ mxfp8_qdq(_f64(W2[i]).T).T) if mxfp8 else dy @ _f64(W2[i])
        s = sigmoid(a)
        da = dh * b * s * (1.0 + a * (1.0 - s))
        db = dh * silu(a)
        if mxfp8:
            dx += (mxfp8_qdq(da) @ mxfp8_qdq(_f64(W1[i]).T).T + mxfp8_qdq(db) @ mxfp8_qdq(_f64(W3[i]).T).T)[0]
        else:
            dx += (da @ _f64(W1[i]) + db @ _f64(W3[i]))[0]
    dlogits = route_backward(p, idx, gate, dgate[None, :], gating, renorm)[0]
    return dx, dgate, dlogits


def _mx_expert_forward(X, W1e, W3e, W2e):
    """MXFP8 forward of one expert's rows (as in forward(mxfp8=True)):
    a, b from quantised x and W1/W3 rows, y from quantised h and W2 rows."""
    xq = mxfp8_qdq(X)
    a = xq @ mxfp8_qdq(W1e).T
    b = xq @ mxfp8_qdq(W3e).T
    y = mxfp8_qdq(silu(a) * b) @ mxfp8_qdq(W2e).T
    return a, b, y


def expert_weight_grads(X_e, gate_e, dout_e, W1e, W3e, W2e, mxfp8: bool = False, mxfp8_wgrad: bool = False):
    """dW1_e, dW3_e, dW2_e of one expert from its rows alone: X_e [R,d] the
    activations of its pairs, gate_e [R] their gates, dout_e [R,d] the output
    gradients of their tokens (row order does not matter, except with
    mxfp8_wgrad, whose blocks of 32 rows need the placement order).  MXFP8 as
    in backward(mxfp8=True, mxfp8_wgrad=...)."""
    X = _f64(X_e)
    if mxfp8:
        a, b, _ = _mx_expert_forward(X, W1e, W3e, W2e)
        h = silu(a) * b
    else:
        a, b, h, _ = expert_ffn(X, W1e, W3e, W2e)
    dy = _f64(gate_e)[:, None] * _f64(dout_e)
    dh = (mxfp8_qdq(dy) @ mxfp8_qdq(_f64(W2e).T).T) if mxfp8 else dy @ _f64(W2e)
    s = sigmoid(a)
    da = dh * b * s * (1.0 + a * (1.0 - s))
    db = dh * silu(a)
    if mxfp8_wgrad:
        if not mxfp8:
            raise ValueError("mxfp8_wgrad needs mxfp8")
        xq = mxfp8_qdq_rows(X)
        return (mxfp8_qdq_rows(bf16_round(da)).T @ xq, mxfp8_qdq_rows(bf16_round(db)).T @ xq,
                mxfp8_qdq_rows(bf16_round(dy)).T @ mxfp8_qdq_rows(bf16_round(h)))
    return da.T @ X, db.T @ X, dy.T @ h
