"""How exactly the gfx950 scaled matrix instruction sums (the MXFP8 GEMMs'
v_mfma_scale_f32_32x32x64_f8f6f4), measured on one block of fixed E4M3 codes
and E8M0 scales against the exact sum of the same products.

Every E4M3 product times its two power-of-two scales is exact in float64, and
so is the sum of 64 of them at the magnitudes used here, so the reference is
the exact value; its nearest fp32 is what an exactly rounded fp32 sum would
give.  The probe reports how far the hardware lands from it.  The only hard
bar is a loose one that any fp32-class accumulation meets; the measured
figures are printed for the record."""
import ctypes
import os

import numpy as np
import pytest
import torch

from oracle import mok_oracle as O
from tests.gpu_case import note

pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "mixture_experts_layer_34_amd",
                   "libmok_diag.so")


def _lib():
    L = ctypes.CDLL(LIB)
    L.mok_diag_mfma_scale_block.restype = ctypes.c_int32
    L.mok_diag_mfma_scale_block.argtypes = [ctypes.c_void_p] * 7
    L.mok_diag_e4m3_check.restype = ctypes.c_int32
    L.mok_diag_e4m3_check.argtypes = [ctypes.c_uint32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32,
                                      ctypes.c_void_p]
    return L


def test_e4m3_conversion_instruction_matches_the_definition():
    """The E4M3 encoding the layer's quantisers use (the conversion
    instruction on the value clamped to +-448, alone and four packed) equals
    the software encoder of the OCP definition on every float32 of magnitude
    below 2^9, both signs: 2.28e9 values."""
    note("e4m3 conversion instruction, exhaustive")
    blocks = 4096
    dev = torch.device("cuda")
    count = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
    first = torch.zeros(blocks * 256, dtype=torch.int32, device=dev)
    assert _lib().mok_diag_e4m3_check(0x44000000, count.data_ptr(), first.data_ptr(), blocks,
                                      torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    bad = int(count.to(torch.int64).sum())
    firsts = [hex(int(v) & 0xFFFFFFFF) for v in first.cpu().numpy() if int(v) != -1][:5]
    assert bad == 0, (bad, firsts)


def _finite_codes(rng, shape):
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] ^= 0x01          # S.1111.111 is NaN: take its neighbour
    return c


def _run(a, b, sa, sb, c_in):
    dev = torch.device("cuda")
    t = [torch.from_numpy(np.ascontiguousarray(v)).to(dev) for v in (a, b, sa, sb, c_in)]
    out = torch.empty((32, 32), dtype=torch.float32, device=dev)
    rc = _lib().mok_diag_mfma_scale_block(*[v.data_ptr() for v in t], out.data_ptr(),
                                          torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def _exact(a, b, sa, sb, c_in):
    va = O.e4m3_decode(a) * np.ldexp(1.0, np.repeat(sa.astype(np.int64) - 127, 32, axis=1))
    vb = O.e4m3_decode(b) * np.ldexp(1.0, np.repeat(sb.astype(np.int64) - 127, 32, axis=1))
    prod = va[:, None, :] * vb[None, :, :]            # [32, 32, 64], each exact
    return c_in.astype(np.float64) + prod.sum(axis=2), np.abs(prod).sum(axis=2) + np.abs(c_in)


def _report(case, hw, exact, mag):
    """Prints how far the hardware sum lands from the exact one: how many
    results differ from the exactly rounded fp32 sum, the largest error in
    units of the result's fp32 spacing, and the largest error relative to the
    element's own sum of magnitudes and to the block's largest."""
    rne = exact.astype(np.float32).astype(np.float64)
    ulp = np.spacing(np.abs(exact).astype(np.float32)).astype(np.float64)
    err = np.abs(hw - exact)
    err_ulp = err / np.maximum(ulp, np.finfo(np.float32).tiny)
    off = int((hw != rne).sum())
    rel_own = float((err / np.maximum(mag, 1e-300)).max())
    note(f"  {case}: {off} of {hw.size} differ from the exactly rounded fp32 sum; max error {err_ulp.max():.1f} ulp "
         f"of the result, {rel_own:.2e} of the element's sum of magnitudes, "
         f"{err.max() / max(mag.max(), 1e-300):.2e} of the block's largest")
    return off, err_ulp


def _codes_with_exponent(rng, shape, lo, hi):
    """Random E4M3 codes whose exponent field lies in [lo, hi] (0: subnormal)."""
    e = rng.integers(lo, hi + 1, size=shape)
    m = rng.integers(0, 8, size=shape)
    m = np.where((e == 15) & (m == 7), 6, m)          # S.1111.111 is NaN
    m = np.where((e == 0) & (m == 0), 1, m)           # no zeros among the subnormals
    s = rng.integers(0, 2, size=shape)
    return ((s << 7) | (e << 3) | m).astype(np.uint8)


def test_normal_operands_sum_exactly_rounded():
    """Normal E4M3 operands only, unit scales: the hardware sum against the
    exactly rounded fp32 sum."""
    rng = np.random.default_rng(1)
    a, b = _codes_with_exponent(rng, (32, 64), 1, 15), _codes_with_exponent(rng, (32, 64), 1, 15)
    sa = np.full((32, 2), 127, np.uint8)
    sb = np.full((32, 2), 127, np.uint8)
    c_in = np.zeros((32, 32), np.float32)
    hw = _run(a, b, sa, sb, c_in)
    exact, mag = _exact(a, b, sa, sb, c_in)
    _report("normal operands", hw, exact, mag)
    assert (np.abs(hw - exact) <= 2.0 ** -12 * mag).all()


def test_subnormal_operands():
    """One non-zero product per output, A subnormal (2^-9 .. 7 * 2^-9), B = 1:
    the value the hardware gives it (exact, or flushed to zero)."""
    a = np.zeros((32, 64), np.uint8)
    for i in range(32):
        a[i, i % 64] = 1 + (i % 7)                     # subnormal codes 0x01 .. 0x07
    b = np.full((32, 64), 0x38, np.uint8)              # 1.0
    sa = np.full((32, 2), 127, np.uint8)
    sb = np.full((32, 2), 127, np.uint8)
    hw = _run(a, b, sa, sb, np.zeros((32, 32), np.float32))
    exact, mag = _exact(a, b, sa, sb, np.zeros((32, 32), np.float32))
    flushed = int((hw == 0).sum())
    exact_n = int((hw == exact).sum())
    note(f"  subnormal A operands: {exact_n} of 1024 results exact, {flushed} are 0 "
         f"(exact values {exact[0, 0]:.3e} ..)")
    _report("subnormal operands", hw, exact, mag)
    assert (np.abs(hw - exact) <= np.abs(exact)).all(), "a subnormal product came out larger than itself"


@pytest.mark.parametrize("case", ["random", "one-large-many-small", "accumulate"])
def test_scaled_mfma_block_against_exact_sum(case):
    """Random codes (subnormals included) and scales; the record of how far
    the result lands from the exact sum, with a loose bar of 2^-10 of the
    block's largest sum of magnitudes."""
    rng = np.random.default_rng({"random": 1, "one-large-many-small": 2, "accumulate": 3}[case])
    a, b = _finite_codes(rng, (32, 64)), _finite_codes(rng, (32, 64))
    sa = rng.integers(124, 131, size=(32, 2)).astype(np.uint8)
    sb = rng.integers(124, 131, size=(32, 2)).astype(np.uint8)
    c_in = np.zeros((32, 32), np.float32)
    if case == "one-large-many-small":
        a[:, 1:] = 0x08 | (a[:, 1:] & 0x80)            # +-2^-6: small terms
        a[:, 0] = 0x70                                 # 2^7 = 128: one large term
        b[:, :] = 0x38 | (b & 0x80)                    # +-1
        sa[:] = 127
        sb[:] = 127
    if case == "accumulate":
        c_in = rng.normal(size=(32, 32)).astype(np.float32) * 64
    hw = _run(a, b, sa, sb, c_in)
    exact, mag = _exact(a, b, sa, sb, c_in)
    _report(case, hw, exact, mag)
    assert (np.abs(hw - exact) <= 2.0 ** -10 * mag.max()).all()


# ------------------------------------------------------------------ E2M1 operands

def _raw(areg, breg, sa_l, sb_l, fa, fb):
    """The instruction on raw lane registers (uint8 [64, 32] each), lane scale
    bytes [64]; returns C [32, 32] (C[m][n], m = A row, n = B row)."""
    L = _lib()
    L.mok_diag_mfma_scale_raw.restype = ctypes.c_int32
    L.mok_diag_mfma_scale_raw.argtypes = [ctypes.c_void_p] * 6 + [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    dev = torch.device("cuda")
    t = [torch.from_numpy(np.ascontiguousarray(v)).to(dev) for v in (areg, breg, sa_l, sb_l)]
    c_in = torch.zeros(64 * 16, dtype=torch.float32, device=dev)
    out = torch.zeros_like(c_in)
    rc = L.mok_diag_mfma_scale_raw(*[v.data_ptr() for v in t], c_in.data_ptr(), out.data_ptr(), fa, fb,
                                   torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy().reshape(64, 16).astype(np.float64)
    C = np.zeros((32, 32))
    for l in range(64):
        for i in range(16):
            C[(i // 4) * 8 + (l // 32) * 4 + i % 4, l % 32] = o[l, i]
    return C


def _fp4_regs(M):
    """E2M1 codes M [32, 64] into lane registers as the MXFP4 kernels feed
    them: lane l holds row l % 32 and K [32 h, 32 h + 32) (h = l / 32) as 16
    packed bytes, element 2i in the low nibble of byte i."""
    regs = np.zeros((64, 32), np.uint8)
    for l in range(64):
        r, h = l % 32, l // 32
        row = M[r, 32 * h:32 * h + 32].astype(np.uint8)
        regs[l, :16] = row[0::2] | (row[1::2] << 4)
    return regs


def _fp8_regs(M):
    regs = np.zeros((64, 32), np.uint8)
    for l in range(64):
        r, h = l % 32, l // 32
        regs[l, :16] = M[r, 16 * h:16 * h + 16]
        regs[l, 16:] = M[r, 32 + 16 * h:48 + 16 * h]
    return regs


def _lane_scales(S):
    return np.array([S[l % 32, l // 32] for l in range(64)], np.uint8)


@pytest.mark.parametrize("fb", [4, 0], ids=["e2m1xe2m1", "e2m1xe4m3"])
def test_e2m1_operand_layout(fb):
    """The register layout the MXFP4 kernels rely on: E2M1 operands as 16
    packed bytes per lane, K [32 h, 32 h + 32) for lanes 32 h .. 32 h + 31,
    low nibble first, the lane group h supplying the scale of K block h.
    Against an E4M3 B operand in its own (established) layout the nibble
    order is fixed too.  E2M1 x E2M1 with scales of 2^-1 .. 2^1: every
    product and partial sum is exact in fp32, so the bar is equality; against
    E4M3 a layout mistake moves results by O(1) of the largest, so the bar
    there is 2^-16 of it."""
    rng = np.random.default_rng(7)
    A = rng.integers(0, 16, (32, 64))
    sa = rng.integers(126, 129, (32, 2)).astype(np.uint8)
    sb = rng.integers(126, 129, (32, 2)).astype(np.uint8)
    if fb == 4:
        B = rng.integers(0, 16, (32, 64))
        breg, vb = _fp4_regs(B), O.e2m1_decode(B)
    else:
        B = _codes_with_exponent(rng, (32, 64), 4, 9)   # 2^-3 .. 2^2
        breg, vb = _fp8_regs(B), O.e4m3_decode(B)
    hw = _raw(_fp4_regs(A), breg, _lane_scales(sa), _lane_scales(sb), 4, fb)
    va = O.e2m1_decode(A) * np.repeat(np.ldexp(1.0, sa.astype(np.int64) - 127), 32, axis=1)
    vb = vb * np.repeat(np.ldexp(1.0, sb.astype(np.int64) - 127), 32, axis=1)
    exact = va @ vb.T
    note(f"  e2m1 x {'e2m1' if fb == 4 else 'e4m3'}: max |hw - exact| {np.abs(hw - exact).max():.3e}")
    if fb == 4:
        np.testing.assert_array_equal(hw, exact)
    else:
        assert np.abs(hw - exact).max() <= 2.0 ** -16 * np.abs(exact).max()
