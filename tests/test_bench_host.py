"""Host logic of bench.py: the traffic record is used only while the kernel
sources it names still hash to the recorded digest."""
import hashlib
import json

import bench


def _write_record(tmp_path, src_text: str, digest: str):
    src = tmp_path / "k.hip"
    src.write_text(src_text)
    rec = {"workload": "wl", "sources": [str(src)], "source_sha256_16": digest,
           "per_launch": {"gemm_x": {"traffic_bytes": 1234}}}
    md = tmp_path / "rec.md"
    md.write_text("# t\n\n```json\n" + json.dumps(rec) + "\n```\n")
    return md


def test_traffic_used_when_sources_match(tmp_path, monkeypatch):
    text = "kernel source"
    md = _write_record(tmp_path, text, hashlib.sha256(text.encode()).hexdigest()[:16])
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {"wl": str(md), "other": str(md)})
    assert bench.measured_traffic("wl", "gemm_x") == 1234
    assert bench.measured_traffic("other", "gemm_x") is None   # the record is the other workload's
    assert bench.measured_traffic("unknown", "gemm_x") is None
    assert bench.measured_traffic("wl", "gemm_y") is None


def test_traffic_null_after_source_change(tmp_path, monkeypatch):
    md = _write_record(tmp_path, "kernel source v2", hashlib.sha256(b"kernel source").hexdigest()[:16])
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {"wl": str(md)})
    assert bench.measured_traffic("wl", "gemm_x") is None


def test_traffic_null_without_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILES", {"wl": str(tmp_path / "missing.md")})
    assert bench.measured_traffic("wl", "gemm_x") is None


def test_gemm_peaks_per_precision():
    """MXFP8 layer: the forward GEMMs and the dH / dX products against the
    MXFP8 peak, the bf16 weight-gradient GEMMs against the bf16 one."""
    for n in ("gemm_up", "gemm_down", "gemm_dh", "gemm_dx"):
        assert bench.gemm_peak("mxfp8", n) == bench.PEAK_TFLOPS["mxfp8"]
    for n in ("gemm_dw2", "gemm_dw13"):
        assert bench.gemm_peak("mxfp8", n) == bench.PEAK_TFLOPS["bf16"]
        assert bench.gemm_peak("bf16", n) == bench.PEAK_TFLOPS["bf16"]


def test_stage_work_mxfp8_bytes():
    """Algorithmic bytes of the MXFP8 training step: one byte per element plus
    one scale per 32 for the quantised operands, bf16 for the rest."""
    import workloads as W
    w = W.get("mxfp8_train")
    P, U = 1024, 200
    flops, nb = bench.stage_work(w, P, U, save_for_backward=True)
    b = W.get("bf16_train")
    fb, nbb = bench.stage_work(b, P, U, save_for_backward=True)
    assert flops == fb                                       # same products
    q, d, F, E = 1 + 1 / 32, w.d, w.F, w.E
    assert nb["dispatch"] == U * d * 2 + P * d * q           # bf16 in, MXFP8 rows out
    assert nb["bwd_gate"] == nbb["bwd_gate"] + P * d * q     # dY also written in MXFP8
    assert nb["gemm_dx"] == 2 * P * F * q + 2 * E * F * d * q + P * d * 2
    assert nb["gemm_up"] == P * d * q + 2 * E * F * d * q + P * F * q + 3 * P * F * 2
    assert nb["gemm_dw13"] == nbb["gemm_dw13"] and nb["gemm_dw2"] == nbb["gemm_dw2"]


def test_stage_work_mxfp8_weight_gradients():
    """With MXFP8 weight gradients: the dW GEMMs read one byte (plus a scale
    per 32) per operand element and count against the MXFP8 peak; the
    regather stage reads dout, the bf16 H, [dA | dB] and x rows and writes the
    row-quantised codes of all four (dY rebuilt from dout and the gates)."""
    import workloads as W
    w = W.get("mxfp8_train")
    P, U = 1024, 200
    q, d, F, E = 1 + 1 / 32, w.d, w.F, w.E
    _, nb = bench.stage_work(w, P, U, save_for_backward=True, mxfp8_wgrad=True)
    assert nb["gemm_dw2"] == P * d * q + P * F * q + E * d * F * 4
    assert nb["gemm_dw13"] == 2 * P * F * q + P * d * q + 2 * E * F * d * 4
    assert nb["regather"] == 3 * P * F * 2 + 2 * U * d * 2 + (2 * d + 3 * F) * P * q
    for n in ("gemm_dw2", "gemm_dw13"):
        assert bench.gemm_peak("mxfp8", n, True) == bench.PEAK_TFLOPS["mxfp8"]


def test_stage_work_mxfp4_forward_bytes():
    """MXFP4 GEMM operands move half a byte per element plus one scale byte
    per 32; the forward saves nothing; the peak is the MXFP4 one."""
    import workloads as W
    w4, w8 = W.get("mxfp4_infer"), W.get("mxfp8_infer")
    P, U, d, F, E = 65536, 8192, w4.d, w4.F, w4.E
    f4, b4 = bench.stage_work(w4, P, U, save_for_backward=False)
    f8, b8 = bench.stage_work(w8, P, U, save_for_backward=False)
    q4, q8 = 0.5 + 1 / 32, 1 + 1 / 32
    assert f4["gemm_up"] == f8["gemm_up"] == 4.0 * P * d * F
    assert abs(b4["gemm_up"] - (P * d * q4 + 2 * E * F * d * q4 + P * F * q4)) < 1
    assert abs(b4["gemm_down"] - (P * F * q4 + E * d * F * q4 + P * d * 2)) < 1
    assert abs(b8["gemm_up"] - (P * d * q8 + 2 * E * F * d * q8 + P * F * q8)) < 1
    assert abs(b4["dispatch"] - (U * d * 2 + P * d * q4)) < 1
    assert bench.gemm_peak("mxfp4", "gemm_up") == 10100.0
