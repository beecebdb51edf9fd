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
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(md))
    assert bench.measured_traffic("wl", "gemm_x") == 1234
    assert bench.measured_traffic("other", "gemm_x") is None
    assert bench.measured_traffic("wl", "gemm_y") is None


def test_traffic_null_after_source_change(tmp_path, monkeypatch):
    md = _write_record(tmp_path, "kernel source v2", hashlib.sha256(b"kernel source").hexdigest()[:16])
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(md))
    assert bench.measured_traffic("wl", "gemm_x") is None


def test_traffic_null_without_record(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("wl", "gemm_x") is None
