"""Host logic of bench.py (no GPU): the HBM-traffic figure it reads from a
committed counter summary is reported only while every source file whose hash
the summary records is unchanged."""
import hashlib
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _summary(tmp_path, lines):
    (tmp_path / "s.md").write_text("# traffic\n\n" + "\n".join(lines) + "\n")
    return "s.md"


def _sha(name):
    return hashlib.sha256(open(os.path.join(bench.CSRC, name), "rb").read()).hexdigest()


def test_traffic_reported_while_every_recorded_source_matches(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    name = _summary(tmp_path, [f"- sha256 decode.hip: `{_sha('decode.hip')}`",
                               f"- sha256 gdn_device.h: `{_sha('gdn_device.h')}`",
                               "- traffic_bytes_per_launch: 846508407"])
    assert bench.measured_traffic(name, "decode.hip") == 846508407


def test_traffic_null_when_any_recorded_source_changed(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    stale = "0" * 64
    name = _summary(tmp_path, [f"- sha256 decode.hip: `{_sha('decode.hip')}`",
                               f"- sha256 gdn_device.h: `{stale}`",
                               "- traffic_bytes_per_launch: 846508407"])
    assert bench.measured_traffic(name, "decode.hip") is None


def test_traffic_null_without_the_kernel_source_hash_or_the_figure(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    only_header = _summary(tmp_path, [f"- sha256 gdn_device.h: `{_sha('gdn_device.h')}`",
                                      "- traffic_bytes_per_launch: 1"])
    assert bench.measured_traffic(only_header, "decode.hip") is None
    no_figure = _summary(tmp_path, [f"- sha256 decode.hip: `{_sha('decode.hip')}`"])
    assert bench.measured_traffic(no_figure, "decode.hip") is None
    assert bench.measured_traffic("missing.md", "decode.hip") is None

