"""Host-side checks of bench.py (CPU; no kernel runs): the one-GPU rule, the
traffic records it reads from the committed profiles, and the algorithmic
figures its roofline divides by."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("kernel", sorted(bench.TRAFFIC_PROFILES))
def test_every_traffic_record_is_in_its_profile(kernel):
    # Each kernel the bench line can name has a traffic_record line in its
    # committed profile, with a byte count and the SHA-256 of its sources.
    path = os.path.join(ROOT, "profiles", bench.TRAFFIC_PROFILES[kernel])
    assert os.path.isfile(path), path
    recs = [line for line in open(path) if line.startswith("traffic_record:") and f"kernel={kernel} " in line]
    assert len(recs) == 1, (kernel, recs)
    fields = dict(kv.split("=", 1) for kv in recs[0].split(":", 1)[1].split())
    assert int(fields["fetch_bytes"]) > 0 and int(fields["write_bytes"]) >= 0
    assert len(fields["sources_sha256"]) == 64


def test_traffic_is_withheld_once_the_sources_change(tmp_path, monkeypatch):
    # A record whose hash does not match the kernel's current sources gives
    # None (the line then reports no traffic), a matching one the byte sum.
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "p.md").write_text(
        f"traffic_record: kernel=hc_down fetch_bytes=100 write_bytes=20 sources_sha256={'a' * 64}\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setitem(bench.TRAFFIC_PROFILES, "hc_down", "p.md")
    monkeypatch.setattr(bench, "sources_sha256", lambda k: "a" * 64)
    assert bench.recorded_traffic("hc_down") == 120
    monkeypatch.setattr(bench, "sources_sha256", lambda k: "0" * 64)
    assert bench.recorded_traffic("hc_down") is None


def test_algorithmic_figures_of_the_workloads():
    # The decode block's bytes and the prefill block's FLOP that the roofline
    # divides by, from the shapes alone (C = 4, H = 2560, R = 320, bf16).
    K, R, C, H = 4 * 2560, 320, 4, 2560
    assert bench.DEC_UP_BYTES == R * K * 2 + H * 2
    assert bench.PF_FLOP == 2 * 8192 * K * (R + C) + 2 * 8192 * R * K
