"""Host-side checks of bench.py (CPU only): the one-GPU guard, the algorithmic
byte counts that the roofline divides by, and the rule that committed counter
traffic is used only for unchanged kernel sources."""
import json
import subprocess
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))
import bench  # noqa: E402
from decayed_recurrence_scans_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_headline_bytes_per_token():
    """Retention at B=8, H=8, T=2048, D=64, bf16: q, k, v in and y out are 512 B per
    token, the fp32 state written once per (b, h) adds 64*64*4 / 2048 = 8 B per token
    (520 B in all), plus the eight per-head factors."""
    cfg = wl.LA_CONFIGS["retention_bf16"]
    tokens = cfg.B * cfg.H * cfg.T
    assert bench.la_algorithmic_bytes(cfg, False, 2) == tokens * 520 + cfg.H * 4 == 68_157_472


def test_normalized_bytes():
    """Normalized, D=128, bf16, carried state and key sum read and written:
    1024 B per token plus 2 * (128*128 + 128) * 4 B per (b, h)."""
    cfg = wl.LA_CONFIGS["normalized_bf16"]
    tokens, units = cfg.B * cfg.H * cfg.T, cfg.B * cfg.H
    assert bench.la_algorithmic_bytes(cfg, True, 2) == tokens * 1024 + units * 2 * (128 * 128 + 128) * 4


def test_wkv_bytes():
    """WKV fp32: k, v in and y out, 12 B per channel-step, plus w, u and the state out."""
    cfg = wl.WKV_CONFIGS["wkv_f32"]
    steps = cfg.B * cfg.T * cfg.C
    assert bench.wkv_algorithmic_bytes(cfg) == steps * 12 + cfg.C * 8 + 3 * cfg.B * cfg.C * 4 == 403_079_168


def test_every_digested_source_exists():
    for kind, names in bench.KERNEL_SOURCES.items():
        for n in names:
            assert (ROOT / "decayed_recurrence_scans_amd" / "csrc" / n).is_file(), (kind, n)


def test_traffic_only_for_unchanged_sources(tmp_path, monkeypatch):
    f = tmp_path / "traffic.json"
    good = bench.source_digest("wkv")
    f.write_text(json.dumps({"wkv_f32": {"source_sha256": good, "bytes_per_launch": 123},
                             "ema_bf16": {"source_sha256": "0" * 64, "bytes_per_launch": 456}}))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", f)
    assert bench.traffic_for("wkv", "wkv_f32") == 123
    assert bench.traffic_for("ema", "ema_bf16") is None        # sources changed since the counters
    assert bench.traffic_for("la", "retention_bf16") is None   # no record

