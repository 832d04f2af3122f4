"""bench.py end to end on small workloads: every mode prints one JSON line with the fields the
measurement contract asks for (value, roofline, and the oracle's CPU rate where the mode has one)."""
from __future__ import annotations

import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args) -> list[dict]:
    print("bench.py " + " ".join(args), flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                       timeout=240, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    return [json.loads(l) for l in r.stdout.splitlines() if l.startswith("{")]


def test_bench_eviction_tiny():
    (b,) = _bench("--config", "tiny", "--steps", "3", "--warmup", "1", "--cpu-seconds", "0.5")
    assert b["value"] > 0 and b["n_gpus"] == 1 and b["steps"] == 3 and b["warmup"] == 1
    assert b["config"]["workload"].startswith("tiny")
    rf = b["roofline"]
    assert rf["bound"] == "hbm" and rf["unit"] == "GB/s" and rf["peak"] == 8000.0
    assert abs(rf["frac"] - rf["achieved"] / rf["peak"]) < 1e-12
    assert 0 < rf["strict"]["frac"] <= rf["frac"]
    assert b["timing"] == "pristine" and abs(b["value"] - b["pristine"]["steps_per_s"]) < 1e-9
    assert b["back_to_back"]["steps_per_s"] > 0
    (bb,) = _bench("--config", "tiny", "--steps", "3", "--warmup", "1", "--timing", "back-to-back",
                   "--no-cpu-baseline")
    assert bb["timing"] == "back-to-back" and abs(bb["value"] - bb["back_to_back"]["steps_per_s"]) < 1e-9
    cb = b["cpu_baseline"]
    assert cb["kind"] == "oracle" and cb["value"] > 0 and cb["cores"] >= 1
    assert b["copy_reference"]["GBs"] > 0


def test_bench_stream_and_fps_round_tiny():
    (s,) = _bench("--stream", "--stream-config", "stream-tiny", "--cpu-seconds", "0.5")
    assert s["value"] > 0 and s["config"]["evictions"] > 0
    assert s["roofline"]["bound"] == "hbm" and 0 < s["roofline"]["frac"]
    assert s["cpu_baseline"]["kind"] == "oracle" and s["cpu_baseline"]["value"] > 0
    assert s["fps_round"]["roofline"]["bound"] == "mfma"
    (f,) = _bench("--fps-round", "--stream-config", "stream-tiny", "--steps", "3", "--cpu-seconds", "0.5")
    assert f["value"] > 0 and f["roofline"]["unit"] == "TFLOP/s" and f["cpu_baseline"]["value"] > 0

