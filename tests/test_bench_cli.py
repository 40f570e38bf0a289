"""bench.py's contract that needs no GPU: one GPU only (refusal with a message for more),
and the committed HBM-traffic summary is used only while the kernel sources it was
taken on are unchanged."""
from __future__ import annotations

import json
import os
import subprocess
import sys
from pathlib import Path

ROOT = Path(__file__).resolve().parents[1]
sys.path.insert(0, str(ROOT))

import bench  # noqa: E402


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, str(ROOT / "bench.py"), *args], capture_output=True, text=True, env=env,
                          timeout=120, cwd=str(ROOT))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_a_multi_rank_launch_is_refused_too():
    r = _run([], {"WORLD_SIZE": "2", "RANK": "1", "LOCAL_RANK": "1"})
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_summary_is_used_only_for_its_kernel_sources():
    if not bench.TRAFFIC_FILE.exists():  # no counters taken on this kernel yet: the bench reports null
        assert bench.traffic_per_launch() is None
        return
    t = json.loads(bench.TRAFFIC_FILE.read_text())
    if t["kernel_source_sha256"] == bench.kernel_source_hash():
        assert bench.traffic_per_launch() == t["hbm_bytes_per_launch"]
    else:  # sources changed since the counters were taken: the bench reports null
        assert bench.traffic_per_launch() is None
    # 4 x 4096 x 1536 bf16 (Q, K, V read, O written) per launch
    assert t["algorithmic_bytes_per_launch"] == 4 * 4096 * 1536 * 2
    assert 1.0 <= t["traffic_over_algorithmic"] < 2.0


def test_traffic_is_null_for_other_sources(monkeypatch):
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.traffic_per_launch() is None
