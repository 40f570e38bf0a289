"""bench.py's contract that needs no GPU: one GPU only (refusal with a message for more),
the committed HBM-traffic summary is used only while the kernel sources it was taken
on are unchanged, and the counter summaries that write profiles/ read rocprofv3's
CSVs as intended."""
from __future__ import annotations

import csv
import json
import os
import subprocess
import sys
from pathlib import Path

import numpy as np

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


def _counter_csv(path, rows):
    """A rocprofv3 counter_collection CSV: (dispatch id, kernel name, grid, counter, value)."""
    cols = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
            "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
            "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        for did, name, grid, counter, value in rows:
            w.writerow([did, did, "Agent 1", 1, 1, 1, grid, 1, name, 512, 0, 0, 0, 0, 0, counter, value, 0, 1])


def test_counter_summaries_on_synthetic_csv(tmp_path, monkeypatch):
    """--write-traffic, --counter-table and --kernel-traffic on hand-made CSVs: counter
    instances of a dispatch are summed, tower-shaped launches of the attention kernel
    are picked by name and grid, the 1 GiB calibration copy sets the scale, and the
    i-th tower launch is layer i mod 50 of the schedule."""
    from vit_perception_encoder_amd import workloads as wl

    att = f"void mgattn::{bench.KERNEL_NAME}(mgattn::KernelArgs)"
    fetch, write = tmp_path / "fetch.csv", tmp_path / "write.csv"
    # two counter instances per dispatch (summed): 3 tower launches of 24,000 KiB of FETCH,
    # one launch of another grid, and the copy reading as 512 MiB (scale 2)
    rows_f = []
    for did in (1, 2, 3):
        rows_f += [(did, att, bench.TOWER_GRID, "FETCH_SIZE", 12000.0)] * 2
    rows_f += [(4, att, 65536, "FETCH_SIZE", 1.0), (5, bench.COPY_KERNEL, 1 << 20, "FETCH_SIZE", 524288.0)]
    rows_w = [(did, att, bench.TOWER_GRID, "WRITE_SIZE", 12000.0) for did in (1, 2, 3)]
    rows_w += [(5, bench.COPY_KERNEL, 1 << 20, "WRITE_SIZE", 1048576.0)]
    _counter_csv(fetch, rows_f)
    _counter_csv(write, rows_w)
    monkeypatch.setattr(bench, "TRAFFIC_FILE", tmp_path / "traffic.json")
    assert bench.write_traffic(str(fetch), str(write)) == 0
    t = json.loads((tmp_path / "traffic.json").read_text())
    assert t["attention_dispatches"] == 3
    assert t["calibration"]["fetch_scale"] == 2.0 and t["calibration"]["write_scale"] == 1.0
    assert t["hbm_fetch_bytes_per_launch"] == 24000 * 1024 * 2
    assert t["hbm_write_bytes_per_launch"] == 12000 * 1024
    assert t["kernel_source_sha256"] == bench.kernel_source_hash()
    # counter table: 52 tower launches, value = layer index; full layers average their indices
    kinds = wl.tower_layer_kinds()
    sq = tmp_path / "sq.csv"
    _counter_csv(sq, [(i + 1, att, bench.TOWER_GRID, "SQ_WAVES", float(i % 50)) for i in range(52)])
    r = _run(["--counter-table", str(sq)])
    assert r.returncode == 0, r.stderr
    line = next(x for x in r.stdout.splitlines() if x.startswith("| SQ_WAVES"))
    idx = [i % 50 for i in range(52)]
    want_full = np.mean([v for v in idx if kinds[v] == "full"])
    want_win = np.mean([v for v in idx if kinds[v] == "window"])
    got = [float(x) for x in line.strip("|").split("|")[1:]]
    assert abs(got[0] - want_full) < 1e-3 * want_full and abs(got[1] - want_win) < 1e-3 * want_win
    # kernel traffic: one row per (kernel, grid), scaled like write_traffic
    r = _run(["--kernel-traffic", str(fetch), str(write)])
    assert r.returncode == 0, r.stderr
    tower_row = next(x for x in r.stdout.splitlines() if f"| {bench.TOWER_GRID} |" in x and "attn_fwd" in x)
    assert "| 3 | 49.15 | 12.29 |" in tower_row, tower_row


def test_trace_table_splits_the_run_into_its_parts(tmp_path, capsys):
    """A synthetic kernel trace of `--steps 2 --warmup 1`: the timed replays (launches
    250..349 of the tower kernel in start order) are the ones whose mean the table
    reports as timed, full layers 100 us and window layers 30 us; other kernels and other
    grids are ignored."""
    from vit_perception_encoder_amd import workloads as wl
    kinds = wl.tower_layer_kinds()
    path = tmp_path / "kernel_trace.csv"
    t = 0
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"])
        # parts: 1 eager warm-up step, 1 side step, 1 graph warm-up, 2 timed, 3 breakdown, 1 per-kind
        for part, nsteps in enumerate((1, 1, 1, 2, 3, 1)):
            for _ in range(nsteps):
                for layer in range(50):
                    dur = (100 if kinds[layer] == "full" else 30) * (1 if part == 3 else 2)
                    w.writerow([f"void mgattn::{bench.KERNEL_NAME}(mgattn::KernelArgs)", bench.TOWER_GRID, t,
                                t + dur * 1000])
                    w.writerow(["other_kernel", 64, t, t + 5000])
                    t += dur * 1000 + 2000
    assert bench.trace_table(str(path), 2, 1) == 0
    out = capsys.readouterr().out
    timed = [line for line in out.splitlines() if "timed graph replays" in line][0].split("|")
    mean_timed = (13 * 100 + 37 * 30) / 50
    assert int(timed[2]) == 100 and abs(float(timed[3]) - mean_timed) < 0.01
    assert "full layers 100.00 us, window layers 30.00 us" in out
