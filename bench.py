#!/usr/bin/env python3
"""Benchmark of the perception-encoder attention on one MI355X.

One step = the whole 50-layer attention schedule of the ViT-G/14 tower at 4096
patch tokens (64x64 grid): 13 full-attention layers (one 4096-token segment) and 37
window layers (four 32x32 = 1024-token windows), H=16, head_dim=96, bf16 inputs with
f32 accumulation, fresh seeded N(0,1) Q/K/V per layer, all resident in HBM before
timing.  Layer kinds follow vllm.cpp issue #1545, second comment ("Two of the three
labelled uncertainties are now resolved").

The 50 launches of a step are captured once into a HIP graph and replayed (--eager
launches them from Python instead).  HIP events on the launch stream bracket the K
timed steps; every launch inside is the attention kernel, so its average launch
duration is the bracketed time over the launches.  The full-layer / window-layer
breakdown replays the layers of each kind as a graph of their own (time per launch),
and an eager pass with events around each launch gives the same split as "ms_events".

Prints ONE JSON line: algorithmic TFLOP/s over the whole step (4*S^2*d*H per
segment), ms per step (= ms per tower), the roofline of the attention kernel, and
the f64 CPU oracle timed on a bounded sample of the same workload on this host.

    python bench.py [--steps K] [--warmup W] [--eager] [--no-cpu-baseline] [--copy-calibration]

Counter summaries from rocprofv3 --pmc runs of this script (no GPU needed):

    python bench.py --write-traffic FETCH_CSV WRITE_CSV   # HBM bytes per launch -> profiles/
    python bench.py --counter-table CSV [CSV ...]         # mean per dispatch, full / window layers
    python bench.py --kernel-traffic FETCH_CSV WRITE_CSV  # HBM MB per dispatch of every kernel
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time
from pathlib import Path

import numpy as np

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

METRIC = "attention TFLOP/s (%bf16 MFMA peak) + ms per 50-layer tower attn @4096 tok"
PEAK_BF16_TFLOPS = 2516.6  # MI355X dense bf16 MFMA (published 2.5 PFLOP/s): 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E (published 8 TB/s)
PEAK_F32_TFLOPS = 157.3    # MI355X dense f32 (published 157.3 TFLOP/s), the f32 path's own peak
THETA = 10000.0
KERNEL_NAME = "attn_fwd_bf16_pipe<96, 8, false, 1>"  # the dense head_dim-96 kernel the tower's layers launch (W, rope, key groups)
TRAFFIC_FILE = ROOT / "profiles" / "attn_fwd_bf16_pipe_96_tower4096_traffic.json"
KERNEL_SOURCES = ["vit_perception_encoder_amd/csrc/attn_bf16_pipe.hpp", "vit_perception_encoder_amd/csrc/attn_bf16.hpp",
                  "vit_perception_encoder_amd/csrc/schedule.hpp", "vit_perception_encoder_amd/csrc/plan.hpp",
                  "vit_perception_encoder_amd/csrc/mgattn.hip"]


def _code_only(text: str) -> str:
    """C++ source with comments removed and whitespace runs collapsed (string literals
    of these sources hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """sha256 of the attention kernel's sources, comments and layout ignored."""
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        h.update(_code_only((ROOT / rel).read_text()).encode())
    return h.hexdigest()


def traffic_per_launch():
    """HBM bytes per launch from the committed rocprofv3 counter summary, or None if
    it is missing or was taken on a different kernel source."""
    if not TRAFFIC_FILE.exists():
        return None
    t = json.loads(TRAFFIC_FILE.read_text())
    if t.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


TOWER_GRID = 256 * 512  # threads of one tower launch: 256 workgroups of 8 waves
COPY_KERNEL = "__amd_rocclr_copyBuffer"  # the runtime's device-to-device copy (--copy-calibration)
COPY_BYTES = 1 << 30


def _dispatches(path):
    """rocprofv3 counter_collection CSV -> [(dispatch id, kernel name, grid size,
    {counter: value summed over the counter's instances})] in dispatch order."""
    d = {}
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            ent = d.setdefault(int(r["Dispatch_Id"]), [r["Kernel_Name"], int(r["Grid_Size"]), {}])
            ent[2][r["Counter_Name"]] = ent[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [(k, v[0], v[1], v[2]) for k, v in sorted(d.items())]


def _is_tower_kernel(name: str, grid: int) -> bool:
    return KERNEL_NAME in name and grid == TOWER_GRID


def write_traffic(fetch_csv: str, write_csv: str) -> int:
    """HBM bytes per launch of the tower's attention kernel from one FETCH_SIZE run and
    one WRITE_SIZE run of `bench.py --eager --copy-calibration` under rocprofv3 --pmc:
    median KiB per dispatch over the tower-shaped launches (full and window layers
    move the same Q, K, V and O), each counter scaled so that the run's 1 GiB device
    copy reads as 1 GiB.  Writes TRAFFIC_FILE, stamped with the current kernel sources'
    hash (the CSVs must come from a build of these sources)."""
    out = {"what": f"HBM traffic of {KERNEL_NAME} per launch on the 50-layer tower schedule at 4096 tokens "
                   "(full and window launches alike move Q, K, V and O of 4096 x 1536 bf16); median over the "
                   "run's tower-shaped launches",
           "kernel_source_sha256": kernel_source_hash(),
           "command_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d DIR -o p -- python3 -u bench.py "
                            "--steps 2 --warmup 1 --no-cpu-baseline --eager --copy-calibration",
           "command_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d DIR -o p -- python3 -u bench.py "
                            "--steps 2 --warmup 1 --no-cpu-baseline --eager --copy-calibration",
           "command_summary": f"python bench.py --write-traffic {fetch_csv} {write_csv}"}
    per = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _dispatches(path)
        att = [c[counter] for _, n, g, c in rows if _is_tower_kernel(n, g) and counter in c]
        cpy = sorted(c[counter] for _, n, _, c in rows if n == COPY_KERNEL and counter in c)[-3:]
        if not att or not cpy:
            print(f"[bench] {path}: no tower launches or no calibration copy", file=sys.stderr)
            return 1
        kib = float(np.median(att))
        scale = round(COPY_BYTES / (float(np.median(cpy)) * 1024.0), 3)
        per[counter] = (kib, scale, len(att))
        key = "fetch" if counter == "FETCH_SIZE" else "write"
        out[f"{key}_kib_per_dispatch_raw"] = kib
        out.setdefault("calibration", {"copy_bytes": COPY_BYTES})[f"{key}_kib_raw"] = float(np.median(cpy))
        out["calibration"][f"{key}_scale"] = scale
    out["attention_dispatches"] = per["FETCH_SIZE"][2]
    fb = int(round(per["FETCH_SIZE"][0] * 1024 * per["FETCH_SIZE"][1]))
    wb = int(round(per["WRITE_SIZE"][0] * 1024 * per["WRITE_SIZE"][1]))
    alg = 4 * 4096 * 16 * 96 * 2
    out.update({"hbm_fetch_bytes_per_launch": fb, "hbm_write_bytes_per_launch": wb, "hbm_bytes_per_launch": fb + wb,
                "algorithmic_bytes_per_launch": alg, "traffic_over_algorithmic": round((fb + wb) / alg, 3)})
    TRAFFIC_FILE.write_text(json.dumps(out, indent=1) + "\n")
    print(json.dumps(out, indent=1))
    return 0


def kernel_traffic(fetch_csv: str, write_csv: str) -> int:
    """Markdown table of HBM traffic per dispatch for every (kernel, grid size) of one
    FETCH_SIZE run and one WRITE_SIZE run (medians, each counter scaled by the run's
    1 GiB calibration copy as in write_traffic)."""
    med = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _dispatches(path)
        cpy = sorted(c[counter] for _, n, _, c in rows if n == COPY_KERNEL and counter in c)[-3:]
        if not cpy:
            print(f"[bench] {path}: no calibration copy", file=sys.stderr)
            return 1
        scale = COPY_BYTES / (float(np.median(cpy)) * 1024.0)
        groups = {}
        for _, n, g, c in rows:
            if counter in c and n != COPY_KERNEL:
                groups.setdefault((n, g), []).append(c[counter] * 1024.0 * scale)
        for key, vals in groups.items():
            med.setdefault(key, {})[counter] = (float(np.median(vals)), len(vals))
    print("| kernel | grid (threads) | dispatches | fetch (MB) | write (MB) |\n|---|---|---|---|---|")
    for (n, g), v in sorted(med.items(), key=lambda kv: (kv[0][0], kv[0][1])):
        f, nf = v.get("FETCH_SIZE", (float("nan"), 0))
        w, _ = v.get("WRITE_SIZE", (float("nan"), 0))
        short = re.sub(r"\(.*", "", n.replace("void ", "").replace("mgattn::", ""))
        print(f"| {short} | {g} | {nf} | {f / 1e6:.2f} | {w / 1e6:.2f} |")
    return 0


def counter_table(paths) -> int:
    """Markdown table of counters per dispatch (summed over instances, mean over
    dispatches) of the tower's attention launches in runs of `bench.py --eager
    --no-token-path`, split into full and window layers: the i-th tower launch of a
    run is layer i mod 50 of the schedule."""
    from vit_perception_encoder_amd import workloads as wl
    kinds = wl.tower_layer_kinds()
    acc = {"full": {}, "window": {}}
    cnt = {"full": {}, "window": {}}
    for path in paths:
        i = 0
        for _, n, g, c in _dispatches(path):
            if not _is_tower_kernel(n, g):
                continue
            kind = kinds[i % len(kinds)]
            i += 1
            for name, v in c.items():
                acc[kind][name] = acc[kind].get(name, 0.0) + v
                cnt[kind][name] = cnt[kind].get(name, 0) + 1
    names = sorted(set(acc["full"]) | set(acc["window"]))
    print("| counter | full | window |\n|---|---|---|")
    for name in names:
        f = acc["full"].get(name, 0.0) / max(cnt["full"].get(name, 0), 1)
        w = acc["window"].get(name, 0.0) / max(cnt["window"].get(name, 0), 1)
        print(f"| {name} | {f:.4g} | {w:.4g} |")
    return 0


def trace_table(path: str, steps: int, warmup: int) -> int:
    """Markdown summary of the tower's attention launches in a rocprofv3 --kernel-trace
    CSV of `bench.py --steps K --warmup W --no-token-path` (graph path): the launches in
    start order fall into the parts main() runs them in -- W eager warm-up steps, one
    side-stream step, W graph warm-up replays, the K timed replays, the eager breakdown
    passes (max(3, min(K, 10)) steps), then the per-kind graphs -- 50 launches per step,
    the i-th launch of a step being layer i of the schedule."""
    from vit_perception_encoder_amd import workloads as wl
    kinds = wl.tower_layer_kinds()
    nl = len(kinds)
    rows = []
    with open(path, newline="") as f:
        for r in csv.DictReader(f):
            grid = int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)
            if _is_tower_kernel(r["Kernel_Name"], grid):
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
    rows.sort()
    nb = max(3, min(steps, 10))
    parts = [("eager warm-up", warmup * nl), ("side-stream warm-up", nl), ("graph warm-up replays", warmup * nl),
             ("**timed graph replays**", steps * nl), ("eager breakdown passes", nb * nl)]
    durs = [(e - s) / 1e3 for s, e in rows]
    print(f"{len(rows)} launches of {KERNEL_NAME}: mean {np.mean(durs):.2f} us, min {np.min(durs):.2f}, "
          f"max {np.max(durs):.2f}\n")
    print("| part | launches | mean kernel (us) | sum of kernels per step (us) | first start to last end per step (us) |")
    print("|---|---|---|---|---|")
    i = 0
    timed = None
    for name, n in parts:
        seg = rows[i:i + n]
        if len(seg) < n:
            print(f"(trace ends inside part '{name}')")
            return 1
        per_step = [seg[s * nl:(s + 1) * nl] for s in range(n // nl)]
        mean_k = np.mean([(e - s) / 1e3 for s, e in seg])
        span = np.mean([(st[-1][1] - st[0][0]) / 1e3 for st in per_step])
        print(f"| {name} | {n} | {mean_k:.2f} | {mean_k * nl:.1f} | {span:.1f} |")
        if "timed" in name:
            timed = seg
        i += n
    print(f"| per-kind graphs | {len(rows) - i} | {np.mean(durs[i:]):.2f} | | |")
    full = [(e - s) / 1e3 for j, (s, e) in enumerate(timed) if kinds[j % nl] == "full"]
    win = [(e - s) / 1e3 for j, (s, e) in enumerate(timed) if kinds[j % nl] == "window"]
    print(f"\nIn the timed replays: full layers {np.mean(full):.2f} us, window layers {np.mean(win):.2f} us per launch.")
    return 0


def host_threads() -> int:
    """Every core this process may run on."""
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:
        return max(1, os.cpu_count() or 1)


def cpu_model() -> str:
    """The host CPU's model name (as lscpu prints it), from /proc/cpuinfo."""
    try:
        for line in Path("/proc/cpuinfo").read_text().splitlines():
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(layer_cases, one_thread_case):
    """The f64 oracle, as it stands, on whole full-attention layers of the schedule,
    on every host core; plus one 1024-token layer on a single thread (a per-core
    figure)."""
    from oracle import oracle as orc

    threads = host_threads()
    outs, flops, t0 = [], 0.0, time.perf_counter()
    for c in layer_cases:
        q, k, v = (x.reshape(c.T, c.H, c.d) for x in (c.q, c.k, c.v))
        outs.append(orc.attention(q, k, v, c.cu_seqlens, c.H, c.d, c.scale, n_threads=threads))
        flops += c.flops()
    dt = time.perf_counter() - t0
    c = one_thread_case
    q, k, v = (x.reshape(c.T, c.H, c.d) for x in (c.q, c.k, c.v))
    t1 = time.perf_counter()
    orc.attention(q, k, v, c.cu_seqlens, c.H, c.d, c.scale, n_threads=1)
    dt1 = time.perf_counter() - t1
    names = ", ".join(c_.name for c_ in layer_cases)
    return outs, {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
                  "seconds": dt, "host_cores": os.cpu_count(), "cpu_model": cpu_model(),
                  "sample": f"{len(layer_cases)} full-attention layers of the schedule ({names}; each 1 segment x "
                            f"4096 tokens, H=16, d=96, bf16 inputs widened to f64), whole outputs, "
                            f"{flops / 1e9:.1f} GFLOP, {threads} threads",
                  "one_thread": {"value": c.flops() / dt1 / 1e12, "unit": "TFLOP/s", "seconds": dt1,
                                 "sample": f"{c.name}: one 1024-token segment, H=16, d=96, bf16 inputs, whole "
                                           f"output, {c.flops() / 1e9:.2f} GFLOP, 1 thread"}}


def time_launches(torch, fn, reps: int = 30, warm: int = 10) -> float:
    """Median milliseconds of fn() (one enqueue on torch's current stream), events
    around each launch, after `warm` untimed calls and at least 5 ms of them (the first
    launches on freshly allocated buffers run up to 20% slower)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    n = 0
    while n < warm or time.perf_counter() - t0 < 5e-3:
        fn()
        n += 1
        if n % 10 == 0:
            torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    stream = torch.cuda.current_stream()
    for a, b in ev:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.median([a.elapsed_time(b) for a, b in ev]))


def time_graph(torch, fn, n: int = 20, reps: int = 10) -> float:
    """Milliseconds per call of fn(stream) with n calls captured into one HIP graph and
    replayed: the kernels' own duration plus the gaps between graph nodes, without the
    host launch overhead that events around a single launch include (several us,
    comparable to a short HBM-bound kernel).  Best of `reps` replays after >= 5 ms of
    warm-up."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            fn(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        cap = torch.cuda.current_stream()
        for _ in range(n):
            fn(cap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 5e-3:
        graph.replay()
        torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) / n)
    return best


def tower_448(torch, mg, wl, reps: int = 10) -> dict:
    """The 448x448 image's tower: every one of its 50 layers attends one 1024-token
    segment (a single 32x32 window).  50 layers of seeded N(0,1) bf16 inputs resident on
    the device, the 50 launches captured into one graph and replayed; milliseconds per
    replay (best of `reps`) and the TFLOP/s of the 50 launches."""
    dev = torch.device("cuda:0")
    T, H, d = 1024, wl.HEADS, wl.HEAD_DIM
    gen = torch.Generator(device=dev)
    gen.manual_seed(448)
    layers = [tuple(torch.randn(T, H * d, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
              for _ in range(wl.N_LAYERS)]
    out = torch.empty(T, H * d, dtype=torch.bfloat16, device=dev)
    cu = [0, T]

    def run(strm):
        for q, k, v in layers:
            mg.mgattn_dense(q, k, v, out, cu, 1, H, d, wl.SCALE, 0, mg.MGATTN_BF16, strm)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            run(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 5e-3:
        graph.replay()
        torch.cuda.synchronize()
    best = float("inf")
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        graph.replay()
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    flops = wl.N_LAYERS * 4.0 * T * T * d * H
    return {"ms": best, "layers": wl.N_LAYERS, "us_per_layer": best * 1e3 / wl.N_LAYERS,
            "block_m": mg.mgattn_dense_plan_block_m(cu, 1, H, d, mg.MGATTN_BF16, 0),
            "tflops": flops / (best * 1e-3) / 1e12, "frac": flops / (best * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def config_times(torch, mg, wl):
    """Each parity workload timed on its own: the f32 256-token segment, the 1024-token
    full layer, the 4 x 1024 window layer, and the ragged batches' full and window
    layers (17,408 and 16,384 tokens).  "ms": per call of 20 calls replayed as one HIP
    graph (kernel time plus the gaps between launches; the inputs stay in the caches
    between calls); "ms_events": events around single launches, median (adds the host
    enqueue gap).  The rate and fraction use "ms" and the peak of the case's own dtype."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    cases = [wl.config_tiny(), wl.config_full448(), wl.config_window896()]
    for which in ("5a", "5b"):
        qkv = wl.ragged_inputs(which)
        cases += [wl.ragged_case(which, "full", qkv), wl.ragged_case(which, "window", qkv)]
    res = {}
    for c in cases:
        if c.dtype == wl.BF16:
            q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (c.q, c.k, c.v))
        else:
            q, k, v = (torch.from_numpy(x).to(dev) for x in (c.q, c.k, c.v))
        out = torch.empty_like(q)
        cu = [int(x) for x in c.cu_seqlens]
        def call(s, q=q, k=k, v=v, out=out, cu=cu, c=c):
            mg.mgattn_dense(q, k, v, out, cu, c.n_seg, c.H, c.d, c.scale, c.causal, c.dtype, s)

        ms_e = time_launches(torch, lambda: call(stream))
        ms = time_graph(torch, call)
        fl = c.flops()
        peak = PEAK_BF16_TFLOPS if c.dtype == wl.BF16 else PEAK_F32_TFLOPS
        res[c.name] = {"ms": ms, "ms_events": ms_e, "tokens": c.T, "segments": c.n_seg,
                       "dtype": "bf16" if c.dtype == wl.BF16 else "f32", "peak_tflops": peak,
                       "tflops": fl / (ms * 1e-3) / 1e12, "frac": fl / (ms * 1e-3) / 1e12 / peak}
    return res


def token_path(torch, mg, wl, layers):
    """The other entry points on the same shapes: the 4096-token full layer read from a
    merged [T, 3*H*d] qkv buffer, and the HBM-bound token-order kernels (window gather
    of a [T, H*d] bf16 tensor, 2D RoPE in place on the q and k columns of a merged qkv
    buffer) at the tower's 64x64 grid and at the 17,408-token ragged batch."""
    dev = torch.device("cuda:0")
    H, d = wl.HEADS, wl.HEAD_DIM
    row = H * d
    stream = torch.cuda.current_stream()
    res = {}
    # merged qkv, full layer 3, beside the same layer from separate tensors timed the
    # same way (events around each launch, median)
    q, k, v, cu, nseg, flops, _ = layers[3]
    T = q.shape[0]
    out = torch.empty(T, row, dtype=torch.bfloat16, device=dev)
    qkv = torch.cat([q, k, v], dim=1).contiguous()

    def separate():
        mg.mgattn_dense(q, k, v, out, cu, nseg, H, d, wl.SCALE, 0, mg.MGATTN_BF16, stream)

    def merged():
        mg.mgattn_dense_strided(qkv[:, :row], qkv[:, row:2 * row], qkv[:, 2 * row:], out, qkv.stride(0),
                                qkv.stride(0), qkv.stride(0), row, cu, nseg, H, d, wl.SCALE, 0, mg.MGATTN_BF16,
                                stream)

    # the two layouts timed in alternation, three rounds, best median of each (the
    # card's clock drifts with temperature over a run)
    best = {"separate": float("inf"), "merged": float("inf")}
    for _ in range(3):
        for name, fn in (("separate", separate), ("merged", merged)):
            best[name] = min(best[name], time_launches(torch, fn))
    for name in ("separate", "merged"):
        ms = best[name]
        res[f"{name}_qkv_full_layer_4096"] = {"ms": ms, "tflops": flops / (ms * 1e-3) / 1e12,
                                             "frac": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    # the tower's RoPE + attention per layer (tokens in 32x32-window order of the 64x64
    # grid, q|k|v merged): the RoPE pass over q and k then the attention, against
    # mgattn_dense_rope2d (k rotated in place, q rotated as the attention loads it)
    grid64 = [(64, 64)]
    for lname, li in (("full_layer_4096", 3), ("window_layer_4x1024", 0)):
        cu_l, nseg_l, fl_l = layers[li][3], layers[li][4], layers[li][5]

        def unfused(s, cu_l=cu_l, nseg_l=nseg_l):
            mg.mgattn_rope2d(qkv[:, :2 * row], qkv.stride(0), grid64, 32, 2 * H, d, THETA, mg.MGATTN_BF16, s)
            mg.mgattn_dense_strided(qkv[:, :row], qkv[:, row:2 * row], qkv[:, 2 * row:], out, qkv.stride(0),
                                    qkv.stride(0), qkv.stride(0), row, cu_l, nseg_l, H, d, wl.SCALE, 0, mg.MGATTN_BF16,
                                    s)

        def fused(s, cu_l=cu_l, nseg_l=nseg_l):
            mg.mgattn_dense_rope2d(qkv[:, :row], qkv[:, row:2 * row], qkv[:, 2 * row:], out, qkv.stride(0),
                                   qkv.stride(0), qkv.stride(0), row, cu_l, nseg_l, H, d, wl.SCALE, 0, mg.MGATTN_BF16,
                                   grid64, 32, THETA, s)

        # alternation, three rounds, best of each: "ms" per call from a graph of 20
        # calls, "ms_events" with events around one call's launches
        bt = {"unfused": float("inf"), "fused": float("inf")}
        be = dict(bt)
        for _ in range(3):
            for name, fn in (("unfused", unfused), ("fused", fused)):
                bt[name] = min(bt[name], time_graph(torch, fn))
                be[name] = min(be[name], time_launches(torch, lambda fn=fn: fn(stream)))
        res[f"rope_attention_{lname}"] = {"unfused_ms": bt["unfused"], "fused_ms": bt["fused"],
                                          "unfused_ms_events": be["unfused"], "fused_ms_events": be["fused"],
                                          "fused_tflops": fl_l / (bt["fused"] * 1e-3) / 1e12}
    # the HBM-bound kernels: "ms" from a graph of 20 calls (per call), "ms_events" with
    # events around single launches (host launch overhead included)
    for name, grids in (("tower_64x64", [(64, 64)]), ("ragged_17408", [(128, 96), (64, 64), (32, 32)])):
        T = sum(gh * gw for gh, gw in grids)
        x = torch.randn(T, row, device=dev).to(torch.bfloat16)
        y = torch.empty_like(x)

        def gather(s):
            mg.mgattn_window_permute(x, y, row * 2, grids, 32, 0, s)

        ms_g = time_graph(torch, gather)
        ms_ge = time_launches(torch, lambda: gather(stream))
        moved = 2 * T * row * 2  # read + write
        qkv3 = torch.randn(T, 3 * row, device=dev).to(torch.bfloat16)

        def rope(s):  # q and k are adjacent in a merged qkv row: one call over their 2H heads
            mg.mgattn_rope2d(qkv3[:, :2 * row], qkv3.stride(0), grids, 32, 2 * H, d, THETA, mg.MGATTN_BF16, s)

        ms_r = time_graph(torch, rope)
        ms_re = time_launches(torch, lambda: rope(stream))
        rot = 2 * 2 * T * row * 2  # q and k, read + write
        res[f"window_gather_{name}"] = {"ms": ms_g, "ms_events": ms_ge, "bytes": moved,
                                        "gbs": moved / (ms_g * 1e-3) / 1e9,
                                        "frac_hbm": moved / (ms_g * 1e-3) / 1e9 / PEAK_HBM_GBS}
        res[f"rope2d_qk_{name}"] = {"ms": ms_r, "ms_events": ms_re, "launches": 1, "bytes": rot,
                                    "gbs": rot / (ms_r * 1e-3) / 1e9,
                                    "frac_hbm": rot / (ms_r * 1e-3) / 1e9 / PEAK_HBM_GBS}
    # text decoder attention (32 query / 2 key-value heads, head size 128, window 2048)
    Hq, Hkv, dt, W = 32, 2, 128, 2048
    L = 8192
    q = torch.randn(L, Hq * dt, device=dev).to(torch.bfloat16)
    k = torch.randn(L, Hkv * dt, device=dev).to(torch.bfloat16)
    v = torch.randn(L, Hkv * dt, device=dev).to(torch.bfloat16)
    o = torch.empty_like(q)
    ms = time_launches(torch, lambda: mg.mgattn_attention_kv(q, k, v, o, Hq * dt, Hkv * dt, Hkv * dt, Hq * dt, [0, L],
                                                            [0, L], 1, Hq, Hkv, dt, dt ** -0.5, W, mg.MGATTN_BF16,
                                                            stream))
    visible = sum(min(i + 1, W) for i in range(L))
    fl = 4.0 * dt * Hq * visible
    res["text_prefill_8192_window2048"] = {"ms": ms, "gflop": fl / 1e9, "tflops": fl / (ms * 1e-3) / 1e12,
                                           "frac": fl / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
    B, Lk = 32, 4096
    qd = torch.randn(B, Hq * dt, device=dev).to(torch.bfloat16)
    kc = torch.randn(B * Lk, Hkv * dt, device=dev).to(torch.bfloat16)
    vc = torch.randn(B * Lk, Hkv * dt, device=dev).to(torch.bfloat16)
    od = torch.empty_like(qd)
    cq = list(range(B + 1))
    ck = [i * Lk for i in range(B + 1)]
    kv_bytes = B * min(Lk, W) * Hkv * dt * 2 * 2  # the window's K and V, read once
    # keys split over several workgroups per (sequence, key/value head), partial results
    # in a workspace (decode kernel + merge kernel), and one workgroup per pair without it
    wsb = mg.mgattn_attention_kv_workspace(cq, ck, B, Hq, Hkv, dt, W, mg.MGATTN_BF16)
    ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=dev)
    def decode_ws(s):
        mg.mgattn_attention_kv_ws(qd, kc, vc, od, Hq * dt, Hkv * dt, Hkv * dt, Hq * dt, cq, ck, B, Hq, Hkv, dt,
                                  dt ** -0.5, W, mg.MGATTN_BF16, ws, wsb, s)

    def decode_plain(s):
        mg.mgattn_attention_kv(qd, kc, vc, od, Hq * dt, Hkv * dt, Hkv * dt, Hq * dt, cq, ck, B, Hq, Hkv, dt,
                               dt ** -0.5, W, mg.MGATTN_BF16, s)

    ms = time_graph(torch, decode_ws)
    ms_e = time_launches(torch, lambda: decode_ws(stream))
    res["text_decode_32x4096_window2048"] = {"ms": ms, "ms_events": ms_e, "kv_bytes": kv_bytes,
                                             "gbs": kv_bytes / (ms * 1e-3) / 1e9,
                                             "frac_hbm": kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                             "workspace_bytes": wsb, "launches": 2 if wsb else 1}
    ms = time_graph(torch, decode_plain)
    res["text_decode_32x4096_window2048_no_workspace"] = {"ms": ms, "kv_bytes": kv_bytes,
                                                          "gbs": kv_bytes / (ms * 1e-3) / 1e9,
                                                          "frac_hbm": kv_bytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}
    return res


def segment_sweep(torch, mg, wl, dev) -> int:
    """Dense kernel on one 4096 x 16 x 96 input cut into equal segments of 256 .. 4096 tokens.

    Every cut gives 256 workgroups (16 heads x 16 query tiles of 256), one per CU, each
    running S/64 steps of 64 keys, so the launch time is a fixed cost plus S/64 times the
    cost of one step; the least-squares line through the points separates the two."""
    c = wl.tower_layer(3)
    q, k, v = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (c.q, c.k, c.v))
    out = torch.empty_like(q)
    T, H, D = c.T, wl.HEADS, wl.HEAD_DIM
    pts = []
    for S in (256, 512, 1024, 2048, 4096):
        cu = list(range(0, T + 1, S))
        n = len(cu) - 1

        def launch():
            mg.mgattn_dense(q, k, v, out, cu, n, H, D, wl.SCALE, 0, mg.MGATTN_BF16, None)

        for _ in range(3):
            launch()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(50):
                launch()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / 50)
        us = min(ts)
        flops = 4 * S * S * D * H * n
        pts.append((S // 64, us))
        print(f"segment {S:5d} x {n:2d}: {us:8.2f} us per launch (50 back to back, best of 5), "
              f"{flops / us / 1e6:7.1f} TFLOP/s, {S // 64:2d} steps per workgroup", flush=True)
    x = np.array([p[0] for p in pts], float)
    y = np.array([p[1] for p in pts], float)
    slope, icept = np.polyfit(x[1:], y[1:], 1)
    print(f"fit over 512..4096: {icept:.2f} us fixed per launch + {slope:.3f} us per 64-key step", flush=True)
    return 0


def shape_sweep(torch, mg, dev) -> int:
    """Dense kernel (bf16) at the tower's row width 1536 split as 24x64, 16x96 or 12x128
    heads, T = 1024..16384 tokens, one segment or 1024-token windows; seeded N(0,1)
    inputs, 30 back-to-back launches after a warm-up, best of 3."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    for d, H in ((64, 24), (96, 16), (128, 12)):
        for T in (1024, 4096, 16384):
            q, k, v = (torch.randn(T, H * d, generator=gen, device=dev).to(torch.bfloat16) for _ in range(3))
            out = torch.empty_like(q)
            for seg in ((T,) if T == 1024 else (T, 1024)):
                cu = list(range(0, T + 1, seg))
                n = len(cu) - 1

                def launch():
                    mg.mgattn_dense(q, k, v, out, cu, n, H, d, d ** -0.5, 0, mg.MGATTN_BF16, None)

                for _ in range(10):
                    launch()
                best = float("inf")
                for _ in range(3):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    for _ in range(30):
                        launch()
                    e1.record()
                    torch.cuda.synchronize()
                    best = min(best, e0.elapsed_time(e1) * 1e3 / 30)
                flops = 4.0 * seg * seg * d * H * n
                print(f"d={d:3d} H={H:2d} T={T:5d} segments {n:2d} x {seg:5d}: {best:8.1f} us "
                      f"{flops / best / 1e6:7.1f} TFLOP/s ({flops / best / 1e6 / PEAK_BF16_TFLOPS:.1%} of peak)",
                      flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager", action="store_true", help="launch the 50 layers eagerly instead of replaying a graph")
    ap.add_argument("--no-token-path", action="store_true",
                    help="skip detail.token_path (profiling runs that count only the tower's launches)")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the traffic summary from two rocprofv3 --pmc counter_collection CSVs and exit")
    ap.add_argument("--kernel-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print HBM traffic per dispatch of every kernel from two rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--counter-table", nargs="+", metavar="CSV",
                    help="print mean counters per tower launch (full / window) from rocprofv3 --pmc CSVs and exit")
    ap.add_argument("--trace-table", nargs=3, metavar=("CSV", "STEPS", "WARMUP"),
                    help="summarise the tower launches of a rocprofv3 --kernel-trace CSV of `bench.py --steps STEPS "
                         "--warmup WARMUP --no-token-path` by part of the run and exit")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (HBM counter calibration under rocprofv3)")
    ap.add_argument("--shape-sweep", action="store_true",
                    help="print the dense kernel's TFLOP/s for head_dim 64/96/128 (rows of 1536), 1024..16384 "
                         "tokens, one segment or 1024-token windows, and exit; no JSON line")
    ap.add_argument("--segment-sweep", action="store_true",
                    help="print the attention kernel's time at 4096 tokens for segment lengths 256..4096 "
                         "(fixed cost per launch vs cost per 64-key step) and exit; no JSON line")
    args = ap.parse_args()
    if args.write_traffic:
        return write_traffic(*args.write_traffic)
    if args.counter_table:
        return counter_table(args.counter_table)
    if args.kernel_traffic:
        return kernel_traffic(*args.kernel_traffic)
    if args.trace_table:
        return trace_table(args.trace_table[0], int(args.trace_table[1]), int(args.trace_table[2]))
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: mgattn has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        return 2

    import torch

    from vit_perception_encoder_amd import mgattn as mg
    from vit_perception_encoder_amd import workloads as wl

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    mg.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    if args.segment_sweep:
        return segment_sweep(torch, mg, wl, dev)
    if args.shape_sweep:
        return shape_sweep(torch, mg, dev)
    print(f"[bench] device {torch.cuda.get_device_name(0)}; generating 50 layers of seeded inputs", file=sys.stderr,
          flush=True)

    layers = []
    cpu_layers = (3, 7, 11, 15)  # the first four full-attention layers
    host_cpu = []
    for l in range(wl.N_LAYERS):
        c = wl.tower_layer(l)
        if l in cpu_layers and not args.no_cpu_baseline:
            host_cpu.append(c)
        dq, dk, dv = (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev) for x in (c.q, c.k, c.v))
        layers.append((dq, dk, dv, [int(x) for x in c.cu_seqlens], c.n_seg, c.flops(), c.meta["kind"]))
    T = layers[0][0].shape[0]
    out = torch.empty(T, wl.HEADS * wl.HEAD_DIM, dtype=torch.bfloat16, device=dev)
    step_flops = sum(x[5] for x in layers)

    def run_step(strm, events=None):
        for i, (q, k, v, cu, nseg, _, _) in enumerate(layers):
            if events is not None:
                events[i][0].record(strm)
            mg.mgattn_dense(q, k, v, out, cu, nseg, wl.HEADS, wl.HEAD_DIM, wl.SCALE, 0, mg.MGATTN_BF16, strm)
            if events is not None:
                events[i][1].record(strm)

    for _ in range(args.warmup):
        run_step(stream)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        # The 50 launches of one step are captured once and replayed: no host launch
        # overhead between layers.
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            run_step(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            run_step(torch.cuda.current_stream())
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
    print(f"[bench] warmup done ({args.warmup} steps, {'eager' if graph is None else 'graph'}); "
          f"timing {args.steps} steps", file=sys.stderr, flush=True)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            run_step(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    # every launch in the timed region is the attention kernel: its average launch
    # duration is the region's time over the launches (gaps between launches included)
    launch_ms_mean = ms_per_step / len(layers)
    flops_per_launch = step_flops / len(layers)
    achieved = flops_per_launch / (launch_ms_mean * 1e-3) / 1e12

    # per-layer-kind breakdown, events around each launch of an eager pass
    nb = max(3, min(args.steps, 10))
    ev = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in layers] for _ in range(nb)]
    for s_ in range(nb):
        run_step(stream, ev[s_])
    torch.cuda.synchronize()
    per_launch = np.array([[ev[s_][i][0].elapsed_time(ev[s_][i][1]) for i in range(len(layers))]
                           for s_ in range(nb)])
    full_idx = [i for i, x in enumerate(layers) if x[6] == "full"]
    win_idx = [i for i, x in enumerate(layers) if x[6] == "window"]
    full_ms_e = float(np.median(per_launch[:, full_idx]))
    win_ms_e = float(np.median(per_launch[:, win_idx]))
    # the same split as the tower graph runs it: the layers of one kind (each on its own
    # inputs) captured into one graph and replayed, time per launch
    def kind_ms(idx):
        def one_pass(strm):
            for i in idx:
                q, k, v, cu, nseg, _, _ = layers[i]
                mg.mgattn_dense(q, k, v, out, cu, nseg, wl.HEADS, wl.HEAD_DIM, wl.SCALE, 0, mg.MGATTN_BF16, strm)
        return time_graph(torch, one_pass, n=1) / len(idx)

    # (--eager launches nothing through graphs: the eager events are the split there, and
    # the i-th tower launch of the run stays layer i mod 50 for the counter summaries)
    if graph is not None:
        full_ms, win_ms = kind_ms(full_idx), kind_ms(win_idx)
    else:
        full_ms, win_ms = full_ms_e, win_ms_e
    full_tf = layers[full_idx[0]][5] / (full_ms * 1e-3) / 1e12
    win_tf = layers[win_idx[0]][5] / (win_ms * 1e-3) / 1e12

    print("[bench] timing the other entry points (merged qkv, window gather, 2D RoPE, text decoder)", file=sys.stderr,
          flush=True)
    token = None if args.no_token_path else token_path(torch, mg, wl, layers)
    configs = None if args.no_token_path else config_times(torch, mg, wl)
    t448 = None if args.no_token_path else tower_448(torch, mg, wl)

    if args.copy_calibration:
        a = torch.empty(1 << 29, dtype=torch.int16, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    hbm = traffic_per_launch()
    roofline = {"bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": achieved / PEAK_BF16_TFLOPS, "traffic": hbm,
                "kernel": KERNEL_NAME, "launch_ms_mean": launch_ms_mean,
                "flops_per_launch": flops_per_launch}

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        print(f"[bench] timing the f64 CPU oracle on {len(host_cpu)} full layers", file=sys.stderr, flush=True)
        wants, cpu = cpu_baseline(host_cpu, wl.config_full448())
        parity = 0.0
        for l, want in zip(cpu_layers, wants):
            q, k, v, cu, nseg, _, _ = layers[l]
            mg.mgattn_dense(q, k, v, out, cu, nseg, wl.HEADS, wl.HEAD_DIM, wl.SCALE, 0, mg.MGATTN_BF16, stream)
            torch.cuda.synchronize()
            got = wl.bf16_bits_to_f32(out.view(torch.int16).cpu().numpy().view(np.uint16)).reshape(want.shape)
            parity = max(parity, float(np.abs(got - want).max()))

    line = {
        "metric": METRIC,
        "value": step_flops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "launch": "eager" if graph is None else "hip_graph",
        "config": {"workload": "tower_4096x50: 13 full layers [4096] + 37 window layers [4x1024], H=16, d=96, "
                               "bf16 N(0,1) seeded per layer, non-causal, scale 1/sqrt(96)",
                   "tokens": T, "layers": len(layers), "heads": wl.HEADS, "head_dim": wl.HEAD_DIM},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "detail": {
            "tower_ms": ms_per_step,
            "frac_of_bf16_peak": step_flops / (ms_per_step * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "full_layer_4096": {"ms": full_ms, "ms_events": full_ms_e, "tflops": full_tf,
                                "frac": full_tf / PEAK_BF16_TFLOPS, "launches": len(full_idx)},
            "window_layer_4x1024": {"ms": win_ms, "ms_events": win_ms_e, "tflops": win_tf,
                                    "frac": win_tf / PEAK_BF16_TFLOPS, "launches": len(win_idx)},
            "step_gflop": step_flops / 1e9,
            "wall_s_timed_region": wall,
            "oracle_parity_full_layers_max_abs_err": parity,
            "token_path": token,
            "configs": configs,
            "tower_448": t448,
            "kernel_source_sha256": kernel_source_hash(),
        },
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
