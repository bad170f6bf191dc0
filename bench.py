#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: SAGA + Atop-N vs the dense GQA kernel.

One step = one saga_decode_attn call (one layer, one decode token) on the
Qwen2.5-1.5B-shaped workload at 128K context, batch 1 (h_q=12, h_k=1, h_v=4, d=128,
N=512, exact threshold every 32 steps), bf16 inputs, seeded synthetic data.

The exact threshold refresh is part of the method's cost: one step in every n
(n = refresh_period) recomputes it. Two graphs of exactly K steps each are timed:
K steps that reuse the threshold (t_steady per step) and K steps that each refresh
it (t_refresh per step). The reported step time is the amortized one,
t_step = ((n - 1) t_steady + t_refresh) / n, whatever K is. A third graph of K
consecutive steps starting at a multiple of n (refreshes at their natural rate,
ceil(K / n) of them) is timed as a cross-check and reported beside it.

Inputs are resident in HBM before timing. R rotating copies of q/K/V/tau (R*bytes(K)
>= 1 GiB, R coprime with the refresh period) keep the 256 MB Infinity Cache from
serving repeated reads, as a model's per-layer caches would. Timed steps are
replayed from a HIP graph and timed with HIP events on the launch stream.

Prints one JSON line. `value` = SAGA decode steps/s = 1 / t_step (refresh cost
amortized as above).
`roofline` is for the dominant kernel, the select kernel of a step that reuses the
threshold (saga_select_gather: K stream and comparison, and the value gather in the
early form): a graph of K launches of it alone is timed with HIP events on its
stream; its algorithmic bytes per launch are bytes(K) in the late value-gather form
(the combining kernel reads the selected V rows) and bytes(K) + bytes(selected V rows,
union per value head) in the early one (`value_gather` names the form). `traffic` is
the HBM traffic of that kernel measured with rocprofv3 counters (recorded in
profiles/ for one build of the kernels; null when the sources differ).
`cpu_baseline` is the CPU oracle timed on this host on the same workload.

Other modes: --probe copy|read (streaming ceilings and counter calibration),
--only <part> (one part, for profiler runs), --rocprof-summary CSV... (per-kernel
averages of a rocprofv3 csv output).
"""
from __future__ import annotations

import argparse
import csv
import json
import math
import os
import sys
import time
from typing import Optional

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn steps/s + % HBM roofline at l_kv=128K, bs=1 (SAGA+Atop-N vs dense GQA)"
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "k_qk_select_qwen128k_traffic.txt")
DEFAULT_WORKLOAD = "qwen2.5-1.5b-shape-l128k"


def dominant_kernel(w, form: str) -> str:
    """Name of the select kernel a workload's step spends most of its time in; `form`
    is the step's value gather, "late" (slot records, the combining kernel gathers) or
    "early" (the select kernel gathers into chunk records)."""
    dims = f"d={w.d}" if w.dv == w.d else f"d_k={w.d}, d_v={w.dv}"
    keys = "speculative keys" if w.batch == 1 else "keys after l_kv"
    out = "slot records" if form == "late" else "gather"
    return f"k_qk_select<{w.dtype}, {dims}, {keys}, {out}> (saga_select_gather)"


def select_kernel_pattern(form: str) -> str:
    """The dominant kernel's name in rocprofv3 output at the default workload (bf16,
    d = 128, speculative keys, contiguous caches)."""
    return f"k_qk_select<unsigned short, 128, 128, 1, {2 if form == 'late' else 1}, false"


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def rotating_sets(bytes_k: int, period: int, want: int) -> int:
    if want > 0:
        return want
    r = max(1, math.ceil((1 << 30) / bytes_k))
    while math.gcd(r, period) != 1:
        r += 1
    return r


def time_graph(torch, fn_steps, reps: int):
    """Capture fn_steps() into a HIP graph; replay once untimed, then `reps` timed
    replays, each bracketed by device synchronisation and HIP events on the stream
    the graph is launched on. Returns the per-replay ms list."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(g, stream=s):
        fn_steps()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1))
    del g
    return out


def pct(xs, p):
    xs = sorted(xs)
    if len(xs) == 1:
        return xs[0]
    k = (len(xs) - 1) * p / 100.0
    lo, hi = int(math.floor(k)), int(math.ceil(k))
    return xs[lo] + (xs[hi] - xs[lo]) * (k - lo)


def cpu_baseline(w, x, seconds: float, one_thread_seconds: Optional[float] = None):
    """The oracle as it stands, on the same inputs, for about `seconds` of host time
    with every host core, then (default: a fifth of that) on one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import saga_oracle as orc

    q64, k64, v64 = x.f64()

    def run(limit_s):
        tau = None
        steps = 0
        t0 = time.perf_counter()
        while True:
            r = orc.saga_decode_step(q64, k64, v64, x.l_kv, w.N, w.refresh_period, steps, tau_in=tau,
                                     keep_logits=False)
            tau = r.tau
            steps += 1
            el = time.perf_counter() - t0
            if el >= limit_s:
                return steps, el

    steps, el = run(seconds)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu_model)
    except OSError:
        pass
    with threadpool_limits(limits=1):
        steps1, el1 = run(seconds / 5 if one_thread_seconds is None else one_thread_seconds)
    return {"value": steps / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "host": {"cpu_model": cpu_model, "logical_cpus": os.cpu_count()},
            "sample": f"{steps} consecutive oracle decode steps (steps 0..{steps - 1}, exact threshold at "
                      f"step % {w.refresh_period} == 0) of the full {w.name} workload, {el:.1f} s of host time; "
                      f"float64 numpy, BLAS threads = cores",
            "single_thread": {"value": steps1 / el1, "unit": "steps/s", "cores": 1,
                              "sample": f"{steps1} steps, {el1:.1f} s, BLAS limited to one thread"}}


def cpu_baselines(args) -> int:
    """The CPU oracle timed on this host, with every core and on one thread, for the
    tiny fp32 case, the Llama- and Qwen-shaped layers and both ends of the sweep's
    context range (4K and 128K keys): one JSON line. Bounded: about
    --cpu-seconds with every core and a third of that on one thread per workload."""
    from sparse_decode_attention_saga_amd import workloads as wl

    cases = [(wl.TINY, None), (wl.LLAMA_32K, None), (wl.QWEN_128K, None),
             (wl.SWEEP, wl.SWEEP_L[0]), (wl.SWEEP, wl.SWEEP_L[-1])]
    rows = []
    for w, L in cases:
        x = wl.generate(w, seed=0) if L is None else wl.generate(w, seed=0, lengths=[L], l_max=L)
        name = w.name if L is None else f"{w.name} at l_kv={L}"
        r = cpu_baseline(w, x, args.cpu_seconds, args.cpu_seconds / 3)
        log(f"cpu oracle {name}: {r['value']:.1f} steps/s on {r['cores']} threads, "
            f"{r['single_thread']['value']:.1f} steps/s on one")
        rows.append({"workload": name, "l_kv": int(x.l_kv.max()), "N": w.N, "refresh_period": w.refresh_period,
                     "dtype": w.dtype, **r})
    print(json.dumps({"cpu_baselines": rows}), flush=True)
    return 0


def copy_probe(torch, reps: int) -> int:
    """torch's device copy of 256 MiB, `reps` times: reads and writes 256 MiB each."""
    n = 256 << 20
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    print(json.dumps({"probe": "copy", "bytes_read": n, "bytes_written": n, "launches": reps + 1,
                      "us_per_copy": us, "read_plus_write_gbs": 2 * n / us / 1e3}), flush=True)
    return 0


def read_probe(torch, reps: int) -> dict:
    """Streaming-read ceilings with the probe kernel of libsaga_probe.so (16-byte loads,
    each block one contiguous range, 8 loads in flight per thread), for 256..2048 blocks
    of 256 threads: one 1 GiB read per launch, and 32 MiB reads (the size of the 128K
    key stream) from 32 different slices, one per launch. Each is timed as a graph of
    launches, like the decode steps; the best grid is reported with the whole table."""
    import ctypes
    from sparse_decode_attention_saga_amd import build
    lib = ctypes.CDLL(build.PROBE_PATH)
    fn = lib.saga_probe_stream_read
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    n = 1 << 30
    x = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
    sink = torch.zeros(4096, dtype=torch.float32, device="cuda:0")

    def launch(off, nbytes, blocks):
        st = fn(x.data_ptr() + off, nbytes, sink.data_ptr(), blocks, torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"saga_probe_stream_read failed ({st})")

    table = {}
    for blocks in (256, 512, 1024, 2048):
        def big():
            for _ in range(4):
                launch(0, n, blocks)

        def small():
            for i in range(32):
                launch(i * (n // 32), n // 32, blocks)

        big()
        small()
        torch.cuda.synchronize()
        ms_big = min(time_graph(torch, big, reps)) / 4
        ms_small = min(time_graph(torch, small, reps)) / 32
        table[blocks] = (n / (ms_big * 1e-3) / 1e9, (n // 32) / (ms_small * 1e-3) / 1e9, ms_small * 1e3)
    best_big = max(table, key=lambda b: table[b][0])
    best_small = max(table, key=lambda b: table[b][1])

    # one read of S bytes per launch, consecutive slices over the whole GiB (so that
    # no slice is still in the 256 MB cache when it is read again): the time of a
    # short launch is a fixed part plus S over a streaming rate
    by_size = {}
    for mib in (2, 4, 8, 16, 32):
        S = mib << 20
        blocks = max(256, min(2048, S // 16384))

        def sized():
            for i in range(n // S):
                launch(i * S, S, blocks)

        sized()
        torch.cuda.synchronize()
        by_size[mib] = min(time_graph(torch, sized, reps)) / (n // S) * 1e3
    xs = np.array([m * 1048576.0 for m in by_size])
    ys = np.array([by_size[m] for m in by_size])
    slope, t0 = np.polyfit(xs, ys, 1)

    # one 32 MiB read per launch (32 slices of the GiB, a graph of 32 launches) for
    # 4, 8, 16 and 32 loads in flight per thread and 1 to 8 blocks per compute unit
    fn_ex = lib.saga_probe_stream_read_ex
    fn_ex.restype = ctypes.c_int
    fn_ex.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                      ctypes.c_void_p, ctypes.c_void_p]
    sink_ex = torch.zeros(65536, dtype=torch.float32, device="cuda:0")
    S32 = n // 32

    def launch_ex(off, blocks, loads, times=None):
        st = fn_ex(x.data_ptr() + off, S32, sink_ex.data_ptr(), blocks, loads,
                   None if times is None else times.data_ptr(), torch.cuda.current_stream().cuda_stream)
        if st != 0:
            raise RuntimeError(f"saga_probe_stream_read_ex failed ({st})")

    sweep = {}
    for loads in (4, 8, 16, 32):
        for blocks in (256, 512, 1024, 2048):
            def run32():
                for i in range(32):
                    launch_ex(i * S32, blocks, loads)
            run32()
            torch.cuda.synchronize()
            sweep[(loads, blocks)] = min(time_graph(torch, run32, reps)) / 32 * 1e3
    best = min(sweep, key=sweep.get)

    # timeline of the best configuration: per launch, the spread of block starts, the
    # first load's arrival, the last block's end (s_memrealtime, 100 MHz), against the
    # launch's share of the graph time
    loads, blocks = best
    times = [torch.zeros(3 * blocks, dtype=torch.int64, device="cuda:0") for _ in range(32)]

    def run32_t():
        for i in range(32):
            launch_ex(i * S32, blocks, loads, times[i])
    run32_t()
    torch.cuda.synchronize()
    us_launch = min(time_graph(torch, run32_t, reps)) / 32 * 1e3
    tl = []
    for t in times:
        a = t.view(blocks, 3).cpu().numpy().astype(np.float64) * 1e-2  # ticks of 10 ns -> us
        start = a[:, 0].min()
        tl.append((a[:, 0].max() - start, np.median(a[:, 1] - a[:, 0]), (a[:, 1] - start).min(),
                   a[:, 2].max() - start))
    tl = np.median(np.array(tl), axis=0)
    timeline = {"loads_per_thread": loads, "blocks": blocks, "us_per_launch_graph": us_launch,
                "us_block_start_spread": float(tl[0]), "us_first_load_median": float(tl[1]),
                "us_first_load_earliest": float(tl[2]), "us_first_to_last_instruction": float(tl[3]),
                "us_outside_kernel_body": us_launch - float(tl[3])}
    return {"kernel": "k_stream_read (libsaga_probe.so)",
            "mib32_sweep_us": {f"{l}x{b}": round(v, 3) for (l, b), v in sweep.items()},
            "mib32_best": {"loads_per_thread": best[0], "blocks": best[1], "us": sweep[best],
                           "gbs": S32 / (sweep[best] * 1e-6) / 1e9},
            "mib32_timeline": timeline,
            "per_launch_us_by_mib": {str(m): round(v, 3) for m, v in by_size.items()},
            "fit_fixed_us": float(t0), "fit_stream_gbs": float(1e-3 / slope),
            "gib_read_gbs": table[best_big][0], "gib_blocks": best_big,
            "mib32_read_gbs": table[best_small][1], "mib32_read_us": table[best_small][2], "mib32_blocks": best_small,
            "by_blocks": {str(b): {"gib_gbs": round(v[0], 1), "mib32_gbs": round(v[1], 1), "mib32_us": round(v[2], 3)}
                          for b, v in table.items()}}


def recorded_traffic():
    """Traffic per launch of the dominant kernel recorded in profiles/, if it was
    measured on the current sources of the kernels; else None (with the reason)."""
    from sparse_decode_attention_saga_amd import build
    if not os.path.exists(TRAFFIC_FILE):
        return None, "no counter record"
    rec = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != build.source_digest():
        return None, "kernel sources changed since the counters were taken"
    return float(rec["traffic_bytes_per_launch"]), os.path.relpath(TRAFFIC_FILE, os.path.dirname(os.path.abspath(__file__)))


def rocprof_summary(paths) -> int:
    """Per-kernel averages of rocprofv3 csv files: kernel_stats (durations) or
    counter_collection (one row per dispatch and counter)."""
    for path in paths:
        with open(path) as f:
            rows = list(csv.DictReader(f))
        if not rows:
            continue
        if "AverageNs" in rows[0]:
            print(f"# {os.path.basename(path)}: kernel, calls, average / min / max duration (us)")
            for r in rows:
                print(f"{r['Name'][:96]:96s} {int(r['Calls']):7d} {float(r['AverageNs']) / 1e3:9.2f} "
                      f"{float(r['MinNs']) / 1e3:9.2f} {float(r['MaxNs']) / 1e3:9.2f}")
        elif "Counter_Name" in rows[0]:
            acc = {}
            for r in rows:
                key = (r["Kernel_Name"], r["Counter_Name"])
                s = acc.setdefault(key, [0.0, 0])
                s[0] += float(r["Counter_Value"])
                s[1] += 1
            print(f"# {os.path.basename(path)}: kernel, counter, dispatches, average value per dispatch")
            for (k, c), (tot, n) in sorted(acc.items()):
                print(f"{k[:96]:96s} {c:12s} {n:7d} {tot / n:14.1f}")
    return 0


def counter_averages(path):
    """{(kernel, counter): (average value per dispatch, dispatches)} of a rocprofv3
    counter_collection csv."""
    acc = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            key = (r["Kernel_Name"], r["Counter_Name"])
            a = acc.setdefault(key, [0.0, 0])
            a[0] += float(r["Counter_Value"])
            a[1] += 1
    return {k: (v[0] / v[1], v[1]) for k, v in acc.items()}


def traffic_record(args) -> int:
    """Writes the HBM-traffic record of the dominant kernel from four rocprofv3
    counter_collection csv files: FETCH_SIZE and WRITE_SIZE of a
    `--only select` run, and FETCH_SIZE and WRITE_SIZE of a `--probe copy` run (a
    256 MiB device copy: 262144 KiB read and written per dispatch, which calibrates the
    two counters to bytes). The record names the kernel sources it was taken on."""
    from sparse_decode_attention_saga_amd import build
    f_sel, w_sel, f_copy, w_copy = args.traffic_record
    copy_kib = 262144.0
    cf = counter_averages(f_copy)
    cw = counter_averages(w_copy)
    cf_copy = next(v for (k, c), v in cf.items() if "copyBuffer" in k and c == "FETCH_SIZE")
    cw_copy = next(v for (k, c), v in cw.items() if "copyBuffer" in k and c == "WRITE_SIZE")
    fetch_scale, write_scale = copy_kib / cf_copy[0], copy_kib / cw_copy[0]
    name = select_kernel_pattern(args.form)
    fs = counter_averages(f_sel)
    ws = counter_averages(w_sel)
    f_k = next(v for (k, c), v in fs.items() if name in k and c == "FETCH_SIZE")
    w_k = next(v for (k, c), v in ws.items() if name in k and c == "WRITE_SIZE")
    traffic = f_k[0] * 1024 * fetch_scale + w_k[0] * 1024 * write_scale
    alg = args.alg_bytes

    def outdir(csv_path):  # the -d directory of the rocprofv3 run that wrote csv_path
        return os.path.relpath(os.path.dirname(os.path.abspath(csv_path)), ROOT)

    kept = "kept-entry slot records (late value gather)" if args.form == "late" else \
        "value gather into chunk records (early value gather)"
    lines = [
        f"# HBM traffic of k_qk_select<bf16, d=128, speculative keys, {kept}> (saga_select_gather),",
        "# the select kernel of a step that reuses the threshold, on the Qwen2.5-1.5B-shaped layer at",
        "# l_kv=128K (rotating input sets, so the caches are read from HBM).",
        "#",
        "# counter passes (repository root), one counter per run:",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {outdir(f_sel)} -o p --output-format csv -- \\",
        "#       python3 -u bench.py --only select --steps 256 --warmup 8 --reps 1 --no-cpu-baseline",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {outdir(w_sel)} -o p --output-format csv -- (the same)",
        f"#   rocprofv3 --pmc FETCH_SIZE -d {outdir(f_copy)} -o p --output-format csv -- \\",
        "#       python3 -u bench.py --probe copy --steps 8",
        f"#   rocprofv3 --pmc WRITE_SIZE -d {outdir(w_copy)} -o p --output-format csv -- (the same)",
        f"#   python3 bench.py --traffic-record <the four counter_collection.csv> --alg-bytes {alg} --form {args.form}",
        "# calibration: a 256 MiB device copy reads and writes 262144 KiB per dispatch;",
        f"#   FETCH_SIZE reads {cf_copy[0]:.1f} KiB (scale {fetch_scale:.5f}), "
        f"WRITE_SIZE reads {cw_copy[0]:.1f} KiB (scale {write_scale:.5f})",
        "# traffic = FETCH_SIZE * 1024 * fetch_scale + WRITE_SIZE * 1024 * write_scale",
    ]
    if alg:
        what = "K stream" if args.form == "late" else "K stream + union of selected V rows"
        lines.append(f"# algorithmic bytes per launch ({what}) = {alg}")
        lines.append(f"#   -> traffic / algorithmic = {traffic / alg:.3f}; reads alone = "
                     f"{f_k[0] * 1024 * fetch_scale / alg:.3f}")
    lines += [
        f"fetch_kib_per_dispatch: {f_k[0]:.1f}",
        f"write_kib_per_dispatch: {w_k[0]:.1f}",
        f"dispatches: {f_k[1]}",
        f"fetch_scale: {fetch_scale:.6f}",
        f"write_scale: {write_scale:.6f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"source_sha256: {build.source_digest()}",
        "#",
        "# averages per dispatch of every kernel of the select runs (KiB):",
    ]
    for (k, c), (v, n) in sorted(list(fs.items()) + list(ws.items())):
        lines.append(f"#   {k[:90]:90s} {c:10s} {n:6d} {v:12.1f}")
    text = "\n".join(lines) + "\n"
    with open(args.out or TRAFFIC_FILE, "w") as f:
        f.write(text)
    print(text, end="")
    return 0


def sweep(torch, args) -> int:
    """Decode step time of SAGA + Atop-N and of the dense GQA kernel over the sweep grid
    (Qwen2.5-1.5B-shaped heads, l_kv in 4K..128K, N in {128, 512, 2048}, refresh period
    in {1, 8, 64}): where sparse selection stops paying off. Each point rotates enough
    input sets that the touched bytes exceed the Infinity Cache."""
    from sparse_decode_attention_saga_amd import api
    from sparse_decode_attention_saga_amd import workloads as wl

    dev = torch.device("cuda:0")
    api.lib()
    base_w = wl.SWEEP
    K, W = args.steps, args.warmup
    rows = []
    for L in wl.SWEEP_L:
        x = wl.generate(base_w, seed=0, lengths=[L], l_max=L)
        q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
        l_kv = torch.from_numpy(x.l_kv).to(dev)
        touched = k0.numel() * 2 + base_w.h_q * max(wl.SWEEP_N) * base_w.d * 2
        R = max(2, math.ceil((768 << 20) / touched))
        while any(math.gcd(R, n) != 1 for n in wl.SWEEP_PERIOD):
            R += 1
        ks = k0.unsqueeze(0).repeat(R, 1, 1, 1, 1)
        vs = v0.unsqueeze(0).repeat(R, 1, 1, 1, 1)
        out = torch.empty_like(q0)
        wsp = None
        wd = base_w.with_(h_k=base_w.dense_h_kv, h_v=base_w.dense_h_kv, workload_id=base_w.workload_id + 100)
        xd = wl.generate(wd, seed=0, lengths=[L], l_max=L)
        qd = xd.q.to(dev)
        Rd = max(2, math.ceil((768 << 20) / (2 * xd.k.numel() * 2)))
        kd = xd.k.to(dev).unsqueeze(0).repeat(Rd, 1, 1, 1, 1)
        vd = xd.v.to(dev).unsqueeze(0).repeat(Rd, 1, 1, 1, 1)
        wsd = api.Workspace(api.make_shape(qd, kd[0], vd[0]), 1, L, dev)
        outd = torch.empty_like(qd)

        def dense_step(t):
            api.dense_gqa_attn(qd, kd[t % Rd], vd[t % Rd], l_kv, max_l_kv=L, out=outd, workspace=wsd)

        for t in range(W):
            dense_step(t)
        torch.cuda.synchronize()
        dense_us = pct([1e3 * m / K for m in time_graph(torch, lambda: [dense_step(t) for t in range(K)],
                                                        args.reps)], 50)
        for N in wl.SWEEP_N:
            wsp = api.Workspace(api.make_shape(q0, k0, v0), N, L, dev)
            for n in wl.SWEEP_PERIOD:
                taus = torch.zeros(R, 1, base_w.h_q, dtype=torch.float32, device=dev)
                for r in range(R):
                    api.refresh_threshold(q0, ks[r], l_kv, taus[r], N=N, max_l_kv=L, workspace=wsp)

                def step(t):
                    r = t % R
                    api.decode_attn(q0, ks[r], vs[r], l_kv, taus[r], N=N, refresh_period=n, step=t,
                                    max_l_kv=L, out=out, workspace=wsp)

                for t in range(W):
                    step(t)
                torch.cuda.synchronize()
                us = pct([1e3 * m / K for m in time_graph(torch, lambda: [step(t) for t in range(W, W + K)],
                                                          args.reps)], 50)
                rows.append({"l_kv": L, "N": N, "refresh_period": n, "saga_us": us, "dense_us": dense_us,
                             "speedup": dense_us / us, "sets": R})
                log(f"l_kv={L:6d} N={N:4d} n={n:2d}: saga {us:7.2f} us  dense {dense_us:7.2f} us  "
                    f"speedup {dense_us / us:5.2f}")
        del ks, vs, kd, vd
        torch.cuda.empty_cache()
    print(json.dumps({"sweep": rows, "steps": K, "warmup": W, "workload": base_w.name,
                      "dense_h_kv": base_w.dense_h_kv}), flush=True)
    return 0


def merge_bench(torch, args) -> int:
    """The GQA-to-SAGA key-head merge (closed-form initialisation) at the Llama 3.2-1B
    shape: D = 2048, h_q = 32, 8 teacher key heads of d = 64 merged into 4, on T
    calibration tokens of random hidden states with random-init projections. Times the
    device part (saga_merge_losses: projections, Grams, per-pair closed form and
    losses; saga_merge_keys) with HIP events, the host matching, and the CPU oracle
    on the same inputs at the smaller T."""
    from sparse_decode_attention_saga_amd import api
    from sparse_decode_attention_saga_amd import workloads as wl

    dev = torch.device("cuda:0")
    api.lib()
    D, h_q, h_k, d = 2048, 32, 8, 64
    res = {}
    for T in args.merge_tokens:
        inp = wl.merge_inputs(T, D, h_q, h_k, d, seed=0)
        x, wq, wk = inp.x.to(dev), inp.w_q.to(dev), inp.w_k.to(dev)
        loss, ws = api.merge_losses(x, wq, wk, h_q=h_q, h_k=h_k)
        partner, total = api.min_weight_pairing(loss.cpu())
        out = api.merge_keys(x, wq, wk, partner, h_q=h_q, h_k=h_k, workspace=ws)
        torch.cuda.synchronize()
        t_loss, t_keys, t_host = [], [], []
        for _ in range(max(args.reps, 3)):
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            torch.cuda.synchronize()
            e0.record()
            api.merge_losses(x, wq, wk, h_q=h_q, h_k=h_k, workspace=ws)
            e1.record()
            api.merge_keys(x, wq, wk, partner, h_q=h_q, h_k=h_k, workspace=ws, out=out)
            e2.record()
            torch.cuda.synchronize()
            t_loss.append(1e3 * e0.elapsed_time(e1))
            t_keys.append(1e3 * e1.elapsed_time(e2))
            h0 = time.perf_counter()
            api.min_weight_pairing(loss.cpu())
            t_host.append(1e6 * (time.perf_counter() - h0))
        n_cols = (h_q + h_k) * d
        flops = 2.0 * T * D * n_cols + 2.0 * (h_k * d * d * (h_q // h_k) * T + (h_k * d) ** 2 * T)
        r = {"us_merge_losses": pct(t_loss, 50), "us_merge_keys": pct(t_keys, 50),
             "us_host_pairing_incl_copy": pct(t_host, 50),
             "projection_and_gram_flop": flops,
             "pairs": sorted((a, b) for a, b in enumerate(partner) if a < b), "total_loss": total}
        log(f"merge T={T}: losses {r['us_merge_losses']:.1f} us, keys {r['us_merge_keys']:.1f} us, "
            f"host pairing {r['us_host_pairing_incl_copy']:.1f} us")
        if not args.no_cpu_baseline and T == min(args.merge_tokens):
            from threadpoolctl import threadpool_info
            from oracle import convert_oracle as cv
            X = inp.x.double().numpy()
            W_Q, W_K = inp.w_q.double().numpy().T, inp.w_k.double().numpy().T
            t0 = time.perf_counter()
            n = 0
            while True:
                cv.convert(X, W_Q, W_K, h_q, h_k, d)
                n += 1
                if time.perf_counter() - t0 >= args.cpu_seconds:
                    break
            el = time.perf_counter() - t0
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            r["cpu_baseline"] = {"value": n / el, "unit": "conversions/s", "cores": int(threads), "kind": "oracle",
                                 "sample": f"{n} full oracle conversions (all 28 pair losses by eq. (13), "
                                           f"merges, matching) of this T={T} input, {el:.1f} s"}
            r["gpu_conversions_per_s"] = 1e6 / (r["us_merge_losses"] + r["us_merge_keys"] +
                                                r["us_host_pairing_incl_copy"])
        res[str(T)] = r
    print(json.dumps({"metric": "GQA-to-SAGA key-head merge time (closed-form initialisation)",
                      "unit": "us", "config": {"workload": "llama3.2-1b-shape key-head merge", "d_model": D,
                                               "h_q": h_q, "h_k_teacher": h_k, "h_k_student": h_k // 2, "d": d,
                                               "inputs": "bf16 random hidden states and projections"},
                      "by_tokens": res}), flush=True)
    return 0


def decompose(torch, args) -> int:
    """Where the SAGA + Atop-N gain comes from, at the Qwen2.5-1.5B-shaped 128K layer:
    the same library's dense attention and Atop-N step, each with grouped-query heads
    (h_k = h_v = 2, the original layer) and with SAGA heads (h_k = 1, h_v = 4)."""
    from sparse_decode_attention_saga_amd import api
    from sparse_decode_attention_saga_amd import workloads as wl

    dev = torch.device("cuda:0")
    api.lib()
    w0 = wl.WORKLOADS[args.workload]
    K, W = args.steps, args.warmup
    L = w0.l_kv
    heads = {"gqa": (w0.dense_h_kv, w0.dense_h_kv), "saga": (w0.h_k, w0.h_v)}
    res = {}
    for name, (h_k, h_v) in heads.items():
        w = w0.with_(h_k=h_k, h_v=h_v, workload_id=w0.workload_id + (100 if name == "gqa" else 0))
        x = wl.generate(w, seed=0)
        q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
        l_kv = torch.from_numpy(x.l_kv).to(dev)
        touched = (k0.numel() + v0.numel()) * k0.element_size()
        R = max(2, math.ceil((1 << 30) / touched))
        while math.gcd(R, w0.refresh_period) != 1:
            R += 1
        ks = k0.unsqueeze(0).repeat(R, 1, 1, 1, 1)
        vs = v0.unsqueeze(0).repeat(R, 1, 1, 1, 1)
        out = torch.empty_like(q0)
        ws = api.Workspace(api.make_shape(q0, k0, v0), w0.N, L, dev)
        taus = torch.zeros(R, w0.batch, w0.h_q, dtype=torch.float32, device=dev)
        for r in range(R):
            api.refresh_threshold(q0, ks[r], l_kv, taus[r], N=w0.N, max_l_kv=L, workspace=ws)

        def dense_step(t):
            api.dense_gqa_attn(q0, ks[t % R], vs[t % R], l_kv, max_l_kv=L, out=out, workspace=ws)

        def sparse_step(t):
            r = t % R
            api.decode_attn(q0, ks[r], vs[r], l_kv, taus[r], N=w0.N, refresh_period=w0.refresh_period, step=t,
                            max_l_kv=L, out=out, workspace=ws)

        for label, fn in (("dense", dense_step), ("atopn", sparse_step)):
            for t in range(W):
                fn(t)
            torch.cuda.synchronize()
            us = pct([1e3 * m / K for m in time_graph(torch, lambda: [fn(t) for t in range(W, W + K)], args.reps)], 50)
            res[f"{name}_{label}_us"] = us
            log(f"{name} (h_k={h_k}, h_v={h_v}) {label}: {us:.2f} us/step")
        del ks, vs
        torch.cuda.empty_cache()
    base = res["gqa_dense_us"]
    line = {"decomposition": w0.name, "N": w0.N, "refresh_period": w0.refresh_period, "steps": K, **res,
            "speedup_saga_heads_dense": base / res["saga_dense_us"],
            "speedup_gqa_atopn": base / res["gqa_atopn_us"],
            "speedup_saga_atopn": base / res["saga_atopn_us"],
            "saga_over_gqa_with_atopn": res["gqa_atopn_us"] / res["saga_atopn_us"]}
    print(json.dumps(line), flush=True)
    return 0


def stages(torch, args) -> int:
    """The stages of the decode step as separate launches, at a workload (default: the
    Qwen2.5-1.5B-shaped 128K layer), each timed alone from a graph of launches over
    rotating input sets: the key stream with the Atop-N comparison (saga_qk_select,
    algorithmic bytes = the keys), the value gather into chunk records followed by the
    combine (saga_sparse_gather over the kept lists of one saga_qk_select call,
    algorithmic bytes = the selected value rows), and the step's own two kernels
    (saga_select_gather, saga_split_combine) in the value-gather form the step takes.
    Under rocprofv3 the same command gives each kernel's duration and counters."""
    from sparse_decode_attention_saga_amd import api
    from sparse_decode_attention_saga_amd import bytemodel
    from sparse_decode_attention_saga_amd import workloads as wl

    dev = torch.device("cuda:0")
    api.lib()
    w = wl.WORKLOADS[args.workload]
    es = 2 if w.dtype == "bf16" else 4
    x = wl.generate(w, seed=0)
    L = int(x.k.shape[2])
    lens = [int(n) for n in x.l_kv]
    bytes_k = bytemodel.key_bytes(w.h_k, w.d, lens, es)
    R = rotating_sets(bytes_k, w.refresh_period, args.sets)
    q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    l_kv = torch.from_numpy(x.l_kv).to(dev)
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    tau = torch.zeros(w.batch, w.h_q, dtype=torch.float32, device=dev)
    out = torch.empty(w.batch, w.h_q, w.dv, dtype=q0.dtype, device=dev)
    ws = api.Workspace(api.make_shape(q0, k0, v0), w.N, L, dev)
    api.refresh_threshold(q0, k0, l_kv, tau, N=w.N, max_l_kv=L, workspace=ws, d_v=w.dv)
    # the selected value rows of the threshold (the union over each value head's query heads)
    cap = 8 * w.N
    sel_count = torch.zeros(w.batch, w.h_q, dtype=torch.int32, device=dev)
    sel_idx = torch.full((w.batch, w.h_q, cap), -1, dtype=torch.int32, device=dev)
    api.decode_attn(q0, k0, v0, l_kv, tau, N=w.N, refresh_period=1 << 30, step=1, max_l_kv=L, out=out,
                    sel_count=sel_count, sel_idx=sel_idx, workspace=ws)
    torch.cuda.synchronize()
    counts, idx = sel_count.cpu().numpy(), sel_idx.cpu().numpy()
    union_rows = []
    for b in range(w.batch):
        for vh in range(w.h_v):
            rows = set()
            for j in range(w.h_q):
                if (j * w.h_v) // w.h_q == vh:
                    rows.update(idx[b, j, : min(counts[b, j], cap)].tolist())
            union_rows.append(len(rows))
    bytes_v = bytemodel.selected_value_bytes(union_rows, w.dv, es)
    K = args.steps

    def timed(fn):
        fn(0)
        torch.cuda.synchronize()
        return pct([1e3 * m / K for m in time_graph(torch, lambda: [fn(t) for t in range(K)], args.reps)], 50)

    res = {}
    res["qk_select"] = timed(lambda t: api.qk_select(q0, ks[t % R], l_kv, tau, max_l_kv=L, workspace=ws, d_v=w.dv))
    api.qk_select(q0, k0, l_kv, tau, max_l_kv=L, workspace=ws, d_v=w.dv)  # the kept lists the gather reads
    res["sparse_gather"] = timed(lambda t: api.sparse_gather(q0, ks[t % R], vs[t % R], l_kv, tau, N=w.N, max_l_kv=L,
                                                             out=out, workspace=ws))
    res["select_gather"] = timed(lambda t: api.select_gather(q0, ks[t % R], vs[t % R], l_kv, tau, N=w.N,
                                                             max_l_kv=L, workspace=ws))
    res["split_combine"] = timed(lambda t: api.split_combine(q0, ks[t % R], vs[t % R], l_kv, tau, N=w.N, max_l_kv=L,
                                                             out=out, workspace=ws))
    for k, v in res.items():
        log(f"{k}: {v:.2f} us/launch")
    form = api.gather_form(api.make_shape(q0, k0, v0), w.N, L)
    # the late gather's select kernel reads the keys, its combining kernel the value rows
    sel_bytes = bytes_k if form == "late" else bytes_k + bytes_v
    line = {"stages": w.name, "rotating_sets": R, "steps": K, "us": res, "value_gather": form,
            "bytes": {"keys": bytes_k, "selected_value_rows": bytes_v},
            "gbs": {"qk_select_keys": bytes_k / res["qk_select"] / 1e3,
                    "sparse_gather_value_rows": bytes_v / res["sparse_gather"] / 1e3,
                    "select_gather_" + ("keys" if form == "late" else "keys_and_rows"):
                        sel_bytes / res["select_gather"] / 1e3}}
    print(json.dumps(line), flush=True)
    return 0


def device_pages(torch, k, v, page_tokens: int, seed: int):
    """Paged copies of contiguous caches k [B, h_k, L, d], v [B, h_v, L, d_v] (L a
    multiple of the page size) on the device, pages in a seeded random order:
    (k_pages [B*L/P, h_k, P, d], v_pages [B*L/P, h_v, P, d_v], table [B, L/P] int32)."""
    B, h_k, L, d = k.shape
    h_v, dv = v.shape[1], v.shape[3]
    P = page_tokens
    n = L // P
    gen = torch.Generator().manual_seed(seed)
    perm = torch.randperm(B * n, generator=gen).to(torch.int64)
    kp = torch.empty((B * n, h_k, P, d), dtype=k.dtype, device=k.device)
    vp = torch.empty((B * n, h_v, P, dv), dtype=v.dtype, device=v.device)
    kp[perm.to(k.device)] = k.reshape(B, h_k, n, P, d).permute(0, 2, 1, 3, 4).reshape(B * n, h_k, P, d)
    vp[perm.to(v.device)] = v.reshape(B, h_v, n, P, dv).permute(0, 2, 1, 3, 4).reshape(B * n, h_v, P, dv)
    table = perm.to(torch.int32).reshape(B, n).to(k.device)
    return kp, vp, table


def paged_timing(torch, api, w, qs, ks, vs, taus, l_kv, L, args) -> list:
    """The decode step and the reuse step over paged copies of the rotating sets."""
    out = []
    R = len(ks)
    K, W = args.steps, args.warmup
    for P in args.paged:
        if L % P:
            log(f"paged: skipping {P}-token pages (l_kv is not a multiple)")
            continue
        sets = [device_pages(torch, ks[r], vs[r], P, seed=r) for r in range(R)]
        tau_p = [t.clone() for t in taus]
        o = torch.empty(w.batch, w.h_q, w.dv, dtype=qs[0].dtype, device=qs[0].device)
        shape = api.make_shape(qs[0], ks[0], vs[0])
        ws = api.Workspace(shape, w.N, L, qs[0].device)

        def step(t, period):
            r = t % R
            kp, vp, tab = sets[r]
            api.decode_attn_paged(qs[r], kp, vp, tab, l_kv, tau_p[r], N=w.N, refresh_period=period, step=t,
                                  max_l_kv=L, out=o, workspace=ws)

        for t in range(W):
            step(t, w.refresh_period)
        torch.cuda.synchronize()
        n = w.refresh_period
        ms = time_graph(torch, lambda: [step(1 + t, 1 << 30) for t in range(W, W + K)], args.reps)
        us_steady = pct([1e3 * m / K for m in ms], 50)
        ms = time_graph(torch, lambda: [step(t, 1) for t in range(W, W + K)], args.reps)
        us_refresh = pct([1e3 * m / K for m in ms], 50)
        us = ((n - 1) * us_steady + us_refresh) / n
        log(f"paged ({P}-token pages): {us:.2f} us/step amortized (steady {us_steady:.2f}, refresh "
            f"{us_refresh:.2f} us/step)")
        out.append({"page_tokens": P, "us_per_step": us, "us_steady_step": us_steady,
                    "us_refresh_step": us_refresh})
        del sets
    return out


def layer_timing(torch, api, wl, w, ks, vs, L, args) -> dict:
    """One decode layer (QKV projection + cache append, attention, W_O) with random
    weights at the workload's model shape: SAGA heads with Atop-N over the rotating
    cache sets, against the dense GQA layer of the original head shape (dense_h_kv
    key and value heads). Weights rotate with the caches. The new token is appended
    at row L - 1, so the attention reads L rows as in the attention-only step."""
    dev = ks[0].device
    R = len(ks)
    K, W = args.steps, args.warmup
    D = w.h_q * w.d
    bf = torch.bfloat16

    def weight_sets(h_k, h_v, n):
        return [wl.layer_inputs(w, seed=r, h_k=h_k, h_v=h_v) for r in range(n)]

    l_kv = torch.full((w.batch,), L - 1, dtype=torch.int32, device=dev)
    l_next = torch.empty_like(l_kv)
    out = {"d_model": D}

    def run(kset, vset, wsets, mode, label):
        n = len(kset)
        xs = [s.x.to(dev) for s in wsets]
        wq = [s.w_qkv.to(dev) for s in wsets]
        wo = [s.w_o.to(dev) for s in wsets]
        taus = [torch.zeros(w.batch, w.h_q, dtype=torch.float32, device=dev) for _ in range(n)]
        y = torch.empty(w.batch, D, dtype=bf, device=dev)
        desc = api.layer_desc(xs[0], kset[0], vset[0], w.h_q, bf)
        lws = api.LayerWorkspace(desc, w.N, L, dev)

        def step(t, period=w.refresh_period):
            r = t % n
            api.decode_layer(xs[r], wq[r], wo[r], kset[r], vset[r], l_kv, l_next, h_q=w.h_q, attention=mode,
                             N=w.N, refresh_period=period, step=t, tau=taus[r], max_l_kv=L, out=y,
                             workspace=lws)

        def proj(t):
            r = t % n
            q = api.qkv_append(xs[r], wq[r], kset[r], vset[r], l_kv, l_next, h_q=w.h_q)
            api.linear(q.reshape(w.batch, -1), wo[r], out=y)

        # every set starts from an exact threshold, as a decode loop would
        for r in range(n):
            api.decode_layer(xs[r], wq[r], wo[r], kset[r], vset[r], l_kv, l_next, h_q=w.h_q, attention=mode,
                             N=w.N, refresh_period=1, step=0, tau=taus[r], max_l_kv=L, out=y, workspace=lws)
        for t in range(W):
            step(t)
        torch.cuda.synchronize()
        # steps that reuse the threshold, and (Atop-N) steps that refresh it, amortized
        # over the refresh period as the attention step is
        ms = time_graph(torch, lambda: [step(1 + t, 1 << 30) for t in range(W, W + K)], args.reps)
        us = pct([1e3 * m / K for m in ms], 50)
        if mode == api.ATTN_ATOPN:
            p = w.refresh_period
            ms = time_graph(torch, lambda: [step(t, 1) for t in range(W, W + K)], args.reps)
            us = ((p - 1) * us + pct([1e3 * m / K for m in ms], 50)) / p
        ms = time_graph(torch, lambda: [proj(t) for t in range(W, W + K)], args.reps)
        us_proj = pct([1e3 * m / K for m in ms], 50)
        wbytes = (wq[0].numel() + wo[0].numel()) * 2
        log(f"layer ({label}): {us:.2f} us/step; its two projections alone {us_proj:.2f} us "
            f"({wbytes / 1e6:.1f} MB of weights)")
        return us, us_proj, wbytes

    us, us_proj, wb = run(ks, vs, weight_sets(w.h_k, w.h_v, R), api.ATTN_ATOPN, "SAGA + Atop-N")
    out.update({"saga_us": us, "saga_projections_us": us_proj, "saga_weight_bytes": wb})
    if w.dense_h_kv:
        wd = w.with_(h_k=w.dense_h_kv, h_v=w.dense_h_kv, workload_id=w.workload_id + 100)
        xd = wl.generate(wd, seed=0)
        Rd = rotating_sets(bytemodel_dense_bytes(wd, L), 1, 0)
        kd = [xd.k.to(dev)]
        vd = [xd.v.to(dev)]
        kd += [kd[0].clone() for _ in range(Rd - 1)]
        vd += [vd[0].clone() for _ in range(Rd - 1)]
        us_d, us_dp, wbd = run(kd, vd, weight_sets(wd.h_k, wd.h_v, Rd), api.ATTN_DENSE,
                               f"dense GQA, h_kv={wd.h_k}")
        out.update({"dense_h_kv": wd.h_k, "dense_us": us_d, "dense_projections_us": us_dp,
                    "dense_weight_bytes": wbd, "speedup": us_d / us})
        del kd, vd
    return out


def bytemodel_dense_bytes(wd, L) -> int:
    from sparse_decode_attention_saga_amd import bytemodel
    return bytemodel.dense_bytes(wd.h_k, wd.d, [L] * wd.batch, 2 if wd.dtype == "bf16" else 4)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--reps", type=int, default=20, help="timed graph replays (median, p10, p90 reported)")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--batch", type=int, default=0, help="override the workload's batch size")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: >= 1 GiB of K)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--paged", type=int, nargs="*", default=[16, 256], metavar="P",
                    help="also time the step over paged caches with P-token pages (none: skip)")
    ap.add_argument("--no-layer", action="store_true", help="skip the decode-layer timing")
    ap.add_argument("--only", choices=["all", "saga", "dense", "select", "steady", "refresh", "paged", "layer"],
                    default="all",
                    help="time only one part (for profiler runs)")
    ap.add_argument("--probe", choices=["none", "copy", "read"], default="none",
                    help="copy: a plain device copy of 256 MiB (counter calibration); read: read ceilings")
    ap.add_argument("--rocprof-summary", nargs="+", metavar="CSV",
                    help="print per-kernel averages of rocprofv3 csv files and exit")
    ap.add_argument("--traffic-record", nargs=4, metavar=("SEL_FETCH", "SEL_WRITE", "COPY_FETCH", "COPY_WRITE"),
                    help="write the dominant kernel's traffic record from four counter_collection csv files")
    ap.add_argument("--alg-bytes", type=int, default=0, help="algorithmic bytes per launch (--traffic-record)")
    ap.add_argument("--form", choices=["late", "early"], default="late",
                    help="value-gather form of the select kernel of --traffic-record")
    ap.add_argument("--out", default=None, help="output file of --traffic-record (default: the profiles record)")
    ap.add_argument("--sweep", action="store_true",
                    help="SAGA vs dense step time over l_kv x N x refresh period (one JSON line)")
    ap.add_argument("--merge", action="store_true",
                    help="GQA-to-SAGA key-head merge at the Llama 3.2-1B shape (one JSON line)")
    ap.add_argument("--merge-tokens", type=int, nargs="+", default=[512, 4096],
                    help="calibration token counts of --merge")
    ap.add_argument("--stages", action="store_true",
                    help="time the stages of the step as separate launches (key stream, value gather, combine)")
    ap.add_argument("--cpu-baselines", action="store_true",
                    help="time the CPU oracle (all cores, one thread) on the tiny, Llama- and Qwen-shaped "
                         "workloads and the sweep's 4K and 128K ends (one JSON line)")
    ap.add_argument("--decompose", action="store_true",
                    help="dense and Atop-N steps with grouped-query and with SAGA heads (one JSON line)")
    args = ap.parse_args()

    if args.rocprof_summary:
        return rocprof_summary(args.rocprof_summary)
    if args.traffic_record:
        return traffic_record(args)
    if args.cpu_baselines:
        return cpu_baselines(args)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode step runs on a single MI355X; "
              "multi-GPU runs are not part of this library.", file=sys.stderr)
        return 2

    import torch

    if args.probe == "copy":
        return copy_probe(torch, max(args.steps, 8))
    if args.probe == "read":
        print(json.dumps({"probe": "read", **read_probe(torch, max(args.reps, 3))}), flush=True)
        return 0
    if args.sweep:
        return sweep(torch, args)
    if args.decompose:
        return decompose(torch, args)
    if args.stages:
        return stages(torch, args)
    if args.merge:
        return merge_bench(torch, args)

    from sparse_decode_attention_saga_amd import api
    from sparse_decode_attention_saga_amd import bytemodel
    from sparse_decode_attention_saga_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if args.batch:
        w = w.with_(batch=args.batch)
    dev = torch.device("cuda:0")
    api.lib()
    es = 2 if w.dtype == "bf16" else 4
    t0 = time.perf_counter()
    x = wl.generate(w, seed=0)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")
    L = int(x.k.shape[2])              # cache capacity: the longest sequence
    lens = [int(n) for n in x.l_kv]
    ragged = len(set(lens)) > 1
    bytes_k = bytemodel.key_bytes(w.h_k, w.d, lens, es)
    R = rotating_sets(bytes_k, w.refresh_period, args.sets)
    dims = f"d={w.d}" if w.dv == w.d else f"d_k={w.d} d_v={w.dv}"
    ctx = f"l_kv={min(lens)}..{max(lens)} (mean {np.mean(lens):.0f})" if ragged else f"l_kv={L}"
    log(f"workload {w.name}: B={w.batch} h_q={w.h_q} h_k={w.h_k} h_v={w.h_v} {dims} {ctx} "
        f"N={w.N} n={w.refresh_period}; {R} rotating sets")
    q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    l_kv = torch.from_numpy(x.l_kv).to(dev)
    qs = [q0] + [q0.clone() for _ in range(R - 1)]
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    taus = [torch.zeros(w.batch, w.h_q, dtype=torch.float32, device=dev) for _ in range(R)]
    out = torch.empty(w.batch, w.h_q, w.dv, dtype=q0.dtype, device=dev)
    shape = api.make_shape(q0, k0, v0)
    form = api.gather_form(shape, w.N, L)
    ws = api.Workspace(shape, w.N, L, dev)
    for r in range(R):
        api.refresh_threshold(qs[r], ks[r], l_kv, taus[r], N=w.N, max_l_kv=L, workspace=ws, d_v=w.dv)
    torch.cuda.synchronize()

    def saga_step(t):
        r = t % R
        api.decode_attn(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, refresh_period=w.refresh_period,
                        step=t, max_l_kv=L, out=out, workspace=ws)

    def steady_step(t):
        r = t % R
        api.decode_attn(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, refresh_period=1 << 30,
                        step=1 + t, max_l_kv=L, out=out, workspace=ws)

    def select_only(t):
        r = t % R
        api.select_gather(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, max_l_kv=L, workspace=ws)

    def combine_only(t):
        r = t % R
        api.split_combine(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, max_l_kv=L, out=out, workspace=ws)

    def refresh_step(t):
        r = t % R
        api.decode_attn(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, refresh_period=1, step=t,
                        max_l_kv=L, out=out, workspace=ws)

    # a refresh reads the threshold passed in as a guess of a window around the new one
    # (a quarter octave either way); alternating q and 4 q (exact in bf16: every logit
    # times 4) on one shared threshold makes every guess miss, the refresh's slowest path
    q4 = [qs[0], qs[0] * 4]
    tau_miss = taus[0].clone()

    def refresh_miss_step(t):
        r = t % R
        api.decode_attn(q4[t % 2], ks[r], vs[r], l_kv, tau_miss, N=w.N, refresh_period=1, step=t,
                        max_l_kv=L, out=out, workspace=ws)

    K, W = args.steps, args.warmup
    n = w.refresh_period
    res = {}
    if args.only in ("all", "saga"):
        for t in range(W):
            saga_step(t)
        torch.cuda.synchronize()
        # K steps that reuse the threshold and K steps that each refresh it
        ms = time_graph(torch, lambda: [steady_step(t) for t in range(W, W + K)], args.reps)
        steady = [1e3 * m / K for m in ms]
        ms = time_graph(torch, lambda: [refresh_step(t) for t in range(W, W + K)], args.reps)
        refresh = [1e3 * m / K for m in ms]
        res["steady_us"] = pct(steady, 50)
        res["refresh_us"] = pct(refresh, 50)
        # amortized step per replay pair: (n - 1) steady steps and one refresh step
        res["saga_us"] = [((n - 1) * a + b) / n for a, b in zip(sorted(steady), sorted(refresh))]
        log(f"steady step (threshold reused): {res['steady_us']:.2f} us/step; refresh step: "
            f"{res['refresh_us']:.2f} us/step; amortized over n={n}: {pct(res['saga_us'], 50):.2f} us/step")
        # cross-check: K consecutive steps from a multiple of n, refreshes at their natural rate
        t0 = -(-W // n) * n
        ms = time_graph(torch, lambda: [saga_step(t) for t in range(t0, t0 + K)], args.reps)
        res["natural_us"] = pct([1e3 * m / K for m in ms], 50)
        res["refresh_steps"] = sum(1 for t in range(t0, t0 + K) if t % n == 0)
        log(f"natural rate: {res['natural_us']:.2f} us/step over {K} steps ({res['refresh_steps']} refresh)")
    if args.only in ("all", "saga", "refresh"):
        Km = min(K, 512)
        ms = time_graph(torch, lambda: [refresh_miss_step(t) for t in range(W, W + Km)], args.reps)
        res["refresh_miss_us"] = pct([1e3 * m / Km for m in ms], 50)
        log(f"refresh step whose guessed window misses: {res['refresh_miss_us']:.2f} us/step")
    if args.only == "steady":
        ms = time_graph(torch, lambda: [steady_step(t) for t in range(W, W + K)], args.reps)
        res["steady_us"] = pct([1e3 * m / K for m in ms], 50)
        log(f"steady step (threshold reused): {res['steady_us']:.2f} us/step")
    if args.only == "refresh":
        ms = time_graph(torch, lambda: [refresh_step(t) for t in range(W, W + K)], args.reps)
        res["refresh_us"] = pct([1e3 * m / K for m in ms], 50)
        log(f"refresh step: {res['refresh_us']:.2f} us/step")
    if args.only in ("all", "select"):
        ms = time_graph(torch, lambda: [select_only(t) for t in range(W, W + K)], args.reps)
        res["select_us"] = pct([1e3 * m / K for m in ms], 50)
        log(f"select kernel alone: {res['select_us']:.2f} us/launch")
        ms = time_graph(torch, lambda: [combine_only(t) for t in range(W, W + K)], args.reps)
        res["combine_us"] = pct([1e3 * m / K for m in ms], 50)
        log(f"combine kernel alone: {res['combine_us']:.2f} us/launch")

    if args.paged and args.only in ("all", "paged"):
        res["paged"] = paged_timing(torch, api, w, qs, ks, vs, taus, l_kv, L, args)

    # survivor statistics at a step that reuses the threshold of set 0
    cap = 8 * w.N
    sel_count = torch.zeros(w.batch, w.h_q, dtype=torch.int32, device=dev)
    sel_idx = torch.full((w.batch, w.h_q, cap), -1, dtype=torch.int32, device=dev)
    flags = torch.zeros(w.batch, w.h_q, dtype=torch.int32, device=dev)
    api.decode_attn(qs[0], ks[0], vs[0], l_kv, taus[0], N=w.N, refresh_period=w.refresh_period,
                    step=1, max_l_kv=L, out=out, sel_count=sel_count, sel_idx=sel_idx, flags=flags, workspace=ws)
    torch.cuda.synchronize()
    counts = sel_count.cpu().numpy()
    idx = sel_idx.cpu().numpy()
    forced = int(((flags.cpu().numpy() & api.FLAG_FORCED) != 0).sum())
    union_rows = []
    for b in range(w.batch):
        for vh in range(w.h_v):
            heads = [j for j in range(w.h_q) if (j * w.h_v) // w.h_q == vh]
            rows = set()
            for j in heads:
                rows.update(idx[b, j, : min(counts[b, j], cap)].tolist())
            union_rows.append(len(rows))
    bytes_v = bytemodel.selected_value_bytes(union_rows, w.dv, es)
    bytes_v_per_head = int(counts.sum()) * w.dv * es
    bytes_step = bytes_k + bytes_v

    dense = {}
    if w.dense_h_kv and args.only in ("all", "dense"):
        wd = w.with_(h_k=w.dense_h_kv, h_v=w.dense_h_kv, workload_id=w.workload_id + 100)
        xd = wl.generate(wd, seed=0, lengths=lens, l_max=L)
        bytes_d = bytemodel.dense_bytes(wd.h_k, wd.d, lens, es)
        Rd = rotating_sets(bytes_d, 1, 0)
        qd = xd.q.to(dev)
        kd = [xd.k.to(dev)]
        vd = [xd.v.to(dev)]
        kd += [kd[0].clone() for _ in range(Rd - 1)]
        vd += [vd[0].clone() for _ in range(Rd - 1)]
        outd = torch.empty_like(qd)
        wsd = api.Workspace(api.make_shape(qd, kd[0], vd[0]), 1, L, dev)

        def dense_step(t):
            r = t % Rd
            api.dense_gqa_attn(qd, kd[r], vd[r], l_kv, max_l_kv=L, out=outd, workspace=wsd)

        for t in range(W):
            dense_step(t)
        torch.cuda.synchronize()
        ms = time_graph(torch, lambda: [dense_step(t) for t in range(W, W + K)], args.reps)
        dense = {"h_kv": wd.h_k, "us": pct([1e3 * m / K for m in ms], 50), "bytes": bytes_d, "sets": Rd}
        log(f"dense GQA (h_kv={wd.h_k}): {dense['us']:.2f} us/step")
        del kd, vd

    if not args.no_layer and args.only in ("all", "layer") and w.dv == w.d and not ragged:
        res["layer"] = layer_timing(torch, api, wl, w, ks, vs, L, args)

    if "paged" in res and "saga_us" in res:
        for p in res["paged"]:
            p["vs_contiguous"] = p["us_per_step"] / pct(res["saga_us"], 50)
    if "saga_us" not in res:
        print(json.dumps({"metric": METRIC, "partial": args.only, **res, "dense": dense}))
        return 0

    ceil = read_probe(torch, 5) if args.only == "all" else None
    if ceil:
        log(f"read ceilings (probe kernel): 1 GiB {ceil['gib_read_gbs']:.0f} GB/s, "
            f"32 MiB {ceil['mib32_read_gbs']:.0f} GB/s")
    us = pct(res["saga_us"], 50)
    t_step = us * 1e-6
    step_gbs = bytes_step / t_step / 1e9
    # the recorded counters are those of the default workload's select kernel
    traffic, traffic_src = recorded_traffic() if w.name == DEFAULT_WORKLOAD else (None, None)
    roof = None
    if "select_us" in res:
        # the late gather's select kernel reads the keys; the early one also the selected value rows
        bytes_sel = bytes_k if form == "late" else bytes_step
        achieved = bytes_sel / (res["select_us"] * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                "kernel": dominant_kernel(w, form),
                "kernel_us": res["select_us"], "bytes_per_launch": bytes_sel,
                "traffic_source": traffic_src}
    line = {
        "metric": METRIC,
        "value": 1.0 / t_step,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": t_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "h_q": w.h_q, "h_k": w.h_k, "h_v": w.h_v,
                   "d": w.d, "d_v": w.dv, "l_kv": L if not ragged else {"min": min(lens), "max": max(lens),
                                                                         "mean": float(np.mean(lens))},
                   "N": w.N, "refresh_period": w.refresh_period,
                   "accumulate": "f32", "rotating_sets": R, "dense_h_kv": w.dense_h_kv},
        "us_per_step": us,
        "us_per_step_p10": pct(res["saga_us"], 10),
        "us_per_step_p90": pct(res["saga_us"], 90),
        "us_steady_step": res.get("steady_us"),
        "us_refresh_step": res.get("refresh_us"),
        "us_refresh_step_guess_missed": res.get("refresh_miss_us"),
        "step_time": "((n-1) * us_steady_step + us_refresh_step) / n, n = refresh_period",
        "us_per_step_natural_rate": res.get("natural_us"),
        "us_select_kernel": res.get("select_us"),
        "us_combine_kernel": res.get("combine_us"),
        "value_gather": form,
        "bytes_per_step": bytes_step,
        "bytes_k": bytes_k,
        "bytes_selected_v_union": bytes_v,
        "bytes_selected_v_per_query_head": bytes_v_per_head,
        "step_gbs": step_gbs,
        "step_roofline_frac": step_gbs / HBM_PEAK_GBS,
        "refresh_steps_timed_natural_rate": res["refresh_steps"],
        "survivors_mean": float(counts.mean()),
        "survivors_max": int(counts.max()),
        "forced_refresh_rows": forced,
        "read_ceiling": ceil,
        "paged": res.get("paged"),
        "layer": res.get("layer"),
        "roofline": roof,
    }
    if dense:
        td = dense["us"] * 1e-6
        line["dense_gqa"] = {"h_kv": dense["h_kv"], "us_per_step": dense["us"], "steps_per_s": 1.0 / td,
                             "bytes_per_step": dense["bytes"], "gbs": dense["bytes"] / td / 1e9,
                             "roofline_frac": dense["bytes"] / td / 1e9 / HBM_PEAK_GBS,
                             "rotating_sets": dense["sets"]}
        line["speedup_vs_dense"] = td / t_step
        if line["layer"] and "speedup" in line["layer"]:
            line["layer"]["attention_only_speedup"] = td / t_step
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
