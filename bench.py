#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X: SAGA + Atop-N vs the dense GQA kernel.

One step = one saga_decode_attn call (one layer, one decode token) on the
Qwen2.5-1.5B-shaped workload at 128K context, batch 1 (h_q=12, h_k=1, h_v=4, d=128,
N=512, exact threshold every 32 steps), bf16 inputs, seeded synthetic data. Refresh
steps occur at their natural rate (one in refresh_period) inside the timed region.

Inputs are resident in HBM before timing. R rotating copies of q/K/V/tau (R*bytes(K)
>= 1 GiB, R coprime with the refresh period) keep the 256 MB Infinity Cache from
serving repeated reads, as a model's per-layer caches would. The K timed steps are
replayed from a HIP graph and timed with HIP events on the launch stream.

Prints one JSON line. `value` = SAGA decode steps/s; `roofline` is for the dominant
kernel (the fused steady-step kernel, timed alone the same way: a step that reuses
the threshold is exactly one launch of it); `cpu_baseline` is the CPU oracle timed on
this host on the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn steps/s + % HBM roofline at l_kv=128K, bs=1 (SAGA+Atop-N vs dense GQA)"
HBM_PEAK_GBS = 8000.0


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
    replays bracketed by device synchronisation. Returns the per-replay ms list."""
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


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def cpu_baseline(w, x, seconds: float):
    """The oracle as it stands, on the same inputs, for about `seconds` of host time."""
    import numpy as np
    from threadpoolctl import threadpool_info
    from oracle import saga_oracle as orc

    q64, k64, v64 = x.f64()
    tau = None
    steps = 0
    t0 = time.perf_counter()
    while True:
        r = orc.saga_decode_step(q64, k64, v64, x.l_kv, w.N, w.refresh_period, steps, tau_in=tau,
                                 keep_logits=False)
        tau = r.tau
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": steps / el, "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{steps} consecutive oracle decode steps (steps 0..{steps - 1}, exact threshold at "
                      f"step % {w.refresh_period} == 0) of the full {w.name} workload, {el:.1f} s of host time; "
                      f"float64 numpy, BLAS threads = cores"}


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


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--reps", type=int, default=5, help="timed graph replays (median reported)")
    ap.add_argument("--workload", default="qwen2.5-1.5b-shape-l128k")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: >= 1 GiB of K)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "saga", "dense", "steady"], default="all",
                    help="time only one part (for profiler runs)")
    ap.add_argument("--probe", choices=["none", "copy"], default="none",
                    help="copy: time a plain device copy of 256 MiB (counter calibration, streaming ceiling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the decode step runs on a single MI355X; "
              "multi-GPU runs are not part of this library.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    if args.probe == "copy":
        return copy_probe(torch, max(args.steps, 8))

    from sparse_decode_attention_saga_amd import api
    from sparse_decode_attention_saga_amd import bytemodel
    from sparse_decode_attention_saga_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    api.lib()
    L = w.l_kv
    es = 2 if w.dtype == "bf16" else 4
    bytes_k = bytemodel.key_bytes(w.h_k, w.d, [L] * w.batch, es)
    R = rotating_sets(bytes_k, w.refresh_period, args.sets)
    log(f"workload {w.name}: B={w.batch} h_q={w.h_q} h_k={w.h_k} h_v={w.h_v} d={w.d} l_kv={L} "
        f"N={w.N} n={w.refresh_period}; {R} rotating sets")

    t0 = time.perf_counter()
    x = wl.generate(w, seed=0)
    log(f"generated inputs in {time.perf_counter() - t0:.1f} s")
    q0, k0, v0 = x.q.to(dev), x.k.to(dev), x.v.to(dev)
    l_kv = torch.from_numpy(x.l_kv).to(dev)
    qs = [q0] + [q0.clone() for _ in range(R - 1)]
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    taus = [torch.zeros(w.batch, w.h_q, dtype=torch.float32, device=dev) for _ in range(R)]
    out = torch.empty(w.batch, w.h_q, w.d, dtype=q0.dtype, device=dev)
    shape = api.make_shape(q0, k0, v0)
    ws = api.Workspace(shape, w.N, L, dev)
    for r in range(R):
        api.refresh_threshold(qs[r], ks[r], l_kv, taus[r], N=w.N, max_l_kv=L, workspace=ws)
    torch.cuda.synchronize()

    def saga_step(t):
        r = t % R
        api.decode_attn(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, refresh_period=w.refresh_period,
                        step=t, max_l_kv=L, out=out, workspace=ws)

    def steady_step(t):
        # a step that reuses the threshold: exactly one launch of the fused kernel
        r = t % R
        api.decode_attn(qs[r], ks[r], vs[r], l_kv, taus[r], N=w.N, refresh_period=1 << 30,
                        step=1 + t, max_l_kv=L, out=out, workspace=ws)

    K, W = args.steps, args.warmup
    res = {}
    if args.only in ("all", "saga"):
        for t in range(W):
            saga_step(t)
        torch.cuda.synchronize()
        ms = time_graph(torch, lambda: [saga_step(t) for t in range(W, W + K)], args.reps)
        res["saga_ms"] = median(ms)
        res["saga_ms_all"] = ms
        res["refresh_steps"] = sum(1 for t in range(W, W + K) if t % w.refresh_period == 0)
        log(f"saga: {1e3 * res['saga_ms'] / K:.2f} us/step over {K} steps ({res['refresh_steps']} refresh)")
    if args.only in ("all", "steady"):
        ms = time_graph(torch, lambda: [steady_step(t) for t in range(W, W + K)], args.reps)
        res["steady_ms"] = median(ms)
        log(f"fused steady-step kernel: {1e3 * res['steady_ms'] / K:.2f} us/launch")

    # survivor statistics at a stale step of set 0 (union of kept rows per value head)
    cap = 8 * w.N
    sel_count = torch.zeros(w.batch, w.h_q, dtype=torch.int32, device=dev)
    sel_idx = torch.full((w.batch, w.h_q, cap), -1, dtype=torch.int32, device=dev)
    api.decode_attn(qs[0], ks[0], vs[0], l_kv, taus[0], N=w.N, refresh_period=w.refresh_period,
                    step=1, max_l_kv=L, out=out, sel_count=sel_count, sel_idx=sel_idx, workspace=ws)
    torch.cuda.synchronize()
    counts = sel_count.cpu().numpy()
    idx = sel_idx.cpu().numpy()
    union_rows = []
    for b in range(w.batch):
        for vh in range(w.h_v):
            heads = [j for j in range(w.h_q) if (j * w.h_v) // w.h_q == vh]
            rows = set()
            for j in heads:
                rows.update(idx[b, j, : min(counts[b, j], cap)].tolist())
            union_rows.append(len(rows))
    bytes_v = bytemodel.selected_value_bytes(union_rows, w.d, es)
    bytes_v_per_head = int(counts.sum()) * w.d * es

    dense = {}
    if w.dense_h_kv and args.only in ("all", "dense"):
        wd = w.with_(h_k=w.dense_h_kv, h_v=w.dense_h_kv, workload_id=w.workload_id + 100)
        xd = wl.generate(wd, seed=0)
        bytes_d = bytemodel.dense_bytes(wd.h_k, wd.d, [L] * wd.batch, es)
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
        dense = {"h_kv": wd.h_k, "ms": median(ms), "bytes": bytes_d, "sets": Rd}
        log(f"dense GQA (h_kv={wd.h_k}): {1e3 * dense['ms'] / K:.2f} us/step")
        del kd, vd

    if "saga_ms" not in res:
        print(json.dumps({"metric": METRIC, "partial": args.only, "steady_ms": res.get("steady_ms"),
                          "dense": dense}))
        return 0

    t_step = res["saga_ms"] / K * 1e-3
    bytes_step = bytes_k + bytes_v
    step_gbs = bytes_step / t_step / 1e9
    st_s = res["steady_ms"] / K * 1e-3 if "steady_ms" in res else None
    achieved = bytes_step / st_s / 1e9 if st_s else None
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
                   "d": w.d, "l_kv": L, "N": w.N, "refresh_period": w.refresh_period,
                   "accumulate": "f32", "rotating_sets": R, "dense_h_kv": w.dense_h_kv},
        "us_per_step": t_step * 1e6,
        "bytes_per_step": bytes_step,
        "bytes_k": bytes_k,
        "bytes_selected_v_union": bytes_v,
        "bytes_selected_v_per_query_head": bytes_v_per_head,
        "step_gbs": step_gbs,
        "step_roofline_frac": step_gbs / HBM_PEAK_GBS,
        "refresh_steps_timed": res["refresh_steps"],
        "survivors_mean": float(counts.mean()),
        "survivors_max": int(counts.max()),
        "saga_ms_replays": res["saga_ms_all"],
        "roofline": {"kernel": "k_decode_fused (steady step: K stream, compare, V gather, merge)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None, "traffic": None,
                     "kernel_us": st_s * 1e6 if st_s else None, "bytes_per_launch": bytes_step},
    }
    if dense:
        td = dense["ms"] / K * 1e-3
        line["dense_gqa"] = {"h_kv": dense["h_kv"], "us_per_step": td * 1e6, "steps_per_s": 1.0 / td,
                             "bytes_per_step": dense["bytes"], "gbs": dense["bytes"] / td / 1e9,
                             "roofline_frac": dense["bytes"] / td / 1e9 / HBM_PEAK_GBS,
                             "rotating_sets": dense["sets"]}
        line["speedup_vs_dense"] = td / t_step
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
